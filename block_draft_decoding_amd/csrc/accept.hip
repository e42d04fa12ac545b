// Block acceptance: the schema validator for primitives (VFlash paper §2.5)
// and greedy longest-prefix verification for text (VFlash paper §2.1; blog
// "Method").  One wavefront per batch row; decisions are exact integer work.
#include <climits>

#include "../../include/fpd.h"
#include "kernels.h"

namespace fpd {
namespace {

__device__ __forceinline__ bool in_set(const int32_t* ids, int n, int t) {
  int lo = 0, hi = n;  // ascending ids: binary search
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (ids[mid] < t)
      lo = mid + 1;
    else
      hi = mid;
  }
  return lo < n && ids[lo] == t;
}

__device__ __forceinline__ int wave_min(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o));
  return v;
}

__global__ __launch_bounds__(64) void validate_kernel(ValidateArgs a) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const int P = a.L - 1;
  const int32_t* tok = a.tokens + (size_t)b * P;
  int first = INT_MAX;
  for (int p0 = 1; p0 < a.L; p0 += 64) {
    const int p = p0 + lane;
    if (p >= a.L) break;
    const int t = tok[p - 1];
    const int s = a.pos_set[p];
    bool ok;
    if (s == -1)
      ok = t >= 0 && t < a.vocab;
    else
      ok = in_set(a.set_ids + a.set_offsets[s], a.set_offsets[s + 1] - a.set_offsets[s], t);
    if (!ok) first = min(first, p - 1);
    const int q = a.partner[p];
    if (q >= 0 && ((t == a.off_id) != (tok[q - 1] == a.off_id))) first = min(first, p - 1);
    const int w = a.field_w[p];
    if (w > 0) {  // FILL^j DIGIT^(w-j), j <= w-1
      bool digits = false;
      for (int i = 0; i < w; ++i) {
        const int ti = tok[p - 1 + i];
        const bool is_digit = ti >= a.digit0_id && ti < a.digit0_id + 10;
        if (is_digit) {
          digits = true;
          continue;
        }
        if (ti == a.fill_id && !digits && i < w - 1) continue;
        first = min(first, p - 1 + i);
        break;
      }
    }
  }
  first = wave_min(first);
  if (lane == 0) {
    a.first_out[b] = first == INT_MAX ? -1 : first;
    a.k_out[b] = first == INT_MAX ? P : 0;
  }
}

__global__ __launch_bounds__(64) void verify_kernel(const int32_t* __restrict__ draft,
                                                    const int32_t* __restrict__ target, int L,
                                                    int32_t* __restrict__ k_out, int32_t* __restrict__ next_out) {
  const int b = blockIdx.x, lane = threadIdx.x;
  const int P = L - 1;
  int k = P;
  for (int i0 = 0; i0 < P; i0 += 64) {
    const int i = i0 + lane;
    const bool miss = i < P && draft[(size_t)b * P + i] != target[(size_t)b * L + i];
    const unsigned long long mask = __ballot(miss);
    if (mask) {
      k = i0 + __ffsll((long long)mask) - 1;
      break;
    }
  }
  if (lane == 0) {
    k_out[b] = k;
    next_out[b] = target[(size_t)b * L + k];
  }
}

}  // namespace

hipError_t validate_primitive(const ValidateArgs& a, hipStream_t st) {
  ProfScope prof("validate", st);
  if (a.B == 0) return hipSuccess;
  hipLaunchKernelGGL(validate_kernel, dim3(a.B), dim3(64), 0, st, a);
  return hipGetLastError();
}

hipError_t verify_prefix(const int32_t* draft, const int32_t* target, int B, int L, int32_t* k_out,
                         int32_t* next_out, hipStream_t st) {
  ProfScope prof("verify", st);
  if (B == 0) return hipSuccess;
  hipLaunchKernelGGL(verify_kernel, dim3(B), dim3(64), 0, st, draft, target, L, k_out, next_out);
  return hipGetLastError();
}

}  // namespace fpd
