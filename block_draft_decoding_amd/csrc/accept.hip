// Block acceptance: the schema validator for primitives (VFlash paper §2.5)
// and greedy longest-prefix verification for text (VFlash paper §2.1; blog
// "Method").  The validator (and box acceptance) runs one workgroup per
// request, verification one wavefront per row; decisions are exact integer
// work.
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

// One workgroup per batch row, one thread per position.  The row's tokens
// and (when they fit) the legal-id sets are staged in LDS first, so every
// position's checks (set membership by binary search, the paired-position
// rule, the digit-field automaton) run in parallel on LDS data and the row's
// answer is a workgroup minimum over the first failing positions.
constexpr int kValThreads = 512;

// Copies n ints to LDS, eight loads in flight per thread (a legal-id table of
// ~5,000 ids would otherwise take one memory round trip per 512 ids).
__device__ __forceinline__ void stage_to_lds(const int32_t* __restrict__ src, int n, int32_t* dst) {
  for (int i0 = threadIdx.x; i0 < n; i0 += 8 * kValThreads) {
    int32_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * kValThreads;
      v[u] = src[min(i, n - 1)];  // clamped, so every load is unconditional
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * kValThreads;
      if (i < n) dst[i] = v[u];
    }
  }
}

__global__ __launch_bounds__(kValThreads) void validate_kernel(ValidateArgs a, int stage_tok, int stage_ids) {
  extern __shared__ int32_t sm[];
  __shared__ int red[2][kValThreads / 64];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int P = a.L - 1;
  const int32_t* gtok = a.tokens + (size_t)b * P;
  const int32_t* tok = gtok;
  const int32_t* ids = a.set_ids;
  if (stage_tok) {
    stage_to_lds(gtok, P, sm);
    tok = sm;
  }
  if (stage_ids) {
    int32_t* sid = sm + (stage_tok ? P : 0);
    stage_to_lds(a.set_ids, a.n_set_ids, sid);
    ids = sid;
  }
  __syncthreads();
  int first = INT_MAX, unc = INT_MAX;
  for (int p = tid + 1; p < a.L; p += kValThreads) {
    // the position's layout entries in one batch of loads (each loaded where
    // it is used, they made a chain of dependent memory round trips)
    const int s = a.pos_set[p], q = a.partner[p], w = a.field_w[p];
    const bool uncertain = a.conf && a.coord[p] && !(a.conf[(size_t)b * P + p - 1] >= a.tau);
    const int t = tok[p - 1];
    // a coordinate is certain only if its confidence reaches tau (NaN fails)
    if (uncertain) unc = min(unc, p - 1);
    bool ok;
    if (s == -1)
      ok = t >= 0 && t < a.vocab;
    else
      ok = in_set(ids + a.set_offsets[s], a.set_offsets[s + 1] - a.set_offsets[s], t);
    if (!ok) first = min(first, p - 1);
    if (q >= 0 && ((t == a.off_id) != (tok[q - 1] == a.off_id))) first = min(first, p - 1);
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
  unc = wave_min(unc);
  if ((tid & 63) == 0) {
    red[0][tid >> 6] = first;
    red[1][tid >> 6] = unc;
  }
  __syncthreads();
  if (tid == 0) {
    int f = red[0][0], u = red[1][0];
#pragma unroll
    for (int i = 1; i < kValThreads / 64; ++i) {
      f = min(f, red[0][i]);
      u = min(u, red[1][i]);
    }
    a.first_out[b] = f == INT_MAX ? -1 : f;
    if (a.conf) {  // keep the drafts before the first failure of either kind
      a.uncertain_out[b] = u == INT_MAX ? -1 : u;
      const int k = min(f, u);
      a.k_out[b] = k == INT_MAX ? P : k;
    } else {
      a.k_out[b] = f == INT_MAX ? P : 0;
    }
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
  constexpr size_t kMaxLds = 64 * 1024;
  const size_t tok_bytes = (size_t)(a.L - 1) * 4, id_bytes = (size_t)a.n_set_ids * 4;
  const int stage_tok = tok_bytes <= kMaxLds;
  const int stage_ids = (stage_tok ? tok_bytes : 0) + id_bytes <= kMaxLds;
  const size_t lds = (stage_tok ? tok_bytes : 0) + (stage_ids ? id_bytes : 0);
  hipLaunchKernelGGL(validate_kernel, dim3(a.B), dim3(kValThreads), lds, st, a, stage_tok, stage_ids);
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
