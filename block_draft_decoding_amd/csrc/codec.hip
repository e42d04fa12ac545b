// Coordinate codec (VFlash paper §2.3 "Token representation"; §3.1 "Base
// VLM"): a coordinate occupies one of 1,001 special tokens -- 2D image
// coordinates normalised to 0..1000, 3D coordinates quantised uniformly over
// a predefined range -- and point-motion numbers are fixed-width fields of a
// sign and five digits whose unused high digits hold a fill token.  One
// thread per value or field; the bin arithmetic runs in double precision so
// that every token is decided exactly as the float64 definition decides it.
#include "../../include/fpd.h"
#include "kernels.h"

namespace fpd {
namespace {

constexpr int kBins = 1001;

__global__ __launch_bounds__(256) void coords_to_tokens_kernel(const float* __restrict__ x, int n, double lo,
                                                               double scale, int base, int32_t* __restrict__ out) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const double v = (double)x[i];
  if (v != v) {
    out[i] = -1;
    return;
  }
  const double b = fmin(fmax(rint((v - lo) * scale), 0.0), (double)(kBins - 1));  // ties to even
  out[i] = base + (int)b;
}

__global__ __launch_bounds__(256) void tokens_to_coords_kernel(const int32_t* __restrict__ t, int n, double lo,
                                                               double width, int base, double* __restrict__ out) {
  // product and sum rounded separately, as the float64 definition computes
  // them: no contraction into a fused multiply-add here
#pragma clang fp contract(off)
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int k = t[i] - base;
  out[i] = (k >= 0 && k < kBins) ? lo + (double)k * width : __builtin_nan("");
}

__global__ __launch_bounds__(256) void ints_to_fields_kernel(const int32_t* __restrict__ v, int n, int plus_id,
                                                             int minus_id, int digit0_id, int fill_id,
                                                             int32_t* __restrict__ out) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  int32_t* f = out + (size_t)i * 6;
  const long long x = v[i];
  const long long a = x < 0 ? -x : x;
  if (a > 99999) {
#pragma unroll
    for (int j = 0; j < 6; ++j) f[j] = -1;
    return;
  }
  f[0] = x < 0 ? minus_id : plus_id;
  long long p10 = 10000;
#pragma unroll
  for (int j = 0; j < 5; ++j, p10 /= 10) {
    const int d = (int)((a / p10) % 10);
    f[1 + j] = (a < p10 && j < 4) ? fill_id : digit0_id + d;  // leading zeros become FILL
  }
}

__global__ __launch_bounds__(256) void fields_to_ints_kernel(const int32_t* __restrict__ fields, int n, int plus_id,
                                                             int minus_id, int digit0_id, int fill_id,
                                                             int32_t* __restrict__ vals, int32_t* __restrict__ ok) {
  const int i = blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int32_t* f = fields + (size_t)i * 6;
  const int sgn = f[0];
  bool good = sgn == plus_id || sgn == minus_id;
  bool in_digits = false;
  int a = 0;
#pragma unroll
  for (int j = 0; j < 5; ++j) {  // FILL^k DIGIT^(5-k), k <= 4
    const int t = f[1 + j];
    if (t >= digit0_id && t < digit0_id + 10) {
      in_digits = true;
      a = a * 10 + (t - digit0_id);
    } else if (!(t == fill_id && !in_digits && j < 4)) {
      good = false;
    }
  }
  vals[i] = good ? (sgn == minus_id ? -a : a) : 0;
  ok[i] = good ? 1 : 0;
}

unsigned blocks(int n) { return (unsigned)((n + 255) / 256); }

}  // namespace

hipError_t coords_to_tokens(const float* x, int n, double lo, double hi, int base, int32_t* out, hipStream_t st) {
  ProfScope prof("codec", st);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(coords_to_tokens_kernel, dim3(blocks(n)), dim3(256), 0, st, x, n, lo, (kBins - 1) / (hi - lo),
                     base, out);
  return hipGetLastError();
}

hipError_t tokens_to_coords(const int32_t* t, int n, double lo, double hi, int base, double* out, hipStream_t st) {
  ProfScope prof("codec", st);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(tokens_to_coords_kernel, dim3(blocks(n)), dim3(256), 0, st, t, n, lo, (hi - lo) / (kBins - 1),
                     base, out);
  return hipGetLastError();
}

hipError_t ints_to_fields(const int32_t* v, int n, int plus_id, int minus_id, int digit0_id, int fill_id,
                          int32_t* out, hipStream_t st) {
  ProfScope prof("codec", st);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(ints_to_fields_kernel, dim3(blocks(n)), dim3(256), 0, st, v, n, plus_id, minus_id, digit0_id,
                     fill_id, out);
  return hipGetLastError();
}

hipError_t fields_to_ints(const int32_t* f, int n, int plus_id, int minus_id, int digit0_id, int fill_id,
                          int32_t* vals, int32_t* ok, hipStream_t st) {
  ProfScope prof("codec", st);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(fields_to_ints_kernel, dim3(blocks(n)), dim3(256), 0, st, f, n, plus_id, minus_id, digit0_id,
                     fill_id, vals, ok);
  return hipGetLastError();
}

}  // namespace fpd
