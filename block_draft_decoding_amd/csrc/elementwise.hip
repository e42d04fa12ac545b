// Row-wise kernels of the drafter: embedding gather, RMSNorm, feature
// concatenation, LM-head row gather.
#include <algorithm>

#include "../../include/fpd.h"
#include "kernels.h"

#include <type_traits>

namespace fpd {
namespace {

// h[m] = E[tok[m]]; an id outside [0, V) embeds as a zero row (never read out of bounds).
template <class T>
__global__ __launch_bounds__(256) void embed_kernel(const int32_t* __restrict__ tok, int M,
                                                    const T* __restrict__ E, int H, int V, float* __restrict__ h) {
  const int m = blockIdx.x;
  const int t = tok[m];
  float* dst = h + (size_t)m * H;
  if (t < 0 || t >= V) {
    for (int k = threadIdx.x; k < H; k += blockDim.x) dst[k] = 0.f;
    return;
  }
  const T* src = E + (size_t)t * H;
  for (int k = threadIdx.x; k < H; k += blockDim.x) dst[k] = Elem<T>::ld(src + k);
}

// Sum of a value over the 256 threads of a workgroup (every thread gets it).
__device__ __forceinline__ float block_sum256(float v, float* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  return red[0] + red[1] + red[2] + red[3];
}

// stores 4 normalised values x * inv * g at dst[0..3] (bf16: one 8-byte store)
template <class T>
__device__ __forceinline__ void store_norm4(T* dst, f32x4_t v, float inv, const T* g);
template <>
__device__ __forceinline__ void store_norm4<bf16_t>(bf16_t* dst, f32x4_t v, float inv, const bf16_t* g) {
  const u32x2_t gw = *(const u32x2_t*)g;
  u32x2_t w;
  w[0] = pack_bf16x2(v[0] * inv * __uint_as_float(gw[0] << 16), v[1] * inv * __uint_as_float(gw[0] & 0xffff0000u));
  w[1] = pack_bf16x2(v[2] * inv * __uint_as_float(gw[1] << 16), v[3] * inv * __uint_as_float(gw[1] & 0xffff0000u));
  *(u32x2_t*)dst = w;
}
template <>
__device__ __forceinline__ void store_norm4<float>(float* dst, f32x4_t v, float inv, const float* g) {
  const f32x4_t gg = *(const f32x4_t*)g;
  *(f32x4_t*)dst = v * inv * gg;
}

// The same with the 4 weights loaded beforehand (so that their load can go
// out with the row's other loads).
template <class T>
struct Gamma4;
template <>
struct Gamma4<bf16_t> {
  u32x2_t w;
  __device__ void load(const bf16_t* g) { w = *(const u32x2_t*)g; }
  __device__ void store(bf16_t* dst, f32x4_t v, float inv) const {
    u32x2_t o;
    o[0] = pack_bf16x2(v[0] * inv * __uint_as_float(w[0] << 16), v[1] * inv * __uint_as_float(w[0] & 0xffff0000u));
    o[1] = pack_bf16x2(v[2] * inv * __uint_as_float(w[1] << 16), v[3] * inv * __uint_as_float(w[1] & 0xffff0000u));
    *(u32x2_t*)dst = o;
  }
};
template <>
struct Gamma4<float> {
  f32x4_t w;
  __device__ void load(const float* g) { w = *(const f32x4_t*)g; }
  __device__ void store(float* dst, f32x4_t v, float inv) const { *(f32x4_t*)dst = v * inv * w; }
};

// One wavefront per output row (4 rows per workgroup), float4 loads:
// y = x / sqrt(mean(x^2) + eps) * g.  H is a multiple of 64.
template <class T>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const float* __restrict__ x, int H, int rows, int per,
                                                      int in_stride, int in_off, const T* __restrict__ g,
                                                      float eps, T* __restrict__ y) {
  const int r = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (r >= rows) return;
  const int lane = threadIdx.x & 63;
  const f32x4_t* src = (const f32x4_t*)(x + ((size_t)(r / per) * in_stride + in_off + r % per) * H);
  const int n4 = H / 4;
  // the row (H <= 4096: at most 16 float4 per lane) and its norm weights are
  // loaded once, all before the first use, and kept in registers for the
  // normalised store (a loop of load-and-wait steps over the row, read twice,
  // cost 20 memory round trips per row at H = 2560)
  constexpr int MAXI = 16;
  f32x4_t v[MAXI];
  Gamma4<T> gw[MAXI];
#pragma unroll
  for (int i = 0; i < MAXI; ++i) {
    const int k = lane + i * 64;
    if (k < n4) {
      v[i] = src[k];
      gw[i].load(g + 4 * k);
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), as the builtin so the compiler's own tracking sees it
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < MAXI; ++i)
    if (lane + i * 64 < n4) ss += v[i][0] * v[i][0] + v[i][1] * v[i][1] + v[i][2] * v[i][2] + v[i][3] * v[i][3];
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  const float inv = 1.0f / sqrtf(ss / (float)H + eps);
  T* dst = y + (size_t)r * H;
#pragma unroll
  for (int i = 0; i < MAXI; ++i) {
    const int k = lane + i * 64;
    if (k < n4) gw[i].store(dst + 4 * k, v[i], inv);
  }
}

// Fused residual update and RMSNorm, one workgroup per row: h[r] +=
// sum_s partial[s][r] (split-K partial products, fixed split order; none when
// partial is null), then out[row'] = RMSNorm(h[r]) * g.  With final_L > 0 only
// rows r = b*L + l with l >= 1 produce output, at row b*(L-1) + l - 1 (the
// drafter's final norm over the masked positions).  H is a multiple of 64
// and at most 4096 (the row stays in registers: 4 float4 per thread).
// Exactly NS (1..8) split-K partials, all loads issued before the sums (a
// runtime-length loop would serialise one memory round trip per split).
template <class T, int NS>
__global__ __launch_bounds__(256) void resid_norm_kernel(const float* __restrict__ partial, int splits, int M, int H,
                                                         float* __restrict__ h, const T* __restrict__ g, float eps,
                                                         T* __restrict__ out, int final_L) {
  __shared__ float red[4];
  const int r = blockIdx.x;
  int orow = r;
  if (final_L > 0) {
    const int l = r % final_L;
    if (l == 0) return;
    orow = (r / final_L) * (final_L - 1) + l - 1;
  }
  f32x4_t* hr = (f32x4_t*)(h + (size_t)r * H);
  const int n4 = H / 4;
  const size_t pstride = (size_t)M * H / 4;
  const f32x4_t* pr = partial ? (const f32x4_t*)partial + (size_t)r * n4 : nullptr;
  // Every load of the row (residual, partials, norm weights) goes out before
  // the first use, and one tracked wait covers them all: one memory round
  // trip, where loading and storing each float4 group in turn cost one per
  // group (and the compiler's own waits then also waited for the stores).
  f32x4_t v[4], parts[4][NS];
  Gamma4<T> gw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int k = threadIdx.x + i * 256;
    if (k < n4) {
      v[i] = hr[k];
      gw[i].load(g + 4 * k);
      if (pr) {
#pragma unroll
        for (int s = 0; s < NS; ++s) parts[i][s] = pr[s * pstride + k];
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), as the builtin so the compiler's own tracking sees it
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int k = threadIdx.x + i * 256;
    if (k < n4) {
      f32x4_t x = v[i];
      if (pr) {
        f32x4_t acc = parts[i][0];
#pragma unroll
        for (int s = 1; s < NS; ++s) acc += parts[i][s];
        x += acc;
        hr[k] = x;
      }
      v[i] = x;
      ss += x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
    }
  }
  const float inv = 1.0f / sqrtf(block_sum256(ss, red) / (float)H + eps);
  T* dst = out + (size_t)orow * H;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int k = threadIdx.x + i * 256;
    if (k < n4) gw[i].store(dst + 4 * k, v[i], inv);
  }
}

// The same for more than 8 split-K partials (small M, where the GEMM splits
// K 16-32 ways): four groups of 256 threads each sum every fourth partial of
// the whole row (loads in batches of 8), the group sums meet in LDS in fixed
// order, and group 0 finishes the row as above.  A single group would make
// ~12 dependent memory round trips per row.
template <class T>
__global__ __launch_bounds__(1024) void resid_norm_many_kernel(const float* __restrict__ partial, int splits, int M,
                                                               int H, float* __restrict__ h, const T* __restrict__ g,
                                                               float eps, T* __restrict__ out, int final_L) {
  __shared__ f32x4_t sums[3][1024];
  __shared__ float red[16];
  const int r = blockIdx.x;
  int orow = r;
  if (final_L > 0) {
    const int l = r % final_L;
    if (l == 0) return;
    orow = (r / final_L) * (final_L - 1) + l - 1;
  }
  const int grp = threadIdx.x >> 8, t = threadIdx.x & 255;
  f32x4_t* hr = (f32x4_t*)(h + (size_t)r * H);
  const int n4 = H / 4;
  const size_t pstride = (size_t)M * H / 4;
  const f32x4_t* pr = (const f32x4_t*)partial + (size_t)r * n4;
  f32x4_t acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int k = t + i * 256;
    acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (k >= n4) continue;
    for (int s0 = grp; s0 < splits; s0 += 32) {  // splits s0, s0 + 4, ..., s0 + 28
      f32x4_t parts[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        parts[j] = s0 + 4 * j < splits ? pr[(size_t)(s0 + 4 * j) * pstride + k] : f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[i] += parts[j];
    }
    if (grp > 0) sums[grp - 1][k] = acc[i];
  }
  __syncthreads();
  f32x4_t v[4];
  float ss = 0.f;
  if (grp == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int k = t + i * 256;
      if (k >= n4) continue;
      f32x4_t x = hr[k];
      x += ((acc[i] + sums[0][k]) + sums[1][k]) + sums[2][k];
      hr[k] = x;
      v[i] = x;
      ss += x[0] * x[0] + x[1] * x[1] + x[2] * x[2] + x[3] * x[3];
    }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
  if (grp != 0) return;
  const float inv = 1.0f / sqrtf((red[0] + red[1] + red[2] + red[3]) / (float)H + eps);
  T* dst = out + (size_t)orow * H;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int k = t + i * 256;
    if (k < n4) store_norm4<T>(dst + 4 * k, v[i], inv, g + 4 * k);
  }
}

// h[m] = E[tok[m]] (ids outside [0, V) embed as zero rows), a[m] = RMSNorm(h[m]) * g;
// one workgroup per row, 4 elements per thread and step.
template <class T>
__global__ __launch_bounds__(256) void embed_norm_kernel(const int32_t* __restrict__ tok, const T* __restrict__ E, int H,
                                                         int V, float* __restrict__ h, const T* __restrict__ g,
                                                         float eps, T* __restrict__ a) {
  __shared__ float red[4];
  const int r = blockIdx.x;
  const int t = tok[r];
  const bool ok = t >= 0 && t < V;
  f32x4_t* hr = (f32x4_t*)(h + (size_t)r * H);
  const int n4 = H / 4;
  // all of the row's loads first, one tracked wait (as in resid_norm_kernel)
  f32x4_t v[4];
  Gamma4<T> gw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int k = threadIdx.x + i * 256;
    if (k < n4) {
      f32x4_t x = {0.f, 0.f, 0.f, 0.f};
      if (ok) {
        const T* src = E + (size_t)t * H + 4 * k;
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = Elem<T>::ld(src + e);
      }
      v[i] = x;
      gw[i].load(g + 4 * k);
    }
  }
  __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0), as the builtin so the compiler's own tracking sees it
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int k = threadIdx.x + i * 256;
    if (k < n4) {
      hr[k] = v[i];
      ss += v[i][0] * v[i][0] + v[i][1] * v[i][1] + v[i][2] * v[i][2] + v[i][3] * v[i][3];
    }
  }
  const float inv = 1.0f / sqrtf(block_sum256(ss, red) / (float)H + eps);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int k = threadIdx.x + i * 256;
    if (k < n4) gw[i].store(a + (size_t)r * H + 4 * k, v[i], inv);
  }
}

// X[b*C + c, t*H + k] = feats[b, t, c, k], copied in 16-byte chunks.
__global__ __launch_bounds__(256) void concat_kernel(const u32x4_t* __restrict__ f, int B, int nt, int C,
                                                     int Hc, u32x4_t* __restrict__ X) {
  const size_t n = (size_t)B * nt * C * Hc;
  for (size_t e = (size_t)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (size_t)gridDim.x * blockDim.x) {
    const int kc = (int)(e % Hc);
    size_t r = e / Hc;
    const int c = (int)(r % C);
    r /= C;
    const int t = (int)(r % nt);
    const int b = (int)(r / nt);
    X[(((size_t)b * C + c) * nt + t) * Hc + kc] = f[e];
  }
}

__global__ __launch_bounds__(256) void gather_rows_kernel(const u32x4_t* __restrict__ W, int Hc,
                                                          const int32_t* __restrict__ ids, int n,
                                                          u32x4_t* __restrict__ out) {
  const int i = blockIdx.x;
  if (i >= n) return;
  const u32x4_t* src = W + (size_t)ids[i] * Hc;
  for (int k = threadIdx.x; k < Hc; k += blockDim.x) out[(size_t)i * Hc + k] = src[k];
}

}  // namespace

hipError_t embed_gather(int dt, const int32_t* tokens, int M, const void* E, int H, int V, float* h,
                        hipStream_t st) {
  ProfScope prof("embed", st);
  if (M == 0) return hipSuccess;
  if (dt == FPD_DTYPE_BF16)
    hipLaunchKernelGGL(embed_kernel<bf16_t>, dim3(M), dim3(256), 0, st, tokens, M, (const bf16_t*)E, H, V, h);
  else
    hipLaunchKernelGGL(embed_kernel<float>, dim3(M), dim3(256), 0, st, tokens, M, (const float*)E, H, V, h);
  return hipGetLastError();
}

hipError_t rmsnorm_rows(int dt, const float* x, int H, int rows, int per, int in_stride, int in_off,
                        const void* g, float eps, void* y, hipStream_t st) {
  ProfScope prof("rmsnorm", st);
  if (rows == 0) return hipSuccess;
  const unsigned grid = (unsigned)((rows + 3) / 4);
  if (dt == FPD_DTYPE_BF16)
    hipLaunchKernelGGL(rmsnorm_kernel<bf16_t>, dim3(grid), dim3(256), 0, st, x, H, rows, per, in_stride, in_off,
                       (const bf16_t*)g, eps, (bf16_t*)y);
  else
    hipLaunchKernelGGL(rmsnorm_kernel<float>, dim3(grid), dim3(256), 0, st, x, H, rows, per, in_stride, in_off,
                       (const float*)g, eps, (float*)y);
  return hipGetLastError();
}

hipError_t residual_norm(int dt, const float* partial, int splits, int M, int H, float* h, const void* g, float eps,
                         void* out, int final_L, hipStream_t st) {
  ProfScope prof("resid_norm", st);
  if (M == 0) return hipSuccess;
  const unsigned grid = (unsigned)M;
  auto launch = [&](auto tag, auto ns) {
    typedef decltype(tag) T;
    hipLaunchKernelGGL((resid_norm_kernel<T, decltype(ns)::value>), dim3(grid), dim3(256), 0, st, partial, splits,
                       M, H, h, (const T*)g, eps, (T*)out, final_L);
  };
  auto by_splits = [&](auto tag) {
    switch (partial ? splits : 1) {
      case 1: launch(tag, std::integral_constant<int, 1>{}); break;
      case 2: launch(tag, std::integral_constant<int, 2>{}); break;
      case 3: launch(tag, std::integral_constant<int, 3>{}); break;
      case 4: launch(tag, std::integral_constant<int, 4>{}); break;
      case 5: launch(tag, std::integral_constant<int, 5>{}); break;
      case 6: launch(tag, std::integral_constant<int, 6>{}); break;
      case 7: launch(tag, std::integral_constant<int, 7>{}); break;
      case 8: launch(tag, std::integral_constant<int, 8>{}); break;
      default: {
        typedef decltype(tag) T;
        hipLaunchKernelGGL(resid_norm_many_kernel<T>, dim3(grid), dim3(1024), 0, st, partial, splits, M, H, h,
                           (const T*)g, eps, (T*)out, final_L);
      }
    }
  };
  if (dt == FPD_DTYPE_BF16)
    by_splits(bf16_t{});
  else
    by_splits(float{});
  return hipGetLastError();
}

hipError_t embed_norm(int dt, const int32_t* tokens, int M, const void* E, int H, int V, float* h, const void* g,
                      float eps, void* a, hipStream_t st) {
  ProfScope prof("embed_norm", st);
  if (M == 0) return hipSuccess;
  if (dt == FPD_DTYPE_BF16)
    hipLaunchKernelGGL(embed_norm_kernel<bf16_t>, dim3(M), dim3(256), 0, st, tokens, (const bf16_t*)E, H, V, h,
                       (const bf16_t*)g, eps, (bf16_t*)a);
  else
    hipLaunchKernelGGL(embed_norm_kernel<float>, dim3(M), dim3(256), 0, st, tokens, (const float*)E, H, V, h,
                       (const float*)g, eps, (float*)a);
  return hipGetLastError();
}

hipError_t concat_features(int dt, const void* feats, int B, int nt, int C, int H, void* X, hipStream_t st) {
  ProfScope prof("concat", st);
  const int esz = dt == FPD_DTYPE_BF16 ? 2 : 4;
  const int Hc = H * esz / 16;
  const size_t n = (size_t)B * nt * C * Hc;
  if (n == 0) return hipSuccess;
  const unsigned grid = (unsigned)std::min<size_t>((n + 255) / 256, 65536);
  hipLaunchKernelGGL(concat_kernel, dim3(grid), dim3(256), 0, st, (const u32x4_t*)feats, B, nt, C, Hc,
                     (u32x4_t*)X);
  return hipGetLastError();
}

hipError_t gather_rows(int dt, const void* W, int H, const int32_t* ids, int n, void* out, hipStream_t st) {
  ProfScope prof("gather_rows", st);
  if (n == 0) return hipSuccess;
  const int esz = dt == FPD_DTYPE_BF16 ? 2 : 4;
  const int Hc = H * esz / 16;
  hipLaunchKernelGGL(gather_rows_kernel, dim3(n), dim3(256), 0, st, (const u32x4_t*)W, Hc, ids, n,
                     (u32x4_t*)out);
  return hipGetLastError();
}

}  // namespace fpd
