// Dense projections of the drafter: Y = A W^T with fused epilogues.
//
// bf16 path: MFMA 32x32x16 (gfx950) tiles, A and W both K-contiguous, staged
// through LDS with a register prefetch of the next K-tile (one barrier per
// K-tile), split-K with a fixed-order reduction when the tile count alone
// cannot fill 256 CUs, and an XCD-aware tile order so the workgroups that
// share a weight tile run on the same XCD.
//
// "Paired" epilogues need two W rows per output (RoPE rotates column i with
// column i + d/2 of a head; SwiGLU combines gate row i with up row I + i).
// Their B tile holds the first members in its first half and the second
// members in its second half, and each wave takes matching sub-tiles from
// both halves, so a lane holds both members of every pair in registers.
#include <algorithm>

#include "../../include/fpd.h"
#include "kernels.h"

namespace fpd {

namespace {

constexpr int BK = 64;
constexpr int LDSW = BK + 8;  // padded LDS row (bf16 elements): conflict-free 16-byte reads

// ---- B-row maps -------------------------------------------------------------
struct MapPlain {  // logical column n -> W row n
  __device__ int row(int n) const { return n; }
};
struct MapRope {   // pair index -> (head * d + i, head * d + i + d/2)
  int half;
  __device__ int first(int p) const { return (p / half) * 2 * half + p % half; }
  __device__ int second(int p) const { return first(p) + half; }
};
struct MapGlu {    // pair index i -> (i, I + i)
  int I;
  __device__ int first(int p) const { return p; }
  __device__ int second(int p) const { return I + p; }
};

// ---- epilogues --------------------------------------------------------------
struct EpiStore {
  float* out;
  int ld;
  __device__ void operator()(int m, int n, float v) const { out[(size_t)m * ld + n] = v; }
};
struct EpiResid {
  float* h;
  int ld;
  __device__ void operator()(int m, int n, float v) const { h[(size_t)m * ld + n] += v; }
};

template <class T>
struct EpiQkv {
  T *q, *k, *vt;
  int L, Lp, nq, nkv, d, half, pos0, rope;
  RopeTab tab;
  __device__ void pair(int m, int p, float x0, float x1) const {
    const int head = p / half, i = p % half;
    const int b = m / L, l = m - b * L;
    if (head < nq + nkv) {
      if (rope) rope_pair(x0, x1, pos0 + l, tab.inv_freq[i]);
      T* dst = head < nq ? q + (((size_t)b * nq + head) * L + l) * d
                         : k + (((size_t)b * nkv + (head - nq)) * L + l) * d;
      Elem<T>::st(dst + i, x0);
      Elem<T>::st(dst + i + half, x1);
    } else {
      T* dst = vt + ((size_t)b * nkv + (head - nq - nkv)) * d * Lp + l;
      Elem<T>::st(dst + (size_t)i * Lp, x0);
      Elem<T>::st(dst + (size_t)(i + half) * Lp, x1);
    }
  }
};

template <class T>
struct EpiCtx {
  T *k, *vt;
  int C, cap, nkv, d, half, pos0, rope;
  RopeTab tab;
  __device__ void pair(int m, int p, float x0, float x1) const {
    const int head = p / half, i = p % half;
    const int b = m / C, c = m - b * C;
    if (head < nkv) {
      if (rope) rope_pair(x0, x1, pos0 + c, tab.inv_freq[i]);
      T* dst = k + (((size_t)b * nkv + head) * cap + c) * d;
      Elem<T>::st(dst + i, x0);
      Elem<T>::st(dst + i + half, x1);
    } else {
      T* dst = vt + ((size_t)b * nkv + (head - nkv)) * d * cap + c;
      Elem<T>::st(dst + (size_t)i * cap, x0);
      Elem<T>::st(dst + (size_t)(i + half) * cap, x1);
    }
  }
};

template <class T>
struct EpiGlu {
  T* u;
  int I;
  __device__ void pair(int m, int p, float g, float up) const {
    Elem<T>::st(u + (size_t)m * I + p, silu_f(g) * up);
  }
};

// ---- bf16 MFMA kernel ---------------------------------------------------------
template <int BM, int BN, int WAVES_M, int WAVES_N, bool PAIRED, class Map, class Epi>
__global__ __launch_bounds__(64 * WAVES_M* WAVES_N) void gemm_bf16_kernel(
    const bf16_t* __restrict__ A, int lda, int M, int K, const bf16_t* __restrict__ W, Map map,
    int ncols, Epi epi, float* __restrict__ partial, int part_ld, int m_tiles, int n_tiles,
    int splits) {
  constexpr int NT = 64 * WAVES_M * WAVES_N;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int A_CH = BM * (BK / 8) / NT;  // 16-byte chunks per thread
  constexpr int B_CH = BN * (BK / 8) / NT;
  static_assert(TM >= 1 && TN >= 1 && A_CH >= 1 && B_CH >= 1, "tile shape");
  static_assert(!PAIRED || (TN % 2 == 0), "paired epilogues need an even number of N sub-tiles");
  constexpr int CPT = PAIRED ? BN / 2 : BN;  // logical columns per tile

  __shared__ __attribute__((aligned(16))) bf16_t As[2][BM * LDSW];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[2][BN * LDSW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int mt = tile % m_tiles;
  const int rest = tile / m_tiles;
  const int nt = rest % n_tiles;
  const int ks = rest / n_tiles;
  const int m0 = mt * BM, c0 = nt * CPT;
  const int KT = K / BK;
  const int kt0 = (int)((long)ks * KT / splits), kt1 = (int)((long)(ks + 1) * KT / splits);

  // per-thread source rows of its A and B chunks (null = zero fill)
  const bf16_t* aptr[A_CH];
  int akc[A_CH], alds[A_CH];
#pragma unroll
  for (int i = 0; i < A_CH; ++i) {
    const int c = tid + i * NT, row = c / (BK / 8), kc = (c % (BK / 8)) * 8;
    const int m = m0 + row;
    aptr[i] = m < M ? A + (size_t)m * lda : nullptr;
    akc[i] = kc;
    alds[i] = row * LDSW + kc;
  }
  const bf16_t* bptr[B_CH];
  int bkc[B_CH], blds[B_CH];
#pragma unroll
  for (int i = 0; i < B_CH; ++i) {
    const int c = tid + i * NT, row = c / (BK / 8), kc = (c % (BK / 8)) * 8;
    int wrow = -1;
    if constexpr (PAIRED) {
      const int p = c0 + (row % (BN / 2));
      if (p < ncols) wrow = row < BN / 2 ? map.first(p) : map.second(p);
    } else {
      const int n = c0 + row;
      if (n < ncols) wrow = map.row(n);
    }
    bptr[i] = wrow >= 0 ? W + (size_t)wrow * K : nullptr;
    bkc[i] = kc;
    blds[i] = row * LDSW + kc;
  }

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  u32x4_t ra[A_CH], rb[B_CH];
  auto gload = [&](int kt) {
    const int k0 = kt * BK;
#pragma unroll
    for (int i = 0; i < A_CH; ++i)
      ra[i] = aptr[i] ? *(const u32x4_t*)(aptr[i] + k0 + akc[i]) : u32x4_t{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < B_CH; ++i)
      rb[i] = bptr[i] ? __builtin_nontemporal_load((const u32x4_t*)(bptr[i] + k0 + bkc[i]))
                      : u32x4_t{0, 0, 0, 0};
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_CH; ++i) *(u32x4_t*)&As[buf][alds[i]] = ra[i];
#pragma unroll
    for (int i = 0; i < B_CH; ++i) *(u32x4_t*)&Bs[buf][blds[i]] = rb[i];
  };

  int bcol[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    if constexpr (PAIRED)
      bcol[j] = j < TN / 2 ? wn * (WN / 2) + j * 32 : BN / 2 + wn * (WN / 2) + (j - TN / 2) * 32;
    else
      bcol[j] = wn * WN + j * 32;
  }
  const int lr = lane & 31, lk = (lane >> 5) * 8;

  if (kt0 < kt1) {
    gload(kt0);
    sstore(0);
    __syncthreads();
  }
  for (int kt = kt0; kt < kt1; ++kt) {
    const int cur = (kt - kt0) & 1;
    if (kt + 1 < kt1) gload(kt + 1);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      bf16x8_t af[TM], bfv[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *(const bf16x8_t*)&As[cur][(wm * WM + i * 32 + lr) * LDSW + kk * 16 + lk];
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bfv[j] = *(const bf16x8_t*)&Bs[cur][(bcol[j] + lr) * LDSW + kk * 16 + lk];
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfv[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < kt1) sstore(cur ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds column (lane % 32) and rows (r/4)*8 + (lane/32)*4 + r%4 of each sub-tile
  float* part = splits > 1 ? partial + (size_t)ks * M * part_ld : nullptr;
#pragma unroll
  for (int i = 0; i < TM; ++i) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + wm * WM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3);
      if (m >= M) continue;
      if constexpr (PAIRED) {
#pragma unroll
        for (int j = 0; j < TN / 2; ++j) {
          const int p = c0 + wn * (WN / 2) + j * 32 + lr;
          if (p >= ncols) continue;
          const float v0 = acc[i][j][r], v1 = acc[i][j + TN / 2][r];
          if (part) {
            part[(size_t)m * part_ld + map.first(p)] = v0;
            part[(size_t)m * part_ld + map.second(p)] = v1;
          } else {
            epi.pair(m, p, v0, v1);
          }
        }
      } else {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int n = c0 + wn * WN + j * 32 + lr;
          if (n >= ncols) continue;
          if (part)
            part[(size_t)m * part_ld + n] = acc[i][j][r];
          else
            epi(m, n, acc[i][j][r]);
        }
      }
    }
  }
}

template <bool PAIRED, class Map, class Epi>
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ partial,
                                                            int splits, int M, int part_ld,
                                                            int ncols, Map map, Epi epi) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= (size_t)M * ncols) return;
  const int m = (int)(idx / ncols), c = (int)(idx % ncols);
  const size_t stride = (size_t)M * part_ld;
  if constexpr (PAIRED) {
    const size_t o0 = (size_t)m * part_ld + map.first(c), o1 = (size_t)m * part_ld + map.second(c);
    float v0 = 0.f, v1 = 0.f;
    for (int s = 0; s < splits; ++s) {
      v0 += partial[s * stride + o0];
      v1 += partial[s * stride + o1];
    }
    epi.pair(m, c, v0, v1);
  } else {
    const size_t o = (size_t)m * part_ld + c;
    float v = 0.f;
    for (int s = 0; s < splits; ++s) v += partial[s * stride + o];
    epi(m, c, v);
  }
}

// ---- f32 SIMT kernel (the fp32 drafter) -----------------------------------------------
template <bool PAIRED, class Map, class Epi>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const float* __restrict__ A, int lda, int M,
                                                       int K, const float* __restrict__ W, Map map,
                                                       int ncols, Epi epi, int m_tiles) {
  constexpr int TS = 64, KS = 16;
  __shared__ float As[KS][TS + 1];
  __shared__ float Bs[KS][TS + 1];
  const int tid = threadIdx.x, tx = tid % 16, ty = tid / 16;
  const int mt = blockIdx.x % m_tiles, nt = blockIdx.x / m_tiles;
  const int m0 = mt * TS;
  const int c0 = nt * (PAIRED ? TS / 2 : TS);
  int col[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) col[j] = PAIRED ? (j < 2 ? 2 * tx + j : TS / 2 + 2 * tx + (j - 2)) : 4 * tx + j;
  // W row of tile column n
  auto wrow = [&](int n) -> int {
    if constexpr (PAIRED) {
      const int p = c0 + (n % (TS / 2));
      if (p >= ncols) return -1;
      return n < TS / 2 ? map.first(p) : map.second(p);
    } else {
      const int c = c0 + n;
      return c < ncols ? map.row(c) : -1;
    }
  };
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += KS) {
    for (int e = tid; e < TS * KS; e += 256) {
      const int r = e / KS, kk = e % KS;
      const int m = m0 + r;
      As[kk][r] = (m < M && k0 + kk < K) ? A[(size_t)m * lda + k0 + kk] : 0.f;
      const int w = wrow(r);
      Bs[kk][r] = (w >= 0 && k0 + kk < K) ? W[(size_t)w * K + k0 + kk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      float a[4], b[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = Bs[kk][col[j]];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] += a[i] * b[j];
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= M) continue;
    if constexpr (PAIRED) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int p = c0 + col[j];
        if (p < ncols) epi.pair(m, p, acc[i][j], acc[i][j + 2]);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = c0 + col[j];
        if (n < ncols) epi(m, n, acc[i][j]);
      }
    }
  }
}

// ---- launch helpers ---------------------------------------------------------------------
template <bool PAIRED, class Map, class Epi>
hipError_t run_bf16(const void* A, int lda, int M, int K, const void* W, Map map, int ncols, int nw,
                    Epi epi, float* partial, size_t partial_bytes, hipStream_t st, const char* tag) {
  GemmPlan pl = plan_gemm_bf16(M, ncols, K, nw, PAIRED);
  if (pl.splits > 1 && pl.partial_floats * sizeof(float) > partial_bytes) pl.splits = 1;
  const int grid = pl.m_tiles * pl.n_tiles * pl.splits;
  if (grid == 0) return hipSuccess;
  const bf16_t* a = (const bf16_t*)A;
  const bf16_t* w = (const bf16_t*)W;
  float* part = pl.splits > 1 ? partial : nullptr;
  {
  ProfScope prof(tag, st);
  if (pl.bm == 128) {
    hipLaunchKernelGGL((gemm_bf16_kernel<128, 128, 2, 2, PAIRED, Map, Epi>), dim3(grid), dim3(256),
                       0, st, a, lda, M, K, w, map, ncols, epi, part, nw, pl.m_tiles, pl.n_tiles,
                       pl.splits);
  } else if (pl.bm == 64) {
    hipLaunchKernelGGL((gemm_bf16_kernel<64, 128, 2, 2, PAIRED, Map, Epi>), dim3(grid), dim3(256),
                       0, st, a, lda, M, K, w, map, ncols, epi, part, nw, pl.m_tiles, pl.n_tiles,
                       pl.splits);
  } else {
    hipLaunchKernelGGL((gemm_bf16_kernel<32, 128, 1, 2, PAIRED, Map, Epi>), dim3(grid), dim3(128),
                       0, st, a, lda, M, K, w, map, ncols, epi, part, nw, pl.m_tiles, pl.n_tiles,
                       pl.splits);
  }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.splits == 1) return e;
  ProfScope prof("splitk_reduce", st);
  const size_t n = (size_t)M * ncols;
  hipLaunchKernelGGL((splitk_reduce_kernel<PAIRED, Map, Epi>), dim3((unsigned)((n + 255) / 256)),
                     dim3(256), 0, st, partial, pl.splits, M, nw, ncols, map, epi);
  return hipGetLastError();
}

template <bool PAIRED, class Map, class Epi>
hipError_t run_f32(const void* A, int lda, int M, int K, const void* W, Map map, int ncols, Epi epi,
                   hipStream_t st, const char* tag) {
  ProfScope prof(tag, st);
  const int m_tiles = (M + 63) / 64;
  const int n_tiles = (ncols + (PAIRED ? 31 : 63)) / (PAIRED ? 32 : 64);
  if (m_tiles == 0 || n_tiles == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_f32_kernel<PAIRED, Map, Epi>), dim3(m_tiles * n_tiles), dim3(256), 0, st,
                     (const float*)A, lda, M, K, (const float*)W, map, ncols, epi, m_tiles);
  return hipGetLastError();
}

}  // namespace

GemmPlan plan_gemm_bf16(int M, int ncols, int K, int nw, bool paired) {
  GemmPlan p;
  p.bm = M <= 32 ? 32 : (M <= 64 ? 64 : 128);
  // prefer 64-row tiles when 128-row tiles leave the GPU under-filled
  const int cpt = paired ? 64 : 128;
  p.n_tiles = (ncols + cpt - 1) / cpt;
  if (p.bm == 128 && ((M + 127) / 128) * p.n_tiles < 256) p.bm = 64;
  p.m_tiles = (M + p.bm - 1) / p.bm;
  const int kt = K / BK;
  int tiles = p.m_tiles * p.n_tiles;
  p.splits = 1;
  while (tiles * p.splits < 320 && kt / (p.splits * 2) >= 4) p.splits *= 2;
  p.partial_floats = p.splits > 1 ? (size_t)p.splits * M * nw : 0;
  return p;
}

hipError_t gemm_store_f32(int dt, const void* A, int lda, int M, int K, const void* W, int N,
                          float* out, int ldo, float* partial, size_t partial_bytes, hipStream_t st,
                          const char* tag) {
  EpiStore e{out, ldo};
  if (dt == FPD_DTYPE_BF16)
    return run_bf16<false>(A, lda, M, K, W, MapPlain{}, N, N, e, partial, partial_bytes, st, tag);
  return run_f32<false>(A, lda, M, K, W, MapPlain{}, N, e, st, tag);
}

hipError_t gemm_residual(int dt, const void* A, int lda, int M, int K, const void* W, int N,
                         float* h, int ldh, float* partial, size_t partial_bytes, hipStream_t st,
                         const char* tag) {
  EpiResid e{h, ldh};
  if (dt == FPD_DTYPE_BF16)
    return run_bf16<false>(A, lda, M, K, W, MapPlain{}, N, N, e, partial, partial_bytes, st, tag);
  return run_f32<false>(A, lda, M, K, W, MapPlain{}, N, e, st, tag);
}

hipError_t gemm_qkv(int dt, const void* A, int M, int K, const void* Wqkv, const QkvOut& o,
                    float* partial, size_t partial_bytes, hipStream_t st) {
  const int half = o.d / 2;
  const int pairs = (o.nq + 2 * o.nkv) * half;
  const int nw = (o.nq + 2 * o.nkv) * o.d;
  if (dt == FPD_DTYPE_BF16) {
    EpiQkv<bf16_t> e{(bf16_t*)o.q, (bf16_t*)o.k, (bf16_t*)o.vt, o.L, o.Lp, o.nq, o.nkv, o.d, half,
                     o.pos0, o.rope, o.tab};
    return run_bf16<true>(A, K, M, K, Wqkv, MapRope{half}, pairs, nw, e, partial, partial_bytes, st,
                          "gemm_qkv");
  }
  EpiQkv<float> e{(float*)o.q, (float*)o.k, (float*)o.vt, o.L, o.Lp, o.nq, o.nkv, o.d, half,
                  o.pos0, o.rope, o.tab};
  return run_f32<true>(A, K, M, K, Wqkv, MapRope{half}, pairs, e, st, "gemm_qkv");
}

hipError_t gemm_ctx_kv(int dt, const void* Zn, int M, int K, const void* Wkv, const CtxOut& o,
                       float* partial, size_t partial_bytes, hipStream_t st) {
  const int half = o.d / 2;
  const int pairs = 2 * o.nkv * half;
  const int nw = 2 * o.nkv * o.d;
  if (dt == FPD_DTYPE_BF16) {
    EpiCtx<bf16_t> e{(bf16_t*)o.k, (bf16_t*)o.vt, o.C, o.cap, o.nkv, o.d, half, o.pos0, o.rope, o.tab};
    return run_bf16<true>(Zn, K, M, K, Wkv, MapRope{half}, pairs, nw, e, partial, partial_bytes, st,
                          "gemm_ctx_kv");
  }
  EpiCtx<float> e{(float*)o.k, (float*)o.vt, o.C, o.cap, o.nkv, o.d, half, o.pos0, o.rope, o.tab};
  return run_f32<true>(Zn, K, M, K, Wkv, MapRope{half}, pairs, e, st, "gemm_ctx_kv");
}

hipError_t gemm_swiglu(int dt, const void* A, int M, int K, const void* Wgu, int I, void* u,
                       float* partial, size_t partial_bytes, hipStream_t st) {
  if (dt == FPD_DTYPE_BF16) {
    EpiGlu<bf16_t> e{(bf16_t*)u, I};
    return run_bf16<true>(A, K, M, K, Wgu, MapGlu{I}, I, 2 * I, e, partial, partial_bytes, st,
                          "gemm_gate_up");
  }
  EpiGlu<float> e{(float*)u, I};
  return run_f32<true>(A, K, M, K, Wgu, MapGlu{I}, I, e, st, "gemm_gate_up");
}

}  // namespace fpd
