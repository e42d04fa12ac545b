// Non-causal grouped-query attention of block queries over
// [context K/V || block K/V] (VFlash paper §2.1: one bidirectional pass,
// target features injected as key/value into every drafter layer).
//
// bf16 path (gfx950 MFMA 32x32x16): the n_q/n_kv query heads that share a
// KV head are packed into one M dimension (rows r = head_in_group * L + l,
// contiguous in the [B, n_q, L, d] query layout).  Each wave owns 32 packed
// query rows; a workgroup of 4 waves shares 64-key K / V^T tiles staged in
// LDS with a register prefetch of the next tile.  Scores are computed
// transposed, S^T = K Q^T, so every lane owns one query: the online softmax
// needs a single cross-lane exchange (lane l with lane l ^ 32).  K rows are
// read with bits 2 and 3 of the row index swapped, which makes the S^T
// accumulator come out exactly in the B-operand layout of the next MFMA, so
// P feeds O^T += V^T P^T with no data movement.  V is stored d-major
// (transposed) so each V^T fragment is one 16-byte LDS read.  The key range
// is split across workgroups when (b, kv-head, query-tile) alone cannot fill
// the GPU; partial (m, l, O) are merged by a log-sum-exp combine.
#include <algorithm>

#include "../../include/fpd.h"
#include "kernels.h"

namespace fpd {
namespace {

constexpr int KT = 64;          // keys per tile
constexpr int D = 128;          // head dim of the bf16 path
constexpr int KLD = D + 8;      // K tile row stride (bf16 elements)
constexpr int VLD = KT + 8;     // V^T tile row stride
constexpr int QROWS = 128;      // packed query rows per workgroup (4 waves x 32)

struct AttnP {
  const bf16_t *q, *kb, *vbt, *ck, *cvt;
  bf16_t* o;
  float* opart;   // [splits, B, nq, L, D]
  float* mlpart;  // [splits, B, nq, L, 2]
  int B, L, Lp, C, cap, nq, nkv, g, R, q_tiles, splits, ctx_tiles, blk_tiles;
  float scale_log2;
};

__device__ __forceinline__ int swap23(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

__global__ __launch_bounds__(256) void attn_bf16_kernel(AttnP p) {
  __shared__ __attribute__((aligned(16))) bf16_t Ks[2][KT * KLD];
  __shared__ __attribute__((aligned(16))) bf16_t Vs[2][D * VLD];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int qt = tile % p.q_tiles;
  const int rest = tile / p.q_tiles;
  const int sp = rest % p.splits;
  const int bh = rest / p.splits;
  const int b = bh / p.nkv, j = bh % p.nkv;
  const int lq = lane & 31, lg = lane >> 5;
  const int r0 = qt * QROWS + wave * 32;
  const bool wave_active = r0 < p.R;
  const int qrow = r0 + lq;
  const bool qvalid = qrow < p.R;

  // query fragments (B operand of S^T = K Q^T): lane holds query qrow, dims kk*16 + lg*8 .. +8
  const bf16_t* qbase = p.q + ((size_t)(b * p.nq + j * p.g) * p.L) * D;
  bf16x8_t qf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    if (qvalid)
      qf[kk] = *(const bf16x8_t*)(qbase + (size_t)qrow * D + kk * 16 + lg * 8);
    else
      qf[kk] = bf16x8_t{};
  }

  const int total = p.ctx_tiles + p.blk_tiles;
  const int t0 = (int)((long)sp * total / p.splits), t1 = (int)((long)(sp + 1) * total / p.splits);
  const size_t bhk = (size_t)b * p.nkv + j;

  // tile source
  auto src = [&](int t, const bf16_t*& kptr, const bf16_t*& vptr, int& ldv, int& key0, int& count) {
    if (t < p.ctx_tiles) {
      key0 = t * KT;
      count = p.C;
      kptr = p.ck + bhk * p.cap * D;
      vptr = p.cvt + bhk * D * p.cap;
      ldv = p.cap;
    } else {
      key0 = (t - p.ctx_tiles) * KT;
      count = p.L;
      kptr = p.kb + bhk * p.L * D;
      vptr = p.vbt + bhk * D * p.Lp;
      ldv = p.Lp;
    }
  };

  u32x4_t rk[4], rv[4];
  int cur_count = 0, cur_key0 = 0;
  auto gload = [&](int t) {
    const bf16_t *kp, *vp;
    int ldv, key0, count;
    src(t, kp, vp, ldv, key0, count);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + i * 256;
      const int krow = c >> 4, kc = (c & 15) * 8;
      rk[i] = (key0 + krow < count) ? *(const u32x4_t*)(kp + (size_t)(key0 + krow) * D + kc)
                                    : u32x4_t{0, 0, 0, 0};
      const int drow = c >> 3, vc = (c & 7) * 8;
      const int kabs = key0 + vc;
      if (kabs < count) {
        u32x4_t v = *(const u32x4_t*)(vp + (size_t)drow * ldv + kabs);
        const int nvalid = count - kabs;  // keys beyond the valid count become exact zeros
        if (nvalid < 8) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int k0e = 2 * e;
            uint32_t w = v[e];
            if (k0e >= nvalid) w = 0;
            else if (k0e + 1 >= nvalid) w &= 0xffffu;
            v[e] = w;
          }
        }
        rv[i] = v;
      } else {
        rv[i] = u32x4_t{0, 0, 0, 0};
      }
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int c = tid + i * 256;
      *(u32x4_t*)&Ks[buf][(c >> 4) * KLD + (c & 15) * 8] = rk[i];
      *(u32x4_t*)&Vs[buf][(c >> 3) * VLD + (c & 7) * 8] = rv[i];
    }
  };

  f32x16_t o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  if (t0 < t1) {
    gload(t0);
    sstore(0);
    __syncthreads();
  }
  for (int t = t0; t < t1; ++t) {
    const int cur = (t - t0) & 1;
    {
      const bf16_t *kp, *vp;
      int ldv;
      src(t, kp, vp, ldv, cur_key0, cur_count);
    }
    if (t + 1 < t1) gload(t + 1);
    if (wave_active) {
      f32x16_t s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
        const int krow = kb * 32 + swap23(lq);
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
          const bf16x8_t kf = *(const bf16x8_t*)&Ks[cur][krow * KLD + kk * 16 + lg * 8];
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[kk], s[kb], 0, 0, 0);
        }
      }
      // register r of sub-block kb holds key kb*32 + (r/8)*16 + lg*8 + r%8 for query lq
      float mloc = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = cur_key0 + kb * 32 + (r >> 3) * 16 + lg * 8 + (r & 7);
          const float x = key < cur_count ? s[kb][r] * p.scale_log2 : -INFINITY;
          s[kb][r] = x;
          mloc = fmaxf(mloc, x);
        }
      mloc = fmaxf(mloc, __shfl_xor(mloc, 32));
      const float m_new = fmaxf(m_run, mloc);
      const float m_use = m_new == -INFINITY ? 0.f : m_new;
      const float alpha = exp2f(m_run - m_use);
      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const float e = exp2f(s[kb][r] - m_use);
          s[kb][r] = e;
          lsum += e;
        }
      l_run = l_run * alpha + lsum;
      m_run = m_new;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          bf16x8_t pf;
#pragma unroll
          for (int e = 0; e < 8; ++e) pf[e] = __builtin_bit_cast(__bf16, f2bf(s[kb][h * 8 + e]));
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt) {
            const bf16x8_t vf =
                *(const bf16x8_t*)&Vs[cur][(dt * 32 + lq) * VLD + kb * 32 + h * 16 + lg * 8];
            o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, o[dt], 0, 0, 0);
          }
        }
    }
    if (t + 1 < t1) sstore(cur ^ 1);
    __syncthreads();
  }

  if (!qvalid) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const int hl = qrow / p.L, l = qrow % p.L;
  const int head = j * p.g + hl;
  if (p.splits == 1) {
    const float inv = 1.0f / l_tot;
    bf16_t* dst = p.o + ((size_t)b * p.L + l) * (size_t)(p.nq * D) + (size_t)head * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = dt * 32 + q4 * 8 + lg * 4;
        u32x2_t w;
        w[0] = pack_bf16x2(o[dt][q4 * 4 + 0] * inv, o[dt][q4 * 4 + 1] * inv);
        w[1] = pack_bf16x2(o[dt][q4 * 4 + 2] * inv, o[dt][q4 * 4 + 3] * inv);
        *(u32x2_t*)(dst + d0) = w;
      }
  } else {
    const size_t row = (((size_t)sp * p.B + b) * p.nq + head) * p.L + l;
    float* dst = p.opart + row * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = dt * 32 + q4 * 8 + lg * 4;
        *(f32x4_t*)(dst + d0) = f32x4_t{o[dt][q4 * 4], o[dt][q4 * 4 + 1], o[dt][q4 * 4 + 2], o[dt][q4 * 4 + 3]};
      }
    if (lg == 0) {
      p.mlpart[row * 2 + 0] = m_run;
      p.mlpart[row * 2 + 1] = l_tot;
    }
  }
}

// Merges split partials: O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s.
template <class T>
__global__ __launch_bounds__(128) void attn_combine_kernel(const float* __restrict__ opart,
                                                           const float* __restrict__ ml, int splits,
                                                           int B, int nq, int L, int d, T* __restrict__ o) {
  const int row = blockIdx.x;  // (b, head, l)
  const int l = row % L, bh = row / L, head = bh % nq, b = bh / nq;
  const size_t rows = (size_t)B * nq * L;
  float M = -INFINITY;
  for (int s = 0; s < splits; ++s) M = fmaxf(M, ml[(s * rows + row) * 2]);
  float den = 0.f;
  for (int s = 0; s < splits; ++s) {
    const float ms = ml[(s * rows + row) * 2];
    if (ms != -INFINITY) den += exp2f(ms - M) * ml[(s * rows + row) * 2 + 1];
  }
  const float inv = 1.0f / den;
  for (int dd = threadIdx.x; dd < d; dd += blockDim.x) {
    float acc = 0.f;
    for (int s = 0; s < splits; ++s) {
      const float ms = ml[(s * rows + row) * 2];
      if (ms != -INFINITY) acc += exp2f(ms - M) * opart[(s * rows + row) * d + dd];
    }
    Elem<T>::st(o + ((size_t)b * L + l) * (size_t)(nq * d) + (size_t)head * d + dd, acc * inv);
  }
}

// ---- f32 path: one wave per (b, head, query); keys split over lanes ------------------------
template <int DD>
__global__ __launch_bounds__(64) void attn_f32_kernel(const float* __restrict__ q, const float* __restrict__ kb,
                                                      const float* __restrict__ vbt, const float* __restrict__ ck,
                                                      const float* __restrict__ cvt, float* __restrict__ o,
                                                      int B, int L, int Lp, int C, int cap, int nq, int nkv,
                                                      float scale) {
  __shared__ float red_o[64][DD + 1];
  __shared__ float red_m[64], red_l[64];
  const int lane = threadIdx.x;
  const int row = blockIdx.x;  // (b, head, l)
  const int l = row % L, bh = row / L, head = bh % nq, b = bh / nq;
  const int j = (head * nkv) / nq;
  const size_t bhk = (size_t)b * nkv + j;
  float qv[DD];
  const float* qp = q + (((size_t)b * nq + head) * L + l) * DD;
#pragma unroll
  for (int e = 0; e < DD; ++e) qv[e] = qp[e];
  float acc[DD];
#pragma unroll
  for (int e = 0; e < DD; ++e) acc[e] = 0.f;
  float m = -INFINITY, lsum = 0.f;
  const int total = C + L;
  for (int key = lane; key < total; key += 64) {
    const float* kp;
    const float* vp;
    int ldv;
    if (key < C) {
      kp = ck + (bhk * cap + key) * DD;
      vp = cvt + bhk * DD * cap + key;
      ldv = cap;
    } else {
      kp = kb + (bhk * L + (key - C)) * DD;
      vp = vbt + bhk * DD * Lp + (key - C);
      ldv = Lp;
    }
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < DD; ++e) s += qv[e] * kp[e];
    s *= scale;
    const float mn = fmaxf(m, s);
    const float a = expf(m - mn), pr = expf(s - mn);
    lsum = lsum * a + pr;
#pragma unroll
    for (int e = 0; e < DD; ++e) acc[e] = acc[e] * a + pr * vp[(size_t)e * ldv];
    m = mn;
  }
  red_m[lane] = m;
  red_l[lane] = lsum;
#pragma unroll
  for (int e = 0; e < DD; ++e) red_o[lane][e] = acc[e];
  __syncthreads();
  float M = -INFINITY;
  for (int i = 0; i < 64; ++i) M = fmaxf(M, red_m[i]);
  float den = 0.f;
  for (int i = 0; i < 64; ++i)
    if (red_m[i] != -INFINITY) den += expf(red_m[i] - M) * red_l[i];
  for (int e = lane; e < DD; e += 64) {
    float v = 0.f;
    for (int i = 0; i < 64; ++i)
      if (red_m[i] != -INFINITY) v += expf(red_m[i] - M) * red_o[i][e];
    o[((size_t)b * L + l) * (size_t)(nq * DD) + (size_t)head * DD + e] = v / den;
  }
}

int attn_splits(int B, int L, int C, int nq, int nkv, int* q_tiles_out, int* total_tiles) {
  const int g = nq / nkv;
  const int R = g * L;
  const int q_tiles = (R + QROWS - 1) / QROWS;
  const int tiles = (C + KT - 1) / KT + (L + KT - 1) / KT;
  const int base = q_tiles * B * nkv;
  int splits = 1;
  while (base * splits < 512 && splits * 2 <= tiles) splits *= 2;
  if (q_tiles_out) *q_tiles_out = q_tiles;
  if (total_tiles) *total_tiles = tiles;
  return splits;
}

}  // namespace

size_t attention_scratch_bytes(int dt, int B, int L, int C, int nq, int nkv, int d) {
  if (dt != FPD_DTYPE_BF16) return 0;
  const int s = attn_splits(B, L, C, nq, nkv, nullptr, nullptr);
  if (s == 1) return 0;
  const size_t rows = (size_t)s * B * nq * L;
  return rows * d * sizeof(float) + rows * 2 * sizeof(float);
}

hipError_t attention(int dt, const AttnArgs& a, void* scratch, size_t scratch_bytes, hipStream_t st) {
  if (dt == FPD_DTYPE_BF16) {
    AttnP p{};
    p.q = (const bf16_t*)a.q;
    p.kb = (const bf16_t*)a.kb;
    p.vbt = (const bf16_t*)a.vbt;
    p.ck = (const bf16_t*)a.ck;
    p.cvt = (const bf16_t*)a.cvt;
    p.o = (bf16_t*)a.o;
    p.B = a.B, p.L = a.L, p.Lp = a.Lp, p.C = a.C, p.cap = a.cap, p.nq = a.nq, p.nkv = a.nkv;
    p.g = a.nq / a.nkv;
    p.R = p.g * a.L;
    int total = 0;
    p.splits = attn_splits(a.B, a.L, a.C, a.nq, a.nkv, &p.q_tiles, &total);
    const size_t rows = (size_t)p.splits * a.B * a.nq * a.L;
    if (p.splits > 1 && rows * (D + 2) * sizeof(float) > scratch_bytes) p.splits = 1;
    p.ctx_tiles = (a.C + KT - 1) / KT;
    p.blk_tiles = (a.L + KT - 1) / KT;
    p.opart = (float*)scratch;
    p.mlpart = (float*)scratch + rows * D;
    p.scale_log2 = a.scale * 1.4426950408889634f;
    const int grid = p.q_tiles * p.splits * a.B * a.nkv;
    {
      ProfScope prof("attention", st);
      hipLaunchKernelGGL(attn_bf16_kernel, dim3(grid), dim3(256), 0, st, p);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1) return e;
    ProfScope prof("attn_combine", st);
    hipLaunchKernelGGL(attn_combine_kernel<bf16_t>, dim3(a.B * a.nq * a.L), dim3(128), 0, st, p.opart,
                       p.mlpart, p.splits, a.B, a.nq, a.L, D, (bf16_t*)a.o);
    return hipGetLastError();
  }
  const int rows = a.B * a.nq * a.L;
  ProfScope prof("attention", st);
  if (a.d == 64)
    hipLaunchKernelGGL(attn_f32_kernel<64>, dim3(rows), dim3(64), 0, st, (const float*)a.q,
                       (const float*)a.kb, (const float*)a.vbt, (const float*)a.ck, (const float*)a.cvt,
                       (float*)a.o, a.B, a.L, a.Lp, a.C, a.cap, a.nq, a.nkv, a.scale);
  else
    hipLaunchKernelGGL(attn_f32_kernel<128>, dim3(rows), dim3(64), 0, st, (const float*)a.q,
                       (const float*)a.kb, (const float*)a.vbt, (const float*)a.ck, (const float*)a.cvt,
                       (float*)a.o, a.B, a.L, a.Lp, a.C, a.cap, a.nq, a.nkv, a.scale);
  return hipGetLastError();
}

}  // namespace fpd
