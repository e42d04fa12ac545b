// Non-causal grouped-query attention of block queries over
// [context K/V || block K/V] (VFlash paper §2.1: one bidirectional pass,
// target features injected as key/value into every drafter layer).
//
// bf16 path (gfx950 MFMA 32x32x16): the n_q/n_kv query heads that share a
// KV head are packed into one M dimension (rows r = head_in_group * L + l,
// contiguous in the [B, n_q, L, d] query layout).  Each wave owns 32 packed
// query rows; a workgroup of 8 waves (256 rows) shares 64-key K / V^T tiles
// that stream global -> LDS through a 3-stage ring of LDS-writing buffer
// loads (two tiles in flight, one barrier per tile).  Scores are computed
// transposed, S^T = K Q^T, so every lane owns one query: the online softmax
// needs a single cross-lane exchange (lane l with lane l ^ 32).  K rows are
// read with bits 2 and 3 of the row index swapped, which makes the S^T
// accumulator come out exactly in the B-operand layout of the next MFMA, so
// P feeds O^T += V^T P^T with no data movement.  V is stored d-major
// (transposed) so each V^T fragment is one 16-byte LDS read, and as fp16
// holding the bf16-rounded values exactly, so that P enters that product in
// fp16 (11 significant bits) rather than bf16 (8) at the same MFMA rate.
// The key range
// is split across workgroups when (b, kv-head, query-tile) alone cannot fill
// the GPU; partial (m, l, O) (O as per-row-scaled fp16) are merged by a
// log-sum-exp combine.  When the packed rows end in a tile of at most 32
// rows (L = 64k + 1 leaves 4), that tail tile runs in workgroups of its own
// where two waves share every key tile (keys 0-31 / 32-63) and merge their
// states at the end: a wave alone per SIMD, each doing half the work of a
// full tile's wave, so the tail takes fewer key splits and frees CUs for
// more splits of the full tiles.
#include <algorithm>
#include <type_traits>

#include "../../include/fpd.h"
#include "kernels.h"
#include "lds_pipe.h"

namespace fpd {
namespace {

constexpr int KT = 64;          // keys per tile
constexpr int D = 128;          // head dim of the bf16 path
constexpr int AW = 8;           // waves per workgroup
constexpr int QROWS = AW * 32;  // packed query rows per workgroup
constexpr int AST = 4;          // depth of the global -> LDS ring (8-wave query tiles; the array holds TST)
constexpr int TST = 5;          // depth of the ring of the tail tile's workgroups
constexpr int KSLOTS = KT * 16; // 16-byte chunks of a K tile (64 keys x 256 bytes)
constexpr int VSLOTS = D * 8;   // 16-byte chunks of a V^T tile (128 dims x 64 keys)
constexpr int ASTAGE = KSLOTS + VSLOTS;
constexpr int APT = KSLOTS / (AW * 64);  // K (and V) loads per thread and stage
constexpr float kRescale = 8.0f;  // lazy rescale: keep the running max until it grows by 2^8

// fp16 pairs (round to nearest even; the first value in the low half), built
// from scalar conversions: a two-element _Float16 vector initialised from two
// conversions came out with both words holding the first pair here.
__device__ __forceinline__ uint32_t pack_f16x2(float lo, float hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)lo) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)hi) << 16);
}
__device__ __forceinline__ float f16lo(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v & 0xffffu));
}
__device__ __forceinline__ float f16hi(uint32_t v) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(v >> 16));
}

struct AttnP {
  const bf16_t *q, *kb, *ck;
  const uint16_t *vbt, *cvt;  // values as fp16 (bf16-rounded values, exactly)
  bf16_t* o;
  uint16_t* opart;  // [splits, B, nq, L, D] fp16: each split's O / (l c), c = its row's max |O / l|
  float* mlpart;    // [splits, B, nq, L, 4]: reference max (log2 units), l, c, unused
  int B, L, Lp, C, cap, nq, nkv, g, R, ctx_tiles, blk_tiles, ctx_bstride;
  int q_tiles;      // query tiles of 8-wave workgroups per (b, kv head)
  int splits;       // their key splits = partial slots per row
  int tail_splits;  // key splits of the tail tile (after the q_tiles), 0 = none
  float scale_log2;
};

// max(x, x of lane l ^ 32) without an LDS round trip: v_permlane32_swap with
// x as both operands returns (x[l mod 32], x[l mod 32 + 32]) in every lane l.
__device__ __forceinline__ float max_lane_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ int swap23(int m) { return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1); }

// LDS tiles hold 16-byte chunks without padding; chunk positions are XOR
// swizzled so the MFMA operand reads (16 rows x 16 bytes per LDS cycle) hit
// distinct banks.  K tile: 64 keys x 16 chunks; V^T tile: 128 dims x 8 chunks.
__device__ __forceinline__ int kslot(int r, int c) { return r * 16 + (c ^ (r & 15)); }
__device__ __forceinline__ int vslot(int d, int c) { return d * 8 + (c ^ ((d >> 1) & 7)); }

// K and V^T tiles stream global -> LDS through an AST-deep ring of
// LDS-writing buffer loads (one descriptor per source segment; per-lane
// offsets are fixed, the tile's key offset is scalar).  Keys past a
// segment's valid count are masked out of the scores; in the (at most two)
// partial tiles of a workgroup their V^T columns are zeroed in LDS before
// use, so padding memory never reaches the P V product.
__global__ __launch_bounds__(AW * 64) void attn_bf16_kernel(AttnP p) {
  __shared__ u32x4_t lds[(AST > TST ? AST : TST) * ASTAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  // Each (b, kv head) owns a contiguous range of tiles: its (query tile,
  // split) pairs of the 8-wave query tiles, query tile fastest, then the
  // splits of the tail tile, whose rows waves 0 and 1 both hold (each takes
  // one 32-key half of every key tile).  A range of tiles runs on one XCD,
  // so all the workgroups that stream one head's keys share its L2.
  const int per_bh = p.q_tiles * p.splits + p.tail_splits;
  const int bh = tile / per_bh, local = tile % per_bh;
  const bool tail = local >= p.q_tiles * p.splits;
  int qt, sp, ns;
  if (!tail) {
    qt = local % p.q_tiles;
    sp = local / p.q_tiles;
    ns = p.splits;
  } else {
    qt = p.q_tiles;
    sp = local - p.q_tiles * p.splits;
    ns = p.tail_splits;
  }
  const int b = bh / p.nkv, j = bh % p.nkv;
  const int lq = lane & 31, lg = lane >> 5;
  const int r0 = qt * QROWS + (tail ? 0 : wave * 32);
  const bool wave_active = tail ? wave < 2 : r0 < p.R;
  const int qrow = r0 + lq;
  const bool qvalid = qrow < p.R;

  // query fragments (B operand of S^T = K Q^T): lane holds query qrow, dims kk*16 + lg*8 .. +8
  const bf16_t* qbase = p.q + ((size_t)(b * p.nq + j * p.g) * p.L) * D;
  bf16x8_t qf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
    qf[kk] = qvalid ? *(const bf16x8_t*)(qbase + (size_t)qrow * D + kk * 16 + lg * 8) : bf16x8_t{};

  const int total = p.ctx_tiles + p.blk_tiles;
  const int t0 = (int)((long)sp * total / ns), t1 = (int)((long)(sp + 1) * total / ns);
  const size_t bhk = (size_t)b * p.nkv + j;
  const size_t cbhk = (size_t)b * p.ctx_bstride * p.nkv + j;  // context segment (shared: b = 0)

  const __amdgpu_buffer_rsrc_t kc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.ck + cbhk * p.cap * D), (short)0, (int)((size_t)p.cap * D * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t kbk = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.kb + bhk * p.L * D), (short)0, (int)((size_t)p.L * D * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t vc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.cvt + cbhk * D * p.cap), (short)0, (int)((size_t)D * p.cap * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t vbk = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(p.vbt + bhk * D * p.Lp), (short)0, (int)((size_t)D * p.Lp * 2), 0x00020000);
  // per-lane source offsets of the slots this lane fills (the swizzle is
  // applied by choosing which global chunk lands in which slot)
  uint32_t koff[APT], voff_c[APT], voff_b[APT];
#pragma unroll
  for (int i = 0; i < APT; ++i) {
    const int sl = (wave * APT + i) * 64 + lane;
    const int kr = sl >> 4, kc_ = (sl & 15) ^ (kr & 15);
    koff[i] = (uint32_t)((kr * D + kc_ * 8) * 2);
    const int dr = sl >> 3, vc_ = (sl & 7) ^ ((dr >> 1) & 7);
    voff_c[i] = (uint32_t)(((size_t)dr * p.cap + vc_ * 8) * 2);
    voff_b[i] = (uint32_t)(((size_t)dr * p.Lp + vc_ * 8) * 2);
  }
  auto tile_key0 = [&](int t) { return t < p.ctx_tiles ? t * KT : (t - p.ctx_tiles) * KT; };
  auto tile_count = [&](int t) { return t < p.ctx_tiles ? p.C : p.L; };
  auto issue = [&](int t, int stage) {
    const bool ctx = t < p.ctx_tiles;
    const int key0 = tile_key0(t);
    u32x4_t* base = lds + stage * ASTAGE;
#pragma unroll
    for (int i = 0; i < APT; ++i) lds_dma16(ctx ? kc : kbk, base + (wave * APT + i) * 64, koff[i], key0 * D * 2);
#pragma unroll
    for (int i = 0; i < APT; ++i)
      lds_dma16(ctx ? vc : vbk, base + KSLOTS + (wave * APT + i) * 64, ctx ? voff_c[i] : voff_b[i], key0 * 2);
  };

  f32x16_t o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[dt][r] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const int krow0 = swap23(lq);

  // The key loop over an ST-deep ring; a wave works on NKB 32-key blocks of
  // each tile starting at block kb0 (NKB = 2, kb0 = 0 in the 8-wave tiles;
  // NKB = 1, kb0 = wave in the tail tile, whose workgroup streams twice the
  // keys of a full tile's and so keeps more tiles in flight).
  auto run = [&](auto nkb_c, auto st_c, int kb0) {
    constexpr int NKB = decltype(nkb_c)::value;
    constexpr int ST = decltype(st_c)::value;
#pragma unroll
    for (int s2 = 0; s2 < ST - 1; ++s2)
      if (t0 + s2 < t1) issue(t0 + s2, s2);
    wait_lgkm0();

    for (int t = t0; t < t1; ++t) {
      const int stage = (t - t0) % ST;
      const int key0 = tile_key0(t), count = tile_count(t);
      wait_stages<2 * APT, ST - 2>(min(ST - 2, t1 - 1 - t));
      barrier_nofence();  // tile t landed for every wave; stage of tile t-1 is free
      u32x4_t* Ks = lds + stage * ASTAGE;
      u32x4_t* Vs = Ks + KSLOTS;
      if (key0 + KT > count) {  // partial tile: zero the V^T columns of keys past the count
        for (int sl = tid; sl < VSLOTS; sl += AW * 64) {
          const int dr = sl >> 3, c = (sl & 7) ^ ((dr >> 1) & 7);
          const int nvalid = count - (key0 + c * 8);
          if (nvalid < 8) {
            u32x4_t v = Vs[sl];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if (2 * e >= nvalid) v[e] = 0;
              else if (2 * e + 1 >= nvalid) v[e] &= 0xffffu;
            }
            Vs[sl] = v;
          }
        }
        wait_lgkm0();
        barrier_nofence();
      }
      if (t + ST - 1 < t1) issue(t + ST - 1, (t - t0 + ST - 1) % ST);
      if (wave_active) {
        const bf16x8_t* Kb = (const bf16x8_t*)Ks;
        const f16x8_t* Vh = (const f16x8_t*)Vs;
        f32x16_t s[NKB];
        if constexpr (NKB == 2) {
#pragma unroll
          for (int i = 0; i < NKB; ++i) {
#pragma unroll
            for (int r = 0; r < 16; ++r) s[i][r] = 0.f;
            const int krow = (kb0 + i) * 32 + krow0;
#pragma unroll
            for (int kk = 0; kk < D / 16; ++kk)
              s[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Kb[kslot(krow, kk * 2 + lg)], qf[kk], s[i], 0, 0, 0);
          }
        } else {
          // one key block: two accumulator chains (even / odd head-dim
          // steps) so that consecutive MFMAs do not wait on each other
          f32x16_t s2;
#pragma unroll
          for (int r = 0; r < 16; ++r) s[0][r] = s2[r] = 0.f;
          const int krow = kb0 * 32 + krow0;
#pragma unroll
          for (int kk = 0; kk < D / 16; kk += 2) {
            s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Kb[kslot(krow, kk * 2 + lg)], qf[kk], s[0], 0, 0, 0);
            s2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Kb[kslot(krow, kk * 2 + 2 + lg)], qf[kk + 1], s2, 0, 0, 0);
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) s[0][r] += s2[r];
        }
        // register r of block kb holds key kb*32 + (r/8)*16 + lg*8 + r%8 for query lq.
        // The running max is kept in raw score units (scale > 0); exponents
        // are fma(s, scale*log2(e), -m*scale*log2(e)).
        float mloc = -INFINITY;
        if (key0 + KT <= count) {
#pragma unroll
          for (int i = 0; i < NKB; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) mloc = fmaxf(mloc, s[i][r]);
        } else {
#pragma unroll
          for (int i = 0; i < NKB; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int key = key0 + (kb0 + i) * 32 + (r >> 3) * 16 + lg * 8 + (r & 7);
              s[i][r] = key < count ? s[i][r] : -INFINITY;
              mloc = fmaxf(mloc, s[i][r]);
            }
        }
        mloc = max_lane_xor32(mloc);
        // keep the reference max unless it would let exponents exceed 2^kRescale
        const bool grow = (mloc - m_run) * p.scale_log2 > kRescale;
        if (__builtin_amdgcn_ballot_w64(grow)) {
          const float m_new = grow ? mloc : m_run;
          const float alpha = grow ? __builtin_amdgcn_exp2f((m_run - m_new) * p.scale_log2) : 1.0f;
          l_run *= alpha;
#pragma unroll
          for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) o[dt][r] *= alpha;
          m_run = m_new;
        }
        const float neg_m = m_run == -INFINITY ? 0.f : -m_run * p.scale_log2;
#pragma unroll
        for (int i = 0; i < NKB; ++i)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float e = __builtin_amdgcn_exp2f(fmaf(s[i][r], p.scale_log2, neg_m));
            s[i][r] = e;
            l_run += e;
          }
        // P in fp16 (values in [0, 2^kRescale]; 11 significant bits) against
        // the fp16 values, which hold the bf16-rounded V exactly
#pragma unroll
        for (int i = 0; i < NKB; ++i)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            f16x8_t pf;
#pragma unroll
            for (int e = 0; e < 8; ++e) pf[e] = (_Float16)s[i][h * 8 + e];
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
              o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(Vh[vslot(dt * 32 + lq, (kb0 + i) * 4 + h * 2 + lg)],
                                                             pf, o[dt], 0, 0, 0);
          }
      }
    }
  };
  if (tail)
    run(std::integral_constant<int, 1>{}, std::integral_constant<int, TST>{}, wave & 1);
  else
    run(std::integral_constant<int, 2>{}, std::integral_constant<int, AST>{}, 0);

  if (tail) {
    // Wave 1 hands its (m, l, O) for the other half of the keys to wave 0
    // through a ring stage that no wave reads any more (the last tile used
    // stage (n - 1) % TST, and every wave has passed the barrier that ended
    // the tile before it).
    float* xch = (float*)(lds + ((t1 - t0) % TST) * ASTAGE);
    if (wave == 1) {
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) xch[(dt * 16 + r) * 64 + lane] = o[dt][r];
      xch[64 * 64 + lane] = m_run;
      xch[65 * 64 + lane] = l_run;
    }
    wait_lgkm0();
    barrier_nofence();
    if (wave != 0) return;
    const float m1 = xch[64 * 64 + lane], l1 = xch[65 * 64 + lane];
    const float mm = fmaxf(m_run, m1);
    const float a0 = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m_run - mm) * p.scale_log2);
    const float a1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m1 - mm) * p.scale_log2);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[dt][r] = o[dt][r] * a0 + xch[(dt * 16 + r) * 64 + lane] * a1;
    l_run = l_run * a0 + l1 * a1;
    m_run = mm;
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
    // The split's output is stored normalised and scaled into [-1, 1] by its
    // row's largest magnitude c, in fp16: 11 significant bits relative to c,
    // finer than the bf16 output it becomes, in half the bytes of f32.
    const size_t row = (((size_t)sp * p.B + b) * p.nq + head) * p.L + l;
    float amax = 0.f;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int r = 0; r < 16; ++r) amax = fmaxf(amax, fabsf(o[dt][r]));
    amax = fmaxf(amax, __shfl_xor(amax, 32));  // the row's other 64 dims
    const float c = amax > 0.f ? amax / l_tot : 1.0f;
    const float inv = amax > 0.f ? 1.0f / amax : 1.0f;
    uint16_t* dst = p.opart + row * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d0 = dt * 32 + q4 * 8 + lg * 4;
        u32x2_t w;
        w[0] = pack_f16x2(o[dt][q4 * 4 + 0] * inv, o[dt][q4 * 4 + 1] * inv);
        w[1] = pack_f16x2(o[dt][q4 * 4 + 2] * inv, o[dt][q4 * 4 + 3] * inv);
        *(u32x2_t*)(dst + d0) = w;
      }
    if (lg == 0) {
      *(f32x4_t*)(p.mlpart + row * 4) = f32x4_t{m_run * p.scale_log2, l_tot, c, 0.f};
      // the tail tile fills fewer slots: its first split marks the rest empty
      if (tail && sp == 0) {
        const size_t rows = (size_t)p.B * p.nq * p.L;
        for (int s2 = ns; s2 < p.splits; ++s2)
          *(f32x4_t*)(p.mlpart + (row + s2 * rows) * 4) = f32x4_t{-INFINITY, 0.f, 1.f, 0.f};
      }
    }
  }
}

// Merges split partials: O = sum_s 2^(m_s - M) O_s / sum_s 2^(m_s - M) l_s, where
// m_s is each split's reference max (log2 units) and O_s = l_s c_s x_s with
// x_s the stored fp16 values.  16 rows per workgroup, 8 dims per thread (one
// 16-byte load per split, one 16-byte bf16 store); the NS splits' loads are
// all issued before any use.
template <int NS>
__global__ __launch_bounds__(256) void attn_combine_kernel(const uint16_t* __restrict__ opart,
                                                           const float* __restrict__ ml, int B, int nq, int L,
                                                           bf16_t* __restrict__ o) {
  const size_t rows = (size_t)B * nq * L;
  const size_t row = (size_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  if (row >= rows) return;
  const int d0 = (threadIdx.x & 15) * 8;
  const int l = (int)(row % L);
  const size_t bh = row / L;
  const int head = (int)(bh % nq), b = (int)(bh / nq);
  float ms[NS], ls[NS], cs[NS];
  u32x4_t v[NS];
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    const f32x4_t x = *(const f32x4_t*)(ml + (s * rows + row) * 4);
    ms[s] = x[0];
    ls[s] = x[1];
    cs[s] = x[2];
    v[s] = *(const u32x4_t*)(opart + (s * rows + row) * D + d0);
  }
  float M = -INFINITY;
#pragma unroll
  for (int s = 0; s < NS; ++s) M = fmaxf(M, ms[s]);
  float den = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < NS; ++s) {
    if (ms[s] == -INFINITY) continue;
    const float w = __builtin_amdgcn_exp2f(ms[s] - M);
    den += w * ls[s];
    const float wl = w * ls[s] * cs[s];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      acc[2 * j] += wl * f16lo(v[s][j]);
      acc[2 * j + 1] += wl * f16hi(v[s][j]);
    }
  }
  const float inv = 1.0f / den;
  u32x4_t w;
#pragma unroll
  for (int j = 0; j < 4; ++j) w[j] = pack_bf16x2(acc[2 * j] * inv, acc[2 * j + 1] * inv);
  *(u32x4_t*)(o + ((size_t)b * L + l) * (size_t)(nq * D) + (size_t)head * D + d0) = w;
}

// ---- f32 path: one wave per (b, head, query); keys split over lanes ------------------------
template <int DD>
__global__ __launch_bounds__(64) void attn_f32_kernel(const float* __restrict__ q, const float* __restrict__ kb,
                                                      const float* __restrict__ vbt, const float* __restrict__ ck,
                                                      const float* __restrict__ cvt, float* __restrict__ o,
                                                      int B, int L, int Lp, int C, int cap, int nq, int nkv,
                                                      int ctx_bstride, float scale) {
  __shared__ float red_o[64][DD + 1];
  __shared__ float red_m[64], red_l[64];
  const int lane = threadIdx.x;
  const int row = blockIdx.x;  // (b, head, l)
  const int l = row % L, bh = row / L, head = bh % nq, b = bh / nq;
  const int j = (head * nkv) / nq;
  const size_t bhk = (size_t)b * nkv + j;
  const size_t cbhk = (size_t)b * ctx_bstride * nkv + j;  // context segment (shared: b = 0)
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
      kp = ck + (cbhk * cap + key) * DD;
      vp = cvt + cbhk * DD * cap + key;
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

// Work split of the bf16 attention.
struct AttnPlan {
  int q_tiles = 1;      // 8-wave query tiles per (b, kv head)
  int splits = 1;       // their key splits = partial slots per row
  int tail_splits = 0;  // key splits of the tail tile, 0 = no tail tile
};

AttnPlan attn_plan(int B, int L, int C, int nq, int nkv) {
  const int g = nq / nkv;
  const int R = g * L;
  const int q_tiles = (R + QROWS - 1) / QROWS;
  const int tiles = (C + KT - 1) / KT + (L + KT - 1) / KT;
  const int base = q_tiles * B * nkv;
  // one workgroup per CU: split the keys until the grid would exceed one
  // pass over the 256 CUs (more splits only add combine traffic), keeping at
  // least two key tiles per split (one-tile splits write a partial O per
  // tile: slower on short blocks over 2,048 keys, measured)
  AttnPlan pl;
  pl.q_tiles = q_tiles;
  while (base * pl.splits * 2 <= 256 && pl.splits * 2 * 2 <= tiles && pl.splits < 32) pl.splits *= 2;
  // A last tile of at most 32 rows (one busy wave) goes to tail workgroups
  // with two key splits, whose two waves (one per SIMD) each take half of
  // every key tile; the full tiles then split as far as the pass allows.
  // Up to 7 splits the tail's 2 * 850-cycle half tiles finish before the
  // full tiles' 3,300-cycle tiles (two waves per SIMD).
  const int rt = R - (q_tiles - 1) * QROWS;
  if (q_tiles >= 2 && rt <= 32) {
    const int nf = (q_tiles - 1) * B * nkv, nt = B * nkv, ts = 2;
    int s = (256 - nt * ts) / nf;
    s = std::min(s, std::min(tiles / 2, 7));
    if (s > pl.splits && s >= ts) {
      pl.q_tiles = q_tiles - 1;
      pl.splits = s;
      pl.tail_splits = ts;
    }
  }
  return pl;
}

}  // namespace

size_t attention_scratch_bytes(int dt, int B, int L, int C, int nq, int nkv, int d) {
  if (dt != FPD_DTYPE_BF16) return 0;
  const int s = attn_plan(B, L, C, nq, nkv).splits;
  if (s == 1) return 0;
  const size_t rows = (size_t)s * B * nq * L;
  return rows * d * sizeof(uint16_t) + rows * 4 * sizeof(float);
}

hipError_t attention(int dt, const AttnArgs& a, void* scratch, size_t scratch_bytes, hipStream_t st) {
  if (dt == FPD_DTYPE_BF16) {
    AttnP p{};
    p.q = (const bf16_t*)a.q;
    p.kb = (const bf16_t*)a.kb;
    p.vbt = (const uint16_t*)a.vbt;
    p.ck = (const bf16_t*)a.ck;
    p.cvt = (const uint16_t*)a.cvt;
    p.o = (bf16_t*)a.o;
    p.B = a.B, p.L = a.L, p.Lp = a.Lp, p.C = a.C, p.cap = a.cap, p.nq = a.nq, p.nkv = a.nkv;
    p.ctx_bstride = a.ctx_bstride;
    p.g = a.nq / a.nkv;
    p.R = p.g * a.L;
    const AttnPlan pl = attn_plan(a.B, a.L, a.C, a.nq, a.nkv);
    p.q_tiles = pl.q_tiles;
    p.splits = pl.splits;
    p.tail_splits = pl.tail_splits;
    const size_t rows = (size_t)p.splits * a.B * a.nq * a.L;
    if (p.splits > 1 && rows * (D * sizeof(uint16_t) + 4 * sizeof(float)) > scratch_bytes) {
      // no room for the partials: one workgroup per query tile covers every key
      p.q_tiles = (p.R + QROWS - 1) / QROWS;
      p.splits = 1;
      p.tail_splits = 0;
    }
    p.ctx_tiles = (a.C + KT - 1) / KT;
    p.blk_tiles = (a.L + KT - 1) / KT;
    p.opart = (uint16_t*)scratch;
    p.mlpart = (float*)((uint16_t*)scratch + rows * D);
    p.scale_log2 = a.scale * 1.4426950408889634f;
    const int grid = (p.q_tiles * p.splits + p.tail_splits) * a.B * a.nkv;
    {
      ProfScope prof("attention", st);
      hipLaunchKernelGGL(attn_bf16_kernel, dim3(grid), dim3(AW * 64), 0, st, p);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.splits == 1) return e;
    ProfScope prof("attn_combine", st);
    const size_t nrows = (size_t)a.B * a.nq * a.L;
    const dim3 cg((unsigned)((nrows + 15) / 16));
    switch (p.splits) {
#define FPD_COMB(NS)                                                                                            \
  case NS:                                                                                                      \
    hipLaunchKernelGGL((attn_combine_kernel<NS>), cg, dim3(256), 0, st, p.opart, p.mlpart, a.B, a.nq, a.L,       \
                       (bf16_t*)a.o);                                                                          \
    break;
      FPD_COMB(2)
      FPD_COMB(3)
      FPD_COMB(4)
      FPD_COMB(5)
      FPD_COMB(6)
      FPD_COMB(7)
      FPD_COMB(8)
      FPD_COMB(16)
      FPD_COMB(32)
#undef FPD_COMB
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  const int rows = a.B * a.nq * a.L;
  ProfScope prof("attention", st);
  if (a.d == 64)
    hipLaunchKernelGGL(attn_f32_kernel<64>, dim3(rows), dim3(64), 0, st, (const float*)a.q,
                       (const float*)a.kb, (const float*)a.vbt, (const float*)a.ck, (const float*)a.cvt,
                       (float*)a.o, a.B, a.L, a.Lp, a.C, a.cap, a.nq, a.nkv, a.ctx_bstride, a.scale);
  else
    hipLaunchKernelGGL(attn_f32_kernel<128>, dim3(rows), dim3(64), 0, st, (const float*)a.q,
                       (const float*)a.kb, (const float*)a.vbt, (const float*)a.ck, (const float*)a.cvt,
                       (float*)a.o, a.B, a.L, a.Lp, a.C, a.cap, a.nq, a.nkv, a.ctx_bstride, a.scale);
  return hipGetLastError();
}

}  // namespace fpd
