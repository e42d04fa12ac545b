// Dense projections of the drafter: Y = A W^T with fused epilogues.
//
// bf16 path: MFMA 32x32x16 (gfx950) tiles, A and W both K-contiguous,
// streamed global -> LDS through a 2-4 stage ring of LDS-writing buffer loads
// (one barrier per K-tile), split-K with a fixed-order reduction when the
// tile count alone cannot fill 256 CUs, an XCD-aware tile order so the
// workgroups that share a weight tile run on the same XCD, and a last row
// tile that can carry up to 16 leftover rows.  W is read row-major or from
// its K-tile-contiguous copy (Wt::tiled: each 32-row group's 64-deep K-tiles
// back to back), which changes only the load addresses.
//
// "Paired" epilogues need two W rows per output (RoPE rotates column i with
// column i + d/2 of a head; SwiGLU combines gate row i with up row I + i).
// Their B tile holds the first members in its first half and the second
// members in its second half, and each wave takes matching sub-tiles from
// both halves, so a lane holds both members of every pair in registers.
#include <algorithm>
#include <type_traits>

#include "../../include/fpd.h"
#include "kernels.h"
#include "lds_pipe.h"

namespace fpd {

namespace {

constexpr int BK = 64;

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
// Plain epilogues store (EpiStore) or add into (EpiResid, kRmw) an f32
// matrix.  Paired epilogues split into col(p), the per-column state a lane
// computes once for the column pairs it holds, and pair(m, col, x0, x1) per
// row, so that nothing per column is re-read after the stores of earlier
// rows (a lane-indexed kernel-argument table would otherwise be re-loaded,
// one memory round trip per output pair).
struct EpiStore {
  static constexpr bool kRmw = false;
  float* out;
  int ld;
  __device__ float load(int, int) const { return 0.f; }
  __device__ void store(int m, int n, float v) const { out[(size_t)m * ld + n] = v; }
  __device__ void operator()(int m, int n, float v) const { store(m, n, v); }
};
struct EpiResid {
  static constexpr bool kRmw = true;
  float* h;
  int ld;
  __device__ float load(int m, int n) const { return h[(size_t)m * ld + n]; }
  __device__ void store(int m, int n, float v) const { h[(size_t)m * ld + n] = v; }
  __device__ void operator()(int m, int n, float v) const { h[(size_t)m * ld + n] += v; }
};

template <class T>
struct EpiQkv {
  T *q, *k, *vt;
  int L, Lp, nq, nkv, d, half, pos0, rope;
  RopeTab tab;
  float inv_L;  // 1 / L (rows m < 2^24 split into (b, l) by divmod_rows)
  struct Col {
    int head, i;
    double inv_rev;
    float cd, sd;  // cos, sin of one position step
  };
  __device__ Col col(int p) const {
    const int i = p % half;
    const float st = (float)tab.inv_rev[i];
    return Col{p / half, i, tab.inv_rev[i], __builtin_amdgcn_cosf(st), __builtin_amdgcn_sinf(st)};
  }
  // Four consecutive rows m0 .. m0 + nv - 1 (nv <= 4) of one column pair:
  // within one request the row offset, the output addresses and the
  // rotation advance by one step per row (the angle of the first row is
  // evaluated, the next three follow by rotating it, ~1e-7 apart).
  __device__ void pair4(int m0, int nv, const Col& c, f32x4_t x0, f32x4_t x1) const {
    int b, l;
    divmod_rows(m0, L, inv_L, b, l);
    if (nv < 4 || l + 3 >= L) {
      for (int r = 0; r < nv; ++r) pair(m0 + r, c, x0[r], x1[r]);
      return;
    }
    if (c.head < nq + nkv) {
      if (rope) {
        float cs, sn;
        rope_cs(pos0 + l, c.inv_rev, cs, sn);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float a0 = x0[r], a1 = x1[r];
          rope_rot(a0, a1, cs, sn);
          x0[r] = a0;
          x1[r] = a1;
          if (r < 3) rope_step(cs, sn, c.cd, c.sd);
        }
      }
      T* dst = (c.head < nq ? q + (((size_t)b * nq + c.head) * L + l) * d
                            : k + (((size_t)b * nkv + (c.head - nq)) * L + l) * d) + c.i;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        Elem<T>::st(dst + (size_t)r * d, x0[r]);
        Elem<T>::st(dst + (size_t)r * d + half, x1[r]);
      }
    } else {
      T* dst = vt + (((size_t)b * nkv + (c.head - nq - nkv)) * d + c.i) * Lp + l;
      T* dst1 = dst + (size_t)half * Lp;
      if constexpr (sizeof(T) == 2) {
        if ((l & 3) == 0 && (Lp & 3) == 0) {  // four values of a d-major row: one 8-byte store each
          u32x2_t w0, w1;
          w0[0] = ValueStore<T>::bits(x0[0]) | ((uint32_t)ValueStore<T>::bits(x0[1]) << 16);
          w0[1] = ValueStore<T>::bits(x0[2]) | ((uint32_t)ValueStore<T>::bits(x0[3]) << 16);
          w1[0] = ValueStore<T>::bits(x1[0]) | ((uint32_t)ValueStore<T>::bits(x1[1]) << 16);
          w1[1] = ValueStore<T>::bits(x1[2]) | ((uint32_t)ValueStore<T>::bits(x1[3]) << 16);
          *(u32x2_t*)dst = w0;
          *(u32x2_t*)dst1 = w1;
          return;
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        ValueStore<T>::st(dst + r, x0[r]);
        ValueStore<T>::st(dst1 + r, x1[r]);
      }
    }
  }
  __device__ void pair(int m, const Col& c, float x0, float x1) const {
    int b, l;
    divmod_rows(m, L, inv_L, b, l);
    if (c.head < nq + nkv) {
      if (rope) rope_pair(x0, x1, pos0 + l, c.inv_rev);
      T* dst = c.head < nq ? q + (((size_t)b * nq + c.head) * L + l) * d
                           : k + (((size_t)b * nkv + (c.head - nq)) * L + l) * d;
      Elem<T>::st(dst + c.i, x0);
      Elem<T>::st(dst + c.i + half, x1);
    } else {
      T* dst = vt + ((size_t)b * nkv + (c.head - nq - nkv)) * d * Lp + l;
      ValueStore<T>::st(dst + (size_t)c.i * Lp, x0);
      ValueStore<T>::st(dst + (size_t)(c.i + half) * Lp, x1);
    }
  }
  __device__ void pair(int m, int p, float x0, float x1) const { pair(m, col(p), x0, x1); }
};

template <class T>
struct EpiCtx {
  T *k, *vt;
  int C, cap, nkv, d, half, pos0, rope;
  RopeTab tab;
  float inv_C;  // 1 / C
  struct Col {
    int head, i;
    double inv_rev;
    float cd, sd;  // cos, sin of one position step
  };
  __device__ Col col(int p) const {
    const int i = p % half;
    const float st = (float)tab.inv_rev[i];
    return Col{p / half, i, tab.inv_rev[i], __builtin_amdgcn_cosf(st), __builtin_amdgcn_sinf(st)};
  }
  // Four consecutive rows (as EpiQkv::pair4).
  __device__ void pair4(int m0, int nv, const Col& cc, f32x4_t x0, f32x4_t x1) const {
    int b, c;
    divmod_rows(m0, C, inv_C, b, c);
    if (nv < 4 || c + 3 >= C) {
      for (int r = 0; r < nv; ++r) pair(m0 + r, cc, x0[r], x1[r]);
      return;
    }
    if (cc.head < nkv) {
      if (rope) {
        float cs, sn;
        rope_cs(pos0 + c, cc.inv_rev, cs, sn);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float a0 = x0[r], a1 = x1[r];
          rope_rot(a0, a1, cs, sn);
          x0[r] = a0;
          x1[r] = a1;
          if (r < 3) rope_step(cs, sn, cc.cd, cc.sd);
        }
      }
      T* dst = k + (((size_t)b * nkv + cc.head) * cap + c) * d + cc.i;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        Elem<T>::st(dst + (size_t)r * d, x0[r]);
        Elem<T>::st(dst + (size_t)r * d + half, x1[r]);
      }
    } else {
      T* dst = vt + (((size_t)b * nkv + (cc.head - nkv)) * d + cc.i) * cap + c;
      T* dst1 = dst + (size_t)half * cap;
      if constexpr (sizeof(T) == 2) {
        if ((c & 3) == 0 && (cap & 3) == 0) {
          u32x2_t w0, w1;
          w0[0] = ValueStore<T>::bits(x0[0]) | ((uint32_t)ValueStore<T>::bits(x0[1]) << 16);
          w0[1] = ValueStore<T>::bits(x0[2]) | ((uint32_t)ValueStore<T>::bits(x0[3]) << 16);
          w1[0] = ValueStore<T>::bits(x1[0]) | ((uint32_t)ValueStore<T>::bits(x1[1]) << 16);
          w1[1] = ValueStore<T>::bits(x1[2]) | ((uint32_t)ValueStore<T>::bits(x1[3]) << 16);
          *(u32x2_t*)dst = w0;
          *(u32x2_t*)dst1 = w1;
          return;
        }
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        ValueStore<T>::st(dst + r, x0[r]);
        ValueStore<T>::st(dst1 + r, x1[r]);
      }
    }
  }
  __device__ void pair(int m, const Col& cc, float x0, float x1) const {
    int b, c;
    divmod_rows(m, C, inv_C, b, c);
    if (cc.head < nkv) {
      if (rope) rope_pair(x0, x1, pos0 + c, cc.inv_rev);
      T* dst = k + (((size_t)b * nkv + cc.head) * cap + c) * d;
      Elem<T>::st(dst + cc.i, x0);
      Elem<T>::st(dst + cc.i + half, x1);
    } else {
      T* dst = vt + ((size_t)b * nkv + (cc.head - nkv)) * d * cap + c;
      ValueStore<T>::st(dst + (size_t)cc.i * cap, x0);
      ValueStore<T>::st(dst + (size_t)(cc.i + half) * cap, x1);
    }
  }
  __device__ void pair(int m, int p, float x0, float x1) const { pair(m, col(p), x0, x1); }
};

template <class T>
struct EpiGlu {
  T* u;
  int I;
  using Col = int;
  __device__ Col col(int p) const { return p; }
  __device__ void pair(int m, int p, float g, float up) const {
    Elem<T>::st(u + (size_t)m * I + p, silu_f(g) * up);
  }
  __device__ void pair4(int m0, int nv, int p, f32x4_t g, f32x4_t up) const {
    T* dst = u + (size_t)m0 * I + p;
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (r < nv) Elem<T>::st(dst + (size_t)r * I, silu_f(g[r]) * up[r]);
  }
};

// Maps the launch index to a tile (row tile fastest, then column tile, then
// K split).  Each XCD runs one contiguous range of tiles (workgroups are
// dispatched to XCDs round-robin), so the row tiles that share a weight tile
// meet in that XCD's L2.  Within the range, tiles whose rows all lie below M
// go first and the last, partly filled row tile of each column (cheap: its
// empty row blocks are skipped) goes last, where it fills the gaps the full
// tiles leave.  m_full = number of full row tiles (m_tiles or m_tiles - 1).
//
// With many row tiles (kGroupMinRows or more, all full) the range instead
// walks groups of kGroupRows row tiles across every column tile, so that the
// ~32 tiles an XCD runs at once are 4 row tiles x 8 column tiles: each A
// K-slab is then read by 8 tiles and each weight K-slab by 4 out of that L2,
// where row tiles first would have 32 tiles stream 32 different A slabs past
// one weight slab, re-reading all of A once per column tile.
constexpr int kGroupRows = 4;
constexpr int kGroupMinRows = 16;
__device__ __forceinline__ int gemm_tile_order(int bid, int grid, int m_tiles, int m_full, int n_tiles) {
  const int x = bid % kXcds, local = bid / kXcds;
  const int per = grid / kXcds, rem = grid % kXcds;
  const int s = x * per + (x < rem ? x : rem);
  const int cnt = per + (x < rem ? 1 : 0);
  if (m_full == m_tiles) {
    const int t = s + local;
    if (m_tiles < kGroupMinRows) return t;
    const int mn = m_tiles * n_tiles, ks = t / mn, r = t % mn;
    const int g = r / (kGroupRows * n_tiles), w = r % (kGroupRows * n_tiles);
    const int gm = min(kGroupRows, m_tiles - g * kGroupRows);  // row tiles of this group
    return ks * mn + (w / gm) * m_tiles + g * kGroupRows + w % gm;
  }
  auto full_before = [&](int t) { return (t / m_tiles) * m_full + min(t % m_tiles, m_full); };
  const int h0 = full_before(s), h1 = full_before(s + cnt);
  if (local < h1 - h0) {
    const int i = h0 + local;
    return (i / m_full) * m_tiles + i % m_full;
  }
  return (s - h0 + local - (h1 - h0)) * m_tiles + m_full;
}

// ---- bf16 MFMA kernel ---------------------------------------------------------
// Operand tiles go global -> LDS directly (an LDS-writing buffer load: lane i
// of a wave instruction fills 16-byte slot base + i) through a STAGES-deep
// ring, so several K-tiles are in flight per workgroup without register
// staging.
// A tile row (BK bf16 = CH chunks of 16 bytes) keeps chunk c at position
// c ^ ((row / (16 / CH)) % CH): the MFMA operand reads (16 rows x 16 bytes
// per LDS cycle) then hit distinct banks.  The swizzle is applied by choosing which
// global chunk each lane loads.  Lanes whose row lies outside the problem
// load a clamped in-range row instead of being switched off, so every loading
// wave issues the same number of loads per stage and vmcnt counts stay exact; the
// outputs of those rows/columns are never stored.
//
// When M = k BM + r with 0 < r <= XR, the last row tile also carries the r
// leftover rows (an (XR x BK) A slab after its BM rows in each stage, filled
// by one 16-byte LDS-writing load per loading wave, multiplied by 16x16x32
// MFMAs whose columns are split over all waves).  A separate row tile for
// them would stream the whole weight column once more from HBM for r rows of
// work.  Two 4-byte loads per wave filled the slab at first: the same bytes,
// but twice the load instructions, and the 385-row gate/up projection took
// ~1 us longer per launch.
//
// Addressing of the A operand (byte offsets for the buffer loads: a per-row
// part fixed per lane, and a per-K-tile part that is scalar).  APlain: row-
// major A [M, K], row m at m * lda.  AFused: the per-layer target features
// [B, n_t, C, H] read in place as their concatenation [B * C, n_t * H] (row
// b * C + c, column t * H + k; lda = n_t * H), which the context fusion's
// projection would otherwise copy out first (a 64-deep K tile never crosses
// a layer, since H is a multiple of 64).  Both parts are unsigned 32-bit
// byte offsets (operands stay under 4 GiB), added by the hardware.
struct APlain {
  __device__ uint32_t row(int m, int lda) const { return (uint32_t)((size_t)m * lda * 2); }
  __device__ uint32_t ktile(int kt, int bk) const { return (uint32_t)(kt * bk * 2); }
};
struct AFused {
  int C, H;  // positions per request, columns of one target layer
  __device__ uint32_t row(int m, int lda) const {
    return (uint32_t)(((size_t)(m / C) * C * lda + (size_t)(m % C) * H) * 2);
  }
  __device__ uint32_t ktile(int kt, int bk) const {
    const int k = kt * bk;
    return (uint32_t)(((size_t)(k / H) * C * H + k % H) * 2);
  }
};

template <int BM, int BN, int BK, int WAVES_M, int WAVES_N, int STAGES, int XR, bool PAIRED, class Map, class Epi,
          class ALay = APlain>
__global__ __launch_bounds__(64 * WAVES_M* WAVES_N) void gemm_bf16_kernel(
    const bf16_t* __restrict__ A, int lda, int M, int K, const bf16_t* __restrict__ W, int w_rows, int w_tiled,
    Map map, int ncols, Epi epi, float* __restrict__ partial, int part_ld, int m_tiles, int n_tiles,
    int splits, ALay alay = {}) {
  constexpr int NW = WAVES_M * WAVES_N;
  constexpr int NT = 64 * NW;
  // Waves that fill the ring.  In 8-wave workgroups only waves 0-3 (one per
  // SIMD) issue the loads and wait for them: the other wave of each SIMD keeps
  // issuing MFMAs meanwhile (2-4% faster than all eight loading; 4-wave
  // workgroups were slower that way).
  constexpr int LW = NW == 8 ? NW / 2 : NW;
  constexpr int LT = 64 * LW;
  constexpr int WM = BM / WAVES_M, WN = BN / WAVES_N;
  constexpr int TM = WM / 32, TN = WN / 32;
  constexpr int CH = BK / 8;        // 16-byte chunks per tile row
  constexpr int AI = BM * CH / LT;  // load instructions per wave and stage (A)
  constexpr int BI = BN * CH / LT;  // (B)
  constexpr int LPS = AI + BI;
  static_assert(BK == 32 || BK == 64, "K tile");
  static_assert(TM >= 1 && TN >= 1 && AI >= 1 && BI >= 1 && BM * CH % LT == 0 && BN * CH % LT == 0, "tile shape");
  static_assert(!PAIRED || (TN % 2 == 0), "paired epilogues need an even number of N sub-tiles");
  static_assert(STAGES >= 2 && STAGES <= 8 && LPS * (STAGES - 1) < 64, "pipeline depth");
  constexpr int CPT = PAIRED ? BN / 2 : BN;  // logical columns per tile
  static_assert(XR == 0 || XR == gemm_extra_rows(BM, BN, BK, NW, PAIRED), "extra rows of this tile shape");
  constexpr int XB = XR ? CPT / (NW * 16) : 0;  // 16-column blocks (pairs when PAIRED) per wave
  constexpr int XA = PAIRED ? 2 * XB : XB;      // their accumulators
  // the extra rows' 128 slots per stage: one 16-byte load per loading wave,
  // waves 2 and 3 repeating the loads of waves 0 and 1
  static_assert(XR == 0 || (XR * CH == 128 && LW % 2 == 0 && XB * NW * 16 == CPT), "extra rows");
  constexpr int AR = BM + XR;                // A rows held per stage
  constexpr int STAGE = (AR + BN) * CH;      // 16-byte slots per stage

  __shared__ u32x4_t lds[STAGES * STAGE];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WAVES_N, wn = wave % WAVES_N;
  const bool loader = wave < LW;
  const int tile = gemm_tile_order(blockIdx.x, gridDim.x, m_tiles, M / BM, n_tiles);
  const int mt = tile % m_tiles;
  const int rest = tile / m_tiles;
  const int nt = rest % n_tiles;
  const int ks = rest / n_tiles;
  const int m0 = mt * BM, c0 = nt * CPT;
  const int KT = K / BK;
  const int kt0 = (int)((long)ks * KT / splits), kt1 = (int)((long)(ks + 1) * KT / splits);
  // only the plan's last row tile carries the rows past m_tiles * BM (any
  // other tile would compute the next tile's first rows a second time, and a
  // residual epilogue would add them twice)
  const bool ext = XR > 0 && mt == m_tiles - 1 && m0 + BM < M;

  // Operands are read through buffer descriptors: the per-lane byte offset
  // (row and swizzled chunk) is fixed, the K-tile offset is a scalar.  The
  // LDS-writing buffer load is also what lets the compiler keep its LDS read
  // waits partial (an LDS-writing global load counts as a flat access, which
  // forces a full LDS wait before every MFMA group).
  const __amdgpu_buffer_rsrc_t arsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)A, (short)0, (int)((size_t)M * lda * 2), 0x00020000);
  // W row-major, or K-tile-contiguous (w_tiled: each 32-row group's 64-deep
  // K-tiles one after another, rows padded to 32)
  const __amdgpu_buffer_rsrc_t brsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)W, (short)0, (int)((size_t)(w_tiled ? (w_rows + 31) / 32 * 32 : w_rows) * K * 2), 0x00020000);
  uint32_t aoff[AI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int sl = (wave * AI + i) * 64 + lane, r = sl / CH, c = (sl % CH) ^ ((r / (16 / CH)) & (CH - 1));
    const int m = min(m0 + r, M - 1);
    aoff[i] = alay.row(m, lda) + (uint32_t)(c * 16);
  }
  uint32_t boff[BI];
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    const int sl = (wave * BI + i) * 64 + lane, r = sl / CH, c = (sl % CH) ^ ((r / (16 / CH)) & (CH - 1));
    int wrow;
    if constexpr (PAIRED) {
      const int pidx = min(c0 + (r % (BN / 2)), ncols - 1);
      wrow = r < BN / 2 ? map.first(pidx) : map.second(pidx);
    } else {
      wrow = map.row(min(c0 + r, ncols - 1));
    }
    boff[i] = w_tiled ? (uint32_t)((((size_t)(wrow / 32) * (K / 64) * 32 + wrow % 32) * 64 + c * 8) * 2)
                      : (uint32_t)(((size_t)wrow * K + c * 8) * 2);
  }
  // extra rows: lane l of a loading wave fills slot (wave & 1) * 64 + l of
  // the XR x BK slab (rows past M clamped to M - 1, so two waves that fill
  // the same slots write the same bytes)
  uint32_t xoff;
  {
    const int q = (wave & 1) * 64 + lane, r = BM + q / CH;
    const int c = (q % CH) ^ ((r / (16 / CH)) & (CH - 1));
    xoff = alay.row(min(m0 + r, M - 1), lda) + (uint32_t)(c * 16);
  }
  // With one row tile every weight tile is read by one workgroup only: the
  // small-row tiles then load it non-temporal (trajectory L = 25 block
  // 0.450 -> 0.440 ms).  Where row tiles share weight tiles through L2 the
  // same hint cost 5% (L = 385), so larger tiles keep the default policy.
  const bool w_once = BM <= 64 && m_tiles == 1;
  auto issue = [&](int kt, int stage, auto ext_c) {
    const int soff = (int)alay.ktile(kt, BK);  // the same 32 bits as a scalar offset
    const int k0 = kt * BK, sb = w_tiled ? (k0 / 64) * 4096 + (k0 % 64) * 2 : k0 * 2;
    if (!loader) return;
    u32x4_t* base = lds + stage * STAGE;
#pragma unroll
    for (int i = 0; i < AI; ++i) lds_dma16(arsrc, base + (wave * AI + i) * 64, aoff[i], soff);
    if (w_once) {
#pragma unroll
      for (int i = 0; i < BI; ++i)
        lds_dma16<kLoadNonTemporal>(brsrc, base + AR * CH + (wave * BI + i) * 64, boff[i], sb);
    } else {
#pragma unroll
      for (int i = 0; i < BI; ++i) lds_dma16(brsrc, base + AR * CH + (wave * BI + i) * 64, boff[i], sb);
    }
    if constexpr (decltype(ext_c)::value) {
      lds_dma16(arsrc, base + BM * CH + (wave & 1) * 64, xoff, soff);
    }
  };

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;
  f32x4_t xacc[XA > 0 ? XA : 1];
#pragma unroll
  for (int b = 0; b < (XA > 0 ? XA : 1); ++b)
#pragma unroll
    for (int r = 0; r < 4; ++r) xacc[b][r] = 0.f;
  // first column (pair index when PAIRED) of this wave's extra-row blocks;
  // block b covers xcol0 + 16 b .. + 15 (PAIRED: first members there, second
  // members at BN / 2 + the same offset)
  const int xcol0 = wave * 16 * XB;

  int bcol[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    if constexpr (PAIRED)
      bcol[j] = j < TN / 2 ? wn * (WN / 2) + j * 32 : BN / 2 + wn * (WN / 2) + (j - TN / 2) * 32;
    else
      bcol[j] = wn * WN + j * 32;
  }
  const int lr = lane & 31, lk = lane >> 5;

  // Row blocks of this wave that contain rows below M (wave-uniform).  The
  // blocks past M are neither read nor multiplied (their outputs are never
  // stored), so a tile that only covers the last rows of M costs a fraction
  // of a full tile; its waves still take part in the loads and barriers.
  const int rows_left = M - (m0 + wm * WM);
  const int nr = rows_left >= WM ? TM : (rows_left <= 0 ? 0 : (rows_left + 31) / 32);

  // The ring holds STAGES K-tiles.  Within a K-tile the operand fragments of
  // step kk+1 are read from LDS while the MFMAs of step kk run (two register
  // sets, order pinned by scheduling barriers).  At the last step each wave
  // drains its own LDS reads and each loading wave waits for its loads of the
  // next K-tile; one
  // barrier then hands the finished stage back to the loads (K-tile kt +
  // STAGES goes into it) and publishes the next K-tile, whose first fragments
  // are read before the last MFMAs of the current one.
  auto mainloop = [&](auto nr_c, auto ext_c) {
    constexpr int NR = decltype(nr_c)::value;
    constexpr bool EXT = decltype(ext_c)::value;
    constexpr int LPSX = LPS + (EXT ? 1 : 0);  // loads per wave and stage
    constexpr int KS = BK / 16;
    bf16x8_t af[2][TM > 0 ? TM : 1], bfv[2][TN];
    // extra rows: fragments of the two 32-deep K steps of a K-tile (j = kk / 2)
    bf16x8_t xa[2], xb[2][XA > 0 ? XA : 1];
#pragma unroll
    for (int s = 0; s < STAGES; ++s)
      if (kt0 + s < kt1) issue(kt0 + s, s, ext_c);
    auto fetch = [&](int stage, int kk, int buf) {
      const u32x4_t* As = lds + stage * STAGE;
      const u32x4_t* Bs = As + AR * CH;
      if constexpr (NR > 0) {
#pragma unroll
        for (int i = 0; i < NR; ++i)
          af[buf][i] = __builtin_bit_cast(bf16x8_t, As[swz<CH>(wm * WM + i * 32 + lr, kk * 2 + lk)]);
#pragma unroll
        for (int j = 0; j < TN; ++j) bfv[buf][j] = __builtin_bit_cast(bf16x8_t, Bs[swz<CH>(bcol[j] + lr, kk * 2 + lk)]);
      }
      if constexpr (EXT) {
        if (kk % 2 == 0) {  // 16x16x32 operands: lane reads row/column lane % 16, K chunk lane / 16
          const int j = kk / 2, kc = kk * 2 + (lane >> 4), r16 = lane & 15;
          xa[j] = __builtin_bit_cast(bf16x8_t, As[swz<CH>(BM + r16, kc)]);
#pragma unroll
          for (int b = 0; b < XA; ++b) {
            const int col = (PAIRED && b >= XB) ? BN / 2 + xcol0 + 16 * (b - XB) : xcol0 + 16 * b;
            xb[j][b] = __builtin_bit_cast(bf16x8_t, Bs[swz<CH>(col + r16, kc)]);
          }
        }
      }
    };
    auto mma = [&](int kk) {
      const int buf = kk & 1;
      if constexpr (NR > 0) {
#pragma unroll
        for (int i = 0; i < NR; ++i)
#pragma unroll
          for (int j = 0; j < TN; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[buf][i], bfv[buf][j], acc[i][j], 0, 0, 0);
      }
      if constexpr (EXT) {
        if (kk % 2 == 1) {
#pragma unroll
          for (int b = 0; b < XA; ++b)
            xacc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa[kk / 2], xb[kk / 2][b], xacc[b], 0, 0, 0);
        }
      }
    };
    if (kt0 >= kt1) return;
    wait_lgkm0();
    if (loader) wait_stages<LPSX, STAGES - 1>(min(STAGES - 1, kt1 - 1 - kt0));
    barrier_nofence();
    fetch(0, 0, 0);
    for (int kt = kt0; kt < kt1; ++kt) {
      const int stage = (kt - kt0) % STAGES;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        if (kk + 1 < KS) {
          fetch(stage, kk + 1, (kk + 1) & 1);
        } else {
          wait_lgkm0();
          if (loader && kt + 1 < kt1) wait_stages<LPSX, STAGES - 2>(min(STAGES - 2, kt1 - 2 - kt));
          barrier_nofence();
          if (kt + STAGES < kt1) issue(kt + STAGES, stage, ext_c);
          if (kt + 1 < kt1) fetch(stage + 1 == STAGES ? 0 : stage + 1, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        mma(kk);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };
  using NoExt = std::false_type;
  bool extended = false;
  if constexpr (XR > 0) {
    if (ext) {
      mainloop(std::integral_constant<int, TM>{}, std::true_type{});
      extended = true;
    }
  }
  if (extended) {
  } else if (nr == TM) {
    mainloop(std::integral_constant<int, TM>{}, NoExt{});
  } else if (nr == 0) {
    mainloop(std::integral_constant<int, 0>{}, NoExt{});
  } else {
    if constexpr (TM > 1) {
      if (nr == 1)
        mainloop(std::integral_constant<int, 1>{}, NoExt{});
      else
        mainloop(std::integral_constant<int, TM>{}, NoExt{});
    }
  }

  // epilogue: lane holds column (lane % 32) and rows (r/4)*8 + (lane/32)*4 + r%4 of each sub-tile
  float* part = splits > 1 ? partial + (size_t)ks * M * part_ld : nullptr;
  if constexpr (XR > 0) {
    // extra rows (16x16 blocks): lane holds column lane % 16, rows 4 (lane / 16) + r
    if (ext) {
      if (part) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = m0 + BM + 4 * (lane >> 4) + r;
          if (m >= M) continue;
#pragma unroll
          for (int b = 0; b < XB; ++b) {
            const int c = c0 + xcol0 + 16 * b + (lane & 15);
            if (c >= ncols) continue;
            if constexpr (PAIRED) {
              part[(size_t)m * part_ld + map.first(c)] = xacc[b][r];
              part[(size_t)m * part_ld + map.second(c)] = xacc[XB + b][r];
            } else {
              part[(size_t)m * part_ld + c] = xacc[b][r];
            }
          }
        }
      } else if constexpr (PAIRED) {
        typename Epi::Col xc[XB];
#pragma unroll
        for (int b = 0; b < XB; ++b) xc[b] = epi.col(min(c0 + xcol0 + 16 * b + (lane & 15), ncols - 1));
        wait_vm0();  // column state loaded before the first store
        const int mx = m0 + BM + 4 * (lane >> 4);  // this lane's four consecutive extra rows
        if (mx < M) {
#pragma unroll
          for (int b = 0; b < XB; ++b)
            if (c0 + xcol0 + 16 * b + (lane & 15) < ncols) epi.pair4(mx, min(4, M - mx), xc[b], xacc[b], xacc[XB + b]);
        }
      } else {
        // residual epilogues read every old value before the first store
        // (unconditional, clamped loads, all in flight at once)
        if constexpr (Epi::kRmw) {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int m = m0 + BM + 4 * (lane >> 4) + r;
#pragma unroll
            for (int b = 0; b < XB; ++b) {
              const int c = c0 + xcol0 + 16 * b + (lane & 15);
              const float old = epi.load(min(m, M - 1), min(c, ncols - 1));
              xacc[b][r] += (m < M && c < ncols) ? old : 0.f;
            }
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = m0 + BM + 4 * (lane >> 4) + r;
#pragma unroll
          for (int b = 0; b < XB; ++b) {
            const int c = c0 + xcol0 + 16 * b + (lane & 15);
            if (m < M && c < ncols) epi.store(m, c, xacc[b][r]);
          }
        }
      }
    }
  }
  auto row_of = [&](int i, int r) { return m0 + wm * WM + i * 32 + (r >> 2) * 8 + (lane >> 5) * 4 + (r & 3); };
  if (part) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = row_of(i, r);
        if (m >= M) continue;
        if constexpr (PAIRED) {
#pragma unroll
          for (int j = 0; j < TN / 2; ++j) {
            const int p = c0 + wn * (WN / 2) + j * 32 + lr;
            if (p >= ncols) continue;
            part[(size_t)m * part_ld + map.first(p)] = acc[i][j][r];
            part[(size_t)m * part_ld + map.second(p)] = acc[i][j + TN / 2][r];
          }
        } else {
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const int n = c0 + wn * WN + j * 32 + lr;
            if (n < ncols) part[(size_t)m * part_ld + n] = acc[i][j][r];
          }
        }
      }
    }
  } else if constexpr (PAIRED) {
    typename Epi::Col cols[TN / 2];
#pragma unroll
    for (int j = 0; j < TN / 2; ++j) cols[j] = epi.col(min(c0 + wn * (WN / 2) + j * 32 + lr, ncols - 1));
    wait_vm0();  // column state loaded before the first store
    // registers 4 q .. 4 q + 3 of a sub-tile hold four consecutive rows
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int m = row_of(i, 4 * q);
        if (m >= M) continue;
#pragma unroll
        for (int j = 0; j < TN / 2; ++j)
          if (c0 + wn * (WN / 2) + j * 32 + lr < ncols) {
            const f32x4_t x0 = {acc[i][j][4 * q], acc[i][j][4 * q + 1], acc[i][j][4 * q + 2], acc[i][j][4 * q + 3]};
            const f32x4_t x1 = {acc[i][j + TN / 2][4 * q], acc[i][j + TN / 2][4 * q + 1], acc[i][j + TN / 2][4 * q + 2],
                                acc[i][j + TN / 2][4 * q + 3]};
            epi.pair4(m, min(4, M - m), cols[j], x0, x1);
          }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      // residual epilogues read a 32-row block's old values before its
      // first store (unconditional, clamped loads: no branch between a load
      // and its use, so they are all in flight at once)
      if constexpr (Epi::kRmw) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = row_of(i, r);
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            const int n = c0 + wn * WN + j * 32 + lr;
            const float old = epi.load(min(m, M - 1), min(n, ncols - 1));
            acc[i][j][r] += (m < M && n < ncols) ? old : 0.f;
          }
        }
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = row_of(i, r);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int n = c0 + wn * WN + j * 32 + lr;
          if (m < M && n < ncols) epi.store(m, n, acc[i][j][r]);
        }
      }
    }
  }
}

// K-tile-contiguous copy (see Wt): one thread per 16-byte piece.
__global__ __launch_bounds__(256) void pack_tiles_kernel(const bf16_t* __restrict__ W, int rows, int K,
                                                         bf16_t* __restrict__ Wt) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int KT = K / 64;
  const size_t groups = (size_t)(rows + 31) / 32;
  if (idx >= groups * KT * 32 * 8) return;
  const int c = (int)(idx % 8);           // 16-byte piece within the 64-deep row segment
  const int r = (int)((idx / 8) % 32);    // row within the group
  const size_t gk = idx / 256;            // group * KT + K-tile
  const int kt = (int)(gk % KT), row = (int)(gk / KT) * 32 + r;
  u32x4_t v = {0u, 0u, 0u, 0u};
  if (row < rows) v = *(const u32x4_t*)(W + (size_t)row * K + kt * 64 + c * 8);
  *(u32x4_t*)(Wt + idx * 8) = v;
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

// Split-K sum + RoPE + scatter for the q/k/v projection, one workgroup per
// (32 rows, one head).  Partial columns of a head are contiguous, so the
// reads coalesce; q/k rows are written d-contiguous, and v goes through an
// LDS transpose so that its d-major rows are written position-contiguous.
template <int NS>
__global__ __launch_bounds__(256) void qkv_reduce_kernel(const float* __restrict__ partial, int M, int nw,
                                                         EpiQkv<bf16_t> e) {
  constexpr int RB = 32, HALF = 64, D = 128;  // rows per workgroup; bf16 heads are 128 wide
  __shared__ float vt[D][RB + 1];
  const int head = blockIdx.y, m0 = blockIdx.x * RB, tid = threadIdx.x;
  const size_t stride = (size_t)M * nw;
  const bool is_v = head >= e.nq + e.nkv;
  const int i0 = (tid % 16) * 4;  // four consecutive rotation pairs per thread
  const int rr = tid / 16;        // rows rr and rr + 16 of the block
  f32x4_t x0[2], x1[2];
  {
    f32x4_t p0[2][NS], p1[2][NS];
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int m = min(m0 + rr + 16 * k, M - 1);
      const size_t o0 = (size_t)m * nw + (size_t)head * D + i0;
#pragma unroll
      for (int sp = 0; sp < NS; ++sp) {
        p0[k][sp] = *(const f32x4_t*)(partial + sp * stride + o0);
        p1[k][sp] = *(const f32x4_t*)(partial + sp * stride + o0 + HALF);
      }
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      x0[k] = p0[k][0];
      x1[k] = p1[k][0];
#pragma unroll
      for (int sp = 1; sp < NS; ++sp) {
        x0[k] += p0[k][sp];
        x1[k] += p1[k][sp];
      }
    }
  }
  if (!is_v) {
    const bool is_q = head < e.nq;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int m = m0 + rr + 16 * k;
      if (m >= M) continue;
      int b, l;
      divmod_rows(m, e.L, e.inv_L, b, l);
      if (e.rope) {
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          float a0 = x0[k][c], a1 = x1[k][c];
          rope_pair(a0, a1, e.pos0 + l, e.tab.inv_rev[i0 + c]);
          x0[k][c] = a0;
          x1[k][c] = a1;
        }
      }
      bf16_t* dst = is_q ? e.q + (((size_t)b * e.nq + head) * e.L + l) * D
                         : e.k + (((size_t)b * e.nkv + (head - e.nq)) * e.L + l) * D;
      u32x2_t w0, w1;
      w0[0] = pack_bf16x2(x0[k][0], x0[k][1]);
      w0[1] = pack_bf16x2(x0[k][2], x0[k][3]);
      w1[0] = pack_bf16x2(x1[k][0], x1[k][1]);
      w1[1] = pack_bf16x2(x1[k][2], x1[k][3]);
      *(u32x2_t*)(dst + i0) = w0;
      *(u32x2_t*)(dst + i0 + HALF) = w1;
    }
    return;
  }
#pragma unroll
  for (int k = 0; k < 2; ++k)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      vt[i0 + c][rr + 16 * k] = x0[k][c];
      vt[i0 + c + HALF][rr + 16 * k] = x1[k][c];
    }
  __syncthreads();
  const int r = tid % RB;
  const int m = m0 + r;
  if (m >= M) return;
  int b, l;
  divmod_rows(m, e.L, e.inv_L, b, l);
  bf16_t* dst = e.vt + ((size_t)b * e.nkv + (head - e.nq - e.nkv)) * D * e.Lp + l;
  for (int dd = tid / RB; dd < D; dd += 256 / RB) dst[(size_t)dd * e.Lp] = bf16_value_as_f16(vt[dd][r]);
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
template <int BM, int BN, int BKT, int WMW, int WNW, int S, bool PAIRED, class Map, class Epi, class ALay>
void launch_cfg(const GemmPlan& pl, const bf16_t* a, int lda, int M, int K, const bf16_t* w, int tiled, Map map,
                int ncols, int nw, Epi epi, float* part, hipStream_t st, ALay alay) {
  const int grid = pl.m_tiles * pl.n_tiles * pl.splits;
  constexpr int XR = gemm_extra_rows(BM, BN, BKT, WMW * WNW, PAIRED);
  // the extended-tile kernel only where the plan folds leftover rows into the
  // last row tile; the plain kernel keeps its smaller code and LDS otherwise
  if constexpr (XR > 0) {
    if (pl.ext) {
      hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, BKT, WMW, WNW, S, XR, PAIRED, Map, Epi, ALay>), dim3(grid),
                         dim3(64 * WMW * WNW), 0, st, a, lda, M, K, w, nw, tiled, map, ncols, epi, part, nw,
                         pl.m_tiles, pl.n_tiles, pl.splits, alay);
      return;
    }
  }
  hipLaunchKernelGGL((gemm_bf16_kernel<BM, BN, BKT, WMW, WNW, S, 0, PAIRED, Map, Epi, ALay>), dim3(grid),
                     dim3(64 * WMW * WNW), 0, st, a, lda, M, K, w, nw, tiled, map, ncols, epi, part, nw, pl.m_tiles,
                     pl.n_tiles, pl.splits, alay);
}

template <bool PAIRED, class Map, class Epi, class ALay = APlain>
hipError_t run_bf16_plan(const GemmPlan& pl, const void* A, int lda, int M, int K, const Wt& W, Map map,
                         int ncols, int nw, Epi epi, float* partial, hipStream_t st, const char* tag,
                         bool reduce = true, ALay alay = {}) {
  const int grid = pl.m_tiles * pl.n_tiles * pl.splits;
  if (grid == 0) return hipSuccess;
  // buffer descriptors address at most 4 GiB per operand
  if ((size_t)M * lda * 2 > 0xffffffffull || (size_t)(nw + 31) / 32 * 32 * K * 2 > 0xffffffffull)
    return hipErrorInvalidValue;
  const bf16_t* a = (const bf16_t*)A;
  const int tiled = W.tiled != nullptr && K % 64 == 0;
  const bf16_t* w = (const bf16_t*)(tiled ? W.tiled : W.w);
  float* part = pl.splits > 1 ? partial : nullptr;
  {
    ProfScope prof(tag, st);
    switch (pl.cfg) {
#define FPD_CFG(E, BM, BN, BKT, WMW, WNW, S) \
  case E: launch_cfg<BM, BN, BKT, WMW, WNW, S, PAIRED>(pl, a, lda, M, K, w, tiled, map, ncols, nw, epi, part, st, alay); \
    break;
      FPD_GEMM_CFGS(FPD_CFG)
#undef FPD_CFG
      default: return hipErrorInvalidValue;
    }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.splits == 1 || !reduce) return e;
  ProfScope prof("splitk_reduce", st);
  const size_t n = (size_t)M * ncols;
  hipLaunchKernelGGL((splitk_reduce_kernel<PAIRED, Map, Epi>), dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                     partial, pl.splits, M, nw, ncols, map, epi);
  return hipGetLastError();
}

template <bool PAIRED, class Map, class Epi, class ALay = APlain>
hipError_t run_bf16(const void* A, int lda, int M, int K, const Wt& W, Map map, int ncols, int nw, Epi epi,
                    float* partial, size_t partial_bytes, hipStream_t st, const char* tag, ALay alay = {}) {
  GemmPlan pl = plan_gemm_bf16(M, ncols, K, nw, PAIRED);
  if (pl.splits > 1 && pl.partial_floats * sizeof(float) > partial_bytes) {
    pl.splits = 1;
    pl.partial_floats = 0;
  }
  return run_bf16_plan<PAIRED>(pl, A, lda, M, K, W, map, ncols, nw, epi, partial, st, tag, true, alay);
}

template <bool PAIRED, class Map, class Epi>
hipError_t run_f32(const void* A, int lda, int M, int K, const Wt& Wm, Map map, int ncols, Epi epi,
                   hipStream_t st, const char* tag) {
  const void* W = Wm.w;
  ProfScope prof(tag, st);
  const int m_tiles = (M + 63) / 64;
  const int n_tiles = (ncols + (PAIRED ? 31 : 63)) / (PAIRED ? 32 : 64);
  if (m_tiles == 0 || n_tiles == 0) return hipSuccess;
  hipLaunchKernelGGL((gemm_f32_kernel<PAIRED, Map, Epi>), dim3(m_tiles * n_tiles), dim3(256), 0, st,
                     (const float*)A, lda, M, K, (const float*)W, map, ncols, epi, m_tiles);
  return hipGetLastError();
}

}  // namespace

namespace {
struct CfgShape {
  int rows, cols, bk, waves;
};
constexpr CfgShape kCfgShape[GEMM_NUM_CFGS] = {
#define FPD_SHAPE(E, BM, BN, BKT, WMW, WNW, S) {BM, BN, BKT, WMW * WNW},
    FPD_GEMM_CFGS(FPD_SHAPE)
#undef FPD_SHAPE
};
}  // namespace

int gemm_cfg_rows(int cfg) { return kCfgShape[cfg].rows; }
int gemm_cfg_cols(int cfg) { return kCfgShape[cfg].cols; }
int gemm_cfg_bk(int cfg) { return kCfgShape[cfg].bk; }
int gemm_cfg_extra_rows(int cfg, bool paired) {
  const CfgShape& c = kCfgShape[cfg];
  return gemm_extra_rows(c.rows, c.cols, c.bk, c.waves, paired);
}

GemmPlan make_plan(int cfg, int M, int ncols, int K, int nw, bool paired, int splits, bool fold) {
  GemmPlan p;
  p.cfg = cfg;
  const int bm = gemm_cfg_rows(cfg), cpt = gemm_cfg_cols(cfg) / (paired ? 2 : 1);
  p.m_tiles = (M + bm - 1) / bm;
  if (fold && M > bm && M % bm != 0 && M % bm <= gemm_cfg_extra_rows(cfg, paired)) {
    p.m_tiles = M / bm;
    p.ext = true;
  }
  p.n_tiles = (ncols + cpt - 1) / cpt;
  p.splits = std::max(1, std::min(splits, K / gemm_cfg_bk(cfg)));
  p.partial_floats = p.splits > 1 ? (size_t)p.splits * M * nw : 0;
  return p;
}

// Tile and split choice, from measured sweeps on MI355X (block rows M = 8,
// 16, 25 and 385 of the 2560-wide drafter, weights streamed from HBM,
// splits 1..32, split-K sums included; M = 40 and 64 checked): M <= 64
// splits K until about one pass of workgroups over the 256 CUs (more splits
// cost more in partial sums than they gain in streaming); larger M
// takes the 128x256 eight-wave tile (one workgroup per CU) when it alone
// nearly fills 256 CUs; deep-K or paired outputs split that tile along K so
// that the row tiles (a partly filled last one counts its share of 32-row
// blocks) cover about 80% of the CUs once; narrow plain outputs take 64x128 tiles
// split along K.
GemmPlan plan_gemm_bf16(int M, int ncols, int K, int nw, bool paired) {
  const int kt = K / 64;
  // Many rows (the 8-request point-motion block, M = 19,464): 256x256 tiles
  // move half the operand bytes per MFMA of 128x256 ones, which is what the
  // per-CU operand fill rate bounds; with the last tile carrying up to 16
  // leftover rows they took gate/up 1.93 -> 1.64 ms, down 1.21 -> 1.02 ms and
  // O 0.61 -> 0.55 ms per launch there, and q/k/v 0.70 -> 0.63 ms once the
  // tile order grouped row tiles.
  const GemmPlan w256 = make_plan(GEMM_256x256_W8_S2, M, ncols, K, nw, paired, 1, /*fold=*/true);
  if (w256.m_tiles * w256.n_tiles >= 512) return w256;
  auto with_splits = [&](int cfg, int lo, int hi) {
    GemmPlan p = make_plan(cfg, M, ncols, K, nw, paired, 1);
    const int tiles = p.m_tiles * p.n_tiles;
    int s2 = 1;
    while (tiles * s2 < lo && s2 * 2 <= 32 && kt / (s2 * 2) >= 2 && tiles * s2 * 2 <= hi) s2 *= 2;
    return make_plan(cfg, M, ncols, K, nw, paired, s2);
  };
  if (M <= 32) return with_splits(GEMM_32x128_S4, 128, 256);
  if (M <= 64) return with_splits(GEMM_64x128_S3, 128, 256);
  const GemmPlan big = make_plan(GEMM_128x256_W8_S3, M, ncols, K, nw, paired, 1);
  const GemmPlan folded = make_plan(GEMM_128x256_W8_S3, M, ncols, K, nw, paired, 1, /*fold=*/true);
  // A few leftover rows would otherwise form a second wave of one-row tiles,
  // each streaming its whole weight column again: carry them in the last
  // full row tile instead when that keeps the grid within one pass.
  if (folded.ext && big.m_tiles * big.n_tiles > 256 && folded.m_tiles * folded.n_tiles >= 224) return folded;
  if (big.m_tiles * big.n_tiles >= 224) return big;
  const GemmPlan one = make_plan(GEMM_128x128_W8_S3, M, ncols, K, nw, paired, 1);
  if (M >= 256 && one.m_tiles * one.n_tiles <= 256) {
    // Two or more full row tiles whose 128x256 tiles leave CUs idle (the QKV,
    // O and down projections of a few hundred rows): 128x128 tiles with 8
    // waves, K split as far as one pass of workgroups allows.  At M = 385 this
    // runs QKV unsplit (no separate split-K sum) and O / down 3-way split,
    // 7-8% faster than 128x256 tiles split 2-6 ways or 4-wave 64x128 tiles.
    // Where even unsplit 128x128 tiles would take a second pass (the fusion
    // map over 2,048 context rows: 320 tiles), the 128x256 rules below are
    // faster (fusion map 218 -> 182 us).
    const int s = std::max(1, std::min({8, 256 / (one.m_tiles * one.n_tiles), kt / 2}));
    return make_plan(GEMM_128x128_W8_S3, M, ncols, K, nw, paired, s);
  }
  if (paired || K >= 8192) {
    const int full = M / 128, rem_blocks = (M - full * 128 + 31) / 32;  // 32-row blocks of the last tile
    const double units = big.n_tiles * (full + 0.25 * rem_blocks);
    const int s = std::max(1, std::min({8, (int)(0.8 * 256 / units), kt / 2}));
    return make_plan(GEMM_128x256_W8_S3, M, ncols, K, nw, paired, s);
  }
  return with_splits(GEMM_64x128_S3, 256, 640);
}

size_t gemm_tiles_elems(int rows, int K) { return (size_t)(rows + 31) / 32 * 32 * (size_t)K; }

hipError_t gemm_pack_tiles(const void* W, int rows, int K, void* Wtiled, hipStream_t st) {
  if (rows <= 0 || K <= 0 || K % 64) return hipErrorInvalidValue;
  const size_t n = gemm_tiles_elems(rows, K) / 8;
  hipLaunchKernelGGL(pack_tiles_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, (const bf16_t*)W, rows,
                     K, (bf16_t*)Wtiled);
  return hipGetLastError();
}

hipError_t gemm_store_f32(int dt, const void* A, int lda, int M, int K, const Wt& W, int N,
                          float* out, int ldo, float* partial, size_t partial_bytes, hipStream_t st,
                          const char* tag) {
  EpiStore e{out, ldo};
  if (dt == FPD_DTYPE_BF16)
    return run_bf16<false>(A, lda, M, K, W, MapPlain{}, N, N, e, partial, partial_bytes, st, tag);
  return run_f32<false>(A, lda, M, K, W, MapPlain{}, N, e, st, tag);
}

hipError_t gemm_store_fused_f32(const void* feats, int B, int n_t, int C, int H, const Wt& W, int N, float* out,
                                int ldo, float* partial, size_t partial_bytes, hipStream_t st, const char* tag) {
  EpiStore e{out, ldo};
  return run_bf16<false>(feats, n_t * H, B * C, n_t * H, W, MapPlain{}, N, N, e, partial, partial_bytes, st, tag,
                         AFused{C, H});
}

hipError_t gemm_residual(int dt, const void* A, int lda, int M, int K, const Wt& W, int N,
                         float* h, int ldh, float* partial, size_t partial_bytes, hipStream_t st,
                         const char* tag) {
  EpiResid e{h, ldh};
  if (dt == FPD_DTYPE_BF16)
    return run_bf16<false>(A, lda, M, K, W, MapPlain{}, N, N, e, partial, partial_bytes, st, tag);
  return run_f32<false>(A, lda, M, K, W, MapPlain{}, N, e, st, tag);
}

hipError_t gemm_residual_norm(int dt, const void* A, int M, int K, const Wt& W, int H, float* h, const void* g,
                              float eps, void* out, int final_L, float* partial, size_t partial_bytes,
                              hipStream_t st, const char* tag) {
  if (dt == FPD_DTYPE_BF16) {
    GemmPlan pl = plan_gemm_bf16(M, H, K, H, false);
    if (pl.splits > 1 && pl.partial_floats * sizeof(float) <= partial_bytes) {
      // split-K partials; the residual sum and the RMSNorm run fused, row-wise
      hipError_t e = run_bf16_plan<false>(pl, A, K, M, K, W, MapPlain{}, H, H, EpiResid{h, H}, partial, st, tag,
                                          /*reduce=*/false);
      if (e != hipSuccess) return e;
      return residual_norm(dt, partial, pl.splits, M, H, h, g, eps, out, final_L, st);
    }
  }
  hipError_t e = gemm_residual(dt, A, K, M, K, W, H, h, H, partial, partial_bytes, st, tag);
  if (e != hipSuccess) return e;
  return residual_norm(dt, nullptr, 1, M, H, h, g, eps, out, final_L, st);
}

hipError_t gemm_qkv(int dt, const void* A, int M, int K, const Wt& Wqkv, const QkvOut& o,
                    float* partial, size_t partial_bytes, hipStream_t st) {
  const int half = o.d / 2;
  const int pairs = (o.nq + 2 * o.nkv) * half;
  const int nw = (o.nq + 2 * o.nkv) * o.d;
  if (dt == FPD_DTYPE_BF16) {
    EpiQkv<bf16_t> e{(bf16_t*)o.q, (bf16_t*)o.k, (bf16_t*)o.vt, o.L, o.Lp, o.nq, o.nkv, o.d, half,
                     o.pos0, o.rope, o.tab, 1.0f / (float)o.L};
    GemmPlan pl = plan_gemm_bf16(M, pairs, K, nw, true);
    if (pl.splits > 1 && pl.partial_floats * sizeof(float) > partial_bytes) {
      pl.splits = 1;
      pl.partial_floats = 0;
    }
    hipError_t err = run_bf16_plan<true>(pl, A, K, M, K, Wqkv, MapRope{half}, pairs, nw, e, partial, st, "gemm_qkv",
                                         /*reduce=*/false);
    if (err != hipSuccess || pl.splits == 1 || M == 0) return err;
    ProfScope prof("qkv_reduce", st);
    const dim3 grid((M + 31) / 32, o.nq + 2 * o.nkv);
    switch (pl.splits) {
#define FPD_QKVR(NS)                                                                                  \
  case NS:                                                                                            \
    hipLaunchKernelGGL((qkv_reduce_kernel<NS>), grid, dim3(256), 0, st, partial, M, nw, e);         \
    break;
      FPD_QKVR(2)
      FPD_QKVR(3)
      FPD_QKVR(4)
      FPD_QKVR(5)
      FPD_QKVR(6)
      FPD_QKVR(7)
      FPD_QKVR(8)
#undef FPD_QKVR
      default: {
        const size_t n = (size_t)M * pairs;
        hipLaunchKernelGGL((splitk_reduce_kernel<true, MapRope, EpiQkv<bf16_t>>), dim3((unsigned)((n + 255) / 256)),
                           dim3(256), 0, st, partial, pl.splits, M, nw, pairs, MapRope{half}, e);
      }
    }
    return hipGetLastError();
  }
  EpiQkv<float> e{(float*)o.q, (float*)o.k, (float*)o.vt, o.L, o.Lp, o.nq, o.nkv, o.d, half,
                  o.pos0, o.rope, o.tab, 1.0f / (float)o.L};
  return run_f32<true>(A, K, M, K, Wqkv, MapRope{half}, pairs, e, st, "gemm_qkv");
}

hipError_t gemm_ctx_kv(int dt, const void* Zn, int M, int K, const Wt& Wkv, const CtxOut& o,
                       float* partial, size_t partial_bytes, hipStream_t st) {
  const int half = o.d / 2;
  const int pairs = 2 * o.nkv * half;
  const int nw = 2 * o.nkv * o.d;
  if (dt == FPD_DTYPE_BF16) {
    EpiCtx<bf16_t> e{(bf16_t*)o.k, (bf16_t*)o.vt, o.C, o.cap, o.nkv, o.d, half, o.pos0, o.rope, o.tab,
                     1.0f / (float)o.C};
    return run_bf16<true>(Zn, K, M, K, Wkv, MapRope{half}, pairs, nw, e, partial, partial_bytes, st,
                          "gemm_ctx_kv");
  }
  EpiCtx<float> e{(float*)o.k, (float*)o.vt, o.C, o.cap, o.nkv, o.d, half, o.pos0, o.rope, o.tab,
                  1.0f / (float)o.C};
  return run_f32<true>(Zn, K, M, K, Wkv, MapRope{half}, pairs, e, st, "gemm_ctx_kv");
}

hipError_t gemm_swiglu(int dt, const void* A, int M, int K, const Wt& Wgu, int I, void* u,
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
