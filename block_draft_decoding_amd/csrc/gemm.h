// Host-side interface of the bf16 / f32 dense projections (internal to
// libfpd): tile configurations, launch plans and the fused-epilogue
// launchers.
#pragma once
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "common.h"

namespace fpd {

// ---- GEMM planning (shared by workspace sizing and launches) --------------
// Tile configurations of the bf16 GEMM: workgroup tile rows x columns, K
// tile, wave grid (rows x columns of waves) and the depth of the
// global -> LDS ring.  X(name, rows, cols, k_tile, waves_m, waves_n, stages).
#define FPD_GEMM_CFGS(X)                          \
  X(GEMM_32x128_S4, 32, 128, 64, 1, 2, 4)         \
  X(GEMM_64x128_S3, 64, 128, 64, 2, 2, 3)         \
  X(GEMM_128x128_W8_S3, 128, 128, 64, 4, 2, 3)    \
  X(GEMM_128x256_W8_S3, 128, 256, 64, 2, 4, 3)    \
  X(GEMM_256x256_W8_S2, 256, 256, 64, 2, 4, 2)
enum GemmCfg {
#define FPD_ENUM(name, ...) name,
  FPD_GEMM_CFGS(FPD_ENUM)
#undef FPD_ENUM
  GEMM_NUM_CFGS
};
struct GemmPlan {
  int cfg = GEMM_128x256_W8_S3;
  int m_tiles = 1, n_tiles = 1, splits = 1;
  bool ext = false;           // the last row tile carries the rows past (m_tiles) * BM
  size_t partial_floats = 0;  // split-K scratch (splits * M * N_w floats) when splits > 1
};
// Rows past BM that the last row tile of a bf16 GEMM configuration can carry
// (so that M = k BM + r, r <= this, needs no extra row tile re-reading the
// weights): 16 where the K tile is 64 wide, BM >= 64 and every wave gets at
// least one 16-column block of the extra rows.
constexpr int gemm_extra_rows(int bm, int bn, int bk, int waves, bool paired) {
  return (bk == 64 && bm >= 64 && (paired ? bn / 2 : bn) >= waves * 16) ? 16 : 0;
}
// fold: let the last row tile carry up to gemm_extra_rows leftover rows
GemmPlan make_plan(int cfg, int M, int ncols, int K, int nw, bool paired, int splits, bool fold = false);
int gemm_cfg_rows(int cfg);
int gemm_cfg_cols(int cfg);
int gemm_cfg_bk(int cfg);
int gemm_cfg_extra_rows(int cfg, bool paired);
// M rows, ncols logical output columns (pairs for paired epilogues), K depth,
// nw = W rows covered (partial row length), paired = two W rows per column.
GemmPlan plan_gemm_bf16(int M, int ncols, int K, int nw, bool paired);

// ---- K-tile-contiguous copies of the weights ----------------------------------
// A projection's weights: row-major W [rows, K] (torch Linear layout) and,
// once the drafter is prepared, the same matrix with each 32-row group's
// 64-deep K-tiles stored one after another (element (r, k) at
// ((r / 32 * K / 64 + k / 64) * 32 + r % 32) * 64 + k % 64), so a
// workgroup's weight tile for one K step is 4 KB-contiguous runs instead of
// 128-byte pieces of rows 2 K bytes apart (nullptr before).
struct Wt {
  const void* w;
  const void* tiled;
};
// Elements (bf16) of the tiled copy of a [rows, K] matrix (rows rounded up to 32).
size_t gemm_tiles_elems(int rows, int K);
// Writes that copy (rows past the matrix are zero).  K must be a multiple of 64.
hipError_t gemm_pack_tiles(const void* W, int rows, int K, void* Wtiled, hipStream_t st);

// ---- Y = A W^T with epilogues --------------------------------------------
// A [M, K] row-major (lda), W [.., K] row-major (ldw = K).  dt: FPD_DTYPE_*.
// `partial`/`partial_bytes`: split-K scratch from the workspace.

// out[m, n] = Y (float).  N outputs.
hipError_t gemm_store_f32(int dt, const void* A, int lda, int M, int K, const Wt& W, int N,
                          float* out, int ldo, float* partial, size_t partial_bytes, hipStream_t st,
                          const char* tag);

// The same (bf16 only) with A the per-layer target features [B, n_t, C, H]
// read in place as their concatenation [B * C, n_t * H] (H a multiple of 64).
hipError_t gemm_store_fused_f32(const void* feats, int B, int n_t, int C, int H, const Wt& W, int N, float* out,
                                int ldo, float* partial, size_t partial_bytes, hipStream_t st, const char* tag);

// h[m, n] += Y (float residual).
hipError_t gemm_residual(int dt, const void* A, int lda, int M, int K, const Wt& W, int N,
                         float* h, int ldh, float* partial, size_t partial_bytes, hipStream_t st,
                         const char* tag);

// h += A W^T, then out = RMSNorm(h) * g (bf16 split-K partials are summed in
// the fused row-wise norm kernel).  final_L > 0: output only rows with
// l = r % final_L >= 1, at b*(L-1) + l - 1.
hipError_t gemm_residual_norm(int dt, const void* A, int M, int K, const Wt& W, int H, float* h, const void* g,
                              float eps, void* out, int final_L, float* partial, size_t partial_bytes,
                              hipStream_t st, const char* tag);

// Fused QKV projection of block rows m = b * L + l: Q [B, nq, L, d],
// K [B, nkv, L, d] (RoPE at pos0 + l), Vt [B, nkv, d, Lp] (transposed).
struct QkvOut {
  void *q, *k, *vt;
  int L, Lp, nq, nkv, d, pos0, rope;
  RopeTab tab;
};
hipError_t gemm_qkv(int dt, const void* A, int M, int K, const Wt& Wqkv, const QkvOut& o,
                    float* partial, size_t partial_bytes, hipStream_t st);

// Context K/V of one drafter layer from the fused features, rows m = b * C + c:
// ctx_k [B, nkv, cap, d] (RoPE at pos0 + c), ctx_vt [B, nkv, d, cap].
struct CtxOut {
  void *k, *vt;
  int C, cap, nkv, d, pos0, rope;
  RopeTab tab;
};
hipError_t gemm_ctx_kv(int dt, const void* Zn, int M, int K, const Wt& Wkv, const CtxOut& o,
                       float* partial, size_t partial_bytes, hipStream_t st);

// u[m, i] = silu(A Wg^T)[m, i] * (A Wu^T)[m, i], W = [gate rows; up rows] ([2I, K]).
hipError_t gemm_swiglu(int dt, const void* A, int M, int K, const Wt& Wgu, int I, void* u,
                       float* partial, size_t partial_bytes, hipStream_t st);

}  // namespace fpd
