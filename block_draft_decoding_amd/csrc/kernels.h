// Host-side launchers of the gfx950 kernels (internal to libfpd).
#pragma once
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "common.h"

namespace fpd {

// Brackets the kernel launches of its lifetime with HIP events on `st` when
// per-launch timing is enabled (fpd_profile_enable); otherwise a no-op.
class ProfScope {
 public:
  ProfScope(const char* tag, hipStream_t st);
  ~ProfScope();

 private:
  hipStream_t st_;
  int idx_;
};

// ---- GEMM planning (shared by workspace sizing and launches) --------------
// Tile configurations of the bf16 GEMM: workgroup tile rows x columns, K
// tile, wave grid (rows x columns of waves) and the depth of the
// global -> LDS ring.  X(name, rows, cols, k_tile, waves_m, waves_n, stages).
#define FPD_GEMM_CFGS(X)                      \
  X(GEMM_128x128_S2, 128, 128, 64, 2, 2, 2)   \
  X(GEMM_64x128_S3, 64, 128, 64, 2, 2, 3)     \
  X(GEMM_32x128_S4, 32, 128, 64, 1, 2, 4)     \
  X(GEMM_64x256_S3, 64, 256, 64, 1, 4, 3)     \
  X(GEMM_128x256_W8_S2, 128, 256, 64, 2, 4, 2) \
  X(GEMM_128x256_W8_S3, 128, 256, 64, 2, 4, 3) \
  X(GEMM_256x128_W8_S3, 256, 128, 64, 4, 2, 3) \
  X(GEMM_128x256_W8_K32_S5, 128, 256, 32, 2, 4, 5)
enum GemmCfg {
#define FPD_ENUM(name, ...) name,
  FPD_GEMM_CFGS(FPD_ENUM)
#undef FPD_ENUM
  GEMM_NUM_CFGS
};
struct GemmPlan {
  int cfg = GEMM_128x128_S2;
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

// ---- Y = A W^T with epilogues --------------------------------------------
// A [M, K] row-major (lda), W [.., K] row-major (ldw = K).  dt: FPD_DTYPE_*.
// `partial`/`partial_bytes`: split-K scratch from the workspace.

// out[m, n] = Y (float).  N outputs.
hipError_t gemm_store_f32(int dt, const void* A, int lda, int M, int K, const void* W, int N,
                          float* out, int ldo, float* partial, size_t partial_bytes, hipStream_t st,
                          const char* tag);

// h[m, n] += Y (float residual).
hipError_t gemm_residual(int dt, const void* A, int lda, int M, int K, const void* W, int N,
                         float* h, int ldh, float* partial, size_t partial_bytes, hipStream_t st,
                         const char* tag);

// h += A W^T, then out = RMSNorm(h) * g (bf16 split-K partials are summed in
// the fused row-wise norm kernel).  final_L > 0: output only rows with
// l = r % final_L >= 1, at b*(L-1) + l - 1.
hipError_t gemm_residual_norm(int dt, const void* A, int M, int K, const void* W, int H, float* h, const void* g,
                              float eps, void* out, int final_L, float* partial, size_t partial_bytes,
                              hipStream_t st, const char* tag);

// Fused QKV projection of block rows m = b * L + l: Q [B, nq, L, d],
// K [B, nkv, L, d] (RoPE at pos0 + l), Vt [B, nkv, d, Lp] (transposed).
struct QkvOut {
  void *q, *k, *vt;
  int L, Lp, nq, nkv, d, pos0, rope;
  RopeTab tab;
};
hipError_t gemm_qkv(int dt, const void* A, int M, int K, const void* Wqkv, const QkvOut& o,
                    float* partial, size_t partial_bytes, hipStream_t st);

// Context K/V of one drafter layer from the fused features, rows m = b * C + c:
// ctx_k [B, nkv, cap, d] (RoPE at pos0 + c), ctx_vt [B, nkv, d, cap].
struct CtxOut {
  void *k, *vt;
  int C, cap, nkv, d, pos0, rope;
  RopeTab tab;
};
hipError_t gemm_ctx_kv(int dt, const void* Zn, int M, int K, const void* Wkv, const CtxOut& o,
                       float* partial, size_t partial_bytes, hipStream_t st);

// u[m, i] = silu(A Wg^T)[m, i] * (A Wu^T)[m, i], W = [gate rows; up rows] ([2I, K]).
hipError_t gemm_swiglu(int dt, const void* A, int M, int K, const void* Wgu, int I, void* u,
                       float* partial, size_t partial_bytes, hipStream_t st);

// ---- elementwise ------------------------------------------------------------
hipError_t embed_gather(int dt, const int32_t* tokens, int M, const void* E, int H, int V, float* h,
                        hipStream_t st);
// y[r] = RMSNorm(x[row(r)]) * g stored in dt, with row(r) = (r / per) * in_stride + in_off + r % per.
hipError_t rmsnorm_rows(int dt, const float* x, int H, int rows, int per, int in_stride, int in_off,
                        const void* g, float eps, void* y, hipStream_t st);
// h[r] += sum_s partial[s][r] (partial may be null), out = RMSNorm(h) * g; see gemm_residual_norm.
hipError_t residual_norm(int dt, const float* partial, int splits, int M, int H, float* h, const void* g, float eps,
                         void* out, int final_L, hipStream_t st);
// h = E[tokens] (ids outside [0, V) embed as zero rows), a = RMSNorm(h) * g.
hipError_t embed_norm(int dt, const int32_t* tokens, int M, const void* E, int H, int V, float* h, const void* g,
                      float eps, void* a, hipStream_t st);
// X[b * C + c, t * H + k] = feats[b, t, c, k]
hipError_t concat_features(int dt, const void* feats, int B, int nt, int C, int H, void* X,
                           hipStream_t st);

// ---- attention ----------------------------------------------------------------
struct AttnArgs {
  const void* q;      // [B, nq, L, d]
  const void* kb;     // [B, nkv, L, d]
  const void* vbt;    // [B, nkv, d, Lp]
  const void* ck;     // [B, nkv, cap, d]  (this layer)
  const void* cvt;    // [B, nkv, d, cap]
  void* o;            // [B, L, nq * d]
  int B, L, Lp, C, cap, nq, nkv, d;
  int ctx_bstride;    // 1: request b reads context b; 0: every request reads context 0 (shared)
  float scale;
};
size_t attention_scratch_bytes(int dt, int B, int L, int C, int nq, int nkv, int d);
hipError_t attention(int dt, const AttnArgs& a, void* scratch, size_t scratch_bytes, hipStream_t st);

// ---- constrained LM head -------------------------------------------------------
constexpr int kMaxHeadSets = 32;
struct HeadSet {
  const void* w;           // legal rows [n_cols, H] (gathered), or W_lm for free positions
  const int32_t* ids;      // ascending ids [n_cols], nullptr = identity (free)
  const int32_t* pos;      // block positions (1..L-1) that use this set
  int n_pos, n_cols, off_col;  // off_col: column of the OFF id, -1 if none
  int n_chunks, part_base;     // column chunks; first chunk slot of this set in a row's partials
};
struct HeadArgs {
  const void* hidden;      // [B, L-1, H]
  int B, L, H, width, n_sets, max_chunks;
  HeadSet sets[kMaxHeadSets];
  float* logits;           // nullable [B, L-1, width]
  float* pval;             // [B*(L-1), max_chunks]
  int32_t* pcol;           // [B*(L-1), max_chunks]
  float* offv;             // [B*(L-1)]
};
int head_chunk_cols(int dt);
hipError_t lm_head_partials(int dt, const HeadArgs& a, hipStream_t st);
// Combines the chunk partials into tokens; applies the OFF pairing rule.
struct ReduceArgs {
  const int32_t* pos_set;   // [L]
  const int32_t* partner;   // [L]: partner of a pair's first position, -2 second, -1 none
  int B, L, off_id, max_chunks, n_sets;
  int set_chunks[kMaxHeadSets + 1];
  int set_offcol[kMaxHeadSets + 1];
  const int32_t* set_ids[kMaxHeadSets + 1];   // nullptr = identity
  int free_slot;            // index used for free positions (-1 if none)
  const float* pval;
  const int32_t* pcol;
  const float* offv;
  int32_t* tokens;
};
hipError_t lm_head_reduce(const ReduceArgs& a, hipStream_t st);
// logits[r, c] = -inf for c >= row_cols[r % P + 1] (P = L - 1).
hipError_t fill_logits_padding(float* logits, int rows, int width, int P, const int32_t* row_cols,
                               hipStream_t st);

// ---- acceptance -------------------------------------------------------------------
struct ValidateArgs {
  const int32_t* tokens;     // [B, L-1]
  const int32_t* pos_set;    // [L]
  const int32_t* set_offsets;
  const int32_t* set_ids;
  int n_set_ids;
  const int32_t* partner;    // [L]
  const int32_t* field_w;    // [L]: width at a field's first digit position, else 0
  int B, L, vocab, off_id, fill_id, digit0_id;
  int32_t* k_out;
  int32_t* first_out;
  // box partial acceptance (optional: conf == nullptr gives all or nothing)
  const float* conf;         // [B, L-1]
  const int32_t* coord;      // [L]: 1 at coordinate positions
  float tau;
  int32_t* uncertain_out;    // [B]
};
hipError_t validate_primitive(const ValidateArgs& a, hipStream_t st);
hipError_t verify_prefix(const int32_t* draft, const int32_t* target, int B, int L, int32_t* k_out,
                         int32_t* next_out, hipStream_t st);
hipError_t gather_rows(int dt, const void* W, int H, const int32_t* ids, int n, void* out,
                       hipStream_t st);

// ---- coordinate codec (codec.hip) -------------------------------------------------
hipError_t coords_to_tokens(const float* x, int n, double lo, double hi, int base, int32_t* out, hipStream_t st);
hipError_t tokens_to_coords(const int32_t* t, int n, double lo, double hi, int base, double* out, hipStream_t st);
hipError_t ints_to_fields(const int32_t* v, int n, int plus_id, int minus_id, int digit0_id, int fill_id,
                          int32_t* out, hipStream_t st);
hipError_t fields_to_ints(const int32_t* f, int n, int plus_id, int minus_id, int digit0_id, int fill_id,
                          int32_t* vals, int32_t* ok, hipStream_t st);

}  // namespace fpd
