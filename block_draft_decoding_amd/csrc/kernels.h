// Host-side launchers of the gfx950 kernels (internal to libfpd).
#pragma once
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "common.h"
#include "gemm.h"  // GEMM plans and launchers

namespace fpd {

// Brackets the kernel launches of its lifetime with HIP events on `st` when
// per-launch timing is enabled (fpd_profile_enable); otherwise a no-op that
// reads one atomic flag (no lock).
class ProfScope {
 public:
  ProfScope(const char* tag, hipStream_t st);
  ~ProfScope();

 private:
  hipStream_t st_;
  int idx_;
};

// While alive, the calling thread's launches record no timing (timing
// creates HIP events, which the allocation-free entry point must not).
class NoTiming {
 public:
  NoTiming();
  ~NoTiming();
};

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
  int chunk_cols;          // columns per chunk: head_chunk_cols(dt, narrow)
  HeadSet sets[kMaxHeadSets];
  float* logits;           // nullable [B, L-1, width]
  float* pval;             // [B*(L-1), max_chunks]
  int32_t* pcol;           // [B*(L-1), max_chunks]
  float* offv;             // [B*(L-1)]
};
// Columns per LM-head work chunk; narrow chunks (bf16) give 4x the work
// items for layouts that would otherwise leave most CUs idle.
int head_chunk_cols(int dt, bool narrow = false);
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
