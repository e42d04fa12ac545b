/*
 * fpd.h -- C ABI of libfpd, the Flash Primitive Decoding block-drafter path
 * for AMD Instinct MI355X (gfx950).
 *
 * What the library computes (the pages are cited by title and section):
 *   - "VFlash: Fast, Accurate Visual Planning via Flash Primitive Decoding"
 *     (the paper, read in its Chinese translation), §2.1: features of
 *     selected target-VLM layers are fused and injected as key/value into
 *     every drafter layer; from the block's observed first token the drafter
 *     predicts every masked position in one bidirectional forward pass.
 *   - same paper, §2.2 and §2.3: a declared schema (type, coordinate
 *     dimensions, length) fixes the block length and each position's role;
 *     coordinates are one of 1,001 special tokens or fixed-width numeric
 *     fields (a sign and five digits, unused high digits filled).
 *   - same paper, §2.5: per-position legal vocabularies and a cross-position
 *     rule pairing off-frame image coordinates act on logits that are
 *     already computed; a structurally valid primitive is accepted by a
 *     schema validator.
 *   - the VFlash blog summary, "Method": text blocks of 16 positions are
 *     verified by the target, keeping the longest matching prefix and the
 *     target's next token.
 *   - "FlashDrive: Flash Vision-Language-Action Inference for Autonomous
 *     Driving", §3.2: fused target hidden states become the draft layers'
 *     KV cache.
 *
 * Conventions shared by every call:
 *   - Every tensor argument is caller-owned device memory, row-major,
 *     contiguous, 16-byte aligned.  bf16 tensors hold IEEE bfloat16; f32
 *     tensors hold float.  "DT" below is the drafter's dtype.
 *   - Weight tensors are BORROWED: the drafter keeps the device pointers,
 *     copies nothing, and the caller keeps the memory alive and unchanged
 *     until fpd_drafter_destroy.  W_lm may alias the embedding.
 *   - The hot-path calls, which take a `stream` (a hipStream_t passed as
 *     void*, NULL = the default stream), only enqueue work: they never
 *     allocate, never synchronise and return as soon as the work is
 *     queued.  The caller synchronises before reading results.
 *   - Arguments are checked on the host before anything is enqueued: a
 *     non-zero status means nothing was written.  FPD_E_HIP reports a
 *     launch failure (text in fpd_last_error); work enqueued before the
 *     failure may have run.
 *   - Handles are immutable after set-up: a drafter may be changed only by
 *     fpd_drafter_prepare, which the caller makes once, before any other
 *     call uses the drafter and from one thread.  After that, calls on
 *     different streams with distinct workspaces may run concurrently.
 *     Calls sharing a workspace must be ordered on one stream.
 *   - The hot-path calls touch no global state except an atomic flag that
 *     says whether per-launch timing (fpd_profile_enable) is on (with it
 *     off they take no lock) and, for fpd_draft_block_noalloc, the table
 *     of each device's static scratch address (read under a lock).
 *   - fpd_last_error() is thread-local and describes the most recent
 *     failing call on the calling thread.
 *   - Size limits: at most 2^24 rows (B x positions) per call, and for BF16
 *     drafters no operand of 4 GiB or more (the kernels address each
 *     operand through a 32-bit byte range): B*L*max(H, n_q*d, I)*2 bytes in
 *     the drafter forward, B*C*n_fused*H*2 in context fusion, B*(L-1)*H*2 in
 *     the LM head, and each weight matrix at creation.  Calls beyond them
 *     return FPD_E_SHAPE (rows) or FPD_E_UNSUPPORTED (bytes) before any work.
 */
#ifndef FPD_H
#define FPD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
enum {
  FPD_OK = 0,
  FPD_E_ARG = 1,          /* null pointer, bad enum, negative size           */
  FPD_E_SHAPE = 2,        /* inconsistent sizes between arguments, or more   */
                          /* than 2^24 rows (B x positions) in one call      */
  FPD_E_DTYPE = 3,        /* unknown dtype                                    */
  FPD_E_SCHEMA = 4,       /* schema expands to an invalid layout              */
  FPD_E_WORKSPACE = 5,    /* workspace smaller than fpd_workspace_size()      */
  FPD_E_UNSUPPORTED = 6,  /* a shape the kernels do not implement, or a bf16 */
                          /* operand of 4 GiB or more                        */
  FPD_E_HIP = 7           /* HIP runtime error (allocation, launch)           */
};

enum { FPD_DTYPE_F32 = 0, FPD_DTYPE_BF16 = 1 };

/* Schema kinds (VFlash paper §2.2-§2.3; blog "Method").  Per-point position
 * orders are this library's choice (the pages' layout table is not
 * available):
 *   TEXT           L = block_len, every position free (whole vocabulary);
 *   TRAJ2D         per waypoint [x, y, DELIM]                   -> L = 1 + 3n;
 *   TRAJ2D3D       per waypoint [u, v, X, Y, Z, DELIM]          -> L = 1 + 6n;
 *                  with off_id >= 0, u and v also allow OFF and (u, v) is a
 *                  pair decided jointly;
 *   POINTS3D_TEXT  per point ([SIGN, D, D, D, D, D] x 3, DELIM) -> L = 1 + 19n;
 *                  SIGN in {PLUS, MINUS}, D in {DIGIT0..DIGIT9, FILL};
 *   BOXES2D        per box [x1, y1, x2, y2, DELIM] (2D image corners) -> L = 1 + 5n;
 *   CUSTOM         explicit legal sets, per-position set indices, pairs and
 *                  fields (block_len = L).                                 */
enum {
  FPD_SCHEMA_TEXT = 0,
  FPD_SCHEMA_TRAJ2D = 1,
  FPD_SCHEMA_TRAJ2D3D = 2,
  FPD_SCHEMA_POINTS3D_TEXT = 3,
  FPD_SCHEMA_CUSTOM = 4,
  FPD_SCHEMA_BOXES2D = 5
};

/* Drafter shape.  H = hidden, heads of dim head_dim, n_q a multiple of n_kv,
 * I = inter (SwiGLU width), V = vocab, n_fused = number of target layers
 * whose features are fused into the context.  RoPE (rotate-half pairing
 * (i, i + d/2), inverse frequency theta^(-2i/d)) is applied to queries and
 * keys when use_rope != 0.  RMSNorm: x / sqrt(mean(x^2) + rms_eps) * g.
 * Supported: F32 with head_dim in {64, 128}; BF16 with head_dim 128.
 * hidden, inter and n_q*head_dim must be multiples of 64; hidden <= 4096. */
typedef struct fpd_config {
  int32_t hidden, n_q, n_kv, head_dim, n_layers, inter, vocab, n_fused;
  int32_t dtype;      /* FPD_DTYPE_*                                          */
  int32_t use_rope;   /* 0 disables rotary embedding                          */
  float rope_theta;
  float rms_eps;
} fpd_config;

/* One drafter layer (torch Linear layout [out, in], Y = X W^T), all DT:
 *   g_attn [H]; w_qkv [(n_q + 2 n_kv) d, H] (Q rows, then K rows, then V rows);
 *   w_o [H, n_q d]; g_mlp [H]; w_gu [2 I, H] (I gate rows, then I up rows);
 *   w_d [H, I].                                                            */
typedef struct fpd_layer_weights {
  const void *g_attn, *w_qkv, *w_o, *g_mlp, *w_gu, *w_d;
} fpd_layer_weights;

/* Whole drafter, all DT: w_fc [H, n_fused H] (fusion map over the
 * concatenated target layers); g_fc [H]; embed [V, H]; w_lm [V, H];
 * g_final [H]; layers: host array of n_layers entries (copied at create). */
typedef struct fpd_weights {
  const void *w_fc, *g_fc, *embed, *w_lm, *g_final;
  const fpd_layer_weights *layers;
} fpd_weights;

/* A declared primitive schema (VFlash paper §2.2: type, coordinate
 * dimensions and range/length; blog "Method": the tool call declares type
 * and length).  Token ids not used by a kind may be -1.  Coordinate ids are
 * coord_base .. coord_base + coord_count - 1; digits are digit0_id ..
 * digit0_id + 9.  CUSTOM fields (host pointers, read during the call only):
 *   set_offsets [n_sets + 1], set_ids [set_offsets[n_sets]] (CSR; each set
 *   is sorted and de-duplicated by the library), pos_set [block_len] with
 *   -2 at position 0 (the anchor), -1 for free positions, else a set index;
 *   pairs [n_pairs, 2] block positions (u, v) decided jointly with OFF;
 *   fields [n_fields, 2] (block position of the first digit, width 5).     */
typedef struct fpd_schema {
  int32_t kind;
  int32_t n_points;
  int32_t block_len;
  int32_t start_id, mask_id, delim_id, off_id, plus_id, minus_id, digit0_id, fill_id;
  int32_t coord_base, coord_count;
  int32_t n_sets;
  const int32_t *set_offsets, *set_ids, *pos_set;
  int32_t n_pairs;
  const int32_t *pairs;
  int32_t n_fields;
  const int32_t *fields;
} fpd_schema;

/* Sizes of an expanded layout.  width = the widest legal set, or V when
 * some position is free (the row width of fpd_constrained_argmax's
 * optional logits).                                                        */
typedef struct fpd_layout_sizes {
  int32_t L, n_sets, n_set_ids, n_pairs, n_fields, width;
} fpd_layout_sizes;

typedef struct fpd_drafter fpd_drafter;
typedef struct fpd_layout fpd_layout;

/* ---- handles ------------------------------------------------------------ */

/* Validates the shape and records the borrowed weight pointers.  Allocates
 * only host memory.  Errors: E_ARG (null), E_DTYPE, E_SHAPE (non-positive
 * or inconsistent sizes), E_UNSUPPORTED (see fpd_config).                  */
int32_t fpd_drafter_create(const fpd_config *cfg, const fpd_weights *w, fpd_drafter **out);
/* Frees the drafter and the tile copies fpd_drafter_prepare made.        */
int32_t fpd_drafter_destroy(fpd_drafter *d);

/* Copies the bf16 projections (w_qkv, w_o, w_gu, w_d of every layer, and
 * w_fc) into device memory owned by the drafter, K-tile-contiguous: within
 * each group of 32 rows, the 64-column K-tiles are stored one after
 * another, so each K step of a GEMM workgroup reads 4 KB-contiguous runs
 * of weights instead of 128-byte pieces of rows that lie 2 K bytes apart.
 * Later calls read the copies (same results: only the addresses change).
 * Call it once, right after fpd_drafter_create and before any other call
 * uses the drafter: it changes the handle, so it must not race with them.
 * The row-major weights stay borrowed (embed, w_lm and the norms are read
 * from them).  No-op for F32 drafters and for a drafter already prepared.
 * Allocating; synchronises `stream` (a hipStream_t, NULL = default).
 * Errors: E_ARG (null), E_HIP.                                            */
int32_t fpd_drafter_prepare(fpd_drafter *d, void *stream);

/* Host only, no GPU call: expands a schema into its layout for vocabulary
 * size `vocab` (VFlash paper §2.3: position alignment -- each position's role
 * is known before decoding).  Sets are numbered in order of first appearance
 * along the block (CUSTOM keeps the given order), each ascending.  Pass NULL
 * arrays to query sizes only; otherwise each array must hold the size
 * reported in `sizes`: pos_set [L], set_offsets [n_sets + 1], set_ids
 * [n_set_ids], pairs [n_pairs * 2], fields [n_fields * 2].
 * Errors: E_ARG, E_SCHEMA (id outside [0, vocab), empty set, bad pos_set,
 * pair or field that does not fit the layout).                            */
int32_t fpd_schema_expand(const fpd_schema *s, int32_t vocab, fpd_layout_sizes *sizes,
                          int32_t *pos_set, int32_t *set_offsets, int32_t *set_ids,
                          int32_t *pairs, int32_t *fields);

/* Expands the schema (as fpd_schema_expand), uploads the layout tables and
 * gathers the legal W_lm rows of every set into one contiguous device
 * buffer, once per layout (so the constrained LM head streams only legal
 * rows).  This, fpd_drafter_create and fpd_drafter_prepare are the only
 * allocating calls; this one synchronises the device before returning.
 * *L_out receives L.                                                      */
int32_t fpd_layout_create(const fpd_drafter *d, const fpd_schema *s, fpd_layout **out,
                          int32_t *L_out);
int32_t fpd_layout_destroy(fpd_layout *lay);
/* Host copies of a created layout's tables (same format as
 * fpd_schema_expand; NULL arrays skip).                                    */
int32_t fpd_layout_masks(const fpd_layout *lay, fpd_layout_sizes *sizes, int32_t *pos_set,
                         int32_t *set_offsets, int32_t *set_ids, int32_t *pairs, int32_t *fields);

/* Bytes of device workspace that any call below needs for batch B, context
 * capacity C and block length L (one workspace serves all of them).       */
int32_t fpd_workspace_size(const fpd_drafter *d, int32_t B, int32_t C, int32_t L, size_t *bytes);

/* ---- hot path ------------------------------------------------------------ */

/* Context fusion (VFlash paper §2.1; FlashDrive §3.2).  feats [B, n_fused,
 * C, H] DT holds the selected target layers' features in layer order.
 *   X = [F_1 | ... | F_nt] (features concatenated), Z = X W_fc^T,
 *   Zn = RMSNorm(Z; g_fc), and for every drafter layer l:
 *   K_c = RoPE(Zn Wk_l^T) at positions pos0 .. pos0 + C - 1, V_c = Zn Wv_l^T,
 * where Wk_l / Wv_l are the K / V rows of layer l's w_qkv.
 * Writes keys 0..C-1 of ctx_k [n_layers, B, n_kv, ctx_cap, d] DT (keys
 * stored after RoPE) and of ctx_v [n_layers, B, n_kv, d, ctx_cap] (values
 * stored d-major, so attention reads them along keys).  ctx_v's element type
 * is the value type VT: float for F32 drafters; for BF16 drafters IEEE fp16
 * holding each value rounded to bf16 (exact for |v| in [2^-17, 65504];
 * larger magnitudes overflow), so that attention multiplies fp16
 * probabilities with them.  ctx_cap >= C and a
 * multiple of 8.  Entries at keys >= C are left untouched and may hold
 * anything (they never reach an output of fpd_draft_block).               */
int32_t fpd_fuse_context_kv(const fpd_drafter *d, const void *feats, int32_t B, int32_t C,
                            int32_t pos0, void *ctx_k, void *ctx_v, int32_t ctx_cap, void *ws,
                            size_t ws_bytes, void *stream);

/* Incremental context (VFlash paper §2.5: after a primitive or text block
 * is committed, the target's forward pass updates the cache and the context
 * features; FlashDrive §3.2, Fig. 4: the drafter is conditioned on the hidden
 * states of the newest target tokens).  feats [B, n_fused, C_new, H] DT hold
 * the selected layers' features of target positions pos0 .. pos0+C_new-1.
 * They are fused exactly as in fpd_fuse_context_kv, and their K/V are written
 * at key rows pos0 .. pos0+C_new-1 of ctx_k / ctx_v (same layouts), with keys
 * rotated at those positions.  Other rows are untouched, so appending the
 * context in pieces gives the caches of one fusion of the whole.  Needs
 * pos0 + C_new <= ctx_cap (a multiple of 8).  Workspace as for
 * fpd_fuse_context_kv with C = C_new.                                      */
int32_t fpd_append_context_kv(const fpd_drafter *d, const void *feats, int32_t B, int32_t C_new,
                              int32_t pos0, void *ctx_k, void *ctx_v, int32_t ctx_cap, void *ws,
                              size_t ws_bytes, void *stream);

/* One drafter forward over a block (VFlash paper §2.1-§2.2): tokens [B, L]
 * int32 = the anchor then the mask token at positions 1..L-1 (any ids in
 * [0, V) are accepted).  h = E[tokens]; then per layer (pre-norm, fp32
 * residual stream): a = RMSNorm(h); Q, K_b, V_b = a W_qkv^T with RoPE on Q
 * and K_b at positions block_pos .. block_pos + L - 1; non-causal grouped
 * attention of every block query over [context rows 0..C-1 || all L block
 * rows] (query head i reads KV head floor(i n_kv / n_q), scale d^-1/2, no
 * mask); h += O W_o^T; m = RMSNorm(h); h += (silu(m Wg^T) * (m Wu^T)) Wd^T.
 * Writes hidden_out [B, L-1, H] DT = RMSNorm(h; g_final) of positions
 * 1..L-1 (position 0 predicts nothing).  ctx_k/ctx_v as written by
 * fpd_fuse_context_kv with the same ctx_cap.  C may be 0.                  */
int32_t fpd_draft_block(const fpd_drafter *d, const int32_t *tokens, int32_t B, int32_t L,
                        const void *ctx_k, const void *ctx_v, int32_t C, int32_t ctx_cap,
                        int32_t block_pos, void *hidden_out, void *ws, size_t ws_bytes,
                        void *stream);

/* The same as fpd_draft_block without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation).  Its scratch is a static
 * 64 MiB device array inside the library, one per GPU, held until the process
 * ends; nothing is allocated or freed, and no per-launch timing is recorded.
 * Every call on one GPU shares that GPU's array and leaves its contents
 * behind (no call needs it cleared), so calls that overlap on one GPU race:
 * order them on one stream.  Errors as fpd_draft_block, plus FPD_E_WORKSPACE
 * when the block needs more scratch than the array holds (fpd_workspace_size
 * reports the need; the 64-waypoint 385-position block over 4,096 context
 * rows takes about 47 MB), FPD_E_UNSUPPORTED beyond device index 63.       */
int32_t fpd_draft_block_noalloc(const fpd_drafter *d, const int32_t *tokens, int32_t B, int32_t L,
                                const void *ctx_k, const void *ctx_v, int32_t C, int32_t ctx_cap,
                                int32_t block_pos, void *hidden_out, void *stream);

/* Several primitives against one shared observation (VFlash paper,
 * conclusion and future work: complementary primitives predicted from one
 * observation).  Same as fpd_draft_block for B blocks of the same length L,
 * except that every block attends to the one context in ctx_k
 * [n_layers, 1, n_kv, ctx_cap, d] / ctx_v [n_layers, 1, n_kv, d, ctx_cap]
 * (written by fpd_fuse_context_kv / fpd_append_context_kv with B = 1).
 * The projections then run on M = B*L rows at the weight bytes of one block.
 * tokens [B, L]: each block's own anchor, then mask tokens.                */
int32_t fpd_draft_blocks_shared_ctx(const fpd_drafter *d, const int32_t *tokens, int32_t B, int32_t L,
                                    const void *ctx_k, const void *ctx_v, int32_t C, int32_t ctx_cap,
                                    int32_t block_pos, void *hidden_out, void *ws, size_t ws_bytes,
                                    void *stream);

/* Constrained decoding (VFlash paper §2.5).  hidden [B, L-1, H] DT from
 * fpd_draft_block.  For each position p the logits z_p[s] = h_p . W_lm[s]
 * are computed only for s in the legal set S_p (every id for free
 * positions); t_p = the lowest id attaining the maximum over S_p (a NaN
 * logit counts as the maximum).  Then every declared pair (u, v) is decided
 * jointly: (OFF, OFF) wins only if z_u[OFF] + z_v[OFF] is strictly greater
 * than the best on-frame z_u[a] + z_v[b]; otherwise the best on-frame ids.
 * Writes tokens_out [B, L-1] int32.  logits_out (nullable) [B, L-1, width]
 * float receives each position's legal logits in ascending id order, padded
 * with -inf (for checking only; it adds the write traffic).               */
int32_t fpd_constrained_argmax(const fpd_drafter *d, const fpd_layout *lay, const void *hidden,
                               int32_t B, int32_t *tokens_out, float *logits_out, void *ws,
                               size_t ws_bytes, void *stream);

/* Schema validator a(y) (VFlash paper §2.5; blog "Why it's interesting":
 * accepted wholesale when the structure matches).  tokens [B, L-1] int32.
 * Valid iff every token lies in its position's legal set (free: [0, V)),
 * every pair is both OFF or both on-frame, and every numeric field's five
 * digit slots read FILL^j DIGIT^(5-j) with 0 <= j <= 4.  Writes k_out [B] =
 * L-1 if valid else 0 (all or nothing) and first_invalid_out [B] = the
 * smallest failing index into tokens (a pair fails at its first position,
 * a field at its first out-of-pattern slot), -1 if valid.                 */
int32_t fpd_validate_primitive(const fpd_layout *lay, const int32_t *tokens, int32_t B,
                               int32_t *k_out, int32_t *first_invalid_out, void *stream);

/* Box partial acceptance (VFlash paper §2.5: the acceptance test adds an
 * external spatial-confidence check for boxes, and the drafts before the
 * first uncertain coordinate are kept; the rest is regenerated by the
 * target).  tokens [B, L-1] int32; conf [B, L-1] float, one externally
 * supplied confidence per drafted position, read only at coordinate
 * positions (legal set inside the schema's coordinate ids, OFF allowed).  A
 * coordinate is uncertain unless conf >= tau (NaN is uncertain).  Runs the
 * schema validator of fpd_validate_primitive and writes first_invalid_out
 * [B] as it does, first_uncertain_out [B] = the smallest uncertain
 * coordinate index into tokens or -1, and k_out [B] = the smaller of the two
 * indices that are >= 0, L-1 when both are -1.  Applies to any layout;
 * trajectories keep their all-or-nothing rule (fpd_validate_primitive).
 * Errors: E_ARG (null, NaN tau), E_SHAPE (B < 1).                         */
int32_t fpd_accept_boxes(const fpd_layout *lay, const int32_t *tokens, const float *conf, float tau, int32_t B,
                         int32_t *k_out, int32_t *first_invalid_out, int32_t *first_uncertain_out, void *stream);

/* Greedy prefix verification (VFlash paper §2.1; blog "Method").  draft
 * [B, L-1] int32 = t_1..t_{L-1}; target [B, L] int32 = g_0..g_{L-1}, g_j the
 * target's greedy token after the anchor and t_1..t_j.  Writes k_out [B] =
 * the number of leading i with t_i = g_{i-1}, and next_out [B] = g_k (the
 * target's own next token, committed after the k accepted drafts).        */
int32_t fpd_verify_prefix(const int32_t *draft, const int32_t *target, int32_t B, int32_t L,
                          int32_t *k_out, int32_t *next_out, void *stream);

/* ---- coordinate codec (VFlash paper §2.3 "Token representation"; §3.1
 * "Base VLM") ------------------------------------------------------------
 * A coordinate occupies one of 1,001 tokens coord_base .. coord_base+1000:
 * 2D image coordinates are normalised to 0..1000 (lo 0, hi 1000), 3D
 * coordinates are quantised uniformly over a predefined range [lo, hi] (its
 * values are not printed, so it is a parameter).  All device arrays, n
 * entries, stream-ordered; nothing allocates.                              */

/* bin = clamp(round-half-even((x - lo) * (1000 / (hi - lo))), 0, 1000)
 * computed in double precision; tokens_out = coord_base + bin, or -1 for a
 * NaN value.  values float [n].  Needs finite lo < hi.                     */
int32_t fpd_coords_to_tokens(const float *values, int32_t n, double lo, double hi, int32_t coord_base,
                             int32_t *tokens_out, void *stream);

/* values_out double [n] = lo + bin * ((hi - lo) / 1000) for a coordinate
 * token (bin = token - coord_base in 0..1000), NaN for any other token.    */
int32_t fpd_tokens_to_coords(const int32_t *tokens, int32_t n, double lo, double hi, int32_t coord_base,
                             double *values_out, void *stream);

/* Fixed-width numeric fields (VFlash paper §2.3): values int32 [n] ->
 * fields_out int32 [n, 6] = sign (plus_id for n >= 0, minus_id below), then
 * |n| as five decimal digits (digit0_id + d) whose leading zeros, except the
 * last digit, are fill_id.  |n| > 99,999 does not fit: six -1 tokens.      */
int32_t fpd_ints_to_fields(const int32_t *values, int32_t n, int32_t plus_id, int32_t minus_id,
                           int32_t digit0_id, int32_t fill_id, int32_t *fields_out, void *stream);

/* Inverse: fields int32 [n, 6] -> values_out [n] and valid_out [n] (1 when
 * the sign slot holds plus_id / minus_id and the digits read
 * fill^j digit^(5-j) with j <= 4, the field rule of the validator; invalid
 * fields give value 0).                                                    */
int32_t fpd_fields_to_ints(const int32_t *fields, int32_t n, int32_t plus_id, int32_t minus_id,
                           int32_t digit0_id, int32_t fill_id, int32_t *values_out, int32_t *valid_out,
                           void *stream);

/* ---- diagnostics -------------------------------------------------------- */
const char *fpd_status_string(int32_t status);
const char *fpd_last_error(void);

/* Per-launch timing for performance measurement (not part of the method).
 * fpd_profile_enable(1) clears earlier records and, from then on, brackets
 * every kernel launch of the hot calls with a pair of HIP events on the
 * call's stream; fpd_profile_enable(0) stops recording (records stay
 * readable until the next enable).  After synchronising the stream,
 * fpd_profile_read(i, ...) returns record i's kernel tag (a static string,
 * e.g. "gemm_gate_up", "attention", "lm_head") and its duration in ms.
 * The events add a little launch overhead, so time throughput separately. */
int32_t fpd_profile_enable(int32_t on);
int32_t fpd_profile_count(int32_t *n);
int32_t fpd_profile_read(int32_t i, const char **tag, float *ms);

#ifdef __cplusplus
}
#endif
#endif /* FPD_H */
