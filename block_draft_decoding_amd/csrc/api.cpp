// libfpd C ABI: argument checking, workspace planning, layouts, and the
// launch sequences of the hot calls.  See include/fpd.h for the contract.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/fpd.h"
#include "kernels.h"
#include "layout.h"

using namespace fpd;

// Static device scratch of fpd_draft_block_noalloc: 64 MiB per GPU, held
// until the process ends (see noalloc_scratch below).
static constexpr size_t kNoallocScratchBytes = size_t(64) << 20;
static __device__ __align__(256) unsigned char g_noalloc_scratch[kNoallocScratchBytes];

namespace {

thread_local std::string g_err;

int32_t fail(int32_t code, const std::string& msg) {
  g_err = msg;
  return code;
}

#define FPD_TRY_HIP(expr)                                                           \
  do {                                                                              \
    hipError_t e_ = (expr);                                                         \
    if (e_ != hipSuccess) return fail(FPD_E_HIP, std::string(#expr) + ": " + hipGetErrorString(e_)); \
  } while (0)

size_t al(size_t x) { return (x + 255) & ~(size_t)255; }
int round8(int x) { return (x + 7) & ~7; }

// Row counts (B x positions) are kept in int arithmetic by the launches;
// beyond 2^24 rows the workspace alone would exceed any GPU's memory.
constexpr int64_t kMaxRows = int64_t(1) << 24;
bool too_many_rows(int32_t B, int32_t n) { return (int64_t)B * n > kMaxRows; }

// The bf16 kernels read every operand through a buffer descriptor whose
// byte range is 32 bits wide, so no single operand of a call may reach
// 4 GiB: per call, the widest activation rows times the row count (drafter
// forward: normed hidden, attention output and SwiGLU output rows of B x L
// positions; context fusion: the n_t layers' feature rows of B x C
// positions; LM head: hidden rows of B x (L - 1) positions), and per drafter
// each weight matrix (rows padded to 32 in the K-tile-contiguous copies).
constexpr int64_t kMaxOperandBytes = 0xffffffffll;
int64_t forward_row_bytes(const fpd_config& c) {
  return c.dtype == FPD_DTYPE_BF16 ? (int64_t)std::max({c.hidden, c.n_q * c.head_dim, c.inter}) * 2 : 0;
}
int64_t fusion_row_bytes(const fpd_config& c) {
  return c.dtype == FPD_DTYPE_BF16 ? (int64_t)c.n_fused * c.hidden * 2 : 0;
}
bool over_4gib(int64_t rows, int64_t row_bytes) { return rows * row_bytes > kMaxOperandBytes; }
int64_t widest_weight_bytes(const fpd_config& c) {
  auto w = [](int64_t rows, int64_t k) { return (rows + 31) / 32 * 32 * k * 2; };
  const int64_t q = (int64_t)c.n_q * c.head_dim, kv = (int64_t)c.n_kv * c.head_dim, H = c.hidden;
  return std::max({w(q + 2 * kv, H), w(H, q), w(2 * (int64_t)c.inter, H), w(H, c.inter),
                   w(H, (int64_t)c.n_fused * H), w(c.vocab, H)});
}

}  // namespace

struct fpd_drafter {
  fpd_config cfg;
  fpd_weights w;
  std::vector<fpd_layer_weights> layers;
  RopeTab tab;
  int esz;
  // K-tile-contiguous copies of the projections (fpd_drafter_prepare): one
  // device buffer; per layer q/k/v, O, gate/up and down, then the fusion map
  void* tiled = nullptr;
  std::vector<const void*> t_qkv, t_o, t_gu, t_d;
  const void* t_fc = nullptr;
};

struct fpd_layout {
  const fpd_drafter* d = nullptr;
  HostLayout host;
  int32_t* dev = nullptr;  // all integer tables
  void* wg = nullptr;      // gathered legal W_lm rows [n_set_ids, H]
  // device table pointers (into dev)
  int32_t *pos_set, *set_offsets, *set_ids, *partner, *field_w, *row_cols, *set_pos, *coord;
  std::vector<int32_t> set_pos_off;  // [n_sets + 2]: positions of set s, then free positions
  std::vector<int32_t> off_col;      // [n_sets]
};

namespace {

// ---- workspace plans --------------------------------------------------------------
struct DraftWs {
  size_t h, a, q, kb, vbt, o, u, partial, attn, total;
  size_t partial_bytes, attn_bytes;
};

size_t gemm_partial_bytes(int dt, int M, int ncols, int K, int nw, bool paired) {
  if (dt != FPD_DTYPE_BF16) return 0;
  return plan_gemm_bf16(M, ncols, K, nw, paired).partial_floats * sizeof(float);
}

DraftWs plan_draft(const fpd_drafter& d, int B, int L, int C) {
  const fpd_config& c = d.cfg;
  const size_t e = d.esz, M = (size_t)B * L, H = c.hidden, dh = c.head_dim;
  const int Lp = round8(L);
  DraftWs w{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += al(bytes);
    return o;
  };
  w.h = take(M * H * 4);
  w.a = take(M * H * e);
  w.q = take((size_t)B * c.n_q * L * dh * e);
  w.kb = take((size_t)B * c.n_kv * L * dh * e);
  w.vbt = take((size_t)B * c.n_kv * dh * Lp * e);
  w.o = take(M * c.n_q * dh * e);
  w.u = take(M * (size_t)c.inter * e);
  const int dt = c.dtype, m = (int)M, qd = c.n_q * c.head_dim;
  size_t pb = 0;
  pb = std::max(pb, gemm_partial_bytes(dt, m, (c.n_q + 2 * c.n_kv) * c.head_dim / 2, c.hidden,
                                       (c.n_q + 2 * c.n_kv) * c.head_dim, true));
  // O and the MLP run on all rows, and in the last layer of a single block on L - 1
  for (const int mr : {m, B == 1 ? L - 1 : m}) {
    pb = std::max(pb, gemm_partial_bytes(dt, mr, c.hidden, qd, c.hidden, false));
    pb = std::max(pb, gemm_partial_bytes(dt, mr, c.inter, c.hidden, 2 * c.inter, true));
    pb = std::max(pb, gemm_partial_bytes(dt, mr, c.hidden, c.inter, c.hidden, false));
  }
  w.partial_bytes = pb;
  w.partial = take(pb);
  w.attn_bytes = attention_scratch_bytes(dt, B, L, C, c.n_q, c.n_kv, c.head_dim);
  w.attn = take(w.attn_bytes);
  w.total = off;
  return w;
}

struct FuseWs {
  size_t x, z, zn, partial, total, partial_bytes;
};

FuseWs plan_fuse(const fpd_drafter& d, int B, int C) {
  const fpd_config& c = d.cfg;
  const size_t e = d.esz, M = (size_t)B * C, H = c.hidden;
  FuseWs w{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += al(bytes);
    return o;
  };
  // bf16 reads the features in place; f32 concatenates them first
  w.x = take(c.n_fused > 1 && c.dtype != FPD_DTYPE_BF16 ? M * c.n_fused * H * e : 0);
  w.z = take(M * H * 4);
  w.zn = take(M * H * e);
  size_t pb = gemm_partial_bytes(c.dtype, (int)M, c.hidden, c.n_fused * c.hidden, c.hidden, false);
  pb = std::max(pb, gemm_partial_bytes(c.dtype, (int)M, c.n_kv * c.head_dim, c.hidden,
                                       2 * c.n_kv * c.head_dim, true));
  w.partial_bytes = pb;
  w.partial = take(pb);
  w.total = off;
  return w;
}

struct HeadWs {
  size_t pval, pcol, offv, total;
};

HeadWs plan_head(int B, int L, int max_chunks) {
  const size_t rows = (size_t)B * (L - 1);
  HeadWs w{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += al(bytes);
    return o;
  };
  w.pval = take(rows * max_chunks * 4);
  w.pcol = take(rows * max_chunks * 4);
  w.offv = take(rows * 4);
  w.total = off;
  return w;
}

int32_t check_ws(const void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return FPD_OK;
  if (!ws) return fail(FPD_E_ARG, "workspace is null");
  if (ws_bytes < need)
    return fail(FPD_E_WORKSPACE, "workspace has " + std::to_string(ws_bytes) + " bytes, needs " +
                                     std::to_string(need));
  return FPD_OK;
}

char* wsp(void* ws, size_t off) { return (char*)ws + off; }

}  // namespace

extern "C" {

const char* fpd_status_string(int32_t s) {
  switch (s) {
    case FPD_OK: return "ok";
    case FPD_E_ARG: return "invalid argument";
    case FPD_E_SHAPE: return "inconsistent shape";
    case FPD_E_DTYPE: return "unknown dtype";
    case FPD_E_SCHEMA: return "invalid schema";
    case FPD_E_WORKSPACE: return "workspace too small";
    case FPD_E_UNSUPPORTED: return "unsupported shape";
    case FPD_E_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* fpd_last_error(void) { return g_err.c_str(); }

int32_t fpd_drafter_create(const fpd_config* cfg, const fpd_weights* w, fpd_drafter** out) {
  if (!cfg || !w || !out) return fail(FPD_E_ARG, "null argument");
  *out = nullptr;
  const fpd_config& c = *cfg;
  if (c.dtype != FPD_DTYPE_F32 && c.dtype != FPD_DTYPE_BF16) return fail(FPD_E_DTYPE, "unknown dtype");
  if (c.hidden <= 0 || c.n_q <= 0 || c.n_kv <= 0 || c.head_dim <= 0 || c.n_layers <= 0 || c.inter <= 0 ||
      c.vocab <= 0 || c.n_fused <= 0)
    return fail(FPD_E_SHAPE, "every size must be positive");
  if (c.n_q % c.n_kv != 0) return fail(FPD_E_SHAPE, "n_q must be a multiple of n_kv");
  if (!(c.rms_eps >= 0.f) || !(c.rope_theta > 0.f)) return fail(FPD_E_ARG, "rms_eps >= 0 and rope_theta > 0 required");
  if (c.hidden % 64 || c.inter % 64 || (c.n_q * c.head_dim) % 64)
    return fail(FPD_E_UNSUPPORTED, "hidden, inter and n_q*head_dim must be multiples of 64");
  if (c.hidden > 4096) return fail(FPD_E_UNSUPPORTED, "hidden above 4096 is not supported");
  if (c.dtype == FPD_DTYPE_BF16 && c.head_dim != 128)
    return fail(FPD_E_UNSUPPORTED, "bf16 drafters need head_dim 128");
  if (c.dtype == FPD_DTYPE_F32 && c.head_dim != 64 && c.head_dim != 128)
    return fail(FPD_E_UNSUPPORTED, "f32 drafters need head_dim 64 or 128");
  if (c.dtype == FPD_DTYPE_BF16 && widest_weight_bytes(c) > kMaxOperandBytes)
    return fail(FPD_E_UNSUPPORTED, "a bf16 weight matrix of 4 GiB or more");
  if (!w->w_fc || !w->g_fc || !w->embed || !w->w_lm || !w->g_final || !w->layers)
    return fail(FPD_E_ARG, "null weight pointer");
  for (int i = 0; i < c.n_layers; ++i) {
    const fpd_layer_weights& l = w->layers[i];
    if (!l.g_attn || !l.w_qkv || !l.w_o || !l.g_mlp || !l.w_gu || !l.w_d)
      return fail(FPD_E_ARG, "null weight pointer in layer " + std::to_string(i));
  }
  fpd_drafter* d = new fpd_drafter;
  d->cfg = c;
  d->w = *w;
  d->layers.assign(w->layers, w->layers + c.n_layers);
  d->w.layers = d->layers.data();
  d->esz = c.dtype == FPD_DTYPE_BF16 ? 2 : 4;
  std::memset(&d->tab, 0, sizeof(d->tab));
  const int half = c.head_dim / 2;
  for (int i = 0; i < half; ++i)
    d->tab.inv_rev[i] = std::pow((double)c.rope_theta, -2.0 * i / (double)c.head_dim) / (2.0 * M_PI);
  *out = d;
  return FPD_OK;
}

int32_t fpd_drafter_destroy(fpd_drafter* d) {
  if (d && d->tiled) (void)hipFree(d->tiled);
  delete d;
  return FPD_OK;
}

int32_t fpd_drafter_prepare(fpd_drafter* d, void* stream) {
  if (!d) return fail(FPD_E_ARG, "null drafter");
  const fpd_config& c = d->cfg;
  if (c.dtype != FPD_DTYPE_BF16 || d->tiled) return FPD_OK;
  const int H = c.hidden, dh = c.head_dim, qd = c.n_q * dh, nqkv = (c.n_q + 2 * c.n_kv) * dh;
  const size_t e_qkv = gemm_tiles_elems(nqkv, H), e_o = gemm_tiles_elems(H, qd),
               e_gu = gemm_tiles_elems(2 * c.inter, H), e_d = gemm_tiles_elems(H, c.inter),
               e_fc = gemm_tiles_elems(H, c.n_fused * H);
  const size_t per_layer = e_qkv + e_o + e_gu + e_d;
  void* buf = nullptr;
  hipError_t e = hipMalloc(&buf, (per_layer * c.n_layers + e_fc) * 2);
  if (e != hipSuccess) return fail(FPD_E_HIP, std::string("tiled weights: ") + hipGetErrorString(e));
  hipStream_t s = (hipStream_t)stream;
  bf16_t* p = (bf16_t*)buf;
  // copies W [rows, K] to the next free place of the buffer and returns it
  auto pack = [&](const void* W, int rows, int K, size_t elems) -> const void* {
    const void* at = p;
    if (e == hipSuccess) e = gemm_pack_tiles(W, rows, K, p, s);
    p += elems;
    return at;
  };
  std::vector<const void*> tq, to, tg, td;
  for (int li = 0; li < c.n_layers; ++li) {
    const fpd_layer_weights& lw = d->layers[li];
    tq.push_back(pack(lw.w_qkv, nqkv, H, e_qkv));
    to.push_back(pack(lw.w_o, H, qd, e_o));
    tg.push_back(pack(lw.w_gu, 2 * c.inter, H, e_gu));
    td.push_back(pack(lw.w_d, H, c.inter, e_d));
  }
  const void* tfc = pack(d->w.w_fc, H, c.n_fused * H, e_fc);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) {
    (void)hipFree(buf);
    return fail(FPD_E_HIP, std::string("tiled weights: ") + hipGetErrorString(e));
  }
  d->tiled = buf;
  d->t_qkv = tq, d->t_o = to, d->t_gu = tg, d->t_d = td, d->t_fc = tfc;
  return FPD_OK;
}

static int32_t copy_sizes_and_tables(const HostLayout& h, fpd_layout_sizes* sizes, int32_t* pos_set,
                                     int32_t* set_offsets, int32_t* set_ids, int32_t* pairs,
                                     int32_t* fields) {
  if (sizes) {
    sizes->L = h.L;
    sizes->n_sets = h.n_sets();
    sizes->n_set_ids = (int32_t)h.set_ids.size();
    sizes->n_pairs = (int32_t)h.pairs.size() / 2;
    sizes->n_fields = (int32_t)h.fields.size() / 2;
    sizes->width = h.width();
  }
  auto cp = [](int32_t* dst, const std::vector<int32_t>& v) {
    if (dst && !v.empty()) std::memcpy(dst, v.data(), v.size() * sizeof(int32_t));
  };
  cp(pos_set, h.pos_set);
  cp(set_offsets, h.set_offsets);
  cp(set_ids, h.set_ids);
  cp(pairs, h.pairs);
  cp(fields, h.fields);
  return FPD_OK;
}

int32_t fpd_schema_expand(const fpd_schema* s, int32_t vocab, fpd_layout_sizes* sizes, int32_t* pos_set,
                          int32_t* set_offsets, int32_t* set_ids, int32_t* pairs, int32_t* fields) {
  if (!s) return fail(FPD_E_ARG, "null schema");
  HostLayout h;
  std::string err;
  const int32_t st = expand_schema(*s, vocab, &h, &err);
  if (st != FPD_OK) return fail(st, err);
  return copy_sizes_and_tables(h, sizes, pos_set, set_offsets, set_ids, pairs, fields);
}

int32_t fpd_layout_create(const fpd_drafter* d, const fpd_schema* s, fpd_layout** out, int32_t* L_out) {
  if (!d || !s || !out) return fail(FPD_E_ARG, "null argument");
  *out = nullptr;
  fpd_layout* lay = new fpd_layout;
  lay->d = d;
  std::string err;
  int32_t st = expand_schema(*s, d->cfg.vocab, &lay->host, &err);
  if (st != FPD_OK) {
    delete lay;
    return fail(st, err);
  }
  const HostLayout& h = lay->host;
  const int L = h.L, ns = h.n_sets();
  if (ns > kMaxHeadSets) {
    delete lay;
    return fail(FPD_E_UNSUPPORTED, "layouts with more than 32 legal sets are not supported");
  }
  // derived tables
  std::vector<int32_t> partner(L, -1), field_w(L, 0), row_cols(L, 0), set_pos;
  for (size_t i = 0; i < h.pairs.size(); i += 2) {
    partner[h.pairs[i]] = h.pairs[i + 1];
    partner[h.pairs[i + 1]] = -2;
  }
  for (size_t i = 0; i < h.fields.size(); i += 2) field_w[h.fields[i]] = h.fields[i + 1];
  for (int p = 1; p < L; ++p)
    row_cols[p] = h.pos_set[p] == -1 ? h.vocab : h.set_offsets[h.pos_set[p] + 1] - h.set_offsets[h.pos_set[p]];
  lay->set_pos_off.assign(ns + 2, 0);
  for (int s2 = 0; s2 <= ns; ++s2) {
    lay->set_pos_off[s2] = (int32_t)set_pos.size();
    const int want = s2 < ns ? s2 : -1;
    for (int p = 1; p < L; ++p)
      if (h.pos_set[p] == want) set_pos.push_back(p);
  }
  lay->set_pos_off[ns + 1] = (int32_t)set_pos.size();
  lay->off_col.assign(ns, -1);
  for (int s2 = 0; s2 < ns; ++s2)
    for (int i = h.set_offsets[s2]; i < h.set_offsets[s2 + 1]; ++i)
      if (h.off_id >= 0 && h.set_ids[i] == h.off_id) lay->off_col[s2] = i - h.set_offsets[s2];

  std::vector<int32_t> all;
  auto put = [&](const std::vector<int32_t>& v) {
    const size_t o = all.size();
    all.insert(all.end(), v.begin(), v.end());
    all.push_back(0);  // keeps every table non-empty
    return o;
  };
  const size_t o_pos = put(h.pos_set), o_off = put(h.set_offsets), o_ids = put(h.set_ids),
               o_par = put(partner), o_fw = put(field_w), o_rc = put(row_cols), o_sp = put(set_pos),
               o_co = put(h.coord);
  hipError_t e = hipMalloc((void**)&lay->dev, all.size() * sizeof(int32_t));
  if (e == hipSuccess) e = hipMemcpy(lay->dev, all.data(), all.size() * sizeof(int32_t), hipMemcpyHostToDevice);
  const size_t nid = h.set_ids.size(), H = d->cfg.hidden;
  if (e == hipSuccess && nid > 0) e = hipMalloc(&lay->wg, nid * H * d->esz);
  if (e == hipSuccess) {
    lay->pos_set = lay->dev + o_pos;
    lay->set_offsets = lay->dev + o_off;
    lay->set_ids = lay->dev + o_ids;
    lay->partner = lay->dev + o_par;
    lay->field_w = lay->dev + o_fw;
    lay->row_cols = lay->dev + o_rc;
    lay->set_pos = lay->dev + o_sp;
    lay->coord = lay->dev + o_co;
    if (nid > 0) e = gather_rows(d->cfg.dtype, d->w.w_lm, (int)H, lay->set_ids, (int)nid, lay->wg, nullptr);
  }
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    fpd_layout_destroy(lay);
    return fail(FPD_E_HIP, std::string("layout upload: ") + hipGetErrorString(e));
  }
  if (L_out) *L_out = L;
  *out = lay;
  return FPD_OK;
}

int32_t fpd_layout_destroy(fpd_layout* lay) {
  if (!lay) return FPD_OK;
  if (lay->dev) (void)hipFree(lay->dev);
  if (lay->wg) (void)hipFree(lay->wg);
  delete lay;
  return FPD_OK;
}

int32_t fpd_layout_masks(const fpd_layout* lay, fpd_layout_sizes* sizes, int32_t* pos_set,
                         int32_t* set_offsets, int32_t* set_ids, int32_t* pairs, int32_t* fields) {
  if (!lay) return fail(FPD_E_ARG, "null layout");
  return copy_sizes_and_tables(lay->host, sizes, pos_set, set_offsets, set_ids, pairs, fields);
}

int32_t fpd_workspace_size(const fpd_drafter* d, int32_t B, int32_t C, int32_t L, size_t* bytes) {
  if (!d || !bytes) return fail(FPD_E_ARG, "null argument");
  if (B < 1 || C < 0 || L < 2) return fail(FPD_E_SHAPE, "need B >= 1, C >= 0, L >= 2");
  if (too_many_rows(B, C) || too_many_rows(B, L)) return fail(FPD_E_SHAPE, "more than 2^24 rows");
  if (over_4gib((int64_t)B * L, forward_row_bytes(d->cfg)) || over_4gib((int64_t)B * C, fusion_row_bytes(d->cfg)))
    return fail(FPD_E_UNSUPPORTED, "a bf16 operand of 4 GiB or more (too many rows for one call)");
  // LM-head partials: wide chunks of the whole vocabulary, or narrow chunks,
  // which are used only while the wide ones number under 128 per launch
  // (at most 4 x 127 narrow chunks in a row)
  const int wide = head_chunk_cols(d->cfg.dtype), narrow = head_chunk_cols(d->cfg.dtype, true);
  const int worst = std::max((d->cfg.vocab + wide - 1) / wide,
                             std::min((d->cfg.vocab + narrow - 1) / narrow, 4 * 127));
  size_t need = plan_draft(*d, B, L, C).total;
  if (C > 0) need = std::max(need, plan_fuse(*d, B, C).total);
  need = std::max(need, plan_head(B, L, worst).total);
  *bytes = need;
  return FPD_OK;
}

}  // extern "C"

namespace {

// Fuses C positions of features and writes their K/V at key rows 0..C-1 of
// the given layer-0 bases (strides from ctx_cap), keys rotated at rope_pos0 + c.
int32_t fuse_rows(const fpd_drafter* d, const void* feats, int32_t B, int32_t C, int32_t rope_pos0, char* kbase,
                  char* vbase, int32_t ctx_cap, void* ws, size_t ws_bytes, void* stream) {
  const FuseWs w = plan_fuse(*d, B, C);
  if (int32_t st = check_ws(ws, ws_bytes, w.total)) return st;
  const fpd_config& c = d->cfg;
  const int dt = c.dtype, H = c.hidden, M = B * C, dh = c.head_dim;
  hipStream_t s = (hipStream_t)stream;
  float* Z = (float*)wsp(ws, w.z);
  float* part = (float*)wsp(ws, w.partial);
  if (dt == FPD_DTYPE_BF16) {
    // the bf16 projection reads the features [B, n_t, C, H] in place as
    // their concatenation [B * C, n_t * H]
    FPD_TRY_HIP(gemm_store_fused_f32(feats, B, c.n_fused, C, H, Wt{d->w.w_fc, d->t_fc}, H, Z, H, part,
                                     w.partial_bytes, s, "gemm_fc"));
  } else {
    const void* X = feats;
    if (c.n_fused > 1) {
      FPD_TRY_HIP(concat_features(dt, feats, B, c.n_fused, C, H, wsp(ws, w.x), s));
      X = wsp(ws, w.x);
    }
    FPD_TRY_HIP(gemm_store_f32(dt, X, c.n_fused * H, M, c.n_fused * H, Wt{d->w.w_fc, d->t_fc}, H, Z, H, part,
                               w.partial_bytes, s, "gemm_fc"));
  }
  void* Zn = wsp(ws, w.zn);
  FPD_TRY_HIP(rmsnorm_rows(dt, Z, H, M, M, 0, 0, d->w.g_fc, c.rms_eps, Zn, s));
  const size_t per_layer = (size_t)B * c.n_kv * ctx_cap * dh * d->esz;
  for (int li = 0; li < c.n_layers; ++li) {
    CtxOut o{};
    o.k = kbase + li * per_layer;
    o.vt = vbase + li * per_layer;
    o.C = C, o.cap = ctx_cap, o.nkv = c.n_kv, o.d = dh, o.pos0 = rope_pos0, o.rope = c.use_rope;
    o.tab = d->tab;
    const char* wkv = (const char*)d->layers[li].w_qkv + (size_t)c.n_q * dh * H * d->esz;
    // the K/V rows start at row n_q * d, a whole 32-row group of the tiled copy
    const void* tkv = d->tiled ? (const char*)d->t_qkv[li] + (size_t)c.n_q * dh * H * d->esz : nullptr;
    FPD_TRY_HIP(gemm_ctx_kv(dt, Zn, M, H, Wt{wkv, tkv}, o, part, w.partial_bytes, s));
  }
  return FPD_OK;
}

}  // namespace

extern "C" {

int32_t fpd_fuse_context_kv(const fpd_drafter* d, const void* feats, int32_t B, int32_t C, int32_t pos0,
                            void* ctx_k, void* ctx_v, int32_t ctx_cap, void* ws, size_t ws_bytes,
                            void* stream) {
  if (!d || !feats || !ctx_k || !ctx_v) return fail(FPD_E_ARG, "null argument");
  if (B < 1 || C < 1 || pos0 < 0) return fail(FPD_E_SHAPE, "need B >= 1, C >= 1, pos0 >= 0");
  if (too_many_rows(B, C)) return fail(FPD_E_SHAPE, "more than 2^24 rows");
  if (over_4gib((int64_t)B * C, fusion_row_bytes(d->cfg)))
    return fail(FPD_E_UNSUPPORTED, "bf16 features of 4 GiB or more (too many rows for one call)");
  if (ctx_cap < C || ctx_cap % 8) return fail(FPD_E_SHAPE, "ctx_cap must be >= C and a multiple of 8");
  return fuse_rows(d, feats, B, C, pos0, (char*)ctx_k, (char*)ctx_v, ctx_cap, ws, ws_bytes, stream);
}

int32_t fpd_append_context_kv(const fpd_drafter* d, const void* feats, int32_t B, int32_t C_new, int32_t pos0,
                              void* ctx_k, void* ctx_v, int32_t ctx_cap, void* ws, size_t ws_bytes,
                              void* stream) {
  if (!d || !feats || !ctx_k || !ctx_v) return fail(FPD_E_ARG, "null argument");
  if (B < 1 || C_new < 1 || pos0 < 0) return fail(FPD_E_SHAPE, "need B >= 1, C_new >= 1, pos0 >= 0");
  if (too_many_rows(B, C_new)) return fail(FPD_E_SHAPE, "more than 2^24 rows");
  if (over_4gib((int64_t)B * C_new, fusion_row_bytes(d->cfg)))
    return fail(FPD_E_UNSUPPORTED, "bf16 features of 4 GiB or more (too many rows for one call)");
  if (ctx_cap % 8 || (int64_t)pos0 + C_new > ctx_cap)
    return fail(FPD_E_SHAPE, "ctx_cap must be a multiple of 8 and hold pos0 + C_new keys");
  // key row pos0 of every (layer, b, kv head) segment: the K rows are d
  // elements long, the d-major V rows one element per key
  const size_t esz = d->esz, dh = d->cfg.head_dim;
  return fuse_rows(d, feats, B, C_new, pos0, (char*)ctx_k + (size_t)pos0 * dh * esz, (char*)ctx_v + (size_t)pos0 * esz,
                   ctx_cap, ws, ws_bytes, stream);
}

}  // extern "C"

namespace {

int32_t draft_impl(const fpd_drafter* d, const int32_t* tokens, int32_t B, int32_t L, const void* ctx_k,
                   const void* ctx_v, int32_t C, int32_t ctx_cap, int32_t block_pos, void* hidden_out, void* ws,
                   size_t ws_bytes, void* stream, bool shared_ctx) {
  if (!d || !tokens || !hidden_out) return fail(FPD_E_ARG, "null argument");
  if (B < 1 || L < 2 || C < 0 || block_pos < 0) return fail(FPD_E_SHAPE, "need B >= 1, L >= 2, C >= 0, block_pos >= 0");
  if (too_many_rows(B, L) || too_many_rows(B, C)) return fail(FPD_E_SHAPE, "more than 2^24 rows");
  if (over_4gib((int64_t)B * L, forward_row_bytes(d->cfg)))
    return fail(FPD_E_UNSUPPORTED, "a bf16 activation of 4 GiB or more (too many rows for one call)");
  if (C > 0 && (!ctx_k || !ctx_v)) return fail(FPD_E_ARG, "null context");
  if (C > 0 && (ctx_cap < C || ctx_cap % 8)) return fail(FPD_E_SHAPE, "ctx_cap must be >= C and a multiple of 8");
  const DraftWs w = plan_draft(*d, B, L, C);
  if (int32_t st = check_ws(ws, ws_bytes, w.total)) return st;
  const fpd_config& c = d->cfg;
  const int dt = c.dtype, H = c.hidden, M = B * L, dh = c.head_dim, qd = c.n_q * dh;
  hipStream_t s = (hipStream_t)stream;
  float* h = (float*)wsp(ws, w.h);
  void* a = wsp(ws, w.a);
  float* part = (float*)wsp(ws, w.partial);
  // h = E[tokens], a = RMSNorm(h) (the first layer's attention norm)
  FPD_TRY_HIP(embed_norm(dt, tokens, M, d->w.embed, H, c.vocab, h, d->layers[0].g_attn, c.rms_eps, a, s));
  const size_t ctx_layer = (size_t)(shared_ctx ? 1 : B) * c.n_kv * (size_t)ctx_cap * dh * d->esz;
  for (int li = 0; li < c.n_layers; ++li) {
    const fpd_layer_weights& lw = d->layers[li];
    QkvOut qo{};
    qo.q = wsp(ws, w.q), qo.k = wsp(ws, w.kb), qo.vt = wsp(ws, w.vbt);
    qo.L = L, qo.Lp = round8(L), qo.nq = c.n_q, qo.nkv = c.n_kv, qo.d = dh, qo.pos0 = block_pos;
    qo.rope = c.use_rope, qo.tab = d->tab;
    const bool tl = d->tiled != nullptr;
    FPD_TRY_HIP(gemm_qkv(dt, a, M, H, Wt{lw.w_qkv, tl ? d->t_qkv[li] : nullptr}, qo, part, w.partial_bytes, s));
    AttnArgs at{};
    at.q = qo.q, at.kb = qo.k, at.vbt = qo.vt;
    at.ck = C > 0 ? (const char*)ctx_k + li * ctx_layer : nullptr;
    at.cvt = C > 0 ? (const char*)ctx_v + li * ctx_layer : nullptr;
    at.o = wsp(ws, w.o);
    at.B = B, at.L = L, at.Lp = qo.Lp, at.C = C, at.cap = ctx_cap, at.nq = c.n_q, at.nkv = c.n_kv, at.d = dh;
    at.ctx_bstride = shared_ctx ? 0 : 1;
    at.scale = (float)(1.0 / std::sqrt((double)dh));
    FPD_TRY_HIP(attention(dt, at, wsp(ws, w.attn), w.attn_bytes, s));
    const bool last = li + 1 == c.n_layers;
    // The last layer's output is read only at positions 1..L-1 (the anchor
    // predicts nothing), so with one block its O projection and MLP run on
    // those L-1 rows alone: the residual rows from row 1 on, the normed MLP
    // input and SwiGLU output packed from row 0, the final norm written
    // straight to hidden_out.  (The anchor's K/V, computed above, is still
    // used by every query.)
    const bool trim = last && B == 1;
    const int Mr = trim ? L - 1 : M;
    const size_t r0 = trim ? 1 : 0;
    float* hr = h + r0 * H;
    // h += O W_o^T, a = RMSNorm(h) for the MLP
    FPD_TRY_HIP(gemm_residual_norm(dt, (const char*)at.o + r0 * qd * d->esz, Mr, qd,
                                   Wt{lw.w_o, tl ? d->t_o[li] : nullptr}, H, hr, lw.g_mlp, c.rms_eps, a, 0, part,
                                   w.partial_bytes, s, "gemm_o"));
    void* u = wsp(ws, w.u);
    FPD_TRY_HIP(gemm_swiglu(dt, a, Mr, H, Wt{lw.w_gu, tl ? d->t_gu[li] : nullptr}, c.inter, u, part, w.partial_bytes,
                            s));
    // h += u W_d^T, then the next layer's attention norm, or the final norm over positions 1..L-1
    FPD_TRY_HIP(gemm_residual_norm(dt, u, Mr, c.inter, Wt{lw.w_d, tl ? d->t_d[li] : nullptr}, H, hr,
                                   last ? d->w.g_final : d->layers[li + 1].g_attn, c.rms_eps,
                                   last ? hidden_out : a, last && !trim ? L : 0, part, w.partial_bytes, s,
                                   "gemm_down"));
  }
  return FPD_OK;
}

// ---- the allocation-free entry point's scratch -----------------------------------
// Device memory of fpd_draft_block_noalloc: one static array per GPU, held
// until the process ends.  Host code never uses the array's name as an
// address (in host code it is a stand-in): each device's address comes from
// hipGetSymbolAddress with that device current, once, and is kept here.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_dev[kMaxDevices] = {};

int32_t noalloc_scratch(void** out) {
  int dev = -1;
  FPD_TRY_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return fail(FPD_E_UNSUPPORTED, "device index beyond 64");
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_dev[dev]) {
    void* ptr = nullptr;
    FPD_TRY_HIP(hipGetSymbolAddress(&ptr, HIP_SYMBOL(g_noalloc_scratch)));
    if (!ptr) return fail(FPD_E_HIP, "hipGetSymbolAddress returned no address for the static scratch");
    g_scratch_dev[dev] = ptr;
  }
  *out = g_scratch_dev[dev];
  return FPD_OK;
}

}  // namespace

extern "C" {

int32_t fpd_draft_block(const fpd_drafter* d, const int32_t* tokens, int32_t B, int32_t L, const void* ctx_k,
                        const void* ctx_v, int32_t C, int32_t ctx_cap, int32_t block_pos, void* hidden_out,
                        void* ws, size_t ws_bytes, void* stream) {
  return draft_impl(d, tokens, B, L, ctx_k, ctx_v, C, ctx_cap, block_pos, hidden_out, ws, ws_bytes, stream, false);
}

int32_t fpd_draft_block_noalloc(const fpd_drafter* d, const int32_t* tokens, int32_t B, int32_t L, const void* ctx_k,
                                const void* ctx_v, int32_t C, int32_t ctx_cap, int32_t block_pos, void* hidden_out,
                                void* stream) {
  if (!d || !tokens || !hidden_out) return fail(FPD_E_ARG, "null argument");
  if (B < 1 || L < 2 || C < 0 || block_pos < 0) return fail(FPD_E_SHAPE, "need B >= 1, L >= 2, C >= 0, block_pos >= 0");
  if (too_many_rows(B, L) || too_many_rows(B, C)) return fail(FPD_E_SHAPE, "more than 2^24 rows");
  const size_t need = plan_draft(*d, B, L, C).total;
  if (need > kNoallocScratchBytes)
    return fail(FPD_E_WORKSPACE, "block needs " + std::to_string(need) + " bytes of scratch; the static scratch holds " +
                                     std::to_string(kNoallocScratchBytes));
  void* scratch_ptr = nullptr;
  if (int32_t st = noalloc_scratch(&scratch_ptr)) return st;
  NoTiming quiet;  // per-launch timing would create HIP events
  return draft_impl(d, tokens, B, L, ctx_k, ctx_v, C, ctx_cap, block_pos, hidden_out, scratch_ptr,
                    kNoallocScratchBytes, stream, false);
}

int32_t fpd_draft_blocks_shared_ctx(const fpd_drafter* d, const int32_t* tokens, int32_t B, int32_t L,
                                    const void* ctx_k, const void* ctx_v, int32_t C, int32_t ctx_cap,
                                    int32_t block_pos, void* hidden_out, void* ws, size_t ws_bytes, void* stream) {
  return draft_impl(d, tokens, B, L, ctx_k, ctx_v, C, ctx_cap, block_pos, hidden_out, ws, ws_bytes, stream, true);
}

int32_t fpd_constrained_argmax(const fpd_drafter* d, const fpd_layout* lay, const void* hidden, int32_t B,
                               int32_t* tokens_out, float* logits_out, void* ws, size_t ws_bytes,
                               void* stream) {
  if (!d || !lay || !hidden || !tokens_out) return fail(FPD_E_ARG, "null argument");
  if (lay->d != d) return fail(FPD_E_ARG, "layout was created for another drafter");
  if (B < 1) return fail(FPD_E_SHAPE, "need B >= 1");
  if (too_many_rows(B, lay->host.L)) return fail(FPD_E_SHAPE, "more than 2^24 rows");
  if (d->cfg.dtype == FPD_DTYPE_BF16 && over_4gib((int64_t)B * (lay->host.L - 1), (int64_t)d->cfg.hidden * 2))
    return fail(FPD_E_UNSUPPORTED, "bf16 hidden states of 4 GiB or more (too many rows for one call)");
  const HostLayout& h = lay->host;
  const fpd_config& c = d->cfg;
  const int L = h.L, ns = h.n_sets();
  // narrow column chunks when the wide ones would give fewer than 128 work
  // items (each then streams ~0.8 MB through one CU); such layouts have at
  // most 4 x 127 narrow chunks per row, within fpd_workspace_size's bound
  long wide_items = 0;
  for (int s2 = 0; s2 <= ns; ++s2) {
    const int npos = lay->set_pos_off[s2 + 1] - lay->set_pos_off[s2];
    const int ncols = s2 < ns ? h.set_offsets[s2 + 1] - h.set_offsets[s2] : c.vocab;
    const int wide = head_chunk_cols(c.dtype);
    wide_items += (long)((B * npos + 31) / 32) * ((ncols + wide - 1) / wide);
  }
  const int chunk = head_chunk_cols(c.dtype, wide_items < 128);
  HeadArgs ha{};
  ha.chunk_cols = chunk;
  ha.hidden = hidden;
  ha.B = B, ha.L = L, ha.H = c.hidden, ha.width = h.width(), ha.logits = logits_out;
  ReduceArgs ra{};
  ra.pos_set = lay->pos_set, ra.partner = lay->partner, ra.B = B, ra.L = L, ra.off_id = h.off_id;
  ra.n_sets = ns, ra.free_slot = ns;
  int max_chunks = 1;
  for (int s2 = 0; s2 <= ns; ++s2) {
    const int npos = lay->set_pos_off[s2 + 1] - lay->set_pos_off[s2];
    const int ncols = s2 < ns ? h.set_offsets[s2 + 1] - h.set_offsets[s2] : c.vocab;
    const int nch = (ncols + chunk - 1) / chunk;
    ra.set_chunks[s2] = nch;
    ra.set_offcol[s2] = s2 < ns ? lay->off_col[s2] : -1;
    ra.set_ids[s2] = s2 < ns ? lay->set_ids + h.set_offsets[s2] : nullptr;
    if (npos == 0) continue;
    HeadSet& hs = ha.sets[ha.n_sets++];
    hs.w = s2 < ns ? (const void*)((const char*)lay->wg + (size_t)h.set_offsets[s2] * c.hidden * d->esz)
                   : d->w.w_lm;
    hs.ids = ra.set_ids[s2];
    hs.pos = lay->set_pos + lay->set_pos_off[s2];
    hs.n_pos = npos, hs.n_cols = ncols, hs.off_col = ra.set_offcol[s2], hs.n_chunks = nch, hs.part_base = 0;
    max_chunks = std::max(max_chunks, nch);
  }
  const HeadWs w = plan_head(B, L, max_chunks);
  if (int32_t st = check_ws(ws, ws_bytes, w.total)) return st;
  ha.max_chunks = ra.max_chunks = max_chunks;
  ha.pval = (float*)wsp(ws, w.pval), ha.pcol = (int32_t*)wsp(ws, w.pcol), ha.offv = (float*)wsp(ws, w.offv);
  ra.pval = ha.pval, ra.pcol = ha.pcol, ra.offv = ha.offv, ra.tokens = tokens_out;
  hipStream_t s = (hipStream_t)stream;
  FPD_TRY_HIP(lm_head_partials(c.dtype, ha, s));
  if (logits_out) FPD_TRY_HIP(fill_logits_padding(logits_out, B * (L - 1), ha.width, L - 1, lay->row_cols, s));
  FPD_TRY_HIP(lm_head_reduce(ra, s));
  return FPD_OK;
}

namespace {
ValidateArgs validate_args(const fpd_layout* lay, const int32_t* tokens, int32_t B, int32_t* k_out,
                           int32_t* first_invalid_out) {
  const HostLayout& h = lay->host;
  ValidateArgs a{};
  a.tokens = tokens, a.pos_set = lay->pos_set, a.set_offsets = lay->set_offsets, a.set_ids = lay->set_ids;
  a.n_set_ids = (int)h.set_ids.size();
  a.partner = lay->partner, a.field_w = lay->field_w;
  a.B = B, a.L = h.L, a.vocab = h.vocab, a.off_id = h.off_id, a.fill_id = h.fill_id, a.digit0_id = h.digit0_id;
  a.k_out = k_out, a.first_out = first_invalid_out;
  return a;
}
}  // namespace

int32_t fpd_validate_primitive(const fpd_layout* lay, const int32_t* tokens, int32_t B, int32_t* k_out,
                               int32_t* first_invalid_out, void* stream) {
  if (!lay || !tokens || !k_out || !first_invalid_out) return fail(FPD_E_ARG, "null argument");
  if (B < 1) return fail(FPD_E_SHAPE, "need B >= 1");
  if (too_many_rows(B, lay->host.L)) return fail(FPD_E_SHAPE, "more than 2^24 rows");
  FPD_TRY_HIP(validate_primitive(validate_args(lay, tokens, B, k_out, first_invalid_out), (hipStream_t)stream));
  return FPD_OK;
}

int32_t fpd_accept_boxes(const fpd_layout* lay, const int32_t* tokens, const float* conf, float tau, int32_t B,
                         int32_t* k_out, int32_t* first_invalid_out, int32_t* first_uncertain_out, void* stream) {
  if (!lay || !tokens || !conf || !k_out || !first_invalid_out || !first_uncertain_out)
    return fail(FPD_E_ARG, "null argument");
  if (std::isnan(tau)) return fail(FPD_E_ARG, "tau is NaN");
  if (B < 1) return fail(FPD_E_SHAPE, "need B >= 1");
  if (too_many_rows(B, lay->host.L)) return fail(FPD_E_SHAPE, "more than 2^24 rows");
  ValidateArgs a = validate_args(lay, tokens, B, k_out, first_invalid_out);
  a.conf = conf, a.coord = lay->coord, a.tau = tau, a.uncertain_out = first_uncertain_out;
  FPD_TRY_HIP(validate_primitive(a, (hipStream_t)stream));
  return FPD_OK;
}

int32_t fpd_verify_prefix(const int32_t* draft, const int32_t* target, int32_t B, int32_t L, int32_t* k_out,
                          int32_t* next_out, void* stream) {
  if (!draft || !target || !k_out || !next_out) return fail(FPD_E_ARG, "null argument");
  if (B < 1 || L < 2) return fail(FPD_E_SHAPE, "need B >= 1 and L >= 2");
  if (too_many_rows(B, L)) return fail(FPD_E_SHAPE, "more than 2^24 rows");
  FPD_TRY_HIP(verify_prefix(draft, target, B, L, k_out, next_out, (hipStream_t)stream));
  return FPD_OK;
}

int32_t fpd_coords_to_tokens(const float* values, int32_t n, double lo, double hi, int32_t coord_base,
                             int32_t* tokens_out, void* stream) {
  if (n < 0) return fail(FPD_E_SHAPE, "need n >= 0");
  if (n > 0 && (!values || !tokens_out)) return fail(FPD_E_ARG, "null argument");
  if (!(hi > lo) || !std::isfinite(lo) || !std::isfinite(hi)) return fail(FPD_E_ARG, "need finite lo < hi");
  FPD_TRY_HIP(coords_to_tokens(values, n, lo, hi, coord_base, tokens_out, (hipStream_t)stream));
  return FPD_OK;
}

int32_t fpd_tokens_to_coords(const int32_t* tokens, int32_t n, double lo, double hi, int32_t coord_base,
                             double* values_out, void* stream) {
  if (n < 0) return fail(FPD_E_SHAPE, "need n >= 0");
  if (n > 0 && (!tokens || !values_out)) return fail(FPD_E_ARG, "null argument");
  if (!(hi > lo) || !std::isfinite(lo) || !std::isfinite(hi)) return fail(FPD_E_ARG, "need finite lo < hi");
  FPD_TRY_HIP(tokens_to_coords(tokens, n, lo, hi, coord_base, values_out, (hipStream_t)stream));
  return FPD_OK;
}

int32_t fpd_ints_to_fields(const int32_t* values, int32_t n, int32_t plus_id, int32_t minus_id, int32_t digit0_id,
                           int32_t fill_id, int32_t* fields_out, void* stream) {
  if (n < 0) return fail(FPD_E_SHAPE, "need n >= 0");
  if (n > 0 && (!values || !fields_out)) return fail(FPD_E_ARG, "null argument");
  FPD_TRY_HIP(ints_to_fields(values, n, plus_id, minus_id, digit0_id, fill_id, fields_out, (hipStream_t)stream));
  return FPD_OK;
}

int32_t fpd_fields_to_ints(const int32_t* fields, int32_t n, int32_t plus_id, int32_t minus_id, int32_t digit0_id,
                           int32_t fill_id, int32_t* values_out, int32_t* valid_out, void* stream) {
  if (n < 0) return fail(FPD_E_SHAPE, "need n >= 0");
  if (n > 0 && (!fields || !values_out || !valid_out)) return fail(FPD_E_ARG, "null argument");
  FPD_TRY_HIP(fields_to_ints(fields, n, plus_id, minus_id, digit0_id, fill_id, values_out, valid_out,
                             (hipStream_t)stream));
  return FPD_OK;
}

}  // extern "C"
