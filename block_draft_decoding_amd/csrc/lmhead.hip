// Constrained LM head (VFlash paper §2.5): logits are computed only for each
// position's legal vocabulary (the legal W_lm rows of a set are gathered once
// per layout into a contiguous buffer; free text positions stream all of
// W_lm), and the masked argmax is fused into the GEMM epilogue as per-chunk
// (value, column) partials.  The column of the OFF id is kept aside so the
// cross-position off-frame rule can compare the pair's joint scores.
//
// Work items are (set, column chunk, row tile) with the row tile fastest, so
// the workgroups that stream the same weight chunk run together on one XCD.
#include <climits>

#include "../../include/fpd.h"
#include "kernels.h"
#include "lds_pipe.h"

namespace fpd {
namespace {

constexpr int BK = 64;
constexpr int HBM = 32;    // rows per tile (bf16)
constexpr int HBN = 128;   // columns per chunk (bf16): 4 waves x 32
constexpr int HBN_NARROW = 32;  // one wave per K group: for layouts whose 128-column chunks give few items
// depth of the global -> LDS ring (bf16): 3 for the wide chunks, so that two
// workgroups fit in a CU's 160 KB of LDS (4 stages come to just over 80 KB
// with the reduction arrays: 183 -> 148 us for a full-vocabulary text block,
// measured); 4 for the narrow ones (32 KB per K group; four K groups come
// to 140 KB, one workgroup per CU)
constexpr int HST_WIDE = 3;
constexpr int HST_NARROW = 4;
constexpr int kCUs = 256;
// K groups of a narrow-chunk item: the most (4, 2 or 1) that divide the K
// tiles and still run every item in one pass of workgroups (LDS holds one
// four-group workgroup per CU, two two-group ones)
int head_k_groups(int items, int H) {
  if (items <= kCUs && H % (BK * 4) == 0) return 4;
  if (items <= 2 * kCUs && H % (BK * 2) == 0) return 2;
  return 1;
}
constexpr int FBM = 16;    // f32 path: rows per tile
constexpr int FBN = 64;    // f32 path: columns per chunk

struct Item {
  int set, chunk, mt;
};

__device__ __forceinline__ Item find_item(const HeadArgs& a, int tile, int bm) {
  for (int s = 0; s < a.n_sets; ++s) {
    const int mts = (a.B * a.sets[s].n_pos + bm - 1) / bm;
    const int cnt = mts * a.sets[s].n_chunks;
    if (tile < cnt) return Item{s, tile / mts, tile % mts};
    tile -= cnt;
  }
  return Item{-1, 0, 0};
}

// hidden row (and output row) of the m-th row of a set: b * (L-1) + p - 1
__device__ __forceinline__ int set_row(const HeadArgs& a, const HeadSet& s, int m) {
  const int b = m / s.n_pos, i = m - b * s.n_pos;
  return b * (a.L - 1) + s.pos[i] - 1;
}

__device__ __forceinline__ void wave_argmax(float& v, int& c, int width) {
  for (int o = 1; o < width; o <<= 1) {
    const float v2 = __shfl_xor(v, o);
    const int c2 = __shfl_xor(c, o);
    if (arg_better(v2, c2, v, c)) {
      v = v2;
      c = c2;
    }
  }
}

// bf16 path: the hidden rows of the set's positions and the set's gathered
// W_lm rows stream global -> LDS through an HST-deep ring of LDS-writing
// buffer loads (K-tile offsets are scalar; each lane's row offset is fixed),
// so several K-tiles are in flight while the MFMAs run.  16-byte chunks are
// bank-swizzled as in the dense GEMM.  One wave per 32 columns of the chunk;
// with KW > 1, KW such groups of waves each take 1/KW of the K range through
// a ring of their own, and their partial tiles are summed in LDS in group
// order before the epilogue (a chunk's single wave would otherwise stream
// the item's whole 330 KB alone).
template <int CN, int HST, int KW>
__global__ __launch_bounds__(2 * CN * KW) void head_bf16_kernel(HeadArgs a) {
  constexpr int HW = CN / 32;                      // column waves of a K group
  constexpr int NT = 64 * HW;                      // threads of a K group
  constexpr int CH = BK / 8;                       // 16-byte chunks per tile row
  constexpr int STAGE = (HBM + CN) * CH;           // chunks per stage
  constexpr int AI = HBM * CH / NT;                // A loads per thread and stage
  constexpr int BI = CN * CH / NT;                 // B loads per thread and stage
  constexpr int LPS = AI + BI;
  static_assert(AI * NT == HBM * CH && BI * NT == CN * CH, "tile shape");
  static_assert(LPS * (HST - 1) < 64, "pipeline depth");
  __shared__ u32x4_t lds[KW * HST * STAGE];
  __shared__ float red_v[HW][HBM];
  __shared__ int red_c[HW][HBM];
  __shared__ int rowmap[HBM];  // hidden / output row of each tile row (rows past the set repeat a valid one)
  const int tid = threadIdx.x, lane = tid & 63;
  const int gwave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kw = gwave / HW, wave = gwave % HW;    // K group, column wave within it
  const int lq = lane & 31, lg = lane >> 5;
  const Item it = find_item(a, xcd_remap(blockIdx.x, gridDim.x), HBM);
  if (it.set < 0) return;
  const HeadSet& S = a.sets[it.set];
  const int M = a.B * S.n_pos, H = a.H;
  const int m0 = it.mt * HBM, c0 = it.chunk * CN;

  const __amdgpu_buffer_rsrc_t arsrc = __builtin_amdgcn_make_buffer_rsrc(
      (void*)a.hidden, (short)0, (int)((size_t)a.B * (a.L - 1) * H * 2), 0x00020000);
  const __amdgpu_buffer_rsrc_t brsrc =
      __builtin_amdgcn_make_buffer_rsrc((void*)S.w, (short)0, (int)((size_t)S.n_cols * H * 2), 0x00020000);
  if (tid < HBM) rowmap[tid] = set_row(a, S, min(m0 + tid, M - 1));
  uint32_t aoff[AI], boff[BI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int sl = (wave * AI + i) * 64 + lane, r = sl / CH, c = (sl % CH) ^ ((r / (16 / CH)) & (CH - 1));
    const int row = set_row(a, S, min(m0 + r, M - 1));
    aoff[i] = (uint32_t)(((size_t)row * H + c * 8) * 2);
  }
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    const int sl = (wave * BI + i) * 64 + lane, r = sl / CH, c = (sl % CH) ^ ((r / (16 / CH)) & (CH - 1));
    const int col = min(c0 + r, S.n_cols - 1);
    boff[i] = (uint32_t)(((size_t)col * H + c * 8) * 2);
  }
  u32x4_t* ring = lds + kw * HST * STAGE;
  // A set whose rows fit one row group reads each weight chunk once per call,
  // and weight rows larger than the 256 MB last-level cache cannot stay there
  // between calls either: such sets (the full vocabulary) load it non-temporal
  // (text block 0.564 -> 0.537 ms, FlashDrive 16-token block 0.316 -> 0.291
  // ms).  Sets of several row groups share each chunk through L2, and small
  // gathered sets stay cached from one call to the next (the hint cost the
  // 64-box block 0.4%): they keep the default policy.
  const bool w_once = M <= HBM && (size_t)S.n_cols * H * 2 > ((size_t)256 << 20);
  auto issue = [&](int kt, int stage) {
    const int soff = kt * BK * 2;
    u32x4_t* base = ring + stage * STAGE;
#pragma unroll
    for (int i = 0; i < AI; ++i) lds_dma16(arsrc, base + (wave * AI + i) * 64, aoff[i], soff);
    if (w_once) {
#pragma unroll
      for (int i = 0; i < BI; ++i)
        lds_dma16<kLoadNonTemporal>(brsrc, base + HBM * CH + (wave * BI + i) * 64, boff[i], soff);
    } else {
#pragma unroll
      for (int i = 0; i < BI; ++i) lds_dma16(brsrc, base + HBM * CH + (wave * BI + i) * 64, boff[i], soff);
    }
  };

  f32x16_t acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  const int KT = H / BK / KW, kt0 = kw * KT;       // this group's K tiles (KW divides H / BK)
#pragma unroll
  for (int s = 0; s < HST; ++s)
    if (s < KT) issue(kt0 + s, s);
  bf16x8_t af[2], bfv[2];
  auto fetch = [&](int stage, int kk, int buf) {
    const u32x4_t* As = ring + stage * STAGE;
    af[buf] = __builtin_bit_cast(bf16x8_t, As[swz<CH>(lq, kk * 2 + lg)]);
    bfv[buf] = __builtin_bit_cast(bf16x8_t, As[HBM * CH + swz<CH>(wave * 32 + lq, kk * 2 + lg)]);
  };
  wait_lgkm0();
  wait_stages<LPS, HST - 1>(min(HST - 1, KT - 1));
  barrier_nofence();
  fetch(0, 0, 0);
  for (int kt = 0; kt < KT; ++kt) {
    const int stage = kt % HST;
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      if (kk + 1 < BK / 16) {
        fetch(stage, kk + 1, (kk + 1) & 1);
      } else {
        wait_lgkm0();
        if (kt + 1 < KT) wait_stages<LPS, HST - 2>(min(HST - 2, KT - 2 - kt));
        barrier_nofence();
        if (kt + HST < KT) issue(kt0 + kt + HST, stage);
        if (kt + 1 < KT) fetch((kt + 1) % HST, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[kk & 1], bfv[kk & 1], acc, 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }

  if constexpr (KW > 1) {  // sum the groups' partial tiles in group order
    __shared__ f32x16_t kpart[KW - 1][HW][64];
    if (kw > 0) kpart[kw - 1][wave][lane] = acc;
    __syncthreads();
    if (kw > 0) {
      __syncthreads();  // the epilogue's barrier below
      return;
    }
#pragma unroll
    for (int g2 = 0; g2 < KW - 1; ++g2) acc += kpart[g2][wave][lane];
  }
  // epilogue: this lane holds column n of rows rr(r)
  const int n = c0 + wave * 32 + lq;
  const bool ncol = n < S.n_cols;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int rr = (r >> 2) * 8 + lg * 4 + (r & 3);
    const int m = m0 + rr;
    const float v = acc[r];
    if (m < M && ncol) {
      const int grow = rowmap[rr];
      if (a.logits) a.logits[(size_t)grow * a.width + n] = v;
      if (n == S.off_col) a.offv[grow] = v;
    }
    float bv = -INFINITY;
    int bc = INT_MAX;
    if (ncol && n != S.off_col) {
      bv = v;
      bc = n;
    }
    wave_argmax(bv, bc, 32);
    if (lq == 0) {
      red_v[wave][rr] = bv;
      red_c[wave][rr] = bc;
    }
  }
  __syncthreads();
  if (tid < HBM) {
    float bv = red_v[0][tid];
    int bc = red_c[0][tid];
    for (int w = 1; w < HW; ++w)
      if (arg_better(red_v[w][tid], red_c[w][tid], bv, bc)) {
        bv = red_v[w][tid];
        bc = red_c[w][tid];
      }
    const int m = m0 + tid;
    if (m < M) {
      const size_t slot = (size_t)rowmap[tid] * a.max_chunks + S.part_base + it.chunk;
      a.pval[slot] = bv;
      a.pcol[slot] = bc;
    }
  }
}

// f32 path: 16 rows x 64 columns per workgroup; thread = (row, 4 columns).
__global__ __launch_bounds__(256) void head_f32_kernel(HeadArgs a) {
  __shared__ float As[FBM][33];
  __shared__ float Bs[FBN][33];
  const int tid = threadIdx.x;
  const Item it = find_item(a, blockIdx.x, FBM);
  if (it.set < 0) return;
  const HeadSet& S = a.sets[it.set];
  const int M = a.B * S.n_pos, H = a.H;
  const int m0 = it.mt * FBM, c0 = it.chunk * FBN;
  const float* hid = (const float*)a.hidden;
  const float* W = (const float*)S.w;
  const int row = tid >> 4, cq = (tid & 15) * 4;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < H; k0 += 32) {
    for (int e = tid; e < FBM * 32; e += 256) {
      const int r = e >> 5, kk = e & 31, m = m0 + r;
      As[r][kk] = m < M ? hid[(size_t)set_row(a, S, m) * H + k0 + kk] : 0.f;
    }
    for (int e = tid; e < FBN * 32; e += 256) {
      const int r = e >> 5, kk = e & 31, n = c0 + r;
      Bs[r][kk] = n < S.n_cols ? W[(size_t)n * H + k0 + kk] : 0.f;
    }
    __syncthreads();
#pragma unroll 8
    for (int kk = 0; kk < 32; ++kk) {
      const float x = As[row][kk];
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] += x * Bs[cq + j][kk];
    }
    __syncthreads();
  }
  const int m = m0 + row;
  float bv = -INFINITY;
  int bc = INT_MAX;
  const int grow = m < M ? set_row(a, S, m) : 0;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int n = c0 + cq + j;
    if (m < M && n < S.n_cols) {
      if (a.logits) a.logits[(size_t)grow * a.width + n] = acc[j];
      if (n == S.off_col)
        a.offv[grow] = acc[j];
      else if (arg_better(acc[j], n, bv, bc)) {
        bv = acc[j];
        bc = n;
      }
    }
  }
  wave_argmax(bv, bc, 16);  // the 16 threads of a row are consecutive lanes
  if ((tid & 15) == 0 && m < M) {
    const size_t slot = (size_t)grow * a.max_chunks + S.part_base + it.chunk;
    a.pval[slot] = bv;
    a.pcol[slot] = bc;
  }
}

// Best (value, column) of a row's chunk partials, one workgroup of RT
// threads per row: threads take every RT-th chunk, four loads in flight each,
// a butterfly reduces each wavefront and, with several wavefronts, their
// results meet in LDS.  Every thread returns the row's best; arg_better is a
// total order, so the result is the same for any split of the chunks.  Rows
// of a free text position have ~1,200 chunks and take 256 threads (text block
// reduce 12.7 -> 7.2 us); the constrained sets' few dozen take one wavefront.
template <int RT>
__device__ __forceinline__ void best_of_row(const ReduceArgs& a, int row, int slot, float& v, int& c) {
  __shared__ float sv[RT / 64];
  __shared__ int sc[RT / 64];
  const int tid = threadIdx.x, lane = tid & 63;
  v = -INFINITY;
  c = INT_MAX;
  const int nc = a.set_chunks[slot];
  const float* pv = a.pval + (size_t)row * a.max_chunks;
  const int32_t* pc = a.pcol + (size_t)row * a.max_chunks;
  for (int k0 = tid; k0 < nc; k0 += 4 * RT) {
    float v2[4];
    int c2[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int k = k0 + u * RT;
      v2[u] = k < nc ? pv[k] : -INFINITY;
      c2[u] = k < nc ? pc[k] : INT_MAX;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (arg_better(v2[u], c2[u], v, c)) {
        v = v2[u];
        c = c2[u];
      }
  }
  wave_argmax(v, c, 64);
  if constexpr (RT > 64) {
    if (lane == 0) {
      sv[tid >> 6] = v;
      sc[tid >> 6] = c;
    }
    __syncthreads();
    v = sv[0];
    c = sc[0];
#pragma unroll
    for (int w = 1; w < RT / 64; ++w)
      if (arg_better(sv[w], sc[w], v, c)) {
        v = sv[w];
        c = sc[w];
      }
    __syncthreads();  // a second call (the pair's partner row) reuses sv / sc
  }
}

__device__ __forceinline__ int col_id(const ReduceArgs& a, int slot, int c) {
  if (c == INT_MAX) return -1;  // no candidate column (cannot happen for a non-empty set)
  return a.set_ids[slot] ? a.set_ids[slot][c] : c;
}

// One workgroup per (request, position); thread 0 writes the decision.
template <int RT>
__global__ __launch_bounds__(RT) void head_reduce_kernel(ReduceArgs a) {
  const int idx = blockIdx.x;
  const int P = a.L - 1;
  if (idx >= a.B * P) return;
  const bool lead = threadIdx.x == 0;
  const int b = idx / P, p = idx % P + 1;
  const int partner = a.partner[p];
  if (partner == -2) return;  // second position of a pair: decided with its first
  const int ps = a.pos_set[p];
  const int slot = ps >= 0 ? ps : a.free_slot;
  float v;
  int c;
  best_of_row<RT>(a, idx, slot, v, c);
  const int offc = a.set_offcol[slot];
  if (partner >= 0) {
    const int q = partner, qrow = b * P + q - 1;
    const int qs = a.pos_set[q];
    const int qslot = qs >= 0 ? qs : a.free_slot;
    float vq;
    int cq;
    best_of_row<RT>(a, qrow, qslot, vq, cq);
    const float on = v + vq;
    const float off = a.offv[idx] + a.offv[qrow];
    if (!lead) return;
    if (off > on) {
      a.tokens[idx] = a.off_id;
      a.tokens[qrow] = a.off_id;
    } else {
      a.tokens[idx] = col_id(a, slot, c);
      a.tokens[qrow] = col_id(a, qslot, cq);
    }
    return;
  }
  if (!lead) return;
  int id = col_id(a, slot, c);
  if (offc >= 0) {
    const float vo = a.offv[idx];
    if (id < 0 || arg_better(vo, a.off_id, v, id)) id = a.off_id;
  }
  a.tokens[idx] = id;
}

__global__ __launch_bounds__(256) void pad_kernel(float* logits, int rows, int width, int P,
                                                  const int32_t* row_cols) {
  const int r = blockIdx.x;
  if (r >= rows) return;
  const int n0 = row_cols[r % P + 1];
  for (int c = n0 + threadIdx.x; c < width; c += blockDim.x) logits[(size_t)r * width + c] = -INFINITY;
}

}  // namespace

int head_chunk_cols(int dt, bool narrow) {
  if (dt != FPD_DTYPE_BF16) return FBN;
  return narrow ? HBN_NARROW : HBN;
}

hipError_t lm_head_partials(int dt, const HeadArgs& a, hipStream_t st) {
  ProfScope prof("lm_head", st);
  const int bm = dt == FPD_DTYPE_BF16 ? HBM : FBM;
  long items = 0;
  for (int s = 0; s < a.n_sets; ++s)
    items += (long)((a.B * a.sets[s].n_pos + bm - 1) / bm) * a.sets[s].n_chunks;
  if (items == 0) return hipSuccess;
  // buffer descriptors address at most 4 GiB per operand
  if ((size_t)a.B * (a.L - 1) * a.H * 2 > 0xffffffffull) return hipErrorInvalidValue;
  for (int s = 0; s < a.n_sets; ++s)
    if ((size_t)a.sets[s].n_cols * a.H * 2 > 0xffffffffull) return hipErrorInvalidValue;
  if (dt == FPD_DTYPE_BF16 && a.chunk_cols == HBN_NARROW) {
    // split K within the item while the items, so multiplied, still fit in
    // one workgroup per CU (a second pass of workgroups costs more)
    const int kw = head_k_groups(items, a.H);
    if (kw == 4)
      hipLaunchKernelGGL((head_bf16_kernel<HBN_NARROW, HST_NARROW, 4>), dim3((unsigned)items), dim3(2 * HBN_NARROW * 4),
                         0, st, a);
    else if (kw == 2)
      hipLaunchKernelGGL((head_bf16_kernel<HBN_NARROW, HST_NARROW, 2>), dim3((unsigned)items), dim3(2 * HBN_NARROW * 2),
                         0, st, a);
    else
      hipLaunchKernelGGL((head_bf16_kernel<HBN_NARROW, HST_NARROW, 1>), dim3((unsigned)items), dim3(2 * HBN_NARROW), 0,
                         st, a);
  } else if (dt == FPD_DTYPE_BF16 && a.chunk_cols == HBN)
    hipLaunchKernelGGL((head_bf16_kernel<HBN, HST_WIDE, 1>), dim3((unsigned)items), dim3(2 * HBN), 0, st, a);
  else if (dt == FPD_DTYPE_BF16)
    return hipErrorInvalidValue;
  else
    hipLaunchKernelGGL(head_f32_kernel, dim3((unsigned)items), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t lm_head_reduce(const ReduceArgs& a, hipStream_t st) {
  ProfScope prof("lm_head_reduce", st);
  const int n = a.B * (a.L - 1);
  if (n == 0) return hipSuccess;
  if (a.max_chunks > 64)
    hipLaunchKernelGGL(head_reduce_kernel<256>, dim3(n), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(head_reduce_kernel<64>, dim3(n), dim3(64), 0, st, a);
  return hipGetLastError();
}

hipError_t fill_logits_padding(float* logits, int rows, int width, int P, const int32_t* row_cols,
                               hipStream_t st) {
  ProfScope prof("logits_padding", st);
  if (rows == 0) return hipSuccess;
  hipLaunchKernelGGL(pad_kernel, dim3(rows), dim3(256), 0, st, logits, rows, width, P, row_cols);
  return hipGetLastError();
}

}  // namespace fpd
