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

namespace fpd {
namespace {

constexpr int BK = 64;
constexpr int LDSW = BK + 8;
constexpr int HBM = 32;    // rows per tile (bf16)
constexpr int HBN = 128;   // columns per chunk (bf16): 4 waves x 32
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

__global__ __launch_bounds__(256) void head_bf16_kernel(HeadArgs a) {
  __shared__ __attribute__((aligned(16))) bf16_t As[2][HBM * LDSW];
  __shared__ __attribute__((aligned(16))) bf16_t Bs[2][HBN * LDSW];
  __shared__ float red_v[4][HBM];
  __shared__ int red_c[4][HBM];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lq = lane & 31, lg = lane >> 5;
  const Item it = find_item(a, xcd_remap(blockIdx.x, gridDim.x), HBM);
  if (it.set < 0) return;
  const HeadSet& S = a.sets[it.set];
  const int M = a.B * S.n_pos, H = a.H;
  const int m0 = it.mt * HBM, c0 = it.chunk * HBN;
  const bf16_t* hid = (const bf16_t*)a.hidden;
  const bf16_t* W = (const bf16_t*)S.w;

  // one A chunk and four B chunks (16 bytes each) per thread and K-tile
  const int arow = tid >> 3, akc = (tid & 7) * 8;
  const bf16_t* aptr = (m0 + arow < M) ? hid + (size_t)set_row(a, S, m0 + arow) * H : nullptr;
  const bf16_t* bptr[4];
  int blds[4], bkc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = tid + i * 256, row = c >> 3;
    bkc[i] = (c & 7) * 8;
    blds[i] = row * LDSW + bkc[i];
    bptr[i] = (c0 + row < S.n_cols) ? W + (size_t)(c0 + row) * H : nullptr;
  }
  u32x4_t ra, rb[4];
  auto gload = [&](int kt) {
    const int k0 = kt * BK;
    ra = aptr ? *(const u32x4_t*)(aptr + k0 + akc) : u32x4_t{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 4; ++i)
      rb[i] = bptr[i] ? __builtin_nontemporal_load((const u32x4_t*)(bptr[i] + k0 + bkc[i]))
                      : u32x4_t{0, 0, 0, 0};
  };
  auto sstore = [&](int buf) {
    *(u32x4_t*)&As[buf][arow * LDSW + akc] = ra;
#pragma unroll
    for (int i = 0; i < 4; ++i) *(u32x4_t*)&Bs[buf][blds[i]] = rb[i];
  };
  f32x16_t acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  const int KT = H / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < KT) gload(kt + 1);
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      const bf16x8_t af = *(const bf16x8_t*)&As[cur][lq * LDSW + kk * 16 + lg * 8];
      const bf16x8_t bfv = *(const bf16x8_t*)&Bs[cur][(wave * 32 + lq) * LDSW + kk * 16 + lg * 8];
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bfv, acc, 0, 0, 0);
    }
    if (kt + 1 < KT) sstore(cur ^ 1);
    __syncthreads();
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
      const int grow = set_row(a, S, m);
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
    for (int w = 1; w < 4; ++w)
      if (arg_better(red_v[w][tid], red_c[w][tid], bv, bc)) {
        bv = red_v[w][tid];
        bc = red_c[w][tid];
      }
    const int m = m0 + tid;
    if (m < M) {
      const size_t slot = (size_t)set_row(a, S, m) * a.max_chunks + S.part_base + it.chunk;
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

__device__ __forceinline__ void best_of_row(const ReduceArgs& a, int row, int slot, float& v, int& c) {
  v = -INFINITY;
  c = INT_MAX;
  const int nc = a.set_chunks[slot];
  for (int k = 0; k < nc; ++k) {
    const float v2 = a.pval[(size_t)row * a.max_chunks + k];
    const int c2 = a.pcol[(size_t)row * a.max_chunks + k];
    if (arg_better(v2, c2, v, c)) {
      v = v2;
      c = c2;
    }
  }
}

__device__ __forceinline__ int col_id(const ReduceArgs& a, int slot, int c) {
  if (c == INT_MAX) return -1;  // no candidate column (cannot happen for a non-empty set)
  return a.set_ids[slot] ? a.set_ids[slot][c] : c;
}

__global__ __launch_bounds__(256) void head_reduce_kernel(ReduceArgs a) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  const int P = a.L - 1;
  if (idx >= a.B * P) return;
  const int b = idx / P, p = idx % P + 1;
  const int partner = a.partner[p];
  if (partner == -2) return;  // second position of a pair: decided with its first
  const int ps = a.pos_set[p];
  const int slot = ps >= 0 ? ps : a.free_slot;
  float v;
  int c;
  best_of_row(a, idx, slot, v, c);
  const int offc = a.set_offcol[slot];
  if (partner >= 0) {
    const int q = partner, qrow = b * P + q - 1;
    const int qs = a.pos_set[q];
    const int qslot = qs >= 0 ? qs : a.free_slot;
    float vq;
    int cq;
    best_of_row(a, qrow, qslot, vq, cq);
    const float on = v + vq;
    const float off = a.offv[idx] + a.offv[qrow];
    if (off > on) {
      a.tokens[idx] = a.off_id;
      a.tokens[qrow] = a.off_id;
    } else {
      a.tokens[idx] = col_id(a, slot, c);
      a.tokens[qrow] = col_id(a, qslot, cq);
    }
    return;
  }
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

int head_chunk_cols(int dt) { return dt == FPD_DTYPE_BF16 ? HBN : FBN; }

hipError_t lm_head_partials(int dt, const HeadArgs& a, hipStream_t st) {
  ProfScope prof("lm_head", st);
  const int bm = dt == FPD_DTYPE_BF16 ? HBM : FBM;
  long items = 0;
  for (int s = 0; s < a.n_sets; ++s)
    items += (long)((a.B * a.sets[s].n_pos + bm - 1) / bm) * a.sets[s].n_chunks;
  if (items == 0) return hipSuccess;
  if (dt == FPD_DTYPE_BF16)
    hipLaunchKernelGGL(head_bf16_kernel, dim3((unsigned)items), dim3(256), 0, st, a);
  else
    hipLaunchKernelGGL(head_f32_kernel, dim3((unsigned)items), dim3(256), 0, st, a);
  return hipGetLastError();
}

hipError_t lm_head_reduce(const ReduceArgs& a, hipStream_t st) {
  ProfScope prof("lm_head_reduce", st);
  const int n = a.B * (a.L - 1);
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(head_reduce_kernel, dim3((n + 255) / 256), dim3(256), 0, st, a);
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
