// Shared device-side definitions for the gfx950 kernels of libfpd.
#pragma once
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>

namespace fpd {

typedef uint16_t bf16_t;  // raw IEEE bfloat16 bits
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kXcds = 8;  // MI355X: 8 accelerator complex dies, round-robin workgroup dispatch

__device__ __forceinline__ float bf2f(bf16_t x) { return __uint_as_float((uint32_t)x << 16); }

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// float -> bfloat16, round to nearest even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16_t f2bf(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Attention values of bf16 drafters: the value is rounded to bfloat16 (its
// storage precision) and kept as the IEEE half with the same value, so the
// P V product can take fp16 probabilities (11 significant bits instead of
// 8) at the bf16 MFMA rate.  Exact for |v| in [2^-17, 65504]; smaller
// magnitudes keep fp16's subnormal spacing 2^-24, larger ones overflow.
__device__ __forceinline__ uint16_t bf16_value_as_f16(float v) {
  return __builtin_bit_cast(uint16_t, (_Float16)bf2f(f2bf(v)));
}

// Element load/store in the storage type, arithmetic in float.
template <class T>
struct Elem;
template <>
struct Elem<float> {
  static __device__ __forceinline__ float ld(const float* p) { return *p; }
  static __device__ __forceinline__ void st(float* p, float v) { *p = v; }
};
template <>
struct Elem<bf16_t> {
  static __device__ __forceinline__ float ld(const bf16_t* p) { return bf2f(*p); }
  static __device__ __forceinline__ void st(bf16_t* p, float v) { *p = f2bf(v); }
};

// Store of an attention value (V, block or context): f32 drafters keep
// float; bf16 drafters keep the bf16-rounded value as fp16 (above).
template <class T>
struct ValueStore;
template <>
struct ValueStore<float> {
  static __device__ __forceinline__ void st(float* p, float v) { *p = v; }
};
template <>
struct ValueStore<bf16_t> {
  static __device__ __forceinline__ uint16_t bits(float v) { return bf16_value_as_f16(v); }
  static __device__ __forceinline__ void st(bf16_t* p, float v) { *p = bf16_value_as_f16(v); }
};

// Maps a linear block index to a tile index so that consecutive tiles land
// on the same XCD (blocks are dispatched to XCDs round-robin): the tiles an
// XCD runs together then share operands through that XCD's L2.
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int per = n / kXcds, rem = n % kXcds;
  const int x = bid % kXcds, local = bid / kXcds;
  return x * per + (x < rem ? x : rem) + local;
}

// Argmax order of the masked decode: a NaN beats any number; among equal
// values (or NaNs) the lower column (= lower token id) wins.
__device__ __forceinline__ bool arg_better(float v1, int c1, float v2, int c2) {
  const bool n1 = v1 != v1, n2 = v2 != v2;
  if (n1 != n2) return n1;
  if (!n1 && v1 != v2) return v1 > v2;
  return c1 < c2;
}

// g / (1 + e^-g) with the hardware reciprocal (about 1 ulp): an IEEE
// division here cost more than the rest of the gate/up epilogue.
__device__ __forceinline__ float silu_f(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// m = q n + r with 0 <= r < n, for 0 <= m < 2^24, from inv_n = 1 / n rounded
// to float: the product m * inv_n is within one of m / n, so one correction
// step makes the quotient exact (checked on the host for n up to 2^24 - 1).
// About six instructions instead of a general integer division.
__device__ __forceinline__ void divmod_rows(int m, int n, float inv_n, int& q, int& r) {
  q = (int)((float)m * inv_n);
  r = m - q * n;
  if (r < 0) {
    --q;
    r += n;
  } else if (r >= n) {
    ++q;
    r -= n;
  }
}

// Rotary embedding constants: the rotation of pair i advances by
// theta^(-2i/d) / (2 pi) turns per position, computed on the host in double
// precision (d/2 <= 64 entries).
struct RopeTab {
  double inv_rev[64];
};

// cos and sin of pos * inv_rev turns, the turn count reduced to [0, 1) in
// double precision and evaluated by the hardware sine/cosine (which take
// turns).
__device__ __forceinline__ void rope_cs(int pos, double inv_rev, float& c, float& s) {
  const double r = (double)pos * inv_rev;
  const float t = (float)(r - floor(r));
  s = __builtin_amdgcn_sinf(t);
  c = __builtin_amdgcn_cosf(t);
}
// (x0, x1) rotated by the angle with cosine c and sine s.
__device__ __forceinline__ void rope_rot(float& x0, float& x1, float c, float s) {
  const float y0 = x0 * c - x1 * s;
  const float y1 = x1 * c + x0 * s;
  x0 = y0;
  x1 = y1;
}
// Advances (c, s) by one position step (cos and sin of inv_rev turns).
__device__ __forceinline__ void rope_step(float& c, float& s, float cd, float sd) {
  const float c2 = c * cd - s * sd;
  s = s * cd + c * sd;
  c = c2;
}

// Rotates the pair (x_i, x_{i + d/2}) by pos * inv_rev turns.  The turn count
// is reduced to [0, 1) in double precision (exact enough for any position
// the int range allows) and the hardware sine/cosine, which take turns,
// evaluate it.
__device__ __forceinline__ void rope_pair(float& x0, float& x1, int pos, double inv_rev) {
  const double r = (double)pos * inv_rev;
  const float t = (float)(r - floor(r));
  const float s = __builtin_amdgcn_sinf(t), c = __builtin_amdgcn_cosf(t);
  const float y0 = x0 * c - x1 * s;
  const float y1 = x1 * c + x0 * s;
  x0 = y0;
  x1 = y1;
}

}  // namespace fpd
