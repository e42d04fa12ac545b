// Device helpers of the global -> LDS pipelines (GEMM, attention, LM head):
// LDS-writing buffer loads, the bank swizzle of 16-byte chunks, fence-free
// workgroup barriers and explicit memory-counter waits.
#pragma once
#include "common.h"

namespace fpd {

// Cache-policy operand of a buffer load: non-temporal (the nt bit).
constexpr int kLoadNonTemporal = 2;

// One 16-byte buffer load per lane written straight into LDS: lane i fills
// the 16 bytes at dst + 16 i (dst is wave-uniform).  POLICY is the load's
// cache-policy operand.  Only the device pass sees the builtin; the host
// pass would otherwise drop the kernel stubs.
template <int POLICY = 0>
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, u32x4_t* dst, uint32_t voff, int soff) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)dst, 16, voff, soff, 0,
                                           POLICY);
#endif
}

template <int CH>  // 16-byte chunks per row (BK / 8)
__device__ __forceinline__ int swz(int r, int c) {
  return r * CH + (c ^ ((r / (16 / CH)) & (CH - 1)));
}

// Workgroup barrier without the memory fence of __syncthreads(): that fence
// makes the compiler wait for every outstanding load (vmcnt(0)), which would
// drain the stages in flight.  LDS hand-over is ordered by the explicit
// vmcnt wait before it; the clobber keeps LDS accesses from moving across.
__device__ __forceinline__ void barrier_nofence() { asm volatile("s_barrier" ::: "memory"); }

// s_waitcnt lgkmcnt(0) (vmcnt and expcnt fields at their maximum), issued
// as the builtin so that the compiler's own wait insertion sees it: scalar
// loads still pending make it treat the LDS counter as out of order and
// fall back to full waits before every MFMA group.
__device__ __forceinline__ void wait_lgkm0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// s_waitcnt vmcnt(0) (expcnt and lgkmcnt fields at their maximum), as the
// builtin: loads it covers count as complete in the compiler's own tracking,
// which otherwise re-waits for them, and for every store issued since, at
// each later use on a path where it could not prove them complete.
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Waits until at most `ahead` later stages (LPS loads each) are outstanding.
template <int LPS, int MAXA>
__device__ __forceinline__ void wait_stages(int ahead) {
  if constexpr (MAXA > 0) {
    if (ahead >= MAXA) {
      wait_vmcnt<LPS * MAXA>();
      return;
    }
    wait_stages<LPS, MAXA - 1>(ahead);
  } else {
    wait_vmcnt<0>();
  }
}

}  // namespace fpd
