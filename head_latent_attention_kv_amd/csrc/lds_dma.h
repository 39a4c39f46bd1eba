// Direct global -> LDS copies and the waits and barriers that go with them
// (gfx950).  Shared by the attention kernels that stream cache tiles through LDS.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

// s_waitcnt with vmcnt = N (expcnt, lgkmcnt left at their maximum), gfx9
// encoding: vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8].
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0xF70);
}

// 16 bytes per lane, global -> LDS (global_load_lds_dwordx4): lane i's bytes land
// at LDS address lds_base + 16*i.  Issued from asm so the compiler does not treat
// every later LDS read as aliasing the in-flight copy (which makes it wait for
// all outstanding loads, prefetches included); callers wait with explicit vmcnt
// counts instead.  No register is written, so nothing is live in flight.
__device__ __forceinline__ void global_to_lds16(const void* sbase, uint32_t voff, uint32_t lds_base) {
  __asm__ __volatile__(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(sbase), "s"(lds_base)
      : "memory", "m0");
}

// The same copy with the non-temporal hint (nt), for data that one workgroup
// reads once per launch and that is far larger than the caches (latent cache
// tiles, projection weights): the caches then keep what is reused instead.
__device__ __forceinline__ void global_to_lds16_stream(const void* sbase, uint32_t voff, uint32_t lds_base) {
  __asm__ __volatile__(
      "s_mov_b32 m0, %2\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1 nt"
      :
      : "v"(voff), "s"(sbase), "s"(lds_base)
      : "memory", "m0");
}

// Workgroup barrier for LDS traffic only: wait for this wave's LDS operations,
// then s_barrier.  Unlike __syncthreads() it does not wait for outstanding
// global loads, so tiles prefetched into other LDS buffers stay in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt, expcnt at maximum
  __builtin_amdgcn_s_barrier();
  __asm__ __volatile__("" ::: "memory");
}

}  // namespace mla
