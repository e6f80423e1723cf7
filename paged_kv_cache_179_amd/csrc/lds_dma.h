// Global-to-LDS DMA and the explicit waits that pipeline it (gfx950).
//
// The decode kernels stream K/V rows straight into LDS with
// global_load_lds_dwordx4 and order each pipeline slot themselves: the
// compiler cannot tell the slots apart and, left to itself, waits for every
// outstanding DMA before any LDS read.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

// s_waitcnt with vmcnt = N (0..63; the field is split over bits 3:0 and
// 15:14), expcnt and lgkmcnt not waited.
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(((N >> 4) << 14) | 0x0F70 | (N & 15));
}

// 16-byte global-to-LDS DMA (non-temporal).  `lds` is the wave-uniform LDS
// destination of lane 0; lane i's 16 bytes land at lds + 16 * i.  Written as
// inline assembly so that the compiler does not treat every later LDS read as
// dependent on every outstanding DMA; the kernels order each slot with
// explicit vmcnt waits.  M0 carries the LDS address; nothing else in these
// kernels keeps a value in M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ inline void dma16(const void* global, const void* lds) {
  const uint32_t off = static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)lds));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off nt"
               :
               : "s"(__builtin_amdgcn_readfirstlane(off)), "v"(global)
               : "memory", "m0");
}

// As dma16, with the global address given as a wave-uniform base (an SGPR
// pair) plus this lane's 32-bit byte offset, so that a lane's address costs
// one 32-bit VGPR instead of 64-bit arithmetic per transfer.
__device__ inline void dma16_sv(const void* base, uint32_t lane_off, const void* lds) {
  const uint32_t off = static_cast<uint32_t>(
      reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const void*)lds));
  // The lane-read builtin returns int: each half goes back through uint32_t,
  // or the low half would be sign-extended into the high one.
  const uint64_t b = static_cast<uint64_t>(reinterpret_cast<uintptr_t>(base));
  const uint32_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(b))));
  const uint32_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(b >> 32))));
  const uint64_t bu = static_cast<uint64_t>(lo) | (static_cast<uint64_t>(hi) << 32);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2 nt"
               :
               : "s"(__builtin_amdgcn_readfirstlane(off)), "v"(lane_off), "s"(bu)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// Makes this wave's LDS writes visible to its own later reads (and orders its
// reads before later DMA into the same slot).
__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace pa
