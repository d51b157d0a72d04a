// LDS staging helpers shared by the MFMA GEMMs (gemm.hip, mx.hip).
#pragma once

#include "common.hpp"

namespace w4a8 {
namespace lds {

// s_waitcnt vmcnt(n) (gfx9 encoding), leaving the other counters alone.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
}

// One 16-byte-per-lane DMA from global memory into LDS: lane i's bytes land
// at lds_dst + 16 i (lds_dst is wave-uniform; the hardware takes it from M0
// when the instruction issues).  Issued as inline assembly so that the
// compiler's wait-count pass, which cannot always tell DMA into one stage
// from reads of another and then drains every DMA before a read, keeps out:
// the kernel waits for its DMAs itself (vmcnt), and the memory clobber keeps
// LDS accesses in program order around it.  M0 is restored afterwards, and
// an SALU write of M0 needs one wait state before an LDS DMA reads it.
__device__ __forceinline__ void dma16(const void* src, const void* lds_dst) {
  const uint32_t lds = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds_dst));
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %[sv], m0\n\t"
      "s_mov_b32 m0, %[lds]\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %[src], off\n\t"
      "s_mov_b32 m0, %[sv]"
      : [sv] "=&s"(saved)
      : [src] "v"(src), [lds] "s"(lds)
      : "memory");
}

// Workgroup barrier that orders nothing in hardware: each wave has already
// waited for its own DMA into the stage (vmcnt) and has consumed every LDS
// read of the previous step before it arrives.  The empty asm statements
// keep the compiler from moving LDS accesses across it.
__device__ __forceinline__ void stage_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

}  // namespace lds
}  // namespace w4a8
