// Direct-to-LDS buffer loads and counted waits for gfx950, shared by the
// GEMM kernels.
//
// The loads are buffer loads: a 128-bit resource (base address, byte size)
// in scalar registers, a per-lane 32-bit byte offset, and a scalar offset
// (typically the K position), so one request costs a scalar add for M0 (the
// LDS destination of the wave's 1 KB: 64 lanes x 16 bytes at consecutive
// addresses) and the load itself.  Issued as inline assembly so the
// compiler's automatic wait insertion does not treat later LDS reads as
// dependent on it: completion is tracked explicitly by the caller
// (wait_vmcnt + barrier).
#pragma once

#include "common.h"

namespace moe {

typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// A byte offset past every resource of at most 2^31 bytes: loads there fill
// LDS with zeros and fetch nothing.
constexpr uint32_t OOB_OFF = 0x80000000u;

// Raw buffer resource: no stride, no swizzle, byte range [0, bytes); word 3
// is the gfx9 raw-buffer format word (32-bit data format, no type
// conversion).  Addresses outside the range read as zero.
__device__ __forceinline__ i32x4 buffer_rsrc(const void* base, uint32_t bytes) {
  const uint64_t b = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r.x = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(b & 0xffffffffu));
  r.y = __builtin_amdgcn_readfirstlane(static_cast<int32_t>((b >> 32) & 0xffffu));
  r.z = __builtin_amdgcn_readfirstlane(static_cast<int32_t>(bytes));
  r.w = 0x00020000;
  return r;
}

__device__ __forceinline__ void lds_dma16(i32x4 rsrc, uint32_t voff, uint32_t soff,
                                          uint32_t m0) {
  asm volatile("buffer_load_dwordx4 %0, %1, %2 offen lds" ::"v"(voff), "s"(rsrc),
               "s"(soff), "{m0}"(m0)
               : "memory");
}

// 16-byte store through a buffer resource over [base, base + bytes).
// Offsets outside the range are dropped by the hardware, so a store of rows
// past a tile's end needs no branch and every lane issues the same number of
// vector-memory instructions (the counted waits of a ring that also holds
// loads rely on that count).  Written with the compiler's builtin, not as
// inline assembly, so that the compiler knows the instruction reads its
// data registers and keeps later writes of them at the required distance.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t store_rsrc(void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(base, 0, static_cast<int>(bytes), 0x00020000);
}

__device__ __forceinline__ void buf_store16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff,
                                            u32x4_t v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, rsrc, static_cast<int>(voff), 0, 0);
}

// s_waitcnt with only the vector-memory counter limited (gfx9 encoding:
// vmcnt bits [3:0] and [15:14]; expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Barrier without the memory fence of __syncthreads: LDS here is written
// only by the DMA loads, whose completion each wave has already waited for.
__device__ __forceinline__ void wg_barrier() { asm volatile("s_barrier" ::: "memory"); }

}  // namespace moe
