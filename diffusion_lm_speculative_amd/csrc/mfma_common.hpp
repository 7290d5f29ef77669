// Device helpers shared by the matrix-core kernels (gfx950, wave64): bf16
// operand vectors, the 16x16x32 bf16 MFMA, explicit s_waitcnt, LDS barriers,
// transposed LDS reads and direct-to-LDS global loads.
#pragma once

#include "simsd_common.hpp"

namespace simsd {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));

#define SIMSD_LDS __attribute__((address_space(3)))
#define SIMSD_GLOBAL __attribute__((address_space(1)))

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 bits_to_bf16x8(const uint16_t (&v)[8]) {
  u16x8 u = {v[0], v[1], v[2], v[3], v[4], v[5], v[6], v[7]};
  return __builtin_bit_cast(bf16x8, u);
}

// s_waitcnt immediate (gfx9 encoding): vmcnt in bits 3:0 and 15:14, expcnt
// 6:4 (left at its maximum), lgkmcnt 11:8.
template <int VM, int LGKM>
__device__ __forceinline__ void wait_counts() {
  static_assert(VM >= 0 && VM <= 63 && LGKM >= 0 && LGKM <= 15, "waitcnt range");
  __builtin_amdgcn_s_waitcnt((VM & 15) | ((VM >> 4) << 14) | (7 << 4) | (LGKM << 8));
}

// Workgroup barrier for LDS written by this kernel.  Each wave first waits
// until its own LDS writes (lgkmcnt 0) and all but its VM newest direct-to-LDS
// loads (vmcnt VM) are done; the empty asm keeps the compiler from moving
// memory accesses across the barrier.
template <int VM>
__device__ __forceinline__ void lds_barrier() {
  wait_counts<VM, 0>();
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Transposed LDS read (ds_read_b64_tr_b16) of the 8 bytes at byte address
// a + OFF.  The ring loads are invisible to the compiler, so it waits only
// for its own LDS traffic before the result is used.
template <int OFF>
__device__ __forceinline__ bf16x4 tr_read(uint32_t a) {
  static_assert(OFF >= 0 && OFF < 65536, "LDS immediate offset");
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(reinterpret_cast<SIMSD_LDS bf16x4*>(static_cast<uintptr_t>(a + OFF)));
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((const SIMSD_LDS void*)p));
}

// One direct-to-LDS load: 16 bytes from `src` per lane into LDS at
// m0 + 16*lane (m0 = `lds`, wave-uniform).  Inline asm keeps the load out of
// the compiler's view: otherwise it makes every later LDS access of the wave
// wait for all such loads in flight.  Completion is tracked by hand with
// s_waitcnt vmcnt, and every path drains the loads before the workgroup ends.
//
// The compiler does not know that the asm is a vector memory instruction, so
// it inserts none of the wait states the CDNA3/CDNA4 ISA requires before one:
// one after an SALU write of M0 (read by a load with the LDS bit), five after
// a VALU write of an SGPR the load reads (its address base, which a
// v_readlane may have just restored from a spill).  The leading s_nop 4
// gives both.
__device__ __forceinline__ void dma16(const void* src, uint32_t lds) {
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}

// The same load from the wave-uniform base `base` (kept in SGPRs) plus the
// per-lane byte offset `voff`.
__device__ __forceinline__ void dma16s(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base),
               "{m0}"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}

// dma16s with the non-temporal cache-policy bit, for data a call reads once.
__device__ __forceinline__ void dma16s_nt(const void* base, uint32_t voff, uint32_t lds) {
  asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(base),
               "{m0}"(__builtin_amdgcn_readfirstlane(lds))
               : "memory");
}

}  // namespace
}  // namespace simsd
