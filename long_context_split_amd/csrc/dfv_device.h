// Device helpers shared by the gfx950 kernels: the E4M3 decode and the
// direct-to-LDS loads.  One definition each, so the kernels cannot drift
// apart in how they decode codes or in the M0 handling of the LDS DMA.
//
// Page cited: [#589] "[Perf] Reduce DFlash2 attention cost and screen exact QK
// reuse", Purpose (one E4M3 decode serves every producer of the KV operands).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace dfv {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half4 __attribute__((ext_vector_type(4)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef int int2v __attribute__((ext_vector_type(2)));
typedef unsigned uint4v __attribute__((ext_vector_type(4)));
typedef unsigned uint2v __attribute__((ext_vector_type(2)));

#define DFV_LDS __attribute__((address_space(3)))

// Eight OCP E4M3 codes (two dwords, code k in byte k) to eight FP16 values,
// two codes per v_cvt_scalef32_pk_f16_fp8 (gfx950 decodes OCP E4M3; every
// finite code is exact in FP16, 0x7F / 0xFF give NaN).  The per-tensor scales
// are applied elsewhere, so the conversion scale is 1.
__device__ __forceinline__ half8 decode8(unsigned lo, unsigned hi) {
  const half2v a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false);
  const half2v b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true);
  const half2v c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false);
  const half2v d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true);
  return half8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

// Direct-to-LDS loads (global_load_lds_*): lane l's element at the uniform base
// plus its own byte offset lands at LDS address dst + size * l.  Written as
// inline asm so the compiler adds no blanket "wait for every LDS DMA" before
// unrelated LDS reads; callers wait on vmcnt themselves (vector loads complete
// in order).  The s_nop covers the wait state between the M0 write and the
// LDS DMA that reads it.  The _nt forms carry the non-temporal hint, for data
// that is read once.
__device__ __forceinline__ void lds_dma16(const void* base, unsigned off, DFV_LDS void* dst) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)dst);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(off), "s"(base), "s"(m0) : "memory", "m0");
}

__device__ __forceinline__ void lds_dma16_nt(const void* base, unsigned off, DFV_LDS void* dst) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)dst);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
               :: "v"(off), "s"(base), "s"(m0) : "memory", "m0");
}

__device__ __forceinline__ void lds_dma4(const void* base, unsigned off, DFV_LDS void* dst) {
  const unsigned m0 = __builtin_amdgcn_readfirstlane((unsigned)(uintptr_t)dst);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :: "v"(off), "s"(base), "s"(m0) : "memory", "m0");
}

}  // namespace dfv
