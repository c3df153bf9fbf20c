// Device-side building blocks shared by the gfx950 kernels of libmha:
// vector types, direct global -> LDS copies, wait counters and LDS reads.
#pragma once

#include "kernels.h"

namespace mha {
namespace dev {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

// Transposing LDS read: within each 16-lane group, lane s reads 4 consecutive
// bf16 (8 bytes) and receives, transposed, 4 values of one column.
__device__ __forceinline__ i16x4 tr_read(const __bf16* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
}

// s_waitcnt vmcnt(N) (gfx9 encoding; expcnt and lgkmcnt left unconstrained)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// s_waitcnt lgkmcnt(0): every LDS read this wave issued has returned its data.
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14)); }

// 16-byte global -> LDS copy per lane from a wave-uniform 64-bit base plus a
// per-lane 32-bit byte offset (no vector address arithmetic); lane l writes
// LDS byte address lds + 16 l.  Inline assembly, so that the compiler does
// not wait for it before every LDS read; kernels wait for it explicitly
// (vmcnt) before the barrier that publishes the data.  The copy takes its
// LDS address from M0, and on this chip family an LDS-DMA instruction must
// not directly follow a scalar write of M0 (one wait state in between); the
// compiler cannot insert that inside an asm block, hence the s_nop.
__device__ __forceinline__ void dma16_s(const void* sbase, unsigned voff, unsigned lds) {
  // The base is wave-uniform; readfirstlane pins it to SGPRs for the saddr operand.
  const unsigned long long p = (unsigned long long)(size_t)sbase;
  // (readfirstlane returns int: widen through unsigned, never sign-extend.)
  const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)(p >> 32));
  const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)p);
  const unsigned long long sp = ((unsigned long long)hi << 32) | (unsigned long long)lo;
  const unsigned ls = (unsigned)__builtin_amdgcn_readfirstlane(lds);  // wave-uniform: pin to an SGPR
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :
               : "s"(ls), "v"(voff), "s"((const void*)(size_t)sp)
               : "memory", "m0");
}

// 4-byte global -> LDS copy per lane (same addressing and M0 wait state as
// dma16_s; lane l writes LDS byte address lds + 4 l): 64 consecutive floats
// per wave.
__device__ __forceinline__ void dma4_s(const void* sbase, unsigned voff, unsigned lds) {
  const unsigned long long p = (unsigned long long)(size_t)sbase;
  const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)(p >> 32));
  const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)p);
  const unsigned long long sp = ((unsigned long long)hi << 32) | (unsigned long long)lo;
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dword %1, %2"
               :
               : "s"(lds), "v"(voff), "s"((const void*)(size_t)sp)
               : "memory", "m0");
}

// A wave-uniform pointer pinned to SGPRs (uniform 64-bit products are
// otherwise formed, and kept, in VGPRs).
template <typename T>
__device__ __forceinline__ T* wave_uniform(T* p) {
  const unsigned long long v = (unsigned long long)(size_t)p;
  const unsigned hi = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)(v >> 32));
  const unsigned lo = (unsigned)__builtin_amdgcn_readfirstlane((unsigned)v);
  return (T*)(size_t)(((unsigned long long)hi << 32) | (unsigned long long)lo);
}

// LDS byte address of a __shared__ object (wave-uniform).
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane(
      (unsigned)(size_t)(const __attribute__((address_space(3))) char*)p);
}

}  // namespace dev
}  // namespace mha
