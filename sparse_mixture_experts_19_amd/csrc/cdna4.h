// CDNA4 (gfx950) device helpers shared by the MFMA kernels of libmoe_mi355x.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// 16-byte chunk c (0..7) of row r of a 128-byte-row LDS tile sits in slot
// c ^ ((r >> 1) & 7): the 16 lanes an LDS cycle serves (16 consecutive rows,
// same chunk) then cover all 64 banks exactly once.
__device__ __forceinline__ int swz128(int r, int c) { return r * 8 + (c ^ ((r >> 1) & 7)); }

// One 16-byte-per-lane DMA global -> LDS (global_load_lds_dwordx4): lane i's
// 16 bytes land at LDS byte address lds + 16 i.  lds must be wave-uniform.
// Issued from asm so that the compiler's LDS-DMA bookkeeping, which merges
// stages conservatively at loop back-edges and then drains the whole queue
// (vmcnt(0)), stays out of software pipelines; completion is waited for
// explicitly (vmcnt) before the barrier that publishes a stage.  The
// instruction writes no VGPR.  M0 is set right before it (one wait state
// apart) and is not used by any other code of these kernels.
__device__ __forceinline__ void dma16(const void* gptr, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :
               : "v"(gptr), "s"(lds)
               : "memory", "m0");
}

// Same with the address split into a wave-uniform base (SGPR pair) and a
// 32-bit per-lane byte offset, which needs no vector ALU work per DMA.  The
// base is pinned to scalar registers (readfirstlane is a plain move when it
// already is scalar), whatever the compiler's divergence analysis concludes.
__device__ __forceinline__ void dma16s(const void* sbase, uint32_t voff, uint32_t lds) {
  const uint64_t b = reinterpret_cast<uintptr_t>(sbase);
  const uint64_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b)));
  const uint64_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b >> 32)));
  const void* s = reinterpret_cast<const void*>(static_cast<uintptr_t>((hi << 32) | lo));
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(s), "s"(lds)
               : "memory", "m0");
}

// 4-byte-per-lane variant (global_load_lds_dword): lane i's 4 bytes land at
// LDS byte address lds + 4 i.
__device__ __forceinline__ void dma4s(const void* sbase, uint32_t voff, uint32_t lds) {
  const uint64_t b = reinterpret_cast<uintptr_t>(sbase);
  const uint64_t lo = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b)));
  const uint64_t hi = static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<uint32_t>(b >> 32)));
  const void* s = reinterpret_cast<const void*>(static_cast<uintptr_t>((hi << 32) | lo));
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :
               : "v"(voff), "s"(s), "s"(lds)
               : "memory", "m0");
}

// Same with a base already in scalar registers (wave-uniform by construction).
__device__ __forceinline__ void dma16p(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds)
               : "memory", "m0");
}

// 4-byte variant with a base already in scalar registers.
__device__ __forceinline__ void dma4p(const void* sbase, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1"
               :
               : "v"(voff), "s"(sbase), "s"(lds)
               : "memory", "m0");
}

// ------------------------------------------------------------------ MXFP8
// OCP MX v1.0 MXFP8: e4m3 elements (bias 7, largest magnitude 448, no
// infinities) sharing one E8M0 scale 2^e per block of 32 values.

// Shared exponent of a block from its largest magnitude: floor(log2 amax) - 8
// (8 = largest exponent of e4m3), clamped to the E8M0 range; a block of zeros
// or of fp32 subnormals takes -127.  Read off the fp32 exponent field.
__device__ __forceinline__ int mx_block_exp(float amax) {
  const int be = static_cast<int>(__float_as_uint(amax) >> 23) & 255;
  return be < 8 ? -127 : be - 135;
}

// 2^-e as fp32, for a block exponent e in [-127, 120]
__device__ __forceinline__ float mx_inv_scale(int e) {
  return __uint_as_float(static_cast<uint32_t>(127 - e) << 23);
}

// e4m3 codes of a*s .. d*s, packed in that order from the low byte: values
// saturate at +-448 and round to the nearest code, ties to the even code
// (v_cvt_pk_fp8_f32 under the default round-to-nearest-even mode); a value
// that rounds to zero gets the code of +0.  s is a power of two, so every
// product is exact (or far below the smallest e4m3 code).
__device__ __forceinline__ uint32_t mx_encode4(float a, float b, float c, float d, float s) {
  auto sat = [](float v) { return __builtin_amdgcn_fmed3f(v, -448.f, 448.f); };
  int r = __builtin_amdgcn_cvt_pk_fp8_f32(sat(a * s), sat(b * s), 0, false);
  r = __builtin_amdgcn_cvt_pk_fp8_f32(sat(c * s), sat(d * s), r, true);
  const uint32_t u = static_cast<uint32_t>(r);
  // 0x80 in every byte whose magnitude bits are nonzero (no carry crosses a byte)
  const uint32_t nz = ((u & 0x7F7F7F7Fu) + 0x7F7F7F7Fu) & 0x80808080u;
  return u & (nz | 0x7F7F7F7Fu);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
      (__attribute__((address_space(3))) const void*)p));
}

// Workgroup barrier without the release/acquire fences of __syncthreads():
// those wait for every outstanding vector-memory op (vmcnt(0)), which would
// drain the prefetch queue.  LDS reads are complete (lgkmcnt(0)) and DMA
// stages are waited for explicitly; the memory clobber keeps the compiler
// from moving LDS accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// s_waitcnt vmcnt(n) for the few n the pipelines need (expcnt / lgkmcnt at
// their maxima; vmcnt is bits [3:0] and [15:14]).  Vector-memory loads of a
// wave complete in issue order, so "at most n outstanding" means every load
// but the newest n has landed, whatever stores are interleaved.
__device__ __forceinline__ void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt(0x0F70); }
__device__ __forceinline__ void wait_vmcnt6() { __builtin_amdgcn_s_waitcnt(0x0F76); }
__device__ __forceinline__ void wait_vmcnt12() { __builtin_amdgcn_s_waitcnt(0x0F7C); }

}  // namespace moe
