// Small device helpers shared by the attention kernels that stage tiles in
// LDS with the LDS-DMA path and run their matrix products as inline-asm MFMAs
// (decode_mfma.hip, prefill.hip).  gfx950 only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) i32x2 lds_i32x2;

// XOR applied to the 16-byte chunk index of tile row r (within each group of
// eight chunks).  For tiles whose row stride is 128 bytes modulo 256 (1152-B
// cache rows, 640-B prefill key rows) it spreads both the operand reads of 16
// rows at one chunk and the transpose reads of 4 rows x 4 chunks over all 64
// LDS banks.
__device__ __forceinline__ int swz(int r) { return (((r >> 1) & 1) << 2) | ((r >> 2) & 3); }

// s_waitcnt vmcnt(N) with expcnt/lgkmcnt left at their maxima (no wait on them)
template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Workgroup barrier that the compiler may not move memory operations across.
// It does not wait for the wave's own outstanding LDS or memory operations.
__device__ __forceinline__ void block_sync() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

// 32x32x16 bf16 MFMAs written as inline asm so that the accumulator's
// register class is fixed: v0 starts a VGPR accumulator at zero, v adds into
// one, a adds into an AGPR accumulator.  The compiler does not see these as
// MFMAs, so it inserts none of the wait states an MFMA needs around it:
//  - before: an MFMA may read a VGPR only two wait states after a VALU
//    instruction wrote it, and the compiler is free to produce an operand
//    with a VALU copy right before the asm (an AGPR read-back when registers
//    run short), so every wrapper opens with s_nop 1;
//  - after: a VALU or LDS access of the result must be padded (pad_mfma).
__device__ __forceinline__ void mfma_v0(f32x16& d, const bf16x8& a, const bf16x8& b) {
  __asm__ volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v(f32x16& d, const bf16x8& a, const bf16x8& b) {
  __asm__ volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_a(f32x16& d, const bf16x8& a, const bf16x8& b) {
  __asm__ volatile("s_nop 1\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
}
// 64 wait states: more than any MFMA result latency on this part
__device__ __forceinline__ void pad_mfma() {
  __asm__ volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
}
// Maximum of three scores with the hardware instruction.  fmaxf would first
// quiet every operand that the compiler cannot prove canonical (one extra
// VALU instruction per score taken straight from an MFMA accumulator); the
// scores are never NaN (masked columns hold -inf), so the hardware maximum
// gives the same value.
__device__ __forceinline__ float max3f(float a, float b, float c) {
  float r;
  __asm__("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}
// Two floats rounded to bf16 (nearest, ties to even), lo in the low half.
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
// Keeps x computed where this stands: the MFMAs are volatile asm, so an empty
// volatile asm that reads and writes x stays between the same two MFMAs.
template <typename T>
__device__ __forceinline__ void pin(T& x) {
  __asm__ volatile("" : "+v"(x));
}

}  // namespace mla
