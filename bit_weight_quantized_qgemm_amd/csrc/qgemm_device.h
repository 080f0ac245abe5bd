// Device-side vector types and the register-level dequantization primitives
// shared by the gfx950 GEMM kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qg {

typedef _Float16 f16;
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f16x2 as_h2(uint32_t x) { return __builtin_bit_cast(f16x2, x); }

// ---- buffer access ----------------------------------------------------------
// Raw buffer resources (base and byte size in SGPRs) let every wave-wide load
// use a constant per-lane VGPR offset plus a wave-uniform SGPR offset, so the
// streaming loops spend no VALU instructions on address arithmetic. Lanes whose
// offset falls outside the resource's byte size read zeros.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcWord3 = 0x00020000;   // gfx9-family raw buffer, 32-bit data format

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}
__device__ __forceinline__ u32x4 load16(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ __forceinline__ u32x2 load8(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0));
}
// The weight stream: each code byte is read once per launch (once per row tile),
// so its loads carry the non-temporal cache policy (NT) and leave the caches to
// the activations, scales and partial sums that are read again. Measured on
// MI355X against plain loads: 3-8 % faster on the 7B-class layers and the 70B
// down projection at M <= 16, and on the 32-row tiles of the up projection.
constexpr int kStreamPolicy = 2;   // NT
__device__ __forceinline__ u32x4 load16_stream(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, kStreamPolicy));
}
__device__ __forceinline__ u32x2 load8_stream(rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, kStreamPolicy));
}
// Device-scope coherent 16-byte access (SC1 cache policy): visible to, and seen
// from, every CU and XCD without whole-cache write-back or invalidation.
constexpr int kCoherentAgent = 16;
__device__ __forceinline__ f32x4 load16_coherent(rsrc_t r, uint32_t voff) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, kCoherentAgent));
}
__device__ __forceinline__ void store16_coherent(f32x4 v, rsrc_t r, uint32_t voff) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, voff, 0, kCoherentAgent);
}

// v_and_or_b32 with the mask in an SGPR and the OR operand in a VGPR: one VALU
// op (gfx9 VOP3 cannot carry two literal constants, so plain C++ would split it).
// Its result must reach an MFMA only through a compiler-generated instruction:
// the compiler does not count inline asm as a VALU write when it inserts the
// wait states an MFMA operand needs after one.
__device__ __forceinline__ uint32_t and_or(uint32_t x, uint32_t mask, uint32_t orv) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(x), "s"(mask), "v"(orv));
  return r;
}
__device__ __forceinline__ f16x8 as_h8(u32x4 x) { return __builtin_bit_cast(f16x8, x); }
__device__ __forceinline__ i32x4 as_i4(u32x4 x) { return __builtin_bit_cast(i32x4, x); }

// Eight 4-bit codes of one blob word -> eight fp16 values (q - z), exact.
//
// The word keeps element e of its 8 consecutive k in nibble sigma(e) (e/2 for
// even e, 4 + (e-1)/2 for odd e), so each 32-bit AND/OR with the fp16 exponent
// of 1024 (0x6400) lifts a pair of elements into two fp16 lanes at once:
//   bits 0-3 / 16-19 give 1024 + q exactly (fp16 ulp at 1024 is 1),
//   bits 4-7 / 20-23 give 1024 + 16 q exactly.
// One packed add of -(1024 + z), or one packed fma with 1/16 and -(64 + z),
// then yields q - z exactly. lo_off = -(1024 + z), hi_off = -(64 + z) in both
// halves. Nine VALU instructions per eight weights.
__device__ __forceinline__ f16x8 dequant_u4x8(uint32_t w, f16x2 lo_off, f16x2 hi_off,
                                              uint32_t magic /* 0x64006400 in a VGPR */) {
  const f16x2 sixteenth = {(f16)0.0625f, (f16)0.0625f};
  const uint32_t w8 = w >> 8;
  const f16x2 p0 = as_h2(and_or(w, 0x000F000Fu, magic)) + lo_off;
  const f16x2 p1 = __builtin_elementwise_fma(as_h2(and_or(w, 0x00F000F0u, magic)), sixteenth, hi_off);
  const f16x2 p2 = as_h2(and_or(w8, 0x000F000Fu, magic)) + lo_off;
  const f16x2 p3 = __builtin_elementwise_fma(as_h2(and_or(w8, 0x00F000F0u, magic)), sixteenth, hi_off);
  f16x8 r;
  r[0] = p0[0]; r[1] = p0[1]; r[2] = p1[0]; r[3] = p1[1];
  r[4] = p2[0]; r[5] = p2[1]; r[6] = p3[0]; r[7] = p3[1];
  return r;
}

__device__ __forceinline__ f16x2 splat_h2(float v) {
  const f16 h = (f16)v;
  f16x2 r = {h, h};
  return r;
}

// fp16 value held in the low (sel = 0) or high (sel = 1) half of a word.
__device__ __forceinline__ float half_of(uint32_t w, int sel) {
  return (float)as_h2(w)[sel];
}

// Select one 16-bit lane (0..7) of a 128-bit register group by a compile-time index.
template <int I>
__device__ __forceinline__ float scale_at(u32x4 v) {
  return half_of(v[I / 2], I % 2);
}

// Release this wave's prior global writes, bump a device-wide arrival counter and
// report whether this wave arrived last. All lanes call; lane 0 does the atomic.
__device__ __forceinline__ bool arrive_last(uint32_t* counter, uint32_t expected_total) {
  __threadfence();
  uint32_t prev = 0;
  if ((threadIdx.x & 63) == 0) prev = atomicAdd(counter, 1u);
  prev = __shfl(prev, 0);
  const bool last = prev == expected_total - 1;
  if (last) __threadfence();
  return last;
}

}  // namespace qg
