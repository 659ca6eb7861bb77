// lt_device.hpp -- device helpers for liblt (gfx950, wave64).
//
// INT4 / INT8 dequantization in packed fp16: a code q becomes the fp16 value
// 1024 + q by OR-ing it into the mantissa of 0x6400 (1024.0); subtracting the
// fp16 value 1024 + zp (or 1024 + 128 + zp for sign-biased INT8 codes) gives
// q - zp exactly (both are integers below 2048), and one fp16 multiply by the
// scale rounds the exact product once, to nearest-even, with fp16 denormals
// kept (the kernel descriptor's fp16 denorm mode is "preserve").  That equals
// rounding (q - zp) * scale computed exactly, which is the definition of the
// dequantized value ("GPU Compression Pipeline - TDD Roadmap", Phase 1.1 and
// Phase 1.2).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lt {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ h2 as_h2(uint32_t v) { return __builtin_bit_cast(h2, v); }
__device__ __forceinline__ uint32_t as_u32(h2 v) { return __builtin_bit_cast(uint32_t, v); }

// fp16 bit pattern of (1024 + k) for k in [-128, 1023]: exact.
__device__ __forceinline__ uint32_t f16_bits_1024_plus(int k) {
  _Float16 v = (_Float16)(1024 + k);
  return (uint32_t)__builtin_bit_cast(uint16_t, v);
}

// Dequantize one 2-code fp16 pair whose halves hold 0x6400 | u (u = biased
// code, 0..255): (u - bias) * s, where c2 = {1024 + bias, 1024 + bias} and
// s2 = {s, s}.  Exact subtraction, one rounding in the multiply.
__device__ __forceinline__ uint32_t deq_pair(uint32_t magic_pair, h2 c2, h2 s2) {
  h2 d = as_h2(magic_pair) - c2;
  return as_u32(d * s2);
}

// 8 INT4 codes (one packed dword, element order = nibble order from the low
// nibble up) -> 4 dwords of fp16 pairs.
__device__ __forceinline__ uint4 deq8_int4(uint32_t w, h2 c2, h2 s2) {
  uint32_t lo = w & 0x0F0F0F0Fu;          // codes 0, 2, 4, 6 in bytes 0..3
  uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;   // codes 1, 3, 5, 7
  // v_perm: result byte i takes pool byte sel_i, pool = {hi:bytes 4..7, lo:bytes 0..3},
  // selector 0x0C yields 0x00.  Pair k = [lo.b_k, 0, hi.b_k, 0].
  uint32_t p0 = __builtin_amdgcn_perm(hi, lo, 0x0C040C00u) | 0x64006400u;
  uint32_t p1 = __builtin_amdgcn_perm(hi, lo, 0x0C050C01u) | 0x64006400u;
  uint32_t p2 = __builtin_amdgcn_perm(hi, lo, 0x0C060C02u) | 0x64006400u;
  uint32_t p3 = __builtin_amdgcn_perm(hi, lo, 0x0C070C03u) | 0x64006400u;
  uint4 r;
  r.x = deq_pair(p0, c2, s2);
  r.y = deq_pair(p1, c2, s2);
  r.z = deq_pair(p2, c2, s2);
  r.w = deq_pair(p3, c2, s2);
  return r;
}

// fp16 bit pattern of the integer k, |k| < 2048: exact.
__device__ __forceinline__ uint32_t f16_bits_int(int k) {
  _Float16 v = (_Float16)k;
  return (uint32_t)__builtin_bit_cast(uint16_t, v);
}

// 8 INT4 codes -> 4 dwords of fp16 pairs, like deq8_int4, with two VALU
// operations per pair before the arithmetic.  Byte j of w holds codes 2j
// (low nibble) and 2j + 1 (high nibble).  One v_perm builds
// [b_j, 0x64, b_j, 0x54] from w and the magic dword 0x54006400; masking then
// keeps the low nibble under 0x64, where 0x6400 | c is 1024 + c, and the high
// nibble at bits 4..7 under 0x54, where 0x5400 | (c << 4) is 64 + c
// (exponent 2^6, mantissa step 1/16).  So c2 must hold {1024 + zp, 64 + zp};
// both subtractions are exact.
// (the selector goes in a scalar register, so the loop-invariant operands
// cost one vector register, the magic dword, instead of one per selector)
__device__ __forceinline__ uint32_t dual_magic(uint32_t w, uint32_t magic, uint32_t sel) {
  uint32_t t;
  asm("v_perm_b32 %0, %1, %2, %3" : "=v"(t) : "v"(magic), "v"(w), "s"(sel));
  return t & 0xFFF0FF0Fu;
}
__device__ __forceinline__ uint4 deq8_int4_dual(uint32_t w, h2 c2, h2 s2) {
  const uint32_t magic = 0x54006400u;   // pool bytes 5 = 0x64, 7 = 0x54
  uint4 r;
  r.x = deq_pair(dual_magic(w, magic, 0x07000500u), c2, s2);
  r.y = deq_pair(dual_magic(w, magic, 0x07010501u), c2, s2);
  r.z = deq_pair(dual_magic(w, magic, 0x07020502u), c2, s2);
  r.w = deq_pair(dual_magic(w, magic, 0x07030503u), c2, s2);
  return r;
}

// 4 INT8 codes (one dword, little-endian) -> 2 dwords of fp16 pairs.  Codes
// are biased to unsigned (q + 128 = q ^ 0x80) so c2 must hold 1024 + 128 + zp.
__device__ __forceinline__ uint2 deq4_int8(uint32_t w, h2 c2, h2 s2) {
  uint32_t u = w ^ 0x80808080u;
  uint32_t p0 = __builtin_amdgcn_perm(0u, u, 0x0C010C00u) | 0x64006400u;
  uint32_t p1 = __builtin_amdgcn_perm(0u, u, 0x0C030C02u) | 0x64006400u;
  uint2 r;
  r.x = deq_pair(p0, c2, s2);
  r.y = deq_pair(p1, c2, s2);
  return r;
}

// One code, for groups that split a lane's codes (general `group`).
__device__ __forceinline__ uint16_t deq1(int q, int z, uint16_t s_bits) {
  _Float16 d = (_Float16)(q - z);           // exact: |q - z| <= 255
  _Float16 s = __builtin_bit_cast(_Float16, s_bits);
  return __builtin_bit_cast(uint16_t, (_Float16)(d * s));
}

__device__ __forceinline__ h2 splat_h2(uint16_t bits) {
  return as_h2((uint32_t)bits | ((uint32_t)bits << 16));
}

}  // namespace lt
