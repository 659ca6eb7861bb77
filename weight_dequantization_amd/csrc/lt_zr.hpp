// lt_zr.hpp -- zero-run decoding of fp16 activations (the zero-run encoding
// of ReLU outputs on page "Openai/692db884-... (section 28)": runs of zeros
// stored instead of full arrays).  Per block of 1024 elements a 128-byte
// bitmap marks the nonzero elements; the nonzero values follow in element
// order, and val_off[b] counts those before block b, so every block decodes
// on its own.
//
// One wave per block, four per workgroup.  The wave checks the block's bit
// count against its val_off span, stages the block's values in LDS with
// 16-byte loads, and expands: lane l writes elements 8l .. 8l+7 of each
// half-block, so every store instruction writes 1 KiB contiguous, and the
// lane's first value is found by a prefix sum of bit counts over the lanes.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lt_lz4.hpp"   // chunk status codes, wave_excl_scan

namespace lt {

constexpr int ZR_BLOCK = 1024;
constexpr int ZR_WAVES = 4;

struct ZrParams {
  const uint32_t *bitmap;   // 32 words per block
  const uint64_t *val_off;  // [nb + 1]
  const uint16_t *vals;     // [n_vals]
  uint64_t n;               // elements
  uint64_t n_vals;
  uint64_t nb;              // blocks
  uint16_t *out;
  int32_t *status;          // optional, per block
};

__global__ void __launch_bounds__(64 * ZR_WAVES) zr_decode_kernel(ZrParams P) {
  __shared__ __attribute__((aligned(16))) uint16_t sv[ZR_WAVES][ZR_BLOCK + 8];
  const uint32_t wave = threadIdx.x / 64, lane = threadIdx.x & 63;
  const uint64_t b = (uint64_t)blockIdx.x * ZR_WAVES + wave;
  if (b >= P.nb) return;   // whole waves; no workgroup barrier below

  // the block's bitmap: lanes 0..31 hold one word each
  const uint32_t word = lane < 32 ? P.bitmap[32 * b + lane] : 0u;
  const uint64_t e0 = b * ZR_BLOCK;
  const uint64_t left = P.n - e0;   // elements in this block, if under 1024
  // bits set for elements past n make the block inconsistent
  uint32_t past = 0;
  if (left < ZR_BLOCK && lane < 32) {
    const uint64_t w0 = 32ull * lane;
    past = w0 >= left ? word : (left - w0 < 32 ? word >> (uint32_t)(left - w0) : 0u);
  }
  uint32_t bits = (uint32_t)__builtin_popcount(word);
  for (int o = 32; o >= 1; o >>= 1) bits += (uint32_t)__shfl_xor((int)bits, o);
  const uint64_t lo = P.val_off[b], hi = P.val_off[b + 1];
  const bool bad = __ballot(past != 0) != 0 || lo > hi || hi > P.n_vals || hi - lo != bits;
  if (bad) {
    if (lane == 0 && P.status) P.status[b] = C_TABLE;
    return;
  }

  // stage vals[lo .. hi) in LDS from its 16-byte aligned start
  const uintptr_t vs = (uintptr_t)(P.vals + lo), ve = (uintptr_t)(P.vals + hi);
  const uintptr_t va = vs & ~(uintptr_t)15;
  const uint32_t off0 = (uint32_t)(vs - va) / 2;
  uint16_t *sw = sv[wave];
  for (uint32_t j = lane; va + 16 * (uintptr_t)j < ve; j += 64)
    *(uint4 *)(sw + 8 * j) = *(const uint4 *)(va + 16 * (uintptr_t)j);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  uint32_t base = off0;
#pragma unroll
  for (int h = 0; h < 2; h++) {
    // lane l's byte of the bitmap: word 16h + l/4, bits 8(l%4) ..
    const uint32_t m = ((uint32_t)__shfl((int)word, 16 * h + (int)(lane >> 2)) >> (8 * (lane & 3))) & 255u;
    const uint32_t pc = (uint32_t)__builtin_popcount(m);
    uint32_t k = base + wave_excl_scan(pc, lane);
    uint32_t v[8];
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const uint32_t bit = (m >> j) & 1u;
      v[j] = bit ? (uint32_t)sw[k] : 0u;
      k += bit;
    }
    uint32_t total = pc;
    for (int o = 32; o >= 1; o >>= 1) total += (uint32_t)__shfl_xor((int)total, o);
    base += total;
    const uint64_t e = e0 + 512 * h + 8 * lane;
    if (e + 8 <= P.n) {
      *(uint4 *)(P.out + e) = make_uint4(v[0] | v[1] << 16, v[2] | v[3] << 16, v[4] | v[5] << 16, v[6] | v[7] << 16);
    } else {
      for (int j = 0; j < 8; j++)
        if (e + j < P.n) P.out[e + j] = (uint16_t)v[j];
    }
  }
  if (lane == 0 && P.status) P.status[b] = C_OK;
}

}  // namespace lt
