// lt_verify_chunks: the XXH3-64 of every chunk's compressed bytes, without
// decoding (the roadmap's container check, page "GPU Compression Pipeline -
// TDD Roadmap", Phase 6.1: a changed stored byte shows up as a checksum
// mismatch).  One wave per chunk, four chunks per workgroup; the wave takes
// the chunk's 1 KiB blocks in order (lane l loads the 8 bytes at 8 l and at
// 8 l + 512 of each), with the loads of four blocks in flight at a time.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lt_lz4.hpp"
#include "lt_xxh.hpp"

namespace lt {

struct XxhParams {
  const uint8_t *comp;
  const uint64_t *comp_off;
  uint64_t comp_bytes;
  uint32_t n;
  const uint64_t *expect;   // optional: compare and report
  uint64_t *got;            // optional: the computed values
  int32_t *status;          // optional
};

constexpr uint32_t XXH_WAVES = 4;

// 8 bytes at p (any alignment) from global memory as a little-endian word.
// Every lane's p has the same alignment mod 4; only the dwords that hold
// the bytes are read.
__device__ __forceinline__ uint64_t global8(const uint8_t *p) {
  const uintptr_t a = (uintptr_t)p;
  const uint32_t *q = (const uint32_t *)(a & ~(uintptr_t)3);
  const uint32_t sh = (uint32_t)(a & 3);
  uint32_t x0 = q[0], x1 = q[1];
  if (sh) {
    const uint32_t x2 = q[2];
    x0 = __builtin_amdgcn_alignbyte(x1, x0, sh);
    x1 = __builtin_amdgcn_alignbyte(x2, x1, sh);
  }
  return ((uint64_t)x1 << 32) | x0;
}

__global__ void __launch_bounds__(64 * XXH_WAVES) xxh_kernel(XxhParams P) {
  const uint32_t lane = threadIdx.x & 63;
  const uint32_t i = blockIdx.x * XXH_WAVES + __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
  if (i >= P.n) return;
  const uint64_t c0 = P.comp_off[i], c1 = P.comp_off[i + 1];
  if (c0 > c1 || c1 > P.comp_bytes) {
    if (lane == 0 && P.status) P.status[i] = C_TABLE;
    return;
  }
  const uint8_t *p = P.comp + c0;
  const uint64_t n = c1 - c0;
  uint64_t h;
  if (n <= xxh::SHORT_MAX) {
    h = xxh::short_hash((uint32_t)n, [&](uint32_t k) { return (uint32_t)p[k]; });
  } else {
    xxh::Wave W;
    W.init(lane);
    const uint64_t nb = (n - 1) / xxh::BLOCK;
    const uint8_t *q = p + 8 * lane;
    uint64_t b = 0;
    for (; b + 4 <= nb; b += 4) {   // the loads of four blocks in flight
      uint64_t v[4][2];
#pragma unroll
      for (int k = 0; k < 4; k++) {
        v[k][0] = global8(q + xxh::BLOCK * (b + k));
        v[k][1] = global8(q + xxh::BLOCK * (b + k) + 512);
      }
      W.block2(v[0][0], v[0][1], v[1][0], v[1][1]);
      W.block2(v[2][0], v[2][1], v[3][0], v[3][1]);
    }
    for (; b < nb; b++) W.block(global8(q + xxh::BLOCK * b), global8(q + xxh::BLOCK * b + 512));
    // the last block's whole stripes, then the final stripe
    const uint32_t ns = (uint32_t)(((n - 1) - xxh::BLOCK * nb) / 64);
    const uint32_t s = lane >> 3;
    const uint64_t v1 = s < ns ? global8(q + xxh::BLOCK * nb) : 0, v2 = s + 8 < ns ? global8(q + xxh::BLOCK * nb + 512) : 0;
    W.partial(v1, v2, lane, ns);
    W.last(global8(p + n - 64 + 8 * (lane & 7)), lane);
    h = W.merge(n);
  }
  if (lane == 0) {
    if (P.got) P.got[i] = h;
    if (P.status) P.status[i] = (P.expect && P.expect[i] != h) ? C_CHECKSUM : C_OK;
  }
}

}  // namespace lt
