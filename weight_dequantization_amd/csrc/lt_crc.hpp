// lt_crc.hpp -- per-chunk CRC-32 of a chunk table's compressed bytes, on the
// device, for validating stored blocks before they are decoded (the block
// checksum of "GPU Compression Pipeline - TDD Roadmap", Phase 6.1; CRC-32
// of the IEEE 802.3 / zlib polynomial, reflected, all-ones initial value
// and final XOR).
//
// One workgroup per chunk.  Write lin(M) for the CRC register after the
// message M from register 0, and shift(v, k) for register v after k zero
// bytes (multiplication by x^(8k) modulo the polynomial).  lin is linear,
// lin(A || B) = shift(lin(A), |B|) ^ lin(B), and zero bytes in front of a
// message leave lin unchanged.  The all-ones start value equals
// complementing the first four message bytes (for shorter messages, the
// unconsumed part of the start value stays in the register).  So the
// chunk's 16-byte aligned body is padded in front with zero blocks to
// 256 * L blocks; thread t takes blocks t, t + 256, ... (each wave reads
// 1 KiB contiguous per load), folding each into its register after
// shifting the register over the 4080 bytes in between (four table
// lookups), then shifts its result over the 16 * (255 - t) bytes that
// follow its last block; the XOR of the 256 results is lin(body), and
// thread 0 adds the unaligned tail byte by byte.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lt_lz4.hpp"   // chunk status codes

namespace lt {

constexpr int CRC_THREADS = 256;
constexpr uint32_t CRC_POLY = 0xEDB88320u;   // x^32 + ... + 1, reflected, x^32 dropped

struct CrcParams {
  const uint8_t *comp;
  const uint64_t *comp_off;
  uint64_t comp_bytes;
  uint32_t n;
  const uint32_t *expect;   // optional: compare and report
  uint32_t *got;            // optional: the computed values
  int32_t *status;          // optional
};

// a * b modulo the polynomial; bit 31 holds the coefficient of x^0.
__host__ __device__ constexpr uint32_t gf_mul(uint32_t a, uint32_t b) {
  uint32_t p = 0;
  for (int i = 0; i < 32; i++) {
    p ^= b & (0u - (a >> 31));
    a <<= 1;
    b = (b >> 1) ^ (CRC_POLY & (0u - (b & 1u)));
  }
  return p;
}

// x^(8 * bytes) modulo the polynomial: the factor of shift(., bytes).
constexpr uint32_t shift_factor(uint64_t bytes) {
  uint32_t m = 0x80000000u, sq = 0x00800000u;   // x^0, x^8
  for (; bytes != 0; bytes >>= 1) {
    if (bytes & 1) m = gf_mul(m, sq);
    sq = gf_mul(sq, sq);
  }
  return m;
}

// The kernel's tables, evaluated by the compiler:
//   T[k][v]  register 0 after byte v and k zero bytes (slicing by 4)
//   U[k][v]  shift(v << 8k, 4080): a register moved over the 255 blocks
//            between two blocks of one thread
//   G[t]     x^(8 * 16 * (255 - t)): thread t's result moved to the end
struct CrcTables {
  uint32_t T[4][256];
  uint32_t U[4][256];
  uint32_t G[CRC_THREADS];
};
constexpr CrcTables make_crc_tables() {
  CrcTables c{};
  for (uint32_t v = 0; v < 256; v++) {
    uint32_t r = v;
    for (int b = 0; b < 8; b++) r = (r >> 1) ^ (CRC_POLY & (0u - (r & 1u)));
    c.T[0][v] = r;
  }
  for (int k = 1; k < 4; k++)
    for (uint32_t v = 0; v < 256; v++) c.T[k][v] = (c.T[k - 1][v] >> 8) ^ c.T[0][c.T[k - 1][v] & 255];
  const uint32_t x4080 = shift_factor(16 * CRC_THREADS - 16);
  for (int k = 0; k < 4; k++)
    for (uint32_t v = 0; v < 256; v++) c.U[k][v] = gf_mul(v << (8 * k), x4080);
  const uint32_t x16 = shift_factor(16);
  c.G[CRC_THREADS - 1] = 0x80000000u;
  for (int t = CRC_THREADS - 2; t >= 0; t--) c.G[t] = gf_mul(c.G[t + 1], x16);
  return c;
}
__constant__ const CrcTables kCrc = make_crc_tables();

// A block among the chunk's first 32 bytes: bytes before the chunk read as
// zero, and the chunk's first four bytes are complemented (the start value).
__device__ __forceinline__ uint4 edge_block(uint4 w, uintptr_t b, uintptr_t a0) {
  uint32_t d[4] = {w.x, w.y, w.z, w.w};
  for (int q = 0; q < 4; q++)
    for (int j = 0; j < 4; j++) {
      const uintptr_t p = b + 4 * q + j;
      if (p < a0)
        d[q] &= ~(0xFFu << (8 * j));
      else if (p < a0 + 4)
        d[q] ^= 0xFFu << (8 * j);
    }
  return make_uint4(d[0], d[1], d[2], d[3]);
}

__global__ void __launch_bounds__(CRC_THREADS) crc_kernel(CrcParams P) {
  __shared__ uint32_t T[4][256];
  __shared__ uint32_t U[4][256];
  __shared__ uint32_t part[CRC_THREADS / 64];
  const uint32_t i = blockIdx.x;
  const uint32_t tid = threadIdx.x;

  const uint64_t c0 = P.comp_off[i], c1 = P.comp_off[i + 1];
  if (c0 > c1 || c1 > P.comp_bytes) {
    if (tid == 0 && P.status) P.status[i] = C_TABLE;
    return;
  }
  for (int k = 0; k < 4; k++) {
    T[k][tid] = kCrc.T[k][tid];
    U[k][tid] = kCrc.U[k][tid];
  }
  __syncthreads();

  const uintptr_t a0 = (uintptr_t)(P.comp + c0), a1 = (uintptr_t)(P.comp + c1);
  const uintptr_t S = a0 & ~(uintptr_t)15, E = a1 & ~(uintptr_t)15;
  uint32_t lin = 0;
  if (E > S) {   // uniform: the whole workgroup takes this branch or none of it
    const uint64_t nblk = (E - S) >> 4;
    const uint64_t L = (nblk + CRC_THREADS - 1) / CRC_THREADS;
    const uintptr_t A0 = E - (uintptr_t)(L * CRC_THREADS * 16);
    uint32_t r = 0;
#pragma unroll 2
    for (uint64_t k = 0; k < L; k++) {
      const uintptr_t b = A0 + (uintptr_t)((tid + k * CRC_THREADS) * 16);
      // blocks before S are the zero padding: a zero block leaves the zero
      // register zero, so they need no load
      uint4 w = make_uint4(0, 0, 0, 0);
      if (b >= S) w = *(const uint4 *)b;
      if (b < S + 32) w = edge_block(w, b, a0);
      r = U[0][r & 255] ^ U[1][(r >> 8) & 255] ^ U[2][(r >> 16) & 255] ^ U[3][r >> 24];
      const uint32_t d[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int q = 0; q < 4; q++) {
        r ^= d[q];
        r = T[3][r & 255] ^ T[2][(r >> 8) & 255] ^ T[1][(r >> 16) & 255] ^ T[0][r >> 24];
      }
    }
    if (r != 0) r = gf_mul(r, kCrc.G[tid]);
    for (int o = 32; o >= 1; o >>= 1) r ^= __shfl_xor(r, o);
    if ((tid & 63) == 0) part[tid >> 6] = r;
    __syncthreads();
    lin = part[0] ^ part[1] ^ part[2] ^ part[3];
  }
  if (tid == 0) {
    // the unaligned tail, byte by byte, first four chunk bytes complemented
    for (uintptr_t b = (E > a0 ? E : a0); b < a1; b++) {
      const uint32_t v = *(const uint8_t *)b ^ (b < a0 + 4 ? 0xFFu : 0u);
      lin = (lin >> 8) ^ T[0][(lin ^ v) & 255];
    }
    const uint64_t n = c1 - c0;
    if (n < 4) lin ^= 0xFFFFFFFFu >> (8 * n);   // the start value's unconsumed bytes
    const uint32_t crc = lin ^ 0xFFFFFFFFu;
    if (P.got) P.got[i] = crc;
    if (P.status) P.status[i] = (P.expect && P.expect[i] != crc) ? C_CHECKSUM : C_OK;
  }
}

}  // namespace lt
