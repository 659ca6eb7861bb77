// XXH3-64 (seed 0, default secret) computed by one wave: the per-chunk
// checksum of the compressed bytes that the roadmap's container format names
// (page "GPU Compression Pipeline - TDD Roadmap", Phase 6.1 HCT Format V2).
// The pages name the hash only; the arithmetic follows its public definition.
//
// Inputs over 240 bytes are hashed in 1 KiB blocks of 16 stripes of 64
// bytes.  Each stripe adds to eight 64-bit accumulators: word i of the
// stripe goes to accumulator i ^ 1, and the product of the two 32-bit
// halves of (word i XOR secret word) to accumulator i.  The additions
// commute, so a block is one parallel step: each lane takes two of its
// words and a butterfly over the lanes sums the block (struct Wave).
// After every whole block the accumulators are scrambled (a nonlinear map,
// so blocks are taken in order).  The input's last partial block, a final
// stripe over its last 64 bytes and the merge of the accumulators end it.
// Inputs of 240 bytes or less take the definition's short forms, computed
// by every lane alike from single bytes.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lt_xxh_secret.h"

namespace lt {
namespace xxh {

__constant__ uint64_t SECRET[24] = {LT_XXH_SECRET_WORDS};
// the accumulators' starting values, in accumulator order
__constant__ uint64_t ACC0[8] = {0xC2B2AE3Dull,          0x9E3779B185EBCA87ull, 0xC2B2AE3D27D4EB4Full,
                                 0x165667B19E3779F9ull,  0x85EBCA77C2B2AE63ull, 0x85EBCA77ull,
                                 0x27D4EB2F165667C5ull,  0x9E3779B1ull};
constexpr uint64_t PR64_1 = 0x9E3779B185EBCA87ull, PR64_2 = 0xC2B2AE3D27D4EB4Full,
                   PR64_3 = 0x165667B19E3779F9ull, PR32_1 = 0x9E3779B1ull;
constexpr uint32_t BLOCK = 1024, SHORT_MAX = 240;

// secret bytes off .. off + 7 as a little-endian word (off + 8 <= 192)
__device__ __forceinline__ uint64_t sec(uint32_t off) {
  const uint32_t w = off >> 3, sh = (off & 7) * 8;
  const uint64_t lo = SECRET[w];
  return sh ? (lo >> sh) | (SECRET[w + 1] << (64 - sh)) : lo;
}
// the 128-bit product of a and b with its halves XORed
__device__ __forceinline__ uint64_t fold(uint64_t a, uint64_t b) { return (a * b) ^ __umul64hi(a, b); }
__device__ __forceinline__ uint64_t finish3(uint64_t h) {
  h ^= h >> 37;
  h *= 0x165667919E3779F9ull;
  return h ^ (h >> 32);
}
__device__ __forceinline__ uint64_t finish64(uint64_t h) {
  h ^= h >> 33;
  h *= PR64_2;
  h ^= h >> 29;
  h *= PR64_3;
  return h ^ (h >> 32);
}
__device__ __forceinline__ uint64_t swap64(uint64_t v) {
  const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
  return ((uint64_t)__builtin_bswap32(lo) << 32) | __builtin_bswap32(hi);
}
__device__ __forceinline__ uint64_t xor_lanes(uint64_t v, int m) {
  const uint32_t lo = (uint32_t)__shfl_xor((int)(uint32_t)v, m), hi = (uint32_t)__shfl_xor((int)(uint32_t)(v >> 32), m);
  return ((uint64_t)hi << 32) | lo;
}

// The accumulators of one wave: lane l holds accumulator i = l % 8 (the
// same value in every lane of that i).  Of each block it takes word i of
// stripes s = l / 8 and s + 8, the 8 bytes at block offsets 8 l and
// 8 l + 512.  Word i's data value belongs to accumulator i ^ 1, so the
// data values change lanes once (l ^ 1) before the sum over the lanes of
// equal i (l ^ 8, l ^ 16, l ^ 32).
struct Wave {
  uint64_t a;        // accumulator i
  uint64_t k1, k2;   // secret words of the lane's two slots in a block
  uint32_t i;

  __device__ __forceinline__ void init(uint32_t lane) {
    i = lane & 7;
    const uint32_t s = lane >> 3;
    a = ACC0[i];
    k1 = SECRET[s + i];
    k2 = SECRET[s + 8 + i];
  }
  // the block's contribution to accumulator i, from the lane's two words
  // (v1 at 8 l, v2 at 8 l + 512) with secret words x1, x2, each counted when
  // its stripe is; every lane must take part
  __device__ __forceinline__ uint64_t part(uint64_t v1, uint64_t v2, uint64_t x1, uint64_t x2, bool on1,
                                          bool on2) {
    const uint64_t d1 = v1 ^ x1, d2 = v2 ^ x2;
    uint64_t p = 0, dv = 0;
    if (on1) {
      p += (d1 & 0xFFFFFFFFull) * (d1 >> 32);
      dv += v1;
    }
    if (on2) {
      p += (d2 & 0xFFFFFFFFull) * (d2 >> 32);
      dv += v2;
    }
    uint64_t t = p + xor_lanes(dv, 1);
    t += xor_lanes(t, 8);
    t += xor_lanes(t, 16);
    t += xor_lanes(t, 32);
    return t;
  }
  __device__ __forceinline__ void scramble() { a = (a ^ (a >> 47) ^ SECRET[16 + i]) * PR32_1; }
  // one whole block, then its scramble
  __device__ __forceinline__ void block(uint64_t v1, uint64_t v2) {
    a += part(v1, v2, k1, k2, true, true);
    scramble();
  }
  // two whole blocks in order (their sums are independent, so both
  // reductions run side by side before the two scrambles)
  __device__ __forceinline__ void block2(uint64_t v1, uint64_t v2, uint64_t w1, uint64_t w2) {
    const uint64_t t = part(v1, v2, k1, k2, true, true), u = part(w1, w2, k1, k2, true, true);
    a += t;
    scramble();
    a += u;
    scramble();
  }
  // the last block's first ns whole stripes (no scramble)
  __device__ __forceinline__ void partial(uint64_t v1, uint64_t v2, uint32_t lane, uint32_t ns) {
    a += part(v1, v2, k1, k2, (lane >> 3) < ns, (lane >> 3) + 8 < ns);
  }
  // the final stripe (the input's last 64 bytes): lanes 0 .. 7 bring word i;
  // its secret words start 7 bytes before the scramble's
  __device__ __forceinline__ void last(uint64_t v, uint32_t lane) {
    a += part(v, 0, sec(121 + 8 * i), 0, lane < 8, false);
  }
  __device__ __forceinline__ uint64_t merge(uint64_t n) {
    const uint64_t o = xor_lanes(a, 1);   // accumulator i ^ 1
    const uint32_t j = i >> 1;
    const uint64_t lo = (i & 1) ? o : a, hi = (i & 1) ? a : o;
    uint64_t m = fold(lo ^ sec(11 + 16 * j), hi ^ sec(19 + 16 * j));
    m += xor_lanes(m, 2);
    m += xor_lanes(m, 4);
    return finish3(n * PR64_1 + m);
  }
};

// Inputs of at most 240 bytes; byte(k) reads input byte k (k < n).
template <class B>
__device__ uint64_t short_hash(uint32_t n, B byte) {
  auto rd = [&](uint32_t k, int len) {
    uint64_t v = 0;
    for (int j = len - 1; j >= 0; j--) v = (v << 8) | byte(k + (uint32_t)j);
    return v;
  };
  auto mix16 = [&](uint32_t k, uint32_t s) { return fold(rd(k, 8) ^ sec(s), rd(k + 8, 8) ^ sec(s + 8)); };
  if (n == 0) return finish64(sec(56) ^ sec(64));
  if (n <= 3) {
    const uint64_t c = ((uint64_t)byte(0) << 16) | ((uint64_t)byte(n >> 1) << 24) | byte(n - 1) | ((uint64_t)n << 8);
    return finish64(c ^ (uint64_t)((uint32_t)sec(0) ^ (uint32_t)sec(4)));
  }
  if (n <= 8) {
    uint64_t h = (rd(n - 4, 4) + (rd(0, 4) << 32)) ^ (sec(8) ^ sec(16));
    h ^= ((h << 49) | (h >> 15)) ^ ((h << 24) | (h >> 40));
    h *= 0x9FB21C651E98DF25ull;
    h ^= (h >> 35) + n;
    h *= 0x9FB21C651E98DF25ull;
    return h ^ (h >> 28);
  }
  if (n <= 16) {
    const uint64_t lo = rd(0, 8) ^ sec(24) ^ sec(32), hi = rd(n - 8, 8) ^ sec(40) ^ sec(48);
    return finish3(n + swap64(lo) + hi + fold(lo, hi));
  }
  uint64_t acc = n * PR64_1;
  if (n <= 128) {
    for (uint32_t j = 0; 32 * j < n; j++) {   // 16-byte pieces from both ends, pair j at secret 32 j
      acc += mix16(16 * j, 32 * j);
      acc += mix16(n - 16 * (j + 1), 32 * j + 16);
    }
    return finish3(acc);
  }
  for (uint32_t j = 0; j < 8; j++) acc += mix16(16 * j, 16 * j);
  acc = finish3(acc);
  for (uint32_t j = 8; j < n / 16; j++) acc += mix16(16 * j, 16 * (j - 8) + 3);
  acc += mix16(n - 16, 119);
  return finish3(acc);
}

}  // namespace xxh
}  // namespace lt
