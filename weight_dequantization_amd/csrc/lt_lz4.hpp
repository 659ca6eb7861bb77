// lt_lz4.hpp -- chunk-parallel LZ4 block decoding on gfx950, one workgroup
// per independently compressed chunk, with three wave roles:
//
//   wave 0  decoder : parses the block's sequences and materializes the
//                     decoded bytes into a 64 KiB LDS history ring (literal
//                     copies from the input ring, match copies from history);
//   wave 1  feeder  : streams the chunk's compressed bytes from HBM into an
//                     8 KiB LDS input ring ahead of the decoder;
//   waves 2+ flushers: take completed 1 KiB tiles of history and write them
//                     out: as bytes (decode-only), or unpacked and
//                     dequantized to fp16 (fused INT4 / INT8), with coalesced
//                     16-byte stores.
//
// The LZ4 block format (the pages name LZ4 for compressed weight blocks but
// do not define it; "GPU Compression Pipeline - TDD Roadmap", Phase 2.1 and
// Phase 3.1): a sequence is a token (high nibble literal count, low nibble
// match length - 4; 15 means more length follows as bytes of 255 closed by a
// byte < 255), the literals, a 2-byte little-endian distance, and the match
// length's extra bytes; the last sequence has literals only.  A match of
// length M at distance d produces out[p + j] = out[p - d + (j mod d)], which
// is what byte-serial copying gives when d < M; every source byte lies before
// p, so all lanes may copy a match at once.
//
// The roles talk through LDS counters (relaxed atomics after an explicit
// lgkmcnt(0) wait, so the data they publish is already in LDS):
//   in_avail  feeder  -> decoder : input bytes present in the ring
//   in_used   decoder -> feeder  : input before this position is consumed
//   out_done  decoder -> flushers: history bytes that are final
//   next_tile flushers -> decoder: tiles below it are written out (ring reuse
//                                  for chunks over 64 KiB)
//   state     decoder -> all     : running / done / failed
// Every wait is bounded: the decoder consumes at least one input byte per
// sequence and stops at the chunk's end or at the first error, and it sets
// `state` before leaving, which releases every other wave.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lt_device.hpp"

namespace lt {

constexpr uint32_t HIST = 1u << 16;   // LZ4 distances reach 65535
constexpr uint32_t HMASK = HIST - 1;
constexpr uint32_t INR = 1u << 13;    // compressed-input ring
constexpr uint32_t IMASK = INR - 1;
constexpr uint32_t TILE = 1024;       // flush granularity (bytes of decoded stream)
constexpr int NFLUSH = 2;
constexpr int NWAVES = 2 + NFLUSH;
constexpr int NTHREADS = 64 * NWAVES;
constexpr uint32_t LEN_CAP = 1u << 31;

enum : uint32_t { ST_RUN = 0, ST_DONE = 1, ST_FAIL = 2 };
enum : int32_t { C_OK = 0, C_TRUNC = 1, C_BADOFF = 2, C_OVERRUN = 3, C_SIZE = 4, C_TABLE = 5 };
enum Mode : int { MODE_BYTES = 0, MODE_INT4 = 1, MODE_INT8 = 2 };

struct Ctl {
  uint32_t in_avail;
  uint32_t in_used;
  uint32_t out_done;
  uint32_t state;
  uint32_t next_tile[NFLUSH];
  int32_t status;
  uint32_t pad;
};

struct Smem {
  uint8_t hist[HIST];
  uint8_t inr[INR];
  Ctl ctl;
};

struct ChunkParams {
  const uint8_t *comp;
  const uint64_t *comp_off;
  const uint64_t *dst_off;
  uint64_t comp_bytes;
  uint64_t total;
  uint32_t n;
  uint32_t max_chunk;
  void *out;                 // bytes (decode-only) or fp16 (fused)
  int32_t *status;
  const uint16_t *scales;
  const int8_t *zp;
  uint64_t group;
};

// ------------------------------------------------------------ LDS sync

__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }  // lgkmcnt(0)

__device__ __forceinline__ uint32_t lds_get(uint32_t *p) {
  uint32_t v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  return __builtin_amdgcn_readfirstlane(v);
}

// Publish a counter after this wave's earlier LDS writes have completed.
__device__ __forceinline__ void lds_put(uint32_t *p, uint32_t v, uint32_t lane) {
  wait_lds();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  if (lane == 0) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// ------------------------------------------------------ LDS byte moves

__device__ __forceinline__ uint4 lds_ld16(const uint8_t *p) {
  uint4 v;
  __builtin_memcpy(&v, p, 16);
  return v;
}

// dword k (0..3) of v, selected without indexing a register array
__device__ __forceinline__ uint32_t dword_of(uint4 v, uint32_t k) {
  uint32_t lo = (k & 1) ? v.y : v.x;
  uint32_t hi = (k & 1) ? v.w : v.z;
  return (k & 2) ? hi : lo;
}

__device__ __forceinline__ uint32_t byte_of(uint4 v, uint32_t b) {
  return (dword_of(v, b >> 2) >> ((b & 3) * 8)) & 0xFFu;
}

// Write the first n (1..16) bytes of v at p, without touching p[n..16).
__device__ __forceinline__ void lds_st_part(uint8_t *p, uint4 v, uint32_t n) {
  if (n == 16) {
    __builtin_memcpy(p, &v, 16);
    return;
  }
  uint32_t o = 0;
  if (n & 8) {
    uint2 a = make_uint2(v.x, v.y);
    __builtin_memcpy(p, &a, 8);
    o = 8;
  }
  if (n & 4) {
    uint32_t a = dword_of(v, o >> 2);
    __builtin_memcpy(p + o, &a, 4);
    o += 4;
  }
  if (n & 2) {
    uint16_t h = (uint16_t)(dword_of(v, o >> 2) >> ((o & 3) * 8));
    __builtin_memcpy(p + o, &h, 2);
    o += 2;
  }
  if (n & 1) p[o] = (uint8_t)byte_of(v, o);
}

// 16 bytes from a ring at arbitrary (wrapping) positions
template <uint32_t MASK>
__device__ __forceinline__ uint4 ring_ld16(const uint8_t *ring, uint32_t pos) {
  uint32_t w[4];
#pragma unroll
  for (int k = 0; k < 4; k++) {
    w[k] = 0;
#pragma unroll
    for (int b = 0; b < 4; b++) w[k] |= (uint32_t)ring[(pos + 4 * k + b) & MASK] << (8 * b);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// first n (1..16) bytes of v to a ring at arbitrary (wrapping) positions
template <uint32_t MASK>
__device__ __forceinline__ void ring_st_part(uint8_t *ring, uint32_t pos, uint4 v, uint32_t n) {
  for (uint32_t b = 0; b < n; b++) ring[(pos + b) & MASK] = (uint8_t)byte_of(v, b);
}

// ---------------------------------------------------------- the decoder

struct Decoder {
  Smem &sm;
  uint32_t lane;
  uint32_t rbase;     // ring index of input position y = 0
  uint32_t y;         // input position (bytes from the 16-aligned block start)
  uint32_t y_end;
  uint32_t op;        // output position within the chunk
  uint32_t N;         // chunk's decoded size
  uint32_t avail;     // cached ctl.in_avail
  uint32_t flushed;   // cached: tiles below this * TILE are written out
  uint32_t wy;        // window start (multiple of 4); window = [wy, wy + 256)
  uint32_t win;       // this lane's dword of the window
  uint32_t used;      // last value published to ctl.in_used

  __device__ void need_input(uint32_t upto) {
    if (upto > y_end) upto = y_end;
    while (avail < upto) {
      avail = lds_get(&sm.ctl.in_avail);
      if (avail < upto) __builtin_amdgcn_s_sleep(1);
    }
  }

  // History positions below `end` may be written once the flushers are past
  // end - HIST (only chunks larger than the ring ever wait here).
  __device__ void need_ring(uint32_t end) {
    if (end <= HIST) return;
    uint32_t need = end - HIST;
    while (flushed < need) {
      uint32_t m = lds_get(&sm.ctl.next_tile[0]);
      for (int f = 1; f < NFLUSH; f++) {
        uint32_t t = lds_get(&sm.ctl.next_tile[f]);
        m = t < m ? t : m;
      }
      flushed = (m >= (0xFFFFFFFFu / TILE)) ? 0xFFFFFFFFu : m * TILE;
      if (flushed < need) __builtin_amdgcn_s_sleep(1);
    }
  }

  __device__ void load_window(uint32_t p) {
    wy = p & ~3u;
    // nothing before the window is read again: tokens, length bytes and
    // distances before p are parsed, and literal runs start at or after p
    if (wy > used) {
      used = wy;
      lds_put(&sm.ctl.in_used, used, lane);
    }
    need_input(wy + 256);
    win = *(const uint32_t *)(sm.inr + ((rbase + wy + 4 * lane) & IMASK));
  }

  // byte at input position p; the window must cover p
  __device__ uint32_t byte_at(uint32_t p) {
    if (p < wy || p >= wy + 256) load_window(p);
    uint32_t rel = p - wy;
    uint32_t d = __builtin_amdgcn_readlane(win, rel >> 2);
    return (d >> ((rel & 3) * 8)) & 0xFFu;
  }

  __device__ void publish_out() { lds_put(&sm.ctl.out_done, op, lane); }

  // copy n literal bytes from input position ys to history position od
  __device__ void copy_from_input(uint32_t ys, uint32_t od, uint32_t n) {
    for (uint32_t base = 0; base < n; base += 64 * 16) {
      uint32_t j = base + 16 * lane;
      if (j < n) {
        uint32_t cnt = n - j < 16 ? n - j : 16;
        uint32_t s = (rbase + ys + j) & IMASK;
        uint32_t d = (od + j) & HMASK;
        uint4 v = (s + 16 <= INR) ? lds_ld16(sm.inr + s) : ring_ld16<IMASK>(sm.inr, s);
        if (d + 16 <= HIST) lds_st_part(sm.hist + d, v, cnt);
        else ring_st_part<HMASK>(sm.hist, d, v, cnt);
      }
    }
  }

  // contiguous history copy: dst od.., src od - dist.., n bytes, where every
  // source byte is final before this call's first write of its 1 KiB step
  __device__ void copy_hist(uint32_t od, uint32_t dist, uint32_t n) {
    for (uint32_t base = 0; base < n; base += 64 * 16) {
      uint32_t j = base + 16 * lane;
      if (j < n) {
        uint32_t cnt = n - j < 16 ? n - j : 16;
        uint32_t s = (od + j - dist) & HMASK;
        uint32_t d = (od + j) & HMASK;
        uint4 v = (s + 16 <= HIST) ? lds_ld16(sm.hist + s) : ring_ld16<HMASK>(sm.hist, s);
        if (d + 16 <= HIST) lds_st_part(sm.hist + d, v, cnt);
        else ring_st_part<HMASK>(sm.hist, d, v, cnt);
      }
    }
  }

  __device__ void fill(uint32_t od, uint32_t byte, uint32_t n) {
    uint32_t w = byte * 0x01010101u;
    uint4 v = make_uint4(w, w, w, w);
    for (uint32_t base = 0; base < n; base += 64 * 16) {
      uint32_t j = base + 16 * lane;
      if (j < n) {
        uint32_t cnt = n - j < 16 ? n - j : 16;
        uint32_t d = (od + j) & HMASK;
        if (d + 16 <= HIST) lds_st_part(sm.hist + d, v, cnt);
        else ring_st_part<HMASK>(sm.hist, d, v, cnt);
      }
    }
  }

  // first min(M, 1 KiB) bytes of an overlapping match, byte by byte:
  // out[op + j] = out[op - dist + (j mod dist)]
  __device__ void copy_periodic_first(uint32_t od, uint32_t dist, uint32_t n) {
    uint32_t j = 16 * lane;
    if (j < n) {
      uint32_t cnt = n - j < 16 ? n - j : 16;
      uint32_t r = j % dist;
      uint32_t src0 = od - dist;
      uint32_t w[4];
#pragma unroll
      for (int k = 0; k < 4; k++) {
        w[k] = 0;
#pragma unroll
        for (int b = 0; b < 4; b++) {
          w[k] |= (uint32_t)sm.hist[(src0 + r) & HMASK] << (8 * b);
          r = (r + 1 == dist) ? 0 : r + 1;
        }
      }
      uint32_t d = (od + j) & HMASK;
      uint4 v = make_uint4(w[0], w[1], w[2], w[3]);
      if (d + 16 <= HIST) lds_st_part(sm.hist + d, v, cnt);
      else ring_st_part<HMASK>(sm.hist, d, v, cnt);
    }
  }

  __device__ void copy_match(uint32_t dist, uint32_t M) {
    // pieces keep the writes within what the ring can hold ahead of the flushers
    const uint32_t PIECE = 32768;
    if (dist == 1) {
      uint32_t b = sm.hist[(op - 1) & HMASK];
      b = __builtin_amdgcn_readfirstlane(b);
      while (M) {
        uint32_t n = M < PIECE ? M : PIECE;
        need_ring(op + n);
        fill(op, b, n);
        op += n;
        M -= n;
        publish_out();
      }
      return;
    }
    uint32_t done = 0;
    if (dist < M && dist < 1024) {
      uint32_t n = M < 1024 ? M : 1024;
      need_ring(op + n);
      copy_periodic_first(op, dist, n);
      op += n;
      done = n;
      publish_out();
      // later bytes repeat with any multiple of dist; the smallest multiple
      // >= 1 KiB keeps each 1 KiB step's sources before the step
      dist = dist * ((1024 + dist - 1) / dist);
    }
    while (done < M) {
      uint32_t n = M - done < PIECE ? M - done : PIECE;
      need_ring(op + n);
      copy_hist(op, dist, n);
      op += n;
      done += n;
      publish_out();
    }
  }

  // Returns the chunk status.
  __device__ int32_t run() {
    int32_t st = C_OK;
    for (;;) {
      if (y >= y_end) { st = C_TRUNC; break; }
      uint32_t token = byte_at(y);
      y++;
      uint32_t L = token >> 4;
      if (L == 15) {
        uint32_t b;
        do {
          if (y >= y_end) { st = C_TRUNC; goto out; }
          b = byte_at(y);
          y++;
          L += b;
          if (L > LEN_CAP) { st = C_OVERRUN; goto out; }
        } while (b == 255);
      }
      if (L > y_end - y) { st = C_TRUNC; break; }
      if (L > N - op) { st = C_OVERRUN; break; }
      while (L) {
        uint32_t piece = L < INR - 64 ? L : INR - 64;
        used = y;
        lds_put(&sm.ctl.in_used, used, lane);
        need_input(y + piece);
        need_ring(op + piece);
        copy_from_input(y, op, piece);
        y += piece;
        op += piece;
        L -= piece;
        publish_out();
      }
      if (y == y_end) break;
      if (y_end - y < 2) { st = C_TRUNC; break; }
      uint32_t dist = byte_at(y);
      dist |= byte_at(y + 1) << 8;
      y += 2;
      if (dist == 0 || dist > op) { st = C_BADOFF; break; }
      uint32_t M = (token & 15) + 4;
      if ((token & 15) == 15) {
        uint32_t b;
        do {
          if (y >= y_end) { st = C_TRUNC; goto out; }
          b = byte_at(y);
          y++;
          M += b;
          if (M > LEN_CAP) { st = C_OVERRUN; goto out; }
        } while (b == 255);
      }
      if (M > N - op) { st = C_OVERRUN; break; }
      copy_match(dist, M);
      used = y;
      lds_put(&sm.ctl.in_used, used, lane);
    }
  out:
    if (st == C_OK && op != N) st = C_SIZE;
    return st;
  }
};

// -------------------------------------------------------------- feeder

__device__ void feeder(Smem &sm, uint32_t lane, const uint8_t *S, uint32_t rbase, uint32_t y_end) {
  constexpr int FU = 4;   // 16-byte blocks per lane per batch (4 KiB per batch)
  uint32_t nblk = (y_end + 15) / 16;
  uint32_t next = 0;
  while (next < nblk) {
    uint32_t used = lds_get(&sm.ctl.in_used);
    uint32_t state = lds_get(&sm.ctl.state);
    if (state != ST_RUN) break;
    uint32_t limit = ((used & ~15u) + INR) / 16;
    if (limit > nblk) limit = nblk;
    if (limit <= next) {
      __builtin_amdgcn_s_sleep(1);
      continue;
    }
    uint32_t cnt = limit - next;
    if (cnt > 64u * FU) cnt = 64u * FU;
    // every lane loads FU blocks (indices clamped into the batch, so all loads
    // are issued back to back and read only blocks of this chunk), then the
    // lanes whose blocks are in the batch write them to the ring
    const uint32_t last = next + cnt - 1;
    uint32_t b0 = next + lane, b1 = b0 + 64, b2 = b0 + 128, b3 = b0 + 192;
    uint4 v0 = *(const uint4 *)(S + 16ull * (b0 < last ? b0 : last));
    uint4 v1 = *(const uint4 *)(S + 16ull * (b1 < last ? b1 : last));
    uint4 v2 = *(const uint4 *)(S + 16ull * (b2 < last ? b2 : last));
    uint4 v3 = *(const uint4 *)(S + 16ull * (b3 < last ? b3 : last));
    if (b0 <= last) *(uint4 *)(sm.inr + ((rbase + 16 * b0) & IMASK)) = v0;
    if (b1 <= last) *(uint4 *)(sm.inr + ((rbase + 16 * b1) & IMASK)) = v1;
    if (b2 <= last) *(uint4 *)(sm.inr + ((rbase + 16 * b2) & IMASK)) = v2;
    if (b3 <= last) *(uint4 *)(sm.inr + ((rbase + 16 * b3) & IMASK)) = v3;
    next += cnt;
    lds_put(&sm.ctl.in_avail, next * 16, lane);
  }
}

// ------------------------------------------------------------- flushers

template <int MODE>
__device__ void flush_tile(Smem &sm, uint32_t lane, const ChunkParams &P, uint64_t dst0,
                           uint32_t t, uint32_t N) {
  uint32_t base = t * TILE;
  if constexpr (MODE == MODE_BYTES) {
    uint8_t *out = (uint8_t *)P.out + dst0;
    uint32_t p = base + 16 * lane;
    if (p < N) {
      uint4 v = *(const uint4 *)(sm.hist + (p & HMASK));
      if (p + 16 <= N) {
        *(uint4 *)(out + p) = v;
      } else {
        for (uint32_t b = 0; b < N - p; b++) out[p + b] = (uint8_t)byte_of(v, b);
      }
    }
  } else if constexpr (MODE == MODE_INT4) {
    uint16_t *out = (uint16_t *)P.out;
    const uint64_t G = P.group;
#pragma unroll
    for (int k = 0; k < 4; k++) {
      uint32_t p = base + 256 * k + 4 * lane;
      if (p < N) {
        uint32_t w = *(const uint32_t *)(sm.hist + (p & HMASK));
        uint64_t e0 = 2 * (dst0 + p);
        uint32_t nb = N - p < 4 ? N - p : 4;
        uint64_t g0 = e0 / G, g1 = (e0 + 2 * nb - 1) / G;
        if (nb == 4 && g0 == g1) {
          uint16_t sb = P.scales[g0];
          int z = P.zp ? (int)P.zp[g0] : 0;
          uint4 r = deq8_int4(w, splat_h2((uint16_t)f16_bits_1024_plus(z)), splat_h2(sb));
          *(uint4 *)(out + e0) = r;
        } else {
          for (uint32_t c = 0; c < 2 * nb; c++) {
            uint64_t e = e0 + c;
            uint64_t g = e / G;
            int q = (w >> (4 * c)) & 15;
            int z = P.zp ? (int)P.zp[g] : 0;
            out[e] = deq1(q, z, P.scales[g]);
          }
        }
      }
    }
  } else {  // MODE_INT8
    uint16_t *out = (uint16_t *)P.out;
    const uint64_t G = P.group;
#pragma unroll
    for (int k = 0; k < 2; k++) {
      uint32_t p = base + 512 * k + 8 * lane;
      if (p < N) {
        uint2 w = *(const uint2 *)(sm.hist + (p & HMASK));
        uint64_t e0 = dst0 + p;
        uint32_t nb = N - p < 8 ? N - p : 8;
        uint64_t g0 = e0 / G, g1 = (e0 + nb - 1) / G;
        if (nb == 8 && g0 == g1) {
          uint16_t sb = P.scales[g0];
          int z = P.zp ? (int)P.zp[g0] : 0;
          h2 c2 = splat_h2((uint16_t)f16_bits_1024_plus(128 + z)), s2 = splat_h2(sb);
          uint2 a = deq4_int8(w.x, c2, s2), b = deq4_int8(w.y, c2, s2);
          *(uint4 *)(out + e0) = make_uint4(a.x, a.y, b.x, b.y);
        } else {
          for (uint32_t c = 0; c < nb; c++) {
            uint64_t e = e0 + c;
            uint64_t g = e / G;
            int q = (int)(int8_t)byte_of(make_uint4(w.x, w.y, 0, 0), c);
            int z = P.zp ? (int)P.zp[g] : 0;
            out[e] = deq1(q, z, P.scales[g]);
          }
        }
      }
    }
  }
}

template <int MODE>
__device__ void flusher(Smem &sm, uint32_t lane, uint32_t f, const ChunkParams &P, uint64_t dst0,
                        uint32_t N) {
  uint32_t ntiles = (N + TILE - 1) / TILE;
  uint32_t done = 0;
  for (uint32_t t = f; t < ntiles; t += NFLUSH) {
    uint32_t t_end = (t + 1) * TILE < N ? (t + 1) * TILE : N;
    while (done < t_end) {
      done = lds_get(&sm.ctl.out_done);
      if (done >= t_end) break;
      if (lds_get(&sm.ctl.state) != ST_RUN) {
        done = lds_get(&sm.ctl.out_done);
        if (done >= t_end) break;
        goto finish;   // the decoder stopped short of this tile (failed chunk)
      }
      __builtin_amdgcn_s_sleep(1);
    }
    flush_tile<MODE>(sm, lane, P, dst0, t, N);
    lds_put(&sm.ctl.next_tile[f], t + NFLUSH, lane);
  }
finish:
  lds_put(&sm.ctl.next_tile[f], 0xFFFFFFFFu, lane);
}

// -------------------------------------------------------------- kernel

template <int MODE>
__global__ void __launch_bounds__(NTHREADS) chunk_kernel(ChunkParams P) {
  __shared__ Smem sm;
  const uint32_t i = blockIdx.x;
  const uint32_t tid = threadIdx.x;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const uint32_t lane = tid & 63;

  uint64_t c0 = P.comp_off[i], c1 = P.comp_off[i + 1];
  uint64_t d0 = P.dst_off[i], d1 = P.dst_off[i + 1];
  bool bad = c0 > c1 || c1 > P.comp_bytes || d0 > d1 || d1 > P.total ||
             (i == 0 && d0 != 0) || (i == P.n - 1 && d1 != P.total) || (d0 & 15) != 0 ||
             d1 - d0 > (uint64_t)P.max_chunk || c1 - c0 > (uint64_t)LEN_CAP;
  if (bad) {
    if (tid == 0 && P.status) P.status[i] = C_TABLE;
    return;
  }
  const uint32_t N = (uint32_t)(d1 - d0);
  // the feeder reads whole 16-byte aligned blocks covering the chunk's bytes
  // (an aligned block never crosses a page, so it is always mapped)
  const uint32_t head = (uint32_t)((uintptr_t)(P.comp + c0) & 15);
  const uint8_t *S = P.comp + (c0 - head);
  const uint32_t rbase = (uint32_t)((uintptr_t)S & IMASK);
  const uint32_t y_end = head + (uint32_t)(c1 - c0);

  if (tid == 0) {
    sm.ctl.in_avail = 0;
    sm.ctl.in_used = 0;
    sm.ctl.out_done = 0;
    sm.ctl.state = ST_RUN;
    for (int f = 0; f < NFLUSH; f++) sm.ctl.next_tile[f] = f;
    sm.ctl.status = 0;
  }
  __syncthreads();

  if (wave == 0) {
    Decoder D{sm, lane, rbase, head, y_end, 0, N, 0, 0, 0xFFFFFF00u, 0, 0};
    int32_t st = (y_end == head) ? C_TRUNC : D.run();
    D.publish_out();
    if (lane == 0) sm.ctl.status = st;
    lds_put(&sm.ctl.state, st == C_OK ? ST_DONE : ST_FAIL, lane);
  } else if (wave == 1) {
    feeder(sm, lane, S, rbase, y_end);
  } else {
    flusher<MODE>(sm, lane, wave - 2, P, d0, N);
  }
  __syncthreads();
  if (tid == 0 && P.status) P.status[i] = sm.ctl.status;
}

}  // namespace lt
