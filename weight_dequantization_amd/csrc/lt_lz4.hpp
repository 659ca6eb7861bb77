// lt_lz4.hpp -- chunk-parallel LZ4 block decoding on gfx950, one workgroup
// per independently compressed chunk, with three wave roles:
//
//   wave 0  decoder : parses the block's sequences and materializes the
//                     decoded bytes into a 64 KiB LDS history ring (literal
//                     copies from the input ring, match copies from history);
//   wave 1  feeder  : streams the chunk's compressed bytes from HBM into an
//                     8 KiB LDS input ring with LDS-DMA loads
//                     (global_load_lds_dwordx4), several 1 KiB segments in
//                     flight;
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
// LDS traffic is kept to naturally aligned accesses: every lane owns an
// aligned 16-byte block of the destination, gathers its source bytes with
// aligned dword reads and v_alignbyte, and writes the partial blocks at the
// ends of a copy with aligned byte / half / dword stores (no read-modify-
// write).  The decoder reads the next parse window together with a
// sequence's literal bytes, so a typical sequence costs one LDS round trip.
//
// The roles talk through LDS counters (relaxed atomics, published only after
// an lgkmcnt(0) / vmcnt wait, so the data they announce is already in LDS):
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
constexpr uint32_t SEG = 1024;        // feeder unit: one 16-byte DMA load per lane
constexpr uint32_t QMAX = INR / SEG;  // segments in flight at most
constexpr uint32_t TILE = 1024;       // flush granularity (bytes of decoded stream)
constexpr int NFLUSH = 2;
constexpr int NWAVES = 2 + NFLUSH;
constexpr int NTHREADS = 64 * NWAVES;
constexpr uint32_t LEN_CAP = 1u << 31;
constexpr uint32_t LIT_ONE_STEP = 960;  // literal runs copied with one gather step

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
  uint32_t group_shift;      // log2(group) when group is a power of two, else 64
};

// ------------------------------------------------------------ LDS sync

__device__ __forceinline__ void wait_lds() { __builtin_amdgcn_s_waitcnt(0xC07F); }  // lgkmcnt(0)

// vmcnt(k), leaving expcnt and lgkmcnt unconstrained (gfx9 encoding)
template <int K>
__device__ __forceinline__ void wait_vm() {
  static_assert(K >= 0 && K < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((K & 15) | ((K >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ void wait_vm_le(uint32_t k) {
  switch (k) {
    case 0: wait_vm<0>(); break;
    case 1: wait_vm<1>(); break;
    case 2: wait_vm<2>(); break;
    case 3: wait_vm<3>(); break;
    case 4: wait_vm<4>(); break;
    case 5: wait_vm<5>(); break;
    case 6: wait_vm<6>(); break;
    default: wait_vm<7>(); break;
  }
}

__device__ __forceinline__ uint32_t lds_get(uint32_t *p) {
  uint32_t v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  return __builtin_amdgcn_readfirstlane(v);
}

__device__ __forceinline__ void lds_set(uint32_t *p, uint32_t v, uint32_t lane) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  if (lane == 0) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// The feeder's counter accesses go through inline asm: its LDS-DMA loads
// would otherwise make the compiler wait for every load in flight before any
// LDS access of that wave.  Each read waits for its own result inside the asm
// block, so its output register is final when the block ends.
__device__ __forceinline__ uint32_t lds_addr(const uint32_t *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) uint32_t *)p;
}

__device__ __forceinline__ uint32_t lds_get_asm(const uint32_t *p) {
  uint32_t v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_addr(p)) : "memory");
  return __builtin_amdgcn_readfirstlane(v);
}

__device__ __forceinline__ void lds_set_asm(uint32_t *p, uint32_t v, uint32_t lane) {
  if (lane == 0) asm volatile("ds_write_b32 %0, %1" : : "v"(lds_addr(p)), "v"(v) : "memory");
}

// Publish a counter after this wave's earlier LDS operations have completed.
__device__ __forceinline__ void lds_put(uint32_t *p, uint32_t v, uint32_t lane) {
  wait_lds();
  lds_set(p, v, lane);
}

// ------------------------------------------------------ LDS byte moves

// 16 bytes starting at ring index si (any alignment), from five aligned
// dword reads; ring sizes are multiples of 4, so no read straddles the end.
template <uint32_t MASK>
__device__ __forceinline__ uint4 gather16(const uint8_t *ring, uint32_t si) {
  const uint32_t *r = (const uint32_t *)ring;
  uint32_t a = si & ~3u, sh = si & 3u;
  uint32_t d0 = r[(a & MASK) >> 2];
  uint32_t d1 = r[((a + 4) & MASK) >> 2];
  uint32_t d2 = r[((a + 8) & MASK) >> 2];
  uint32_t d3 = r[((a + 12) & MASK) >> 2];
  uint32_t d4 = r[((a + 16) & MASK) >> 2];
  return make_uint4(__builtin_amdgcn_alignbyte(d1, d0, sh), __builtin_amdgcn_alignbyte(d2, d1, sh),
                    __builtin_amdgcn_alignbyte(d3, d2, sh), __builtin_amdgcn_alignbyte(d4, d3, sh));
}

// bytes [lo, hi) of dword d, which sits at p + base (base multiple of 4)
__device__ __forceinline__ void st_dword_part(uint8_t *p, uint32_t d, uint32_t base, uint32_t lo,
                                              uint32_t hi) {
  uint32_t s = lo > base ? lo : base;
  uint32_t e = hi < base + 4 ? hi : base + 4;
  if (s >= e) return;
  if (s == base && e == base + 4) {
    *(uint32_t *)(p + base) = d;
    return;
  }
  uint32_t x = d >> (8 * (s - base));
  if (s & 1) {
    p[s] = (uint8_t)x;
    s++;
    x >>= 8;
  }
  if (e - s >= 2) {
    *(uint16_t *)(p + s) = (uint16_t)x;
    s += 2;
    x >>= 16;
  }
  if (s < e) p[s] = (uint8_t)x;
}

// bytes [lo, hi) (0 <= lo < hi <= 16) of v into the 16-byte aligned block p,
// with naturally aligned stores only
__device__ __forceinline__ void st_block(uint8_t *p, uint4 v, uint32_t lo, uint32_t hi) {
  if (lo == 0 && hi == 16) {
    *(uint4 *)p = v;
    return;
  }
  st_dword_part(p, v.x, 0, lo, hi);
  st_dword_part(p, v.y, 4, lo, hi);
  st_dword_part(p, v.z, 8, lo, hi);
  st_dword_part(p, v.w, 12, lo, hi);
}

// ---------------------------------------------------------- the decoder

struct Decoder {
  Smem &sm;
  Ctl &ctl;
  uint32_t lane;
  uint32_t y;          // input position (bytes from the 16-aligned block start)
  uint32_t y_end;
  uint32_t op;         // output position within the chunk
  uint32_t N;          // chunk's decoded size
  uint32_t avail;      // cached ctl.in_avail
  uint32_t flushed;    // cached: history below this is written out
  uint32_t wy;         // window start (multiple of 4); window = [wy, wy + 256)
  uint32_t win;        // this lane's dword of the window
  uint32_t used;       // last value published to ctl.in_used
  uint32_t last_byte;  // the decoded byte at op - 1
  uint4 cur;           // the 16-byte block holding op; bytes below op are final

  // While every position written so far is below HIST (the first pass
  // through the ring), copies write whole aligned blocks: bytes past a copy's
  // end are future positions, rewritten before any match or flush reads
  // them.  Past that point a block may still hold bytes a long match needs,
  // so copies write exactly their own bytes.
  __device__ bool whole_blocks(uint32_t end) const { return end + 15 <= HIST; }

  static __device__ __forceinline__ uint4 readlane4(uint4 v, uint32_t l) {
    return make_uint4(__builtin_amdgcn_readlane(v.x, l), __builtin_amdgcn_readlane(v.y, l),
                      __builtin_amdgcn_readlane(v.z, l), __builtin_amdgcn_readlane(v.w, l));
  }

  // bytes [0, keep) from c, the rest from v (keep = 0 leaves v unchanged)
  static __device__ __forceinline__ uint4 merge_head(uint4 c, uint4 v, uint32_t keep) {
    uint32_t m[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
      uint32_t k = keep > 4u * j ? keep - 4u * j : 0u;
      m[j] = k >= 4 ? 0xFFFFFFFFu : ((1u << (8 * k)) - 1u);
    }
    return make_uint4((c.x & m[0]) | (v.x & ~m[0]),
                      (c.y & m[1]) | (v.y & ~m[1]), (c.z & m[2]) | (v.z & ~m[2]),
                      (c.w & m[3]) | (v.w & ~m[3]));
  }

  // Whole-block copy of history [od, od + n): block P's bytes come from
  // src(P); the head block keeps cur's bytes below od.  Each 64-block step
  // reads all its sources before writing.  Leaves cur / last_byte at the end.
  template <class Src>
  __device__ void put_blocks(uint32_t od, uint32_t n, Src src) {
    const uint32_t A = od & ~15u, end = od + n, keep = od & 15u;
    const uint32_t nb = (end - A + 15) >> 4;
    uint4 last = cur;
    for (uint32_t b0 = 0; b0 < nb; b0 += 64) {
      const uint32_t b = b0 + lane;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (b < nb) v = src(A + 16 * b);
      v = merge_head(cur, v, b == 0 ? keep : 0u);
      if (b < nb) *(uint4 *)(sm.hist + A + 16 * b) = v;
      const uint32_t lb = nb - 1 - b0;
      if (lb < 64) last = readlane4(v, lb);
    }
    cur = last;
    const uint32_t q = (end - 1) & 15u;
    const uint32_t d = q < 4 ? last.x : q < 8 ? last.y : q < 12 ? last.z : last.w;
    last_byte = (d >> (8 * (q & 3))) & 0xFFu;
  }

  __device__ void need_input(uint32_t upto) {
    if (upto > y_end) upto = y_end;
    while (avail < upto) {
      avail = lds_get(&ctl.in_avail);
      if (avail < upto) __builtin_amdgcn_s_sleep(1);
    }
  }

  // History positions below `end` may be written once the flushers are past
  // end - HIST (only chunks larger than the ring ever wait here).
  __device__ void need_ring(uint32_t end) {
    if (end <= HIST) return;
    uint32_t need = end - HIST;
    while (flushed < need) {
      uint32_t m = lds_get(&ctl.next_tile[0]);
      for (int f = 1; f < NFLUSH; f++) {
        uint32_t t = lds_get(&ctl.next_tile[f]);
        m = t < m ? t : m;
      }
      flushed = (m >= (0xFFFFFFFFu / TILE)) ? 0xFFFFFFFFu : m * TILE;
      if (flushed < need) __builtin_amdgcn_s_sleep(1);
    }
  }

  // Announce progress; cheap right after a wait that already completed this
  // wave's earlier LDS operations.
  __device__ void publish(uint32_t new_used) {
    wait_lds();
    lds_set(&ctl.out_done, op, lane);
    if (new_used > used) {
      used = new_used;
      lds_set(&ctl.in_used, used, lane);
    }
  }

  __device__ void load_window(uint32_t p) {
    wy = p & ~3u;
    // nothing before the window is read again: tokens, length bytes and
    // distances before p are parsed, and literal runs start at or after p
    if (wy > used) {
      used = wy;
      lds_put(&ctl.in_used, used, lane);
    }
    need_input(wy + 256);
    win = *(const uint32_t *)(sm.inr + ((wy + 4 * lane) & IMASK));
    // wait here, on this path only: otherwise the compiler waits at every
    // byte_at for all outstanding LDS writes, whether the window reloaded or not
    wait_lds();
  }

  // byte at input position p (reloads the window when p is outside it)
  __device__ uint32_t byte_at(uint32_t p) {
    if (p < wy || p >= wy + 256) load_window(p);
    uint32_t rel = p - wy;
    uint32_t d = __builtin_amdgcn_readlane(win, rel >> 2);
    return (d >> ((rel & 3) * 8)) & 0xFFu;
  }

  // history [od, od + n) from ring R at index src0 + (P - od); every source
  // byte is final before each 64-block step writes
  template <uint32_t MASK>
  __device__ void copy_blocks(const uint8_t *R, uint32_t src0, uint32_t od, uint32_t n) {
    const uint32_t A = od & ~15u, end = od + n;
    const uint32_t nb = (end - A + 15) >> 4;
    for (uint32_t b0 = 0; b0 < nb; b0 += 64) {
      uint32_t b = b0 + lane;
      if (b < nb) {
        uint32_t P = A + 16 * b;
        uint32_t lo = od > P ? od - P : 0;
        uint32_t hi = end - P < 16 ? end - P : 16;
        uint4 v = gather16<MASK>(R, src0 + (P - od));
        st_block(sm.hist + (P & HMASK), v, lo, hi);
      }
    }
  }

  __device__ void fill(uint32_t od, uint32_t byte, uint32_t n) {
    const uint32_t w = byte * 0x01010101u;
    const uint4 v = make_uint4(w, w, w, w);
    const uint32_t A = od & ~15u, end = od + n;
    const uint32_t nb = (end - A + 15) >> 4;
    for (uint32_t b = lane; b < nb; b += 64) {
      uint32_t P = A + 16 * b;
      uint32_t lo = od > P ? od - P : 0;
      uint32_t hi = end - P < 16 ? end - P : 16;
      st_block(sm.hist + (P & HMASK), v, lo, hi);
    }
  }

  // the first n (<= 1 KiB) bytes of an overlapping match, byte by byte:
  // out[od + j] = out[od - dist + (j mod dist)]
  __device__ void copy_periodic(uint32_t od, uint32_t dist, uint32_t n) {
    const uint32_t A = od & ~15u, end = od + n;
    const uint32_t nb = (end - A + 15) >> 4;
    for (uint32_t b = lane; b < nb; b += 64) {
      uint32_t P = A + 16 * b;
      uint32_t lo = od > P ? od - P : 0;
      uint32_t hi = end - P < 16 ? end - P : 16;
      uint32_t r = (P + lo - od) % dist;
      uint32_t w0 = 0, w1 = 0, w2 = 0, w3 = 0;
#pragma unroll
      for (uint32_t q = 0; q < 16; q++) {
        if (q >= lo && q < hi) {
          uint32_t v = sm.hist[(od - dist + r) & HMASK];
          uint32_t sv = v << (8 * (q & 3));
          if (q < 4) w0 |= sv;
          else if (q < 8) w1 |= sv;
          else if (q < 12) w2 |= sv;
          else w3 |= sv;
          r = (r + 1 == dist) ? 0 : r + 1;
        }
      }
      st_block(sm.hist + (P & HMASK), make_uint4(w0, w1, w2, w3), lo, hi);
    }
  }

  __device__ void copy_match(uint32_t dist, uint32_t M) {
    // pieces keep the writes within what the ring can hold ahead of the flushers
    const uint32_t PIECE = 32768;
    if (dist == 1) {
      const uint32_t w = last_byte * 0x01010101u;
      while (M) {
        uint32_t n = M < PIECE ? M : PIECE;
        need_ring(op + n);
        if (whole_blocks(op + n)) put_blocks(op, n, [&](uint32_t) { return make_uint4(w, w, w, w); });
        else fill(op, last_byte, n);
        op += n;
        M -= n;
        if (M) publish(used);
      }
      return;
    }
    uint32_t done = 0;
    bool exact = false;
    if (dist < M && dist < 1024) {
      uint32_t n = M < 1024 ? M : 1024;
      need_ring(op + n);
      if (whole_blocks(op + n)) {
        const uint32_t od = op;
        put_blocks(od, n, [&](uint32_t P) {
          uint32_t lo = od > P ? od - P : 0;
          uint32_t r = (P + lo - od) % dist;
          uint32_t w0 = 0, w1 = 0, w2 = 0, w3 = 0;
#pragma unroll
          for (uint32_t q = 0; q < 16; q++) {
            if (q >= lo) {
              uint32_t sv = (uint32_t)sm.hist[(od - dist + r) & HMASK] << (8 * (q & 3));
              if (q < 4) w0 |= sv;
              else if (q < 8) w1 |= sv;
              else if (q < 12) w2 |= sv;
              else w3 |= sv;
              r = (r + 1 == dist) ? 0 : r + 1;
            }
          }
          return make_uint4(w0, w1, w2, w3);
        });
      } else {
        copy_periodic(op, dist, n);
        exact = true;
      }
      op += n;
      done = n;
      publish(used);
      // later bytes repeat with any multiple of dist; the smallest multiple
      // >= 1 KiB keeps each 1 KiB step's sources before the step
      dist = dist * ((1024 + dist - 1) / dist);
    }
    while (done < M) {
      uint32_t n = M - done < PIECE ? M - done : PIECE;
      need_ring(op + n);
      if (whole_blocks(op + n)) {
        const uint32_t dd = dist;
        put_blocks(op, n, [&](uint32_t P) { return gather16<HMASK>(sm.hist, P - dd); });
      } else {
        copy_blocks<HMASK>(sm.hist, op - dist, op, n);
        exact = true;
      }
      op += n;
      done += n;
      if (done < M) publish(used);
    }
    if (exact) last_byte = __builtin_amdgcn_readfirstlane(sm.hist[(op - 1) & HMASK]);
  }

  // literal run of L bytes at input y: copy, advance y / op, and leave the
  // window covering the bytes that follow
  __device__ void literals(uint32_t L) {
    const uint32_t ye = y + L;
    if (L <= LIT_ONE_STEP && whole_blocks(op + L)) {
      const uint32_t nw = ye & ~3u;
      need_input((ye > nw + 256) ? ye : nw + 256);
      const uint32_t A = op & ~15u, end = op + L, keep = op & 15u;
      const uint32_t nb = (end - A + 15) >> 4;   // <= 62
      const uint32_t P = A + 16 * lane;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (lane < nb) v = gather16<IMASK>(sm.inr, y + (P - op));
      const uint32_t nwin = *(const uint32_t *)(sm.inr + ((nw + 4 * lane) & IMASK));
      publish(y);   // waits for the reads above (and so for every earlier write)
      v = merge_head(cur, v, lane == 0 ? keep : 0u);
      if (lane < nb) *(uint4 *)(sm.hist + P) = v;
      cur = readlane4(v, nb - 1);
      const uint32_t q = (end - 1) & 15u;
      const uint32_t d = q < 4 ? cur.x : q < 8 ? cur.y : q < 12 ? cur.z : cur.w;
      last_byte = (d >> (8 * (q & 3))) & 0xFFu;
      win = nwin;
      wy = nw;
      y = ye;
      op += L;
      return;
    }
    uint32_t left = L;
    bool exact = false;
    while (left) {
      // the feeder fills whole segments up to QMAX past the segment holding
      // `used`, so a piece of INR - 2 * SEG bytes is always deliverable
      uint32_t piece = left < INR - 2 * SEG ? left : INR - 2 * SEG;
      used = y;
      lds_put(&ctl.in_used, used, lane);
      need_input(y + piece);
      need_ring(op + piece);
      if (whole_blocks(op + piece)) {
        const uint32_t ys = y, od = op;
        put_blocks(op, piece, [&](uint32_t Pb) { return gather16<IMASK>(sm.inr, ys + (Pb - od)); });
      } else {
        copy_blocks<IMASK>(sm.inr, y, op, piece);
        exact = true;
      }
      y += piece;
      op += piece;
      left -= piece;
      publish(used);
    }
    if (exact) last_byte = byte_at(ye - 1);
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
      if (L) literals(L);
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
    }
  out:
    if (st == C_OK && op != N) st = C_SIZE;
    return st;
  }
};

// -------------------------------------------------------------- feeder

// Streams the chunk's 16-byte aligned blocks into the input ring, one 1 KiB
// segment (one LDS-DMA load per lane) at a time, keeping up to QMAX segments
// in flight within the ring space the decoder has released.
__device__ void feeder(Smem &sm, Ctl &ctl, uint32_t lane, const uint8_t *S, uint32_t y_end) {
  const uint32_t nblk = (y_end + 15) / 16;
  const uint32_t nseg = (y_end + SEG - 1) / SEG;
  uint32_t issued = 0, landed = 0;
  while (landed < nseg) {
    if (lds_get_asm(&ctl.state) != ST_RUN) break;
    uint32_t used = lds_get_asm(&ctl.in_used);
    uint32_t limit = used / SEG + QMAX;
    if (limit > nseg) limit = nseg;
    while (issued < limit && issued - landed < QMAX) {
      uint32_t blk = issued * (SEG / 16) + lane;
      if (blk >= nblk) blk = nblk - 1;   // stay within the chunk's blocks
      __builtin_amdgcn_global_load_lds((const void *)(S + 16ull * blk),
                                       (__attribute__((address_space(3))) void *)(sm.inr + ((issued * SEG) & IMASK)),
                                       16, 0, 0);
      issued++;
    }
    if (issued == landed) {
      __builtin_amdgcn_s_sleep(1);
      continue;
    }
    wait_vm_le(issued - landed - 1);   // the oldest segment in flight has landed
    landed++;
    lds_set_asm(&ctl.in_avail, landed * SEG, lane);
  }
  wait_vm<0>();   // no LDS-DMA write outlives this wave
}

// ------------------------------------------------------------- flushers

struct Meta4 {
  uint32_t s[4];
  uint32_t z[4];
};

// scales / zero points of one INT4 tile (fast path: group is a power of two
// >= 8, so each lane's 8 codes share one group).  The loads are issued here
// and consumed only after the wait for the tile (see meta_ready).
__device__ __forceinline__ Meta4 int4_meta(const ChunkParams &P, uint64_t dst0, uint32_t t,
                                           uint32_t lane, uint32_t N) {
  Meta4 m;
  // without zero points, read any valid byte and discard it (no branch)
  const int8_t *zsrc = P.zp ? P.zp : (const int8_t *)P.scales;
#pragma unroll
  for (int k = 0; k < 4; k++) {
    uint32_t p = t * TILE + 256 * k + 4 * lane;
    if (p >= N) p = 0;   // any valid group; unused
    uint64_t g = (2 * (dst0 + p)) >> P.group_shift;
    m.s[k] = P.scales[g];
    m.z[k] = (uint32_t)(int32_t)zsrc[g];
  }
  return m;
}

// Make the tile's scale registers opaque here, so the compiler consumes (and
// waits for) them at this point instead of right after issuing the loads.
__device__ __forceinline__ void meta_ready(Meta4 &m, bool has_zp) {
#pragma unroll
  for (int k = 0; k < 4; k++) {
    asm volatile("" : "+v"(m.s[k]), "+v"(m.z[k]));
    if (!has_zp) m.z[k] = 0;
  }
}

template <int MODE>
__device__ void flush_tile(Smem &sm, uint32_t lane, const ChunkParams &P, uint64_t dst0,
                           uint32_t t, uint32_t N, const Meta4 &m, bool fast) {
  uint32_t base = t * TILE;
  if constexpr (MODE == MODE_BYTES) {
    uint8_t *out = (uint8_t *)P.out + dst0;
    uint32_t p = base + 16 * lane;
    if (p < N) {
      uint4 v = *(const uint4 *)(sm.hist + (p & HMASK));
      if (p + 16 <= N) {
        *(uint4 *)(out + p) = v;
      } else {
#pragma unroll
        for (uint32_t b = 0; b < 16; b++) {
          uint32_t d = b < 4 ? v.x : b < 8 ? v.y : b < 12 ? v.z : v.w;
          if (p + b < N) out[p + b] = (uint8_t)(d >> ((b & 3) * 8));
        }
      }
    }
  } else if constexpr (MODE == MODE_INT4) {
    uint16_t *out = (uint16_t *)P.out;
    const uint64_t G = P.group;
    uint32_t w[4];
#pragma unroll
    for (int k = 0; k < 4; k++) {
      uint32_t p = base + 256 * k + 4 * lane;
      w[k] = (p < N) ? *(const uint32_t *)(sm.hist + (p & HMASK)) : 0u;
    }
#pragma unroll
    for (int k = 0; k < 4; k++) {
      uint32_t p = base + 256 * k + 4 * lane;
      if (p >= N) continue;
      uint64_t e0 = 2 * (dst0 + p);
      if (fast && p + 4 <= N) {
        uint4 r = deq8_int4(w[k], splat_h2((uint16_t)f16_bits_1024_plus((int)m.z[k])),
                            splat_h2((uint16_t)m.s[k]));
        *(uint4 *)(out + e0) = r;
      } else {
        uint32_t nb = N - p < 4 ? N - p : 4;
        for (uint32_t c = 0; c < 2 * nb; c++) {
          uint64_t e = e0 + c;
          uint64_t g = e / G;
          int q = (w[k] >> (4 * c)) & 15;
          int z = P.zp ? (int)P.zp[g] : 0;
          out[e] = deq1(q, z, P.scales[g]);
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
            uint32_t word = c < 4 ? w.x : w.y;
            int q = (int)(int8_t)(word >> ((c & 3) * 8));
            int z = P.zp ? (int)P.zp[g] : 0;
            out[e] = deq1(q, z, P.scales[g]);
          }
        }
      }
    }
  }
}

template <int MODE>
__device__ void flusher(Smem &sm, Ctl &ctl, uint32_t lane, uint32_t f, const ChunkParams &P,
                        uint64_t dst0, uint32_t N) {
  const uint32_t ntiles = (N + TILE - 1) / TILE;
  const bool fast = MODE == MODE_INT4 && P.group_shift < 64 && P.group >= 8;
  uint32_t done = 0;
  for (uint32_t t = f; t < ntiles; t += NFLUSH) {
    // the tile's scales are fetched before waiting for the tile, so their
    // latency overlaps the wait for the decoder
    Meta4 cur{};
    if (fast) cur = int4_meta(P, dst0, t, lane, N);
    uint32_t t_end = (t + 1) * TILE < N ? (t + 1) * TILE : N;
    while (done < t_end) {
      done = lds_get(&ctl.out_done);
      if (done >= t_end) break;
      if (lds_get(&ctl.state) != ST_RUN) {
        done = lds_get(&ctl.out_done);
        if (done >= t_end) break;
        goto finish;   // the decoder stopped short of this tile (failed chunk)
      }
      __builtin_amdgcn_s_sleep(1);
    }
    if (fast) meta_ready(cur, P.zp != nullptr);
    flush_tile<MODE>(sm, lane, P, dst0, t, N, cur, fast);
    lds_put(&ctl.next_tile[f], t + NFLUSH, lane);
  }
finish:
  lds_put(&ctl.next_tile[f], 0xFFFFFFFFu, lane);
}

// -------------------------------------------------------------- kernel

template <int MODE>
__global__ void __launch_bounds__(NTHREADS) chunk_kernel(ChunkParams P) {
  __shared__ __attribute__((aligned(16))) Smem sm;
  __shared__ Ctl ctl;
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
  const uint32_t y_end = head + (uint32_t)(c1 - c0);

  if (tid == 0) {
    ctl.in_avail = 0;
    ctl.in_used = 0;
    ctl.out_done = 0;
    ctl.state = ST_RUN;
    for (int f = 0; f < NFLUSH; f++) ctl.next_tile[f] = f;
    ctl.status = 0;
  }
  __syncthreads();

  if (wave == 0) {
    Decoder D{sm, ctl, lane, head, y_end, 0, N, 0, 0, 0xFFFFFF00u, 0, 0, 0, make_uint4(0, 0, 0, 0)};
    int32_t st = (y_end == head) ? C_TRUNC : D.run();
    D.publish(D.used);
    if (lane == 0) ctl.status = st;
    lds_put(&ctl.state, st == C_OK ? ST_DONE : ST_FAIL, lane);
  } else if (wave == 1) {
    feeder(sm, ctl, lane, S, y_end);
  } else {
    flusher<MODE>(sm, ctl, lane, wave - 2, P, d0, N);
  }
  __syncthreads();
  if (tid == 0 && P.status) P.status[i] = ctl.status;
}

}  // namespace lt
