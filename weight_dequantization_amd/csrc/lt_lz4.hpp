// lt_lz4.hpp -- chunk-parallel LZ4 block decoding on gfx950, one workgroup
// per independently compressed chunk, with four wave roles that form a
// pipeline through LDS:
//
//   wave 0  walker  : the only serial part.  It hops from token to token
//                     (the length nibbles, the 255-run extension bytes and
//                     the distance, read with one 16-byte LDS load per
//                     sequence in an assembly loop for the common shapes)
//                     and appends one raw entry per sequence (where the
//                     literals start, literal count, match length, distance)
//                     to an LDS chain.  It checks nothing it does not need
//                     to find the next token.  When the table carries a
//                     sequence index (the input offset of every token), the
//                     walker instead parses up to 64 listed sequences at once,
//                     one per lane, and checks that each one ends where the
//                     index says the next one starts.
//   wave 1  recorder: takes up to 64 chain entries at a time, one per lane,
//                     validates them (distance within the decoded prefix and
//                     the declared window, lengths within the chunk) and
//                     turns them into records with absolute positions by a
//                     wave-wide prefix scan, then publishes them to an LDS
//                     record ring.
//   wave 2  feeder  : streams the chunk's compressed bytes from HBM into an
//                     LDS input ring (8 KiB beside the long history, 16 KiB
//                     beside the short one) with LDS-DMA loads
//                     (global_load_lds_dwordx4), up to a ring's worth of
//                     1 KiB segments in flight.
//   waves 3+ builders: take the aligned 1 KiB tiles of the decoded stream in
//                     increasing order from a shared counter.  From the
//                     records a builder builds its tile in an LDS history
//                     ring, all 64 lanes at once (each lane owns 16 bytes of
//                     the tile), and then writes the tile out: as bytes
//                     (decode-only), or unpacked and dequantized to fp16
//                     (fused INT4 / INT8), with coalesced 16-byte stores.
//
// The history ring holds 64 KiB of decoded bytes for any LZ4 block, or
// 16 KiB when the chunk table declares that no match reaches further back
// than LT_SMALL_WINDOW bytes; the smaller ring lets more workgroups share a
// CU, and with it more chunks decode at once.  A match beyond the declared
// window is reported as a bad offset.
//
// The LZ4 block format (the pages name LZ4 for compressed weight blocks but
// do not define it; "GPU Compression Pipeline - TDD Roadmap", Phase 2.1 and
// Phase 3.1): a sequence is a token (high nibble literal count, low nibble
// match length - 4; 15 means more length follows as bytes of 255 closed by a
// byte < 255), the literals, a 2-byte little-endian distance, and the match
// length's extra bytes; the last sequence has literals only.  A match of
// length M at distance d produces out[p + j] = out[p - d + (j mod d)], which
// is what byte-serial copying gives when d < M.
//
// Building a tile.  Most tiles hold a few sequences whose matches are runs of
// one byte (distance 1, the byte carried in the record) or copies from before
// the part of the match that lies in the tile.  Such a tile is built in one
// pass: each lane walks the pieces (literal run, match) that meet its 16
// bytes, gathers each piece's bytes with aligned dword reads and
// v_alignbyte, and merges them; the whole tile is then written with one
// 16-byte LDS store per lane.  Where a match reads bytes of the same tile,
// the pass is repeated once per such match, each pass reading what the
// previous one wrote (all of a pass's reads precede its stores).  Tiles with
// many sequences or short-distance overlapping matches are built sequence by
// sequence instead.
//
// The roles talk through LDS counters (relaxed atomics; one wave's LDS
// operations complete in program order, so a counter written after data is
// seen after that data):
//   in_avail     feeder   -> all     : input bytes present in the ring
//   need[0]      walker   -> feeder  : first input byte the walker still reads
//   need[1 + b]  builder  -> feeder  : first input byte builder b still reads
//   wcnt, rcons  walker  <-> recorder: chain entries written / taken
//   nrec, cov    recorder -> builders: records written and the decoded bytes
//                                      they cover, published as one 8-byte word
//   bk[b]        builder  -> recorder: first record builder b still reads
//   built[b]     builder  -> builders: the tile builder b holds, moved on
//                                      as soon as that tile's history bytes
//                                      are final; every tile below the
//                                      smallest of these is built
//   next_tile[b] builder  -> builders: the same, moved on only after the
//                                      tile's write-out (which reads its
//                                      history slot) as well; all ones once
//                                      b has left
//   tile_ctr     builders          : the next tile nobody has taken
//   pstate       recorder -> all     : running / done / failed
// Every wait ends, by the argument below; as a backstop against a protocol
// mistake each wave's polls are also counted, and a wave that polls past its
// budget fails the chunk (C_STALL) instead of hanging the GPU.  The walker
// consumes at least one input byte per
// sequence and stops at the chunk's end, at a malformed length, or when the
// recorder has stopped; the recorder stops at the first invalid sequence;
// builders stop when the records stop short of their next tile.  A literal
// run longer than the input ring is handed over in two parts (its start is
// announced before the walker waits for its end), so the builders that need
// those literals keep consuming input while the walker waits.  The ring sizes
// are chosen so that a waiting wave never holds what the wave it waits for
// needs: the record ring holds more records than one tile can overlap, and
// decoded chunks are at most 1 MiB, so a length field's extra bytes (about
// 1/255 of the length) fit in the input ring beside the oldest tile's
// literals.  A tile's copies read only built tiles; its write-out is not on
// that path, so the next tile's build can start while it runs.  A tile
// overwrites the history slot of the tile one ring length back, so its
// builder first waits until the old tile's write-out is done and every tile
// that may read that slot is built: with a declared window of w bytes
// (r = ceil(w / 1 KiB) tiles) that stays short of the ring, the tiles up to
// r places after the old one; otherwise every earlier tile.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lt_device.hpp"
#include "lt_xxh.hpp"

namespace lt {

constexpr uint32_t SEG = 1024;        // feeder unit: one 16-byte DMA load per lane
constexpr uint32_t TILE = 1024;       // build / write-out unit (bytes of decoded stream)
// Sequence records in flight (recorder -> builders).  A 1 KiB tile overlaps
// at most 257 records (every non-final sequence decodes to >= 4 bytes), and
// the recorder must be able to hold all of them while the oldest tile's
// builder waits for the tile's coverage, so the ring holds more than 258;
// beyond that, a longer ring lets the walker run further ahead of the
// builders on blocks of many short sequences.  (Four workgroups must fit
// in one CU's LDS with the 16 KiB history, which bounds it: 40,880 bytes
// each.)
constexpr uint32_t RING = 368;
constexpr int NB = 5;                 // builder waves
constexpr int NWAVES = 3 + NB;        // walker, recorder, feeder, builders
constexpr int NTHREADS = 64 * NWAVES;
constexpr uint32_t NSLOT = 8;         // counter array length (>= NB + 1)
// A tile is built in passes (one, plus one per copy that reads the tile
// itself) when it has at most BULK_RECS records, or when its passes number
// at most one per BULK_RATIO records; otherwise record by record.  A pass
// over a whole tile costs about as much as two records built alone (short
// pieces take one byte per lane there).
constexpr uint32_t BULK_RECS = 16;
constexpr uint32_t BULK_RATIO = 2;
// Poll intervals (s_sleep units of 64 cycles).  Waiting waves share the CU's
// scalar unit and LDS with the walkers, so they poll no faster than the
// walk can change what they wait for.
constexpr int SLEEP_COV = 6;          // builder waiting for records
constexpr int SLEEP_DONE = 3;         // builder waiting for earlier tiles
constexpr int SLEEP_FEED = 2;         // feeder waiting for ring space
constexpr uint32_t LEN_CAP = 1u << 31;

enum : uint32_t { ST_RUN = 0, ST_DONE = 1, ST_FAIL = 2 };
enum : int32_t { C_OK = 0, C_TRUNC = 1, C_BADOFF = 2, C_OVERRUN = 3, C_SIZE = 4, C_TABLE = 5, C_CHECKSUM = 6,
                 C_STALL = 7 };
// Every wait ends.  The walker, the recorder and the feeder may each poll
// at most this many times per chunk (or the table's spin_limit, when
// nonzero) before they give up; a wave that gives up marks the chunk stalled
// (it then reports C_STALL) and failed, and leaves its role.  Builders wait
// only for those three and for older tiles (no cycle among builders), and
// every builder wait also ends once the chunk has failed, so one wave giving
// up lets every wave reach the kernel's end.  Legitimate waits take far
// fewer polls (a whole 1 MiB chunk decodes in well under a million poll
// intervals), so the bound only ends what would otherwise never end.
constexpr uint32_t SPIN_DEFAULT = 1u << 24;
// MODE_INT4G is MODE_INT4 for groups that are a power of two of at least
// 128 codes, where a tile spans at most 17 groups (its own kernel, with a
// leaner scale / zero-point fetch).
// MODE_GEMV is MODE_INT4G whose whole tiles are dotted with a vector and
// added to y instead of being written.
// MODE_GEMM takes a table whose bytes are INT4 codes in tiles of 16 rows x
// 128 columns (1 KiB, each row's 64 bytes in turn) and multiplies every
// tile with the matching 128 columns of a batch of 16 or 32 vectors on the
// matrix cores; each builder keeps its partial products, and a second
// kernel sums them per row block in a fixed order.
enum Mode : int { MODE_BYTES = 0, MODE_INT4 = 1, MODE_INT8 = 2, MODE_INT4G = 3, MODE_GEMV = 4, MODE_GEMM = 5 };
constexpr uint32_t GEMM_SLOTS = NB + 1;   // partial-product slots per chunk (one per builder)

struct __attribute__((aligned(16))) Ctl {
  uint32_t need[NSLOT];       // first input byte still read: [0] walker, [1 + b] builder b
  uint32_t bk[NSLOT];         // builder b: first record it may still read
  uint32_t next_tile[NSLOT];  // builder b: its next tile (all ones once it has left)
  uint32_t built[NSLOT];      // builder b: its first tile whose history bytes are not final
  uint32_t in_avail;          // feeder: input bytes present in the ring
  uint32_t pstate;            // recorder: running / done / failed
  uint32_t nrec;              // recorder: records written ...
  uint32_t cov;               // ... and the decoded bytes they cover (one 8-byte word)
  uint32_t wcnt;              // walker: chain entries written
  uint32_t rcons;             // recorder: chain entries taken
  uint32_t nfinished;         // builders that have left
  uint32_t tile_ctr;          // builders: the next tile nobody has taken
  int32_t status;
  uint32_t stall;             // any wave: a bounded wait gave up (the chunk fails with C_STALL)
  uint32_t xbad;              // feeder: the block's bytes do not match their checksum
};

// The history ring holds 2^HLOG decoded bytes: 64 KiB for any LZ4 block
// (distances reach 65535), 16 KiB for tables that declare a short window.
// The compressed-input ring is as large as two workgroups per CU allow with
// the long history (8 KiB) and twice that with the short one: the longer
// the ring, the further the feeder's loads run ahead of the builders.
template <int HLOG>
struct Smem {
  static constexpr uint32_t INR = HLOG >= 16 ? 1u << 13 : 1u << 14;
  static constexpr uint32_t IMASK = INR - 1;
  static constexpr uint32_t QMAX = INR / SEG;   // segments in flight at most
  // walker -> recorder entries in flight (a longer chain lets the indexed
  // walk hand over bigger batches)
  static constexpr uint32_t CHAIN = HLOG >= 16 ? 32u : 128u;
  uint8_t hist[1u << HLOG];
  uint8_t inr[INR];
  uint4 recs[RING];
  uint4 chain[CHAIN];
};

// four workgroups of the 16 KiB-history class share one CU's 160 KiB of LDS
static_assert(sizeof(Smem<14>) + sizeof(Ctl) <= 160u * 1024u / 4u, "LDS per workgroup");

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
  uint32_t dmax;             // largest match distance the table allows (65535: any)
  const uint64_t *seq_off;   // optional sequence index (NULL: none)
  const uint32_t *seq_pos;
  uint64_t n_seq;            // entries in seq_pos
  // A launch may cover a slice of a table (a batch of a streamed table, a
  // chunk range): comp_off values count from comp_base, and every chunk of
  // the slice lies within dst_off d_first .. d_last, the first starting at
  // d_first and the last ending at d_last.
  uint64_t comp_base;
  uint64_t d_first, d_last;
  // MODE_GEMV (INT4 groups of 128 codes or more, rows a multiple of 512
  // codes, chunks a multiple of 1 KiB): instead of writing fp16, each tile
  // adds its dot products with x to y (zeroed beforehand).
  const uint16_t *gemv_x;    // fp16 [cols]
  float *gemv_y;             // fp32 [rows]
  uint64_t cols;
  uint32_t spin;             // polls each wave may make per chunk (>= 1)
  // MODE_GEMM: partial products [chunk][GEMM_SLOTS][gemm_nbt][16 x 16]
  // fp32, x fp16 [16 gemm_nbt][cols] in gemv_x, tiles per 16-row block
  float *gemm_part;
  uint32_t gemm_nbt;
  uint64_t gemm_tpr;
  const uint32_t *order;     // workgroup k decodes chunk order[k] (NULL: chunk k)
  const uint64_t *xxh;       // expected XXH3-64 of each chunk's compressed bytes (NULL: not checked)
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

// Counter reads stay in program order with this wave's other LDS accesses
// (the hardware executes one wave's LDS operations in order; the fences keep
// the compiler from moving loads across the read).
__device__ __forceinline__ uint32_t lds_get(uint32_t *p) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  uint32_t v = __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  return __builtin_amdgcn_readfirstlane(v);
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void *)p;
}

// Counter stores are made by lane 0 alone.  The exec mask is narrowed inside
// the asm block rather than by a branch on the lane index, so the caller's
// control flow stays uniform and a serial loop around a store stays a scalar
// loop (a lane-dependent branch inside it would make the compiler treat the
// loop's values as per-lane).  One wave's LDS operations complete in order,
// so a store made here is seen after every LDS store the wave made before it.
// The stores below narrow the exec mask to lane 0 (or to lanes 0 .. n-1)
// inside their asm block, whatever the caller's mask: they are correct only
// where the call is wave-uniform, lane 0 active and the address and value
// the same in every active lane (lds_store_lanes: lanes 0 .. n-1 active).
// An LT_DEBUG build checks this at every call and counts each violation in
// a device counter (read with lt_debug_violations), with the first one's
// source line; release builds check nothing.
#ifdef LT_DEBUG
__device__ uint32_t g_debug_count;
__device__ uint32_t g_debug_line;
__device__ __forceinline__ void debug_flag(bool bad, uint32_t line) {
  const uint64_t ex = __builtin_amdgcn_read_exec();
  const uint32_t me = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  if (__ballot(bad) && me == (uint32_t)__builtin_ctzll(ex)) {
    atomicAdd(&g_debug_count, 1u);
    atomicCAS(&g_debug_line, 0u, line);
  }
}
__device__ __forceinline__ void debug_uniform(uint32_t a, uint32_t v, uint32_t line) {
  const bool lane0 = (__builtin_amdgcn_read_exec() & 1ull) != 0;
  const bool differs = a != (uint32_t)__builtin_amdgcn_readfirstlane(a) || v != (uint32_t)__builtin_amdgcn_readfirstlane(v);
  debug_flag(!lane0 || differs, line);
}
#define LT_UNIFORM(a, v) debug_uniform((a), (v), __LINE__)
#define LT_LANES(n) debug_flag((__builtin_amdgcn_read_exec() & ((n) >= 64 ? ~0ull : ((1ull << (n)) - 1))) != \
                                   ((n) >= 64 ? ~0ull : ((1ull << (n)) - 1)), __LINE__)
#else
#define LT_UNIFORM(a, v) ((void)0)
#define LT_LANES(n) ((void)0)
#endif

__device__ __forceinline__ void lds_set(uint32_t *p, uint32_t v, uint32_t = 0) {
  LT_UNIFORM(lds_addr(p), v);
  uint64_t sv;
  asm volatile("s_mov_b64 %0, exec\n\ts_mov_b64 exec, 1\n\tds_write_b32 %1, %2\n\ts_mov_b64 exec, %0"
               : "=&s"(sv) : "v"(lds_addr(p)), "v"(v) : "memory");
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// lanes 0 .. n-1 (n <= 64) each store 16 bytes at their own address; the
// exec mask is narrowed inside the asm block, as for lds_set
__device__ __forceinline__ void lds_store_lanes(uint32_t addr, u32x4 v, uint32_t n) {
  LT_LANES(n);
  uint64_t sv, m;
  asm volatile("s_bfm_b64 %1, %4, 0\n\ts_cmp_eq_u32 %4, 64\n\ts_cselect_b64 %1, -1, %1\n\t"
               "s_mov_b64 %0, exec\n\ts_mov_b64 exec, %1\n\tds_write_b128 %2, %3\n\ts_mov_b64 exec, %0"
               : "=&s"(sv), "=&s"(m) : "v"(addr), "v"(v), "s"(n) : "scc", "memory");
}

// lane 0 stores a 16-byte entry and then a counter
__device__ __forceinline__ void lds_set_entry(void *e, u32x4 v, uint32_t *p, uint32_t c) {
  LT_UNIFORM(lds_addr(e), v.x ^ v.y ^ v.z ^ v.w);
  LT_UNIFORM(lds_addr(p), c);
  uint64_t sv;
  asm volatile("s_mov_b64 %0, exec\n\ts_mov_b64 exec, 1\n\tds_write_b128 %1, %2\n\t"
               "ds_write_b32 %3, %4\n\ts_mov_b64 exec, %0"
               : "=&s"(sv) : "v"(lds_addr(e)), "v"(v), "v"(lds_addr(p)), "v"(c) : "memory");
}

// nrec and cov are written together with one 8-byte store and read with one
// 8-byte load, so a reader never sees coverage by records it does not count.
__device__ __forceinline__ void publish_rec(Ctl &c, uint32_t nrec, uint32_t cov, uint32_t = 0) {
  LT_UNIFORM(nrec, cov);
  uint64_t sv;
  const uint64_t v = ((uint64_t)cov << 32) | nrec;
  asm volatile("s_mov_b64 %0, exec\n\ts_mov_b64 exec, 1\n\tds_write_b64 %1, %2\n\ts_mov_b64 exec, %0"
               : "=&s"(sv) : "v"(lds_addr(&c.nrec)), "v"(v) : "memory");
}

__device__ __forceinline__ uint2 read_rec(Ctl &c) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  const uint64_t v = __hip_atomic_load((uint64_t *)&c.nrec, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  return make_uint2(__builtin_amdgcn_readfirstlane((uint32_t)v), __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32)));
}

// a value every lane holds, stated so the compiler keeps it in a scalar register
__device__ __forceinline__ uint32_t uni(uint32_t v) { return __builtin_amdgcn_readfirstlane(v); }

// Issue priority from a chunk's progress (done of total, wave-uniform): 3 in
// its first quarter down to 0 in its last.  Every wave of a chunk of a
// sequence-dense table (the kernels with LPF) calls it as it advances, so the
// chunks resident on a CU move forward together instead of oldest first.
// Such chunks vary widely in how long they live, and the launch ends with
// the slowest: decode-only on ReLU activations is 8% faster with it, greedy
// LZ4 blocks of a weight layer 2%; on the packer's weight tables the same
// was 9% slower (13% without the index), as oldest-first frees each CU's
// slots early, which the second round of chunks needs.
__device__ __forceinline__ void prio_by_progress(uint32_t done, uint32_t total) {
  const uint32_t d4 = 4u * __builtin_amdgcn_readfirstlane(done), t = __builtin_amdgcn_readfirstlane(total);
  if (d4 < t) __builtin_amdgcn_s_setprio(3);
  else if (d4 < 2 * t) __builtin_amdgcn_s_setprio(2);
  else if (d4 < 3 * t) __builtin_amdgcn_s_setprio(1);
  else __builtin_amdgcn_s_setprio(0);
}

// A load from device memory through a global (not flat) address: a flat
// load also counts in the LDS wait counter, so every LDS wait after it would
// wait for the memory round trip too.
__device__ __forceinline__ uint32_t gload(const uint32_t *p) {
  return *(const __attribute__((address_space(1))) uint32_t *)p;
}

// One poll of a bounded wait: true while this wave's poll budget lasts.  Once
// it is spent the chunk is marked stalled and failed, and the caller leaves.
__device__ __forceinline__ bool spin_ok(uint32_t &budget, Ctl &ctl) {
  if (budget != 0) {
    budget = uni(budget - 1);
    return true;
  }
  lds_set(&ctl.stall, 1u);
  lds_set(&ctl.pstate, ST_FAIL);
  return false;
}

// Minimum of an 8-entry counter array (16-byte aligned), read at once.  Like
// every counter access of the feeder wave, it goes through inline asm: that
// wave's LDS-DMA loads would otherwise make the compiler wait for every load
// in flight before any LDS access.  The read waits for its own result inside
// the asm block, so its output registers are final when the block ends.
__device__ __forceinline__ uint32_t min8(const uint32_t *a) {
  uint4 u, v;
  asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %2 offset:16\n\ts_waitcnt lgkmcnt(0)"
               : "=v"(u), "=v"(v) : "v"(lds_addr(a)) : "memory");
  uint32_t m0 = min(min(u.x, u.y), min(u.z, u.w));
  uint32_t m1 = min(min(v.x, v.y), min(v.z, v.w));
  return __builtin_amdgcn_readfirstlane(min(m0, m1));
}

__device__ __forceinline__ uint32_t lds_get_asm(const uint32_t *p) {
  uint32_t v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(lds_addr(p)) : "memory");
  return __builtin_amdgcn_readfirstlane(v);
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

// keep the first c bytes of dword acc and take the rest from v (c may be
// negative: take all of v; or 4 and more: keep all of acc)
__device__ __forceinline__ uint32_t merge_from(uint32_t acc, uint32_t v, int c) {
  const uint32_t m = c <= 0 ? 0xFFFFFFFFu : (c >= 4 ? 0u : (0xFFFFFFFFu << (8 * c)));
  return (v & m) | (acc & ~m);
}

// ----------------------------------------------------------- sequences

// A sequence record, written by the recorder into an LDS ring and read by the
// builders: the decoded-stream position where the sequence's literals start,
// the input position of the literals, their count, and the match (distance,
// fill byte for distance 1 when known, flags).  A record's match ends where
// the next record starts; the last record written ends at ctl.cov.
constexpr uint32_t F_MATCH = 1u << 24;  // match fields are final
constexpr uint32_t F_FILL = 2u << 24;   // distance 1 and bits 16..23 hold the byte it repeats
constexpr uint32_t F_LAST = 4u << 24;   // literal-only last sequence

__device__ __forceinline__ uint32_t ridx(uint32_t j) { return j % RING; }
// ring slot of record base + lane for a wave-uniform base: the modulo is
// taken once on the scalar unit, the lane offset wraps at most once
__device__ __forceinline__ uint32_t ridx_lane(uint32_t base, uint32_t lane) {
  const uint32_t r = __builtin_amdgcn_readfirstlane(base % RING) + lane;
  return r >= RING ? r - RING : r;
}
__device__ __forceinline__ uint32_t rec_dist(uint32_t info) { return info & 0xFFFFu; }
__device__ __forceinline__ uint32_t rec_fill(uint32_t info) { return (info >> 16) & 0xFFu; }

// --------------------------------------------------- walker and recorder

// The parse is split in two.  The walker follows the chain of sequence
// starts, which is the only part of LZ4 decoding that is inherently serial:
// from a token it needs the literal count (and its extra bytes), and from the
// literal run's end the match length's extra bytes, to find the next token.
// Reading the distance there as well, it writes one chain entry per sequence
// {literal start, literal count, match length, distance | last literal byte
// << 16 | flags << 24}.  The recorder takes up to 64 chain entries at once,
// one lane per sequence: it forms the decoded positions with a wave prefix
// sum, applies the checks that need them and writes the records the builders
// consume.  It never reads the input.

constexpr uint32_t W_LAST = 1u << 24;   // literal-only last sequence
constexpr uint32_t W_END = 2u << 24;    // the walk stopped here; the status is in the match field
constexpr uint32_t W_LIT = 4u << 24;    // a literal run whose match is still being read ...
constexpr uint32_t W_CONT = 8u << 24;   // ... and, in the next entry, that match (M, distance)

// exclusive prefix sum of v over the wave's lanes
// with DPP moves (no LDS traffic): inclusive sums within each 16-lane row
// by shifts of 1, 2, 4 and 8 lanes (lanes shifted in from outside the row
// read 0), then row 0's total added to row 1 and row 2's to row 3 (row
// broadcast of lane 15), then rows 0..1's total added to rows 2 and 3 (row
// broadcast of lane 31)
__device__ __forceinline__ uint32_t wave_excl_scan(uint32_t v, uint32_t) {
  uint32_t x = v;
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, true);   // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, true);   // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, true);   // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, true);   // row_shr:8
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x - v;
}

// the value of the lane below (lane 0 reads 0), by a DPP wave shift
__device__ __forceinline__ uint32_t lane_below(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x138, 0xF, 0xF, true);   // wave_shr:1
}

// Turns sequence entries into records: the recorder wave's work on entries
// from the chain, and the walker's own when the chunk has a sequence index
// (entries in registers, entry i in lane i).
template <class SM>
struct Rec {
  SM &sm;
  uint32_t dmax;
  Ctl &ctl;
  uint32_t lane;
  uint32_t N;
  uint32_t nrec;        // records written
  uint32_t op;          // decoded bytes described by the records
  uint32_t rec_free;    // cached: records below this may be overwritten
  uint32_t fill_ok;     // the last record ends with a known byte (distance-1 run) ...
  uint32_t fill;        // ... which is this
  uint32_t pending;     // the last record's match is still to come (a W_CONT entry)
  uint32_t spin = 0;    // polls left (set from ChunkParams::spin)

  // the entry after an announced literal run (ent wave-uniform): its match,
  // or the end of the walk.  Returns the chunk's final status, or -1.
  __device__ __forceinline__ int32_t cont(uint4 ent) {
    if (ent.w & W_END) return (int32_t)ent.z;
    const uint32_t M = ent.z, dist = ent.w & 0xFFFFu, lastlit = (ent.w >> 16) & 0xFFu;
    if (dist == 0 || dist > op || dist > dmax) return C_BADOFF;
    if (M > N - op) return C_OVERRUN;
    uint32_t info = F_MATCH | dist;
    if (dist == 1) info |= F_FILL | (lastlit << 16);   // the announced run has literals
    if (lane == 0) sm.recs[(nrec - 1) % RING].w = info;
    op += M;
    fill_ok = dist == 1;
    fill = lastlit;
    pending = 0;
    publish_rec(ctl, nrec, op, lane);
    return -1;
  }

  // Up to n (1 .. 64) entries, entry i in lane i (none of them the one after
  // an announced literal run).  Writes records for as many as the ring has
  // room for, up to and including an announced literal run, and up to the
  // first invalid one; returns how many it took, and in st the chunk's final
  // status when the chunk ends with them (else -1).
  __device__ __forceinline__ uint32_t batch(uint4 ent, uint32_t n, int32_t &st) {
    // record ring space (with every builder gone, bk is all ones and
    // nothing is read any more)
    while (nrec - rec_free >= RING) {
      rec_free = min8(ctl.bk);
      if (rec_free == 0xFFFFFFFFu) rec_free = nrec;
      if (nrec - rec_free < RING) break;
      if (!spin_ok(spin, ctl)) {
        st = C_STALL;
        return 0;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    const uint32_t space = RING - (nrec - rec_free);
    n = n < space ? n : space;
    // a batch ends with an announced literal run (its match comes later)
    const uint64_t lits = __ballot(lane < n && (ent.w & W_LIT) != 0);
    if (lits) n = (uint32_t)__builtin_ctzll(lits) + 1;
    const bool act = lane < n;
    const uint32_t ys = ent.x, L = ent.y, M = ent.z;
    const bool last = (ent.w & W_LAST) != 0, end = (ent.w & W_END) != 0;
    const bool lit = (ent.w & W_LIT) != 0;
    const uint32_t dist = ent.w & 0xFFFFu, lastlit = (ent.w >> 16) & 0xFFu;
    // decoded positions
    const uint32_t len = act && !end ? L + (last || lit ? 0u : M) : 0u;
    const uint32_t o = op + wave_excl_scan(len, lane);
    // checks that need the decoded position (the walker did the rest)
    int32_t err = C_OK;
    if (act) {
      if (end) err = (int32_t)M;
      else if (L > N - o) err = C_OVERRUN;
      else if (last) err = (o + L == N) ? C_OK : C_SIZE;
      else if (lit) err = C_OK;
      else if (dist == 0 || dist > o + L || dist > dmax) err = C_BADOFF;
      else if (M > N - o - L) err = C_OVERRUN;
    }
    const uint64_t bad = __ballot(err != C_OK);
    const uint32_t f = bad ? (uint32_t)__builtin_ctzll(bad) : n;   // records before the first failure
    // fill byte of distance-1 runs: the last literal, or, when this record
    // has no literals, the byte the previous record's run repeats (so a
    // chain of runs without literals between them carries it on)
    uint32_t fok, fb;
    if (L > 0) {
      fok = 1;
      fb = lastlit;
    } else if (lane == 0) {
      fok = fill_ok;
      fb = fill;
    } else {
      fok = 0;
      fb = 0;
    }
    {
      const bool inherits = L == 0 && lane > 0;
      const bool run = dist == 1 && !lit && !last;
      for (;;) {
        const uint32_t po = lane_below(run && fok ? 1u : 0u);
        const uint32_t pb = lane_below(fb);
        const bool take = inherits && !fok && po != 0;
        if (!__ballot(take)) break;
        if (take) {
          fok = 1;
          fb = pb;
        }
      }
    }
    uint32_t info = last ? F_LAST : (lit ? 0u : (F_MATCH | dist));
    if (!last && !lit && dist == 1 && fok) info |= F_FILL | (fb << 16);
    if (lane < f) sm.recs[ridx_lane(nrec, lane)] = make_uint4(o, ys, L, info);
    // state after the records written
    if (f > 0) {
      const uint32_t lf = f - 1;
      const uint32_t l_o = __builtin_amdgcn_readlane(o, lf), l_len = __builtin_amdgcn_readlane(len, lf);
      const uint32_t l_info = __builtin_amdgcn_readlane(info, lf);
      op = l_o + l_len;
      fill_ok = (l_info & F_FILL) ? 1u : 0u;
      fill = rec_fill(l_info);
      pending = __builtin_amdgcn_readlane(lit ? 1u : 0u, lf);
      nrec += f;
      publish_rec(ctl, nrec, op, lane);
    }
    st = -1;
    if (f < n) st = (int32_t)__builtin_amdgcn_readlane((uint32_t)err, f);
    else if (__ballot(act && last)) st = C_OK;
    return f;
  }
};

// Wave 0.  Structural checks only (everything that keeps the walk inside the
// block); distances and decoded positions are the recorder's.  Input waits
// always end: the feeder keeps filling the ring while the walk is open, and
// the walker announces a literal run before it waits for the bytes after it,
// so the builders can release the ring.  Only the chain wait can end with the
// recorder gone (a failed chunk): then the walk stops.
// LPF: the issue priority follows the walk's progress (prio_by_progress)
template <class SM, bool LPF = false>
struct Walker {
  static constexpr uint32_t INR = SM::INR, IMASK = SM::IMASK, CHAIN = SM::CHAIN;
  SM &sm;
  Ctl &ctl;
  uint32_t lane;
  uint32_t y;           // input position of the next token
  uint32_t y_end;
  uint32_t N;
  uint32_t avail;       // cached ctl.in_avail
  uint32_t wy;          // window start (multiple of 4); window = [wy, wy + 256)
  uint32_t win;         // this lane's dword of the window
  uint32_t cnt;         // chain entries written
  uint32_t cons;        // cached ctl.rcons: entries the recorder has taken
  uint32_t stop;        // the recorder is gone: the walk ends
  uint64_t tw;          // bytes y .. y + 7 (when have_tw)
  uint32_t have_tw;
  uint32_t pub;         // last position published in need[0] by the fast step
  uint32_t pend;        // the current literal run [pend_ys, + pend_L) is not announced yet
  uint32_t split;       // it was announced on its own (W_LIT)
  uint32_t pend_ys, pend_L;
  const uint32_t *ix;   // this chunk's sequence index (block offsets), or NULL
  uint32_t icnt;        // its entries
  uint32_t ij;          // the next entry to walk
  uint32_t head;        // block offset 0 sits at input position head
  uint32_t wbase;       // entries wbase .. wbase + 63 sit in lane order in iw,
  uint32_t iw, iw2;     // the next 64 in iw2
  Rec<SM> rec;          // with an index the walker makes the records itself ...
  uint32_t direct;      // ... (and no recorder wave runs)
  int32_t fin;          // (direct) the chunk's final status once known, else -1
  uint32_t spin = 0;    // polls left (set from ChunkParams::spin)
  uint32_t stalled = 0; // a wait for input gave up: the walk ends
  uint32_t iw3 = 0;     // the 64 entries after iw2, in flight while iw and iw2 are read

  __device__ __forceinline__ void emit(uint32_t ys, uint32_t L, uint32_t M, uint32_t w) {
    if (direct) {
      int32_t st;
      if (w & W_END) st = (int32_t)M;
      else if (w & W_CONT) st = rec.cont(make_uint4(ys, L, M, w));
      else rec.batch(make_uint4(ys, L, M, w), 1, st);
      if (st >= 0) {
        fin = st;
        stop = 1;
      }
      return;
    }
    while (cnt - cons >= CHAIN) {
      cons = lds_get(&ctl.rcons);
      if (cnt - cons < CHAIN) break;
      if (lds_get(&ctl.pstate) != ST_RUN || !spin_ok(spin, ctl)) {
        stop = 1;
        return;
      }
      __builtin_amdgcn_s_sleep(1);
    }
    const uint32_t slot = cnt % CHAIN;
    cnt = uni(cnt + 1);
    // the entry first, then the count (one wave's LDS writes land in order)
    lds_set_entry(&sm.chain[slot], u32x4{ys, L, M, w}, &ctl.wcnt, cnt);
  }

  __device__ __forceinline__ void need_input(uint32_t upto) {
    upto = upto < y_end ? upto : y_end;
    if (avail >= upto || stalled) return;
    avail = lds_get(&ctl.in_avail);
    if (avail >= upto) return;
    if (pend) {
      // announce the literal run before waiting: its builders consume it
      // and release the input ring, which may be what the wait needs
      pend = 0;
      split = 1;
      emit(pend_ys, pend_L, 0, W_LIT);
    }
    while (avail < upto) {
      if (!spin_ok(spin, ctl)) {
        // the bytes never came: the walk ends (what it reads from here on
        // is not input, but every read stays inside the ring and the walk
        // stops at its next step)
        stalled = 1;
        stop = 1;
        return;
      }
      __builtin_amdgcn_s_sleep(1);
      avail = lds_get(&ctl.in_avail);
    }
  }

  // Nothing before the window start is read again by the walker (the
  // builders announce their own needs).
  __device__ void load_window(uint32_t p) {
    wy = uni(p & ~3u);
    lds_set(&ctl.need[0], wy, lane);
    need_input(wy + 256);
    win = *(const uint32_t *)(sm.inr + ((wy + 4 * lane) & IMASK));
    wait_lds();
  }

  // byte p of the block (p < y_end)
  __device__ uint32_t byte_at(uint32_t p) {
    if (p < wy || p >= wy + 256) load_window(p);
    const uint32_t rel = p - wy;
    return uni((__builtin_amdgcn_readlane(win, rel >> 2) >> ((rel & 3) * 8)) & 0xFFu);
  }

  // bytes p .. p + 7 from the window (p >= wy, p + 12 <= wy + 256)
  __device__ uint64_t peek8(uint32_t p) {
    const uint32_t r = p - wy, i = r >> 2, sh = (r & 3) * 8;
    const uint32_t d0 = __builtin_amdgcn_readlane(win, i);
    const uint32_t d1 = __builtin_amdgcn_readlane(win, i + 1);
    const uint32_t d2 = __builtin_amdgcn_readlane(win, i + 2);
    const uint32_t lo = (uint32_t)((((uint64_t)d1 << 32) | d0) >> sh);
    const uint32_t hi = (uint32_t)((((uint64_t)d2 << 32) | d1) >> sh);
    return ((uint64_t)hi << 32) | lo;
  }

  // Extra length bytes from q on (each 255 continues the run), added to
  // len; q ends after the run.  The checks are the byte-serial ones: the
  // block may not end inside the run, and a length past the chunk fails at
  // once (which also bounds how far the walk reads ahead inside a run).
  __device__ int32_t ext_run(uint32_t &q, uint32_t &len) {
    for (;;) {
      if (q >= y_end) return C_TRUNC;
      const uint32_t b = byte_at(q);
      q = uni(q + 1);
      len = uni(len + b);
      if (len > N) return C_OVERRUN;
      if (b != 255) return C_OK;
    }
  }

  // the entry of a finished sequence (announced on its own or not)
  __device__ __forceinline__ void finish(uint32_t ys, uint32_t L, uint32_t M, uint32_t w) {
    pend = 0;
    if (split) emit(0, 0, M, w | W_CONT);
    else emit(ys, L, M, w);
  }

  // Bytes p .. p + 7 of the block, read straight from the input ring with
  // one unaligned LDS read (the caller checks that they are present and do
  // not wrap around the ring's end).
  __device__ uint64_t ring8(uint32_t p) {
    uint2 v;
    __builtin_memcpy(&v, sm.inr + (p & IMASK), 8);
    return ((uint64_t)uni(v.y) << 32) | uni(v.x);
  }

  // The common-shape walk, written out in assembly: the compiler's version
  // of this loop spends most of its instructions on branch and lane-mask
  // bookkeeping, and the walk is the chunk's only serial work.
  //
  // A sequence of the common shape has a literal count whose extra bytes
  // end within the 8 bytes carried for the token (tw), a match length whose
  // extra bytes end within 8 bytes of its start, its literal run's end at
  // least 16 bytes before the block's end, and those 16 bytes already in the
  // ring.  Per sequence: the literal count from tw (a find-first-set on the
  // inverted word measures the run of 255-bytes), one 16-byte LDS read from
  // the literal run's last byte on (that byte, the distance, the match
  // length's extra bytes, and the next token with the bytes after it), and
  // the chain entry {literal start, literal count, match length, distance |
  // last literal << 16}, collected in lane k of four registers and written
  // to the chain for all collected sequences at once when the loop ends.
  //
  // Ends after nmax sequences (st 0), when the next token's eight bytes lie
  // beyond the read (st 4: tw must be reloaded), when the ring does not
  // hold the bytes yet (st 2), or at a sequence of another shape (st 1); in
  // the last two cases that sequence is not consumed.  Every iteration
  // advances y by at least 3 bytes, and a walk that crosses a KiB since the
  // last publication publishes y in need[0].
  __device__ __forceinline__ uint32_t fast_run(uint32_t nmax, uint32_t &n) {
    uint32_t st;
    // every scalar operand must be wave-uniform in the compiler's view too
    y = uni(y);
    pub = uni(pub);
    cnt = uni(cnt);
    tw = ((uint64_t)uni((uint32_t)(tw >> 32)) << 32) | uni((uint32_t)tw);
    const uint32_t yend = uni(y_end), av = uni(avail);
    nmax = uni(nmax);
    asm volatile(
        "s_mov_b64 s[46:47], %[tw]\n\t"
        "s_mov_b32 %[n], 0\n\t"
        "s_mov_b32 %[st], 0\n"
        "L_top%=:\n\t"
        // literal count: token nibble, then the run of 255s in bytes 1..7
        "s_and_b32 s48, s46, 0xff\n\t"
        "s_lshr_b64 s[40:41], s[46:47], 8\n\t"
        "s_or_b32 s41, s41, 0xff000000\n\t"
        "s_not_b64 s[40:41], s[40:41]\n\t"
        "s_ff1_i32_b64 s49, s[40:41]\n\t"
        "s_lshr_b32 s49, s49, 3\n\t"
        "s_cmpk_lt_u32 s48, 0xf0\n\t"
        "s_cbranch_scc1 L_short%=\n\t"
        "s_cmp_gt_u32 s49, 6\n\t"
        "s_cbranch_scc1 L_bail%=\n\t"
        "s_lshl_b32 s50, s49, 3\n\t"
        "s_add_u32 s50, s50, 8\n\t"
        "s_lshr_b64 s[40:41], s[46:47], s50\n\t"
        "s_and_b32 s40, s40, 0xff\n\t"
        "s_mul_i32 s51, s49, 0xff\n\t"
        "s_add_u32 s51, s51, s40\n\t"
        "s_add_u32 s51, s51, 15\n\t"            // L
        "s_add_u32 s52, %[y], s49\n\t"
        "s_add_u32 s52, s52, 2\n"               // literal start
        "L_lit%=:\n\t"
        "s_add_u32 s53, s52, s51\n\t"           // q: the literal run's end
        "s_add_u32 s50, s53, 16\n\t"
        "s_cmp_gt_u32 s50, %[yend]\n\t"
        "s_cbranch_scc1 L_bail%=\n\t"
        "s_sub_u32 s54, s53, 1\n\t"             // read from q - 1
        "s_and_b32 s50, s54, %[imask]\n\t"
        "s_cmp_gt_u32 s50, %[rlast]\n\t"          // would wrap around the ring's end
        "s_cbranch_scc1 L_bail%=\n\t"
        "s_add_u32 s55, s54, 16\n\t"
        "s_cmp_gt_u32 s55, %[avail]\n\t"
        "s_cbranch_scc1 L_avail%=\n\t"
        "s_add_u32 s50, s50, %[inr]\n\t"
        "v_mov_b32 v44, s50\n\t"
        "ds_read_b128 v[40:43], v44\n\t"
        "s_sub_u32 s55, s54, %[pub]\n\t"
        "s_cmpk_gt_u32 s55, 0x3ff\n\t"
        "s_cbranch_scc1 L_pub%=\n"
        "L_pubd%=:\n\t"
        "s_waitcnt lgkmcnt(0)\n\t"
        "v_readfirstlane_b32 s42, v40\n\t"
        "v_readfirstlane_b32 s43, v41\n\t"
        "v_readfirstlane_b32 s44, v42\n\t"
        "v_readfirstlane_b32 s45, v43\n\t"
        // match length: nibble, then the run of 255s in bytes q+2 .. q+9
        "s_and_b32 s55, s48, 15\n\t"
        "s_cmp_lg_u32 s55, 15\n\t"
        "s_cbranch_scc1 L_nom%=\n\t"
        "s_lshr_b64 s[40:41], s[42:43], 24\n\t"
        "s_lshl_b32 s50, s44, 8\n\t"
        "s_or_b32 s41, s41, s50\n\t"
        "s_not_b64 s[58:59], s[40:41]\n\t"
        "s_ff1_i32_b64 s49, s[58:59]\n\t"
        "s_lshr_b32 s49, s49, 3\n\t"
        "s_cmp_gt_u32 s49, 7\n\t"
        "s_cbranch_scc1 L_bail%=\n\t"
        "s_lshl_b32 s50, s49, 3\n\t"
        "s_lshr_b64 s[58:59], s[40:41], s50\n\t"
        "s_and_b32 s58, s58, 0xff\n\t"
        "s_mul_i32 s56, s49, 0xff\n\t"
        "s_add_u32 s56, s56, s58\n\t"
        "s_add_u32 s56, s56, 19\n\t"            // M
        "s_add_u32 s49, s49, 1\n"               // its extra bytes
        "L_mdone%=:\n\t"
        // distance | last literal << 16 (no literal: 0)
        "s_bfe_u32 s57, s42, 0x100008\n\t"
        "s_and_b32 s50, s42, 0xff\n\t"
        "s_cmp_eq_u32 s51, 0\n\t"
        "s_cselect_b32 s50, 0, s50\n\t"
        "s_lshl_b32 s50, s50, 16\n\t"
        "s_or_b32 s57, s57, s50\n\t"
        "s_mov_b32 m0, %[n]\n\t"
        "v_writelane_b32 v48, s52, m0\n\t"
        "v_writelane_b32 v49, s51, m0\n\t"
        "v_writelane_b32 v50, s56, m0\n\t"
        "v_writelane_b32 v51, s57, m0\n\t"
        "s_add_u32 %[n], %[n], 1\n\t"
        // the next token: q + 2 + extra bytes, o = 3 + extra bytes into the read
        "s_add_u32 %[y], s53, 2\n\t"
        "s_add_u32 %[y], %[y], s49\n\t"
        "s_add_u32 s50, s49, 3\n\t"
        "s_cmp_gt_u32 s50, 7\n\t"
        "s_cbranch_scc1 L_notw%=\n\t"
        "s_lshl_b32 s50, s50, 3\n\t"
        "s_lshr_b64 s[46:47], s[42:43], s50\n\t"
        "s_sub_u32 s50, 64, s50\n\t"
        "s_lshl_b64 s[40:41], s[44:45], s50\n\t"
        "s_or_b64 s[46:47], s[46:47], s[40:41]\n\t"
        "s_cmp_lt_u32 %[n], %[nmax]\n\t"
        "s_cbranch_scc1 L_top%=\n\t"
        "s_branch L_flush%=\n"
        "L_short%=:\n\t"
        "s_lshr_b32 s51, s48, 4\n\t"
        "s_add_u32 s52, %[y], 1\n\t"
        "s_branch L_lit%=\n"
        "L_nom%=:\n\t"
        "s_add_u32 s56, s55, 4\n\t"
        "s_mov_b32 s49, 0\n\t"
        "s_branch L_mdone%=\n"
        "L_pub%=:\n\t"
        "s_mov_b32 %[pub], %[y]\n\t"
        "v_mov_b32 v45, %[y]\n\t"
        "v_mov_b32 v46, %[need0]\n\t"
        "s_mov_b64 s[58:59], exec\n\t"
        "s_mov_b64 exec, 1\n\t"
        "ds_write_b32 v46, v45\n\t"
        "s_mov_b64 exec, s[58:59]\n\t"
        "s_branch L_pubd%=\n"
        "L_notw%=:\n\t"
        "s_mov_b32 %[st], 4\n\t"
        "s_branch L_flush%=\n"
        "L_avail%=:\n\t"
        "s_mov_b32 %[st], 2\n\t"
        "s_branch L_flush%=\n"
        "L_bail%=:\n\t"
        "s_mov_b32 %[st], 1\n"
        // entries of lanes 0 .. n-1 to chain slots cnt .. cnt+n-1, then the count
        "L_flush%=:\n\t"
        "s_cmp_eq_u32 %[n], 0\n\t"
        "s_cbranch_scc1 L_end%=\n\t"
        "v_add_u32 v45, %[cnt], %[vlane]\n\t"
        "v_and_b32 v45, %[cmask], v45\n\t"
        "v_lshlrev_b32 v45, 4, v45\n\t"
        "v_add_u32 v45, %[chain], v45\n\t"
        "s_add_u32 %[cnt], %[cnt], %[n]\n\t"
        "v_mov_b32 v46, %[cnt]\n\t"
        "v_mov_b32 v47, %[wcnt]\n\t"
        "s_bfm_b64 s[40:41], %[n], 0\n\t"
        "s_mov_b64 s[58:59], exec\n\t"
        "s_mov_b64 exec, s[40:41]\n\t"
        "ds_write_b128 v45, v[48:51]\n\t"
        "s_mov_b64 exec, 1\n\t"
        "ds_write_b32 v47, v46\n\t"
        "s_mov_b64 exec, s[58:59]\n"
        "L_end%=:\n\t"
        "s_mov_b64 %[tw], s[46:47]"
        : [y] "+s"(y), [tw] "+s"(tw), [pub] "+s"(pub), [cnt] "+s"(cnt), [n] "=&s"(n), [st] "=&s"(st)
        : [yend] "s"(yend), [avail] "s"(av), [inr] "s"(uni(lds_addr(sm.inr))),
          [need0] "s"(uni(lds_addr(&ctl.need[0]))), [nmax] "s"(nmax), [chain] "s"(uni(lds_addr(sm.chain))),
          [wcnt] "s"(uni(lds_addr(&ctl.wcnt))), [vlane] "v"(lane), [imask] "s"(IMASK), [rlast] "s"(INR - 16),
          [cmask] "s"(CHAIN - 1)
        : "s40", "s41", "s42", "s43", "s44", "s45", "s46", "s47", "s48", "s49", "s50", "s51", "s52",
          "s53", "s54", "s55", "s56", "s57", "s58", "s59", "v40", "v41", "v42", "v43", "v44", "v45",
          "v46", "v47", "v48", "v49", "v50", "v51", "m0", "scc", "memory");
    return st;
  }

  // Walks common-shape sequences; false, with nothing consumed, when the
  // next sequence needs the general step.
  __device__ __forceinline__ bool fast_step() {
    if (!have_tw) {
      if (((y & IMASK) > INR - 8) | (y + 8 > y_end)) return false;
      if (avail < y + 8) {
        avail = lds_get(&ctl.in_avail);
        if (avail < y + 8) return false;
      }
      tw = ring8(y);
      have_tw = 1;
    }
    if (cnt - cons >= CHAIN) {
      cons = lds_get(&ctl.rcons);
      if (cnt - cons >= CHAIN) {
        if (lds_get(&ctl.pstate) != ST_RUN || !spin_ok(spin, ctl)) stop = 1;
        else __builtin_amdgcn_s_sleep(1);
        return true;
      }
    }
    const uint32_t room = CHAIN - (cnt - cons);
    uint32_t n;
    const uint32_t st = fast_run(room < 4 ? room : 4u, n);
    if (st == 4) have_tw = 0;
    if (st == 2) {
      const uint32_t a = avail;
      avail = lds_get(&ctl.in_avail);
      return n > 0 || avail != a;
    }
    if (st == 1) return n > 0;
    return true;
  }

  // One sequence byte by byte, with the byte-serial checks.  Returns false
  // when the walk ends: after the literal-only last sequence, at a
  // structural error (an END entry carries the status), or when the
  // recorder is gone.
  __device__ __forceinline__ bool slow_step() {
    int32_t st = C_OK;
    uint32_t ys = 0, L = 0, M = 0, w = 0, e = 0, token = 0;
    if (y >= y_end) st = C_TRUNC;
    if (st == C_OK) {
      token = byte_at(y);
      y = uni(y + 1);
      L = token >> 4;
      if (L == 15) st = ext_run(y, L);
    }
    if (st == C_OK && L > y_end - y) st = C_TRUNC;
    if (st == C_OK) {
      ys = y;
      e = uni(y + L);
      if (e == y_end) {   // literal-only last sequence
        emit(ys, L, 0, W_LAST);
        return false;
      }
      if (y_end - e < 2) st = C_TRUNC;
    }
    if (st == C_OK) {
      pend = L > 0;
      split = 0;
      pend_ys = ys;
      pend_L = L;
      const uint32_t lastlit = L ? byte_at(e - 1) : 0u;
      const uint32_t d0 = byte_at(e), d1 = byte_at(e + 1);
      w = d0 | (d1 << 8) | (lastlit << 16);
      y = uni(e + 2);
      M = (token & 15) + 4;
      if ((token & 15) == 15) st = ext_run(y, M);
    }
    if (st != C_OK) {
      pend = 0;
      emit(0, 0, (uint32_t)st, W_END);
      return false;
    }
    finish(ys, L, M, w);
    return stop == 0;
  }

  // first byte != 255 among the low `bytes` bytes of w (== bytes when none)
  static __device__ uint32_t first_not255(uint32_t w, uint32_t bytes) {
    const uint32_t nz = ~w & (bytes >= 4 ? 0xFFFFFFFFu : ((1u << (8 * bytes)) - 1));
    return nz ? (uint32_t)__builtin_ctz(nz) / 8 : bytes;
  }

  // Up to 64 listed sequences side by side, one per lane.  Lane l takes
  // the sequence listed at entry ij + l, which starts at p and must end
  // where entry ij + l + 1 starts (pn): it decodes the token and the literal
  // count from the 16 bytes at p and the distance and match length from the
  // 16 bytes at the literal run's last byte, all from the input ring.  The
  // batch stops before the first sequence whose bytes are not all in the
  // ring yet or whose length fields run past those 16 bytes, and before the
  // last listed sequence (the general step checks the block's end).  A
  // sequence that does not end where the next listed one starts means the
  // index does not describe the block: the chunk fails.  Returns false,
  // with nothing consumed, when the next sequence needs the general step.
  __device__ __forceinline__ bool index_batch() {
    if (!direct && cnt - cons >= CHAIN) {
      cons = lds_get(&ctl.rcons);
      if (cnt - cons >= CHAIN) {
        if (lds_get(&ctl.pstate) != ST_RUN || !spin_ok(spin, ctl)) stop = 1;
        else __builtin_amdgcn_s_sleep(1);
        return true;
      }
    }
    const uint32_t room = direct ? 64u : CHAIN - (cnt - cons), left = icnt - ij;
    uint32_t nmax = room < left - 1 ? room : left - 1;
    nmax = nmax < 64 ? nmax : 64u;
    if (nmax == 0) return false;
    while (ij >= wbase + 64) {          // slide the index window
      iw = iw2;
      iw2 = iw3;
      wbase += 64;
      iw3 = gload(ix + min(wbase + 128 + lane, icnt - 1));
    }
    const uint32_t e = ij + (lane < nmax ? lane : nmax - 1);
    const uint32_t p = head + entry(e), pn = head + entry(e + 1);
    if (uni(p) != y) return false;                 // reported by the general step
    const uint32_t hi = pn + 16 < y_end ? pn + 16 : y_end;
    // the cached count may be behind: more may have landed since
    if (__builtin_amdgcn_readlane(hi, nmax - 1) > avail) avail = lds_get(&ctl.in_avail);
    if (uni(hi) > avail) {
      // the first sequence's bytes are not all here: wait for them when
      // they fit well within the ring (polling only the count, with the
      // batch's setup kept), else walk it with the general step
      if (uni(pn) - y + 16 > INR / 2) return false;
      avail = lds_get(&ctl.in_avail);
      if (uni(hi) > avail) {
        pub = y;
        lds_set(&ctl.need[0], pub);
        do {
          if (!spin_ok(spin, ctl)) {
            stalled = 1;
            stop = 1;
            fin = C_STALL;
            return true;
          }
          __builtin_amdgcn_s_sleep(1);
          avail = lds_get(&ctl.in_avail);
        } while (uni(hi) > avail);
      }
    }
    // the token and the literal count's extra bytes
    const uint4 a = gather16<IMASK>(sm.inr, p);
    const uint32_t token = a.x & 0xFFu;
    const bool l15 = token >= 0xF0u;
    const uint32_t w0 = (a.x >> 8) | (a.y << 24), w1 = (a.y >> 8) | (a.z << 24);
    const uint32_t w2 = (a.z >> 8) | (a.w << 24), w3 = a.w >> 8;
    uint32_t nl = first_not255(w0, 4);
    if (nl == 4) nl = 4 + first_not255(w1, 4);
    if (nl == 8) nl = 8 + first_not255(w2, 4);
    if (nl == 12) nl = 12 + first_not255(w3, 3);   // bytes 1 .. 15
    const uint32_t nlc = nl < 14 ? nl : 14u;
    const uint32_t lb = (nlc < 4 ? w0 >> (8 * nlc) : nlc < 8 ? w1 >> (8 * (nlc - 4))
                         : nlc < 12 ? w2 >> (8 * (nlc - 8)) : w3 >> (8 * (nlc - 12))) & 0xFFu;
    const uint32_t L = l15 ? 15 + 255 * nlc + lb : token >> 4;
    const uint32_t ys = p + (l15 ? nlc + 2 : 1u);
    const uint32_t q = ys + L;
    // the literal run's last byte, the distance and the match length
    const uint4 b = gather16<IMASK>(sm.inr, q - 1);
    const uint32_t lastlit = L ? b.x & 0xFFu : 0u;
    const uint32_t mn = token & 15u;
    const uint32_t v0 = (b.x >> 24) | (b.y << 8), v1 = (b.y >> 24) | (b.z << 8);
    const uint32_t v2 = (b.z >> 24) | (b.w << 8);
    uint32_t nm = first_not255(v0, 4);
    if (nm == 4) nm = 4 + first_not255(v1, 4);
    if (nm == 8) nm = 8 + first_not255(v2, 4);   // bytes q + 2 .. q + 13
    const uint32_t nmc = nm < 11 ? nm : 11u;
    const uint32_t mb = (nmc < 4 ? v0 >> (8 * nmc) : nmc < 8 ? v1 >> (8 * (nmc - 4)) : v2 >> (8 * (nmc - 8))) & 0xFFu;
    const bool m15 = mn == 15;
    const uint32_t M = m15 ? 19 + 255 * nmc + mb : mn + 4;
    const uint32_t nxt = q + 2 + (m15 ? nmc + 1 : 0u);
    const bool hard = (l15 && nl > 13) || (m15 && nm > 10);
    const bool ok = lane < nmax && hi <= avail && !hard;
    const uint64_t stops = __ballot(!ok);
    const uint32_t n = stops ? (uint32_t)__builtin_ctzll(stops) : 64u;
    if (n == 0) return false;
    const uint64_t bad = __ballot(nxt != pn) & (n >= 64 ? ~0ull : ((1ull << n) - 1));
    if (bad) {
      emit(0, 0, (uint32_t)C_TABLE, W_END);
      stop = 1;
      return true;
    }
    const uint32_t dw = ((b.x >> 8) & 0xFFFFu) | (lastlit << 16);
    uint32_t took = n;
    if (direct) {
      int32_t st;
      took = rec.batch(make_uint4(ys, L, M, dw), n, st);
      if (st >= 0) {
        fin = st;
        stop = 1;
        return true;
      }
    } else {
      const uint32_t slot = lds_addr(&sm.chain[(cnt + lane) % CHAIN]);
      lds_store_lanes(slot, u32x4{ys, L, M, dw}, n);
      cnt = uni(cnt + n);
      lds_set(&ctl.wcnt, cnt);
    }
    ij += took;
    y = uni(__builtin_amdgcn_readlane(pn, took - 1));
    if constexpr (LPF) prio_by_progress(y, y_end);
    if (y - pub >= SEG) {
      pub = y;
      lds_set(&ctl.need[0], pub);
    }
    return true;
  }

  // index entry x, for wbase <= x < wbase + 128 (from the two windows)
  __device__ uint32_t entry(uint32_t x) {
    const uint32_t d = x - wbase;
    const uint32_t a = __builtin_amdgcn_ds_bpermute(4 * (d & 63), iw);
    const uint32_t b = __builtin_amdgcn_ds_bpermute(4 * (d & 63), iw2);
    return d < 64 ? a : b;
  }

  // The walk guided by the sequence index: listed sequences in batches,
  // the others (and the last) with the general step, each checked against
  // its listed position.
  __device__ __forceinline__ void run_indexed() {
    wbase = 0;
    iw = gload(ix + min(lane, icnt - 1));
    iw2 = gload(ix + min(64 + lane, icnt - 1));
    iw3 = gload(ix + min(128 + lane, icnt - 1));
    for (;;) {
      if (ij == icnt) {                 // the block goes on past the index
        emit(0, 0, (uint32_t)C_TABLE, W_END);
        return;
      }
      if (index_batch()) {
        if (stop) return;
        continue;
      }
      if (y != head + gload(ix + ij)) {
        emit(0, 0, (uint32_t)C_TABLE, W_END);
        return;
      }
      ij++;
      have_tw = 0;
      if (!slow_step()) return;
    }
  }

  __device__ __forceinline__ void run() {
    if constexpr (LPF) prio_by_progress(0, 1);
    if (icnt) {
      run_indexed();
    } else {
      for (;;) {
        y = uni(y);
        if (fast_step()) {
          if (stop) break;
          if constexpr (LPF) prio_by_progress(y, y_end);
          continue;
        }
        have_tw = 0;
        if (!slow_step()) break;
      }
    }
    if (stalled && direct) fin = C_STALL;
    lds_set(&ctl.need[0], 0xFFFFFFFFu, lane);
  }
};

// Wave 1 (chunks without a sequence index).  Turns chain entries into
// records, 64 at a time.
template <class SM>
__device__ __forceinline__ int32_t recorder(Rec<SM> &r, SM &sm, Ctl &ctl, uint32_t lane) {
  constexpr uint32_t CHAIN = SM::CHAIN;
  uint32_t taken = 0, avail_entries = 0;
  for (;;) {
    // entries to take
    while (avail_entries == taken) {
      avail_entries = lds_get(&ctl.wcnt);
      if (avail_entries != taken) break;
      // the recorder owns pstate: a failed state here is a stalled wave's
      if (lds_get(&ctl.pstate) == ST_FAIL || !spin_ok(r.spin, ctl)) return C_STALL;
      __builtin_amdgcn_s_sleep(1);
    }
    if (r.pending) {
      const uint4 ent = make_uint4(__builtin_amdgcn_readfirstlane(sm.chain[taken % CHAIN].x),
                                   __builtin_amdgcn_readfirstlane(sm.chain[taken % CHAIN].y),
                                   __builtin_amdgcn_readfirstlane(sm.chain[taken % CHAIN].z),
                                   __builtin_amdgcn_readfirstlane(sm.chain[taken % CHAIN].w));
      const int32_t st = r.cont(ent);
      if (st >= 0) return st;
      taken++;
      lds_set(&ctl.rcons, taken, lane);
      continue;
    }
    uint32_t n = avail_entries - taken;
    n = n < 64 ? n : 64;
    uint4 ent = make_uint4(0u, 0u, 0u, W_END);
    if (lane < n) ent = sm.chain[(taken + lane) % CHAIN];
    int32_t st;
    taken += r.batch(ent, n, st);
    if (st >= 0) return st;
    lds_set(&ctl.rcons, taken, lane);
  }
}

// -------------------------------------------------------------- feeder

// Waits until at most K LDS-DMA segments are still in flight, publishes
// in_avail = v, and returns the minimum of the eight need counters.  The
// counters are read before the wait, in the same asm block, so the read
// overlaps the segment's latency; an older minimum is a smaller one, so the
// bound it gives is safe.  (The reads wait for their own results inside the
// block, so their output registers are final when it ends.)
template <int K>
__device__ __forceinline__ uint32_t land_and_bound(const uint32_t *need, uint32_t *in_avail, uint32_t v) {
  uint4 a, b;
  uint64_t sv;
  asm volatile(
      "ds_read_b128 %0, %3\n\t"
      "ds_read_b128 %1, %3 offset:16\n\t"
      "s_waitcnt vmcnt(%6)\n\t"
      "s_mov_b64 %2, exec\n\t"
      "s_mov_b64 exec, 1\n\t"
      "ds_write_b32 %4, %5\n\t"
      "s_mov_b64 exec, %2\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(a), "=&v"(b), "=&s"(sv)
      : "v"(lds_addr(need)), "v"(lds_addr(in_avail)), "v"(v), "n"(K)
      : "memory");
  const uint32_t m0 = min(min(a.x, a.y), min(a.z, a.w));
  const uint32_t m1 = min(min(b.x, b.y), min(b.z, b.w));
  return __builtin_amdgcn_readfirstlane(min(m0, m1));
}

// land_and_bound for a run-time count of loads still allowed in flight
__device__ __forceinline__ uint32_t land_and_bound_k(uint32_t k, const uint32_t *need, uint32_t *in_avail,
                                                     uint32_t v) {
  switch (k) {
    case 0: return land_and_bound<0>(need, in_avail, v);
    case 1: return land_and_bound<1>(need, in_avail, v);
    case 2: return land_and_bound<2>(need, in_avail, v);
    case 3: return land_and_bound<3>(need, in_avail, v);
    case 4: return land_and_bound<4>(need, in_avail, v);
    case 5: return land_and_bound<5>(need, in_avail, v);
    case 6: return land_and_bound<6>(need, in_avail, v);
    case 7: return land_and_bound<7>(need, in_avail, v);
    case 8: return land_and_bound<8>(need, in_avail, v);
    case 9: return land_and_bound<9>(need, in_avail, v);
    case 10: return land_and_bound<10>(need, in_avail, v);
    case 11: return land_and_bound<11>(need, in_avail, v);
    case 12: return land_and_bound<12>(need, in_avail, v);
    case 13: return land_and_bound<13>(need, in_avail, v);
    case 14: return land_and_bound<14>(need, in_avail, v);
    default: return land_and_bound<15>(need, in_avail, v);
  }
}

// 8 input bytes from ring position pos (any alignment) as a little-endian
// word; every lane's pos has the same alignment
template <class SM>
__device__ __forceinline__ uint64_t ring8(const SM &sm, uint32_t pos) {
  constexpr uint32_t WM = SM::IMASK >> 2;
  const uint32_t *R = (const uint32_t *)sm.inr;
  const uint32_t w = pos >> 2, sh = pos & 3;
  uint32_t x0 = R[w & WM], x1 = R[(w + 1) & WM];
  if (sh) {
    const uint32_t x2 = R[(w + 2) & WM];
    x0 = __builtin_amdgcn_alignbyte(x1, x0, sh);
    x1 = __builtin_amdgcn_alignbyte(x2, x1, sh);
  }
  return ((uint64_t)x1 << 32) | x0;
}

// Wave 2.  Streams the chunk's 16-byte aligned blocks into the input ring,
// one 1 KiB segment (one LDS-DMA load per lane) at a time, keeping up to QMAX
// segments in flight within the ring space that every reader has released.
// Each landed segment costs one LDS round trip, overlapped with the wait for
// the segment: the readers' bound is read while the segment is in flight,
// and the exit check (every reader gone: a failed chunk) is made only when
// nothing is in flight.  With a checksum (`whole`) the block is streamed to
// its end in any case, for the hasher.
template <class SM, bool LPF>
__device__ __forceinline__ void feeder(SM &sm, Ctl &ctl, uint32_t lane, const uint8_t *S, uint32_t y_end, uint32_t nb,
                                       uint32_t spin, bool whole) {
  constexpr uint32_t IMASK = SM::IMASK, QMAX = SM::QMAX;
  static_assert(QMAX <= 16, "land_and_bound_k waits for up to 15 loads in flight");
  const uint32_t nblk = (y_end + 15) / 16;
  const uint32_t nseg = (y_end + SEG - 1) / SEG;
  uint32_t issued = 0, landed = 0;
  uint32_t limit = QMAX < nseg ? QMAX : nseg;   // every reader starts at input byte 0
  if constexpr (LPF) prio_by_progress(0, 1);
  for (;;) {
    while (issued < limit && issued - landed < QMAX) {
      uint32_t blk = issued * (SEG / 16) + lane;
      if (blk >= nblk) blk = nblk - 1;   // stay within the chunk's blocks
      __builtin_amdgcn_global_load_lds((const void *)(S + 16ull * blk),
                                       (__attribute__((address_space(3))) void *)(sm.inr + ((issued * SEG) & IMASK)),
                                       16, 0, 0);
      issued++;
    }
    if (issued == landed) {
      if (landed == nseg) break;
      // the window is closed and nothing is in flight: nobody reads input
      // once the walk has ended and every builder has left
      if (!whole && lds_get_asm(&ctl.nfinished) == nb && lds_get_asm(&ctl.need[0]) == 0xFFFFFFFFu) break;
      const uint32_t used = min8(ctl.need);
      limit = used / SEG + QMAX;
      if (limit > nseg) limit = nseg;
      if (issued == limit) {
        if (!spin_ok(spin, ctl)) break;
        __builtin_amdgcn_s_sleep(SLEEP_FEED);
      }
      continue;
    }
    // the oldest segment in flight has landed once at most k loads remain
    const uint32_t k = issued - landed - 1;
    landed++;
    const uint32_t used = land_and_bound_k(k, ctl.need, &ctl.in_avail, landed * SEG);
    if constexpr (LPF) prio_by_progress(landed, nseg);
    limit = used / SEG + QMAX;
    if (limit > nseg) limit = nseg;
  }
  wait_vm<0>();   // no LDS-DMA write outlives this wave
}

// The hasher (a table with checksums): XXH3-64 of the chunk's compressed
// bytes, read from the input ring as the feeder lands them, whole 1 KiB
// blocks in order (two at a time when both have landed).  It is one more
// reader of the ring: need[HSLOT] holds the first byte it still reads, so
// the feeder reloads no slot before it is hashed.  A hash that differs from
// `want` marks the chunk (ctl.xbad); the hasher gives up only when a wave
// has stalled or its own polls run out.
constexpr uint32_t HSLOT = NSLOT - 1;
template <class SM>
__device__ __forceinline__ void hasher(SM &sm, Ctl &ctl, uint32_t lane, uint32_t head, uint32_t y_end, uint64_t want,
                                       uint32_t spin) {
  constexpr uint32_t IMASK = SM::IMASK;
  const uint32_t n = y_end - head;   // the chunk's compressed bytes
  const uint32_t hblocks = n > xxh::SHORT_MAX ? (n - 1) / xxh::BLOCK : 0u;
  const uint32_t tail = n > xxh::SHORT_MAX ? min(xxh::BLOCK * hblocks, n - 64) : 0u;
  xxh::Wave H;
  H.init(lane);
  uint32_t hb = 0, avail = 0;
  auto wait_for = [&](uint32_t upto) -> bool {
    while (avail < upto) {
      avail = lds_get(&ctl.in_avail);
      if (avail >= upto) break;
      if (lds_get(&ctl.stall) || !spin_ok(spin, ctl)) return false;
      __builtin_amdgcn_s_sleep(1);
    }
    return true;
  };
  bool ok = true;
  while (ok && hb < hblocks) {
    ok = wait_for(head + xxh::BLOCK * (hb + 1));
    while (ok && hb < hblocks && head + xxh::BLOCK * (hb + 1) <= avail) {
      const uint32_t q = head + xxh::BLOCK * hb + 8 * lane;
      if (hb + 1 < hblocks && head + xxh::BLOCK * (hb + 2) <= avail) {
        H.block2(ring8(sm, q), ring8(sm, q + 512), ring8(sm, q + xxh::BLOCK), ring8(sm, q + xxh::BLOCK + 512));
        hb += 2;
      } else {
        H.block(ring8(sm, q), ring8(sm, q + 512));
        hb++;
      }
    }
    lds_set(&ctl.need[HSLOT], head + (hb < hblocks ? xxh::BLOCK * hb : tail), lane);
  }
  if (ok) ok = wait_for(y_end);
  if (ok) {
    uint64_t h;
    if (n <= xxh::SHORT_MAX) {
      h = xxh::short_hash(n, [&](uint32_t k) { return (uint32_t)sm.inr[(head + k) & IMASK]; });
    } else {
      const uint32_t ns = ((n - 1) - xxh::BLOCK * hblocks) / 64;   // whole stripes of the last block
      const uint32_t q = head + xxh::BLOCK * hblocks + 8 * lane;
      H.partial(ring8(sm, q), ring8(sm, q + 512), lane, ns);
      H.last(ring8(sm, head + n - 64 + 8 * (lane & 7)), lane);
      h = H.merge(n);
    }
    if (h != want) lds_set(&ctl.xbad, 1u, lane);
  }
  lds_set(&ctl.need[HSLOT], 0xFFFFFFFFu, lane);
}

// ------------------------------------------------------------ write-out

struct Meta4 {
  uint32_t s[4];
  uint32_t z[4];
  uint32_t g0;   // (few groups) the group lane 0 fetched
};

// The groups of INT4 dword k of lane `lane` in tile t (fast path: the group
// is a power of two >= 8, so each lane's 8 codes share one group).
__device__ __forceinline__ uint64_t int4_group(const ChunkParams &P, uint64_t dst0, uint32_t t,
                                               uint32_t lane, uint32_t N, int k) {
  uint32_t p = t * TILE + 256 * k + 4 * lane;
  if (p >= N) p = 0;   // any valid group; unused
  return (2 * (dst0 + p)) >> P.group_shift;
}

// Scales / zero points of one INT4 tile.  The loads are issued here and
// consumed only after the tile is built (see meta_ready).  With groups of
// 128 codes or more a tile spans at most 17 groups: lanes 0 .. 31 then
// fetch groups g0 .. g0 + 31 with one load each of scale and zero point,
// and meta_ready hands each lane its four; smaller groups fetch per lane.
__device__ __forceinline__ Meta4 int4_meta(const ChunkParams &P, uint64_t dst0, uint32_t t,
                                           uint32_t lane, uint32_t N, bool few) {
  Meta4 m{};
  // without zero points, read any valid byte and discard it (no branch)
  const int8_t *zsrc = P.zp ? P.zp : (const int8_t *)P.scales;
  if (few) {
    const uint64_t ng = (2 * P.total + (1ull << P.group_shift) - 1) >> P.group_shift;
    m.g0 = (uint32_t)((2 * (dst0 + (uint64_t)t * TILE)) >> P.group_shift);
    uint64_t g = (uint64_t)m.g0 + (lane & 31);
    g = g < ng ? g : ng - 1;
    m.s[0] = P.scales[g];
    m.z[0] = (uint32_t)(uint8_t)zsrc[g];
    return m;
  }
#pragma unroll
  for (int k = 0; k < 4; k++) {
    const uint64_t g = int4_group(P, dst0, t, lane, N, k);
    m.s[k] = P.scales[g];
    m.z[k] = (uint32_t)(int32_t)zsrc[g];
  }
  return m;
}

// Make the tile's scale registers opaque here, so the compiler consumes (and
// waits for) them at this point instead of right after issuing the loads.
__device__ __forceinline__ void meta_ready(Meta4 &m, bool has_zp, const ChunkParams &P, uint64_t dst0,
                                           uint32_t t, uint32_t lane, uint32_t N, bool few) {
#pragma unroll
  for (int k = 0; k < 4; k++) asm volatile("" : "+v"(m.s[k]), "+v"(m.z[k]));
  if (few) {
    const uint32_t pk = (m.s[0] & 0xFFFFu) | (m.z[0] << 16);
#pragma unroll
    for (int k = 0; k < 4; k++) {
      const uint32_t i = (uint32_t)int4_group(P, dst0, t, lane, N, k) - m.g0;
      const uint32_t v = __builtin_amdgcn_ds_bpermute(4 * i, pk);
      m.s[k] = v & 0xFFFFu;
      m.z[k] = (uint32_t)(int32_t)(int8_t)(v >> 16);
    }
  }
#pragma unroll
  for (int k = 0; k < 4; k++)
    if (!has_zp) m.z[k] = 0;
}

// MODE_INT4G: lanes 0 .. 31 fetch the scale and zero point of groups
// g0 .. g0 + 31 of tile t (the last valid group repeats past the end), from
// a tile-uniform base and a per-lane offset.
struct MetaG {
  uint32_t s, z;
};
__device__ __forceinline__ MetaG int4g_meta(const ChunkParams &P, uint64_t dst0, uint32_t t, uint32_t lane31,
                                            uint64_t ng) {
  const uint64_t g0 = (2 * (dst0 + (uint64_t)t * TILE)) >> P.group_shift;
  const uint64_t left = ng - g0;   // >= 1
  const uint32_t li = lane31 < left ? lane31 : (uint32_t)left - 1;
  // without zero points, read any valid byte and discard it (no branch)
  const int8_t *zsrc = (P.zp ? P.zp : (const int8_t *)P.scales) + g0;
  MetaG m;
  m.s = P.scales[g0 + li];
  m.z = (uint32_t)(uint8_t)zsrc[li];
  return m;
}

// (few groups) lanes 0 .. 31 turn their group's scale and zero point into
// the two packed constants of deq8_int4_dual: s[1] = {s, s} and
// z[1] = {1024 + zp, 64 + zp}.
__device__ __forceinline__ void meta_pack_few(Meta4 &m, bool has_zp) {
  asm volatile("" : "+v"(m.s[0]), "+v"(m.z[0]));
  const int z = has_zp ? (int)(int8_t)m.z[0] : 0;
  m.s[1] = (m.s[0] & 0xFFFFu) * 0x10001u;
  m.z[1] = f16_bits_int(1024 + z) | (f16_bits_int(64 + z) << 16);
}

// Write-out of a whole INT4 tile whose groups hold 128 codes or more (a
// power of two).  Lane l's dword k holds codes 512 k + 8 l .. + 7 of the
// tile, one group, whose constants come from lane (group - g0) by
// ds_bpermute.  Each store instruction writes 1 KiB of contiguous fp16.
template <int MODE, int HLOG>
__device__ __forceinline__ void flush_int4_few(Smem<HLOG> &sm, uint32_t lane, const ChunkParams &P,
                                               uint64_t dst0, uint32_t T, const Meta4 &m) {
  constexpr uint32_t HMASK = (1u << HLOG) - 1;
  const uint8_t *src = sm.hist + (T & HMASK) + 4 * lane;   // a tile never wraps the ring
  uint32_t w[4];
#pragma unroll
  for (int k = 0; k < 4; k++) w[k] = *(const uint32_t *)(src + 256 * k);
  const uint64_t e = 2 * (dst0 + T);   // the tile's first code
  const uint32_t off = (uint32_t)(e & (P.group - 1)) + 8 * lane;
  if constexpr (MODE == MODE_GEMV) {
    // the tile's fp16 weights dotted with x.  Rows are a multiple of 512
    // codes, so each 512-code block k (lane l holds codes 512 k + 8 l ..)
    // lies in one row; a tile inside one row sums all four blocks first.
    const uint64_t row0 = e / P.cols, row3 = (e + 1536) / P.cols;
    float acc[4];
#pragma unroll
    for (int k = 0; k < 4; k++) {
      const uint64_t ek = e + 512 * k;
      const uint64_t rk = ek / P.cols;
      const uint4 xv = *((const uint4 *)(P.gemv_x + (ek - rk * P.cols)) + lane);
      const uint32_t i = (off + 512 * k) >> P.group_shift;
      const h2 c2 = as_h2((uint32_t)__builtin_amdgcn_ds_bpermute(4 * i, m.z[1]));
      const h2 s2 = as_h2((uint32_t)__builtin_amdgcn_ds_bpermute(4 * i, m.s[1]));
      const uint4 wv = deq8_int4_dual(w[k], c2, s2);
      float a = 0.0f;
      a = __builtin_amdgcn_fdot2(as_h2(wv.x), as_h2(xv.x), a, false);
      a = __builtin_amdgcn_fdot2(as_h2(wv.y), as_h2(xv.y), a, false);
      a = __builtin_amdgcn_fdot2(as_h2(wv.z), as_h2(xv.z), a, false);
      a = __builtin_amdgcn_fdot2(as_h2(wv.w), as_h2(xv.w), a, false);
      acc[k] = a;
    }
    if (row0 == row3) {
      float a = (acc[0] + acc[1]) + (acc[2] + acc[3]);
      for (int o = 32; o >= 1; o >>= 1) a += __shfl_xor(a, o);
      if (lane == 0) atomicAdd(P.gemv_y + row0, a);
    } else {
#pragma unroll
      for (int k = 0; k < 4; k++) {
        float a = acc[k];
        for (int o = 32; o >= 1; o >>= 1) a += __shfl_xor(a, o);
        if (lane == 0) atomicAdd(P.gemv_y + (e + 512 * k) / P.cols, a);
      }
    }
    return;
  }
  uint4 *out = (uint4 *)((uint16_t *)P.out + e) + lane;
#pragma unroll
  for (int k = 0; k < 4; k++) {
    const uint32_t i = (off + 512 * k) >> P.group_shift;
    const h2 c2 = as_h2((uint32_t)__builtin_amdgcn_ds_bpermute(4 * i, m.z[1]));
    const h2 s2 = as_h2((uint32_t)__builtin_amdgcn_ds_bpermute(4 * i, m.s[1]));
    out[64 * k] = deq8_int4_dual(w[k], c2, s2);
  }
}

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));

// (MODE_GEMM) the scale and zero point of the tile row lane l multiplies:
// row l % 16 of the tile's 16-row block, whose 128 columns lie in one group
__device__ __forceinline__ MetaG gemm_meta(const ChunkParams &P, uint64_t dst0, uint32_t t, uint32_t lane) {
  const uint64_t tg = (dst0 + (uint64_t)t * TILE) / TILE;   // the tile's index in the table
  const uint64_t rb = tg / P.gemm_tpr, kc = tg - rb * P.gemm_tpr;
  const uint64_t g = ((16 * rb + (lane & 15)) * P.cols + 128 * kc) >> P.group_shift;
  // without zero points, read any valid byte and discard it (no branch)
  const int8_t *zsrc = P.zp ? P.zp : (const int8_t *)P.scales;
  MetaG m;
  m.s = P.scales[g];
  m.z = (uint32_t)(uint8_t)zsrc[g];
  return m;
}

// (MODE_GEMM) one tile times the batch: D[w][b] += sum_k W[w][k] x[b][k]
// over the tile's 16 rows w and 128 columns k, for batch blocks of 16
// vectors b.  The matrix cores' 16x16x32 fp16 product takes, in lane l,
// row l % 16 of A with its columns 8 (l / 16) .. + 7, and column l % 16 of
// B with those rows; A is the tile (lane l dequantizes the 8 codes of its
// row at columns 32 j + 8 (l / 16) .. + 7: one dword of the history, the
// write-out's two-magic arithmetic, so the values are the fused kernel's
// fp16 outputs), B the transposed batch (lane l loads 8 values of vector
// l % 16).  The products are exact in fp32, the sums are fp32.
template <int HLOG>
__device__ __forceinline__ void gemm_block(Smem<HLOG> &sm, uint32_t lane, const ChunkParams &P, uint32_t T,
                                           const uint16_t *xs, uint32_t c2, uint32_t s2, float4_t &acc) {
  constexpr uint32_t HMASK = (1u << HLOG) - 1;
  uint4 xv[4];
#pragma unroll
  for (int j = 0; j < 4; j++) xv[j] = *(const uint4 *)(xs + 32 * j);
  const uint8_t *src = sm.hist + (T & HMASK) + 64 * (lane & 15) + 4 * (lane >> 4);   // a tile never wraps
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const uint4 a = deq8_int4_dual(*(const uint32_t *)(src + 16 * j), as_h2(c2), as_h2(s2));
    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, a), __builtin_bit_cast(half8_t, xv[j]),
                                                 acc, 0, 0, 0);
  }
}

template <int HLOG>
__device__ __forceinline__ void gemm_tile(Smem<HLOG> &sm, uint32_t lane, const ChunkParams &P, uint64_t dst0,
                                          uint32_t T, const MetaG &m, float4_t (&acc)[2]) {
  const uint64_t tg = (dst0 + T) / TILE;
  const uint64_t kc = tg % P.gemm_tpr;
  const uint16_t *xs = P.gemv_x + (uint64_t)(lane & 15) * P.cols + 128 * kc + 8 * (lane >> 4);
  const uint32_t s2 = (m.s & 0xFFFFu) * 0x10001u;
  const int z = P.zp ? (int)(int8_t)m.z : 0;
  const uint32_t c2 = f16_bits_int(1024 + z) | (f16_bits_int(64 + z) << 16);
  // one batch block of 16 vectors at a time (the second re-reads the codes)
  gemm_block<HLOG>(sm, lane, P, T, xs, c2, s2, acc[0]);
  if (P.gemm_nbt > 1) gemm_block<HLOG>(sm, lane, P, T, xs + 16 * P.cols, c2, s2, acc[1]);
}

// (MODE_GEMM) a builder's partial products into its slot of the chunk: lane
// l holds D[4 (l / 16) + v][l % 16] of each batch block
__device__ __forceinline__ void gemm_store(const ChunkParams &P, uint32_t chunk, uint32_t slot, uint32_t lane,
                                           const float4_t (&acc)[2]) {
  float *part = P.gemm_part + ((uint64_t)chunk * GEMM_SLOTS + slot) * 256 * P.gemm_nbt;
  const uint32_t r = lane & 15, q = lane >> 4;
#pragma unroll
  for (uint32_t bt = 0; bt < 2; bt++) {
    if (bt >= P.gemm_nbt) break;
#pragma unroll
    for (int v = 0; v < 4; v++) part[256 * bt + (4 * q + v) * 16 + r] = acc[bt][v];
  }
}

template <int MODE, int HLOG>
__device__ __forceinline__ void flush_tile(Smem<HLOG> &sm, uint32_t lane, const ChunkParams &P, uint64_t dst0,
                           uint32_t t, uint32_t N, const Meta4 &m, bool fast) {
  constexpr uint32_t HMASK = (1u << HLOG) - 1;
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
  } else if constexpr (MODE == MODE_GEMV) {
    // never reached: the prologue admits only chunks of whole tiles
  } else if constexpr (MODE == MODE_INT4 || MODE == MODE_INT4G) {
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

// ------------------------------------------------------------ builders

// Waves 3 .. 3 + NB - 1.  Builder b starts with tile b and then takes the
// next untaken tile each time it starts one.  SPEC: tiles whose sources are
// not yet built may be built speculatively (see run()).
template <int MODE, int HLOG, bool SPEC, bool LPF>
struct Builder {
  static constexpr uint32_t HIST = 1u << HLOG, HMASK = HIST - 1, HTILES = HIST / TILE;
  static constexpr uint32_t IMASK = Smem<HLOG>::IMASK;
  Smem<HLOG> &sm;
  Ctl &ctl;
  const ChunkParams &P;
  uint64_t dst0;
  uint32_t lane;
  uint32_t b;
  uint32_t N;
  uint32_t k;          // first record that may overlap the current tile (announced in bk[b])
  uint32_t nrec;       // cached ctl.nrec
  uint32_t cov;        // cached ctl.cov
  uint32_t avail;      // cached ctl.in_avail
  uint32_t done;       // cached: tiles below this are built
  uint32_t fdone;      // cached: tiles below this are built and written out
  uint32_t need_pub;   // announced in need[1 + b]
  uint32_t chunk = 0;  // the chunk's index in the table (MODE_GEMM's partial-product slot)
  uint32_t nbs = 0;    // builders in this chunk

  __device__ void refresh() {
    const uint2 r = read_rec(ctl);
    nrec = r.x;
    cov = r.y;
  }

  // false if the chunk failed first (the feeder gave up)
  __device__ __forceinline__ bool need_input(uint32_t upto) {
    while (avail < upto) {
      avail = lds_get(&ctl.in_avail);
      if (avail < upto) {
        if (lds_get(&ctl.pstate) == ST_FAIL) return false;
        __builtin_amdgcn_s_sleep(1);
      }
    }
    return true;
  }

  // true if the tiles below `tiles` are built and those below `written`
  // written out too (one look, no wait)
  __device__ __forceinline__ bool ready(uint32_t tiles, uint32_t written) {
    if (done < tiles || fdone < written) {
      done = min8(ctl.built);
      fdone = min8(ctl.next_tile);
    }
    return done >= tiles && fdone >= written;
  }

  // wait until tiles [0, tiles) are final; false if the chunk failed first
  // Wait until the tiles below `tiles` are built and those below `written`
  // are written out too; false if the chunk failed first.
  __device__ __forceinline__ bool wait_done(uint32_t tiles, uint32_t written) {
    while (done < tiles || fdone < written) {
      done = min8(ctl.built);
      fdone = min8(ctl.next_tile);
      if (done >= tiles && fdone >= written) break;
      if (lds_get(&ctl.pstate) == ST_FAIL) return false;
      __builtin_amdgcn_s_sleep(SLEEP_DONE);
    }
    return true;
  }

  // Advance k to the last record starting at or before T, the one that
  // contains T once the records reach that far (records are sorted by
  // start), and announce that records below it are no longer read.
  __device__ __forceinline__ void find_k(uint32_t T) {
    uint32_t kk = k;
    for (;;) {   // records from k on are protected by bk[b] <= k
      const uint32_t j = kk + lane;
      const uint32_t x = (j < nrec) ? sm.recs[ridx_lane(kk, lane)].x : 0xFFFFFFFFu;
      const uint64_t bal = __ballot(x <= T);   // lanes 0 .. h
      const uint32_t h = 63 - __builtin_clzll(bal | 1ull);
      kk += h;
      if (h < 63) break;
    }
    if (kk > k) {
      k = kk;
      lds_set(&ctl.bk[b], kk, lane);
    }
  }

  // Announce the first input byte still read: the literal byte of record k
  // at position T, or the end of record k's literals when T lies past them
  // (later records' literals follow in the input).
  __device__ __forceinline__ void announce(uint32_t T) {
    const uint4 r = rec(k);
    uint32_t off = T > r.x ? T - r.x : 0u;
    off = off < r.z ? off : r.z;
    const uint32_t nd = r.y + off;
    if (nd > need_pub) {
      need_pub = nd;
      lds_set(&ctl.need[1 + b], nd, lane);
    }
  }

  // announce() for record k already read: {start, input position, literal count}
  __device__ void announce_rec(uint32_t T, uint32_t os, uint32_t src, uint32_t L) {
    uint32_t off = T > os ? T - os : 0u;
    off = off < L ? off : L;
    const uint32_t nd = src + off;
    if (nd > need_pub) {
      need_pub = nd;
      lds_set(&ctl.need[1 + b], nd, lane);
    }
  }

  // the next untaken tile: the atomic is issued here and its result read by
  // grab_take, so its latency overlaps the work in between
  __device__ uint32_t grab_issue() {
    uint32_t v = 0;
    if (lane == 0) v = __hip_atomic_fetch_add(&ctl.tile_ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    return v;
  }
  __device__ uint32_t grab_take(uint32_t v) { return __builtin_amdgcn_readlane(v, 0); }

  // wait until records cover [T, Tend); false if the records stopped short.
  // The recorder publishes its final state after its last records, so
  // records read after a final state has been seen are final.
  __device__ __forceinline__ bool wait_cov(uint32_t T, uint32_t Tend) {
    while (cov < Tend) {
      refresh();
      if (cov >= Tend) break;
      if (lds_get(&ctl.pstate) != ST_RUN) {
        refresh();
        return cov >= Tend;
      }
      // move past the records that end before T (nrec may be newer than
      // cov, so the search looks at the records' starts, not at cov)
      if (nrec > 0) {
        find_k(T);
        announce(T);
      }
      __builtin_amdgcn_s_sleep(SLEEP_COV);
    }
    return true;
  }

  // record j's four words (broadcast read)
  __device__ uint4 rec(uint32_t j) {
    uint4 r = sm.recs[ridx(j)];
    return make_uint4(__builtin_amdgcn_readfirstlane(r.x), __builtin_amdgcn_readfirstlane(r.y),
                      __builtin_amdgcn_readfirstlane(r.z), __builtin_amdgcn_readfirstlane(r.w));
  }
  __device__ uint32_t rec_start(uint32_t j) {
    return j < nrec ? __builtin_amdgcn_readfirstlane(sm.recs[ridx(j)].x) : cov;
  }

  // ---- sequence-by-sequence path (exact writes, any match)

  template <uint32_t MASK>
  __device__ void copy_exact(const uint8_t *R, uint32_t src0, uint32_t a, uint32_t n) {
    const uint32_t A = a & ~15u, end = a + n;
    const uint32_t nb = (end - A + 15) >> 4;
    for (uint32_t b0 = 0; b0 < nb; b0 += 64) {
      uint32_t bb = b0 + lane;
      if (bb < nb) {
        uint32_t Pp = A + 16 * bb;
        uint32_t lo = a > Pp ? a - Pp : 0;
        uint32_t hi = end - Pp < 16 ? end - Pp : 16;
        st_block(sm.hist + (Pp & HMASK), gather16<MASK>(R, src0 + (Pp - a)), lo, hi);
      }
    }
  }

  __device__ void fill_exact(uint32_t a, uint32_t byte, uint32_t n) {
    const uint32_t w = byte * 0x01010101u;
    const uint4 v = make_uint4(w, w, w, w);
    const uint32_t A = a & ~15u, end = a + n;
    const uint32_t nb = (end - A + 15) >> 4;
    for (uint32_t bb = lane; bb < nb; bb += 64) {
      uint32_t Pp = A + 16 * bb;
      uint32_t lo = a > Pp ? a - Pp : 0;
      uint32_t hi = end - Pp < 16 ? end - Pp : 16;
      st_block(sm.hist + (Pp & HMASK), v, lo, hi);
    }
  }

  // bytes [a, a + n) of a match with distance dist < n that started at or
  // before a: the match repeats with period dist, so out[q] = out[a - dist +
  // ((q - a) mod dist)], whose sources lie in the dist bytes before a (recent
  // enough to be in the history ring however long the match is)
  __device__ void periodic_exact(uint32_t dist, uint32_t a, uint32_t n) {
    const uint32_t A = a & ~15u, end = a + n;
    const uint32_t nb = (end - A + 15) >> 4;
    for (uint32_t bb = lane; bb < nb; bb += 64) {
      uint32_t Pp = A + 16 * bb;
      uint32_t lo = a > Pp ? a - Pp : 0;
      uint32_t hi = end - Pp < 16 ? end - Pp : 16;
      uint32_t r = (Pp + lo - a) % dist;
      // every byte's source index first (bytes outside [lo, hi) read any
      // byte of the ring and are not stored), so the loads issue back to
      // back, eight at a time, and wait once per eight
      uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (uint32_t h = 0; h < 2; h++) {
        uint32_t b[8];
#pragma unroll
        for (uint32_t i = 0; i < 8; i++) {
          const uint32_t q = 8 * h + i;
          b[i] = sm.hist[(a - dist + r) & HMASK];
          const uint32_t rn = (r + 1 == dist) ? 0 : r + 1;
          r = q >= lo ? rn : r;
        }
#pragma unroll
        for (uint32_t i = 0; i < 8; i++) w[2 * h + i / 4] |= b[i] << (8 * (i & 3));
      }
      st_block(sm.hist + (Pp & HMASK), make_uint4(w[0], w[1], w[2], w[3]), lo, hi);
    }
  }

  // Up to 64 bytes, one per lane: lane i writes byte a + i.  A literal run
  // reads the input ring at src + i; a match reads the history at
  // a - dist + (i mod dist), which lies before a however the match
  // overlaps itself (a match repeats with period dist).  One read and one
  // write instruction, however short the piece.
  __device__ __forceinline__ void lit_lanes(uint32_t src, uint32_t a, uint32_t n) {
    if (lane < n) sm.hist[(a + lane) & HMASK] = sm.inr[(src + lane) & IMASK];
  }
  __device__ __forceinline__ void match_lanes(uint32_t dist, uint32_t a, uint32_t n) {
    // lane mod dist for lane < 64: a multiply by ceil(2^16 / dist) is exact
    // below dist 64, and from 64 on the lane is its own remainder
    const uint32_t mq = 65535u / dist + 1u;
    const uint32_t r = dist >= 64 ? lane : lane - dist * ((lane * mq) >> 16);
    if (lane < n) sm.hist[(a + lane) & HMASK] = sm.hist[(a - dist + r) & HMASK];
  }

  // the match bytes [a, a + n) of a record (the match started at or before a)
  __device__ void match_exact(uint32_t info, uint32_t a, uint32_t n) {
    const uint32_t dist = rec_dist(info);
    if (n <= 64 && !(info & F_FILL)) {
      match_lanes(dist, a, n);
    } else if (dist == 1) {   // every byte of the run equals the one before a
      uint32_t bb = (info & F_FILL) ? rec_fill(info)
                                    : __builtin_amdgcn_readfirstlane(sm.hist[(a - 1) & HMASK]);
      fill_exact(a, bb, n);
    } else if (dist >= n) {
      copy_exact<HMASK>(sm.hist, a - dist, a, n);   // sources q - dist < a are final
    } else {
      periodic_exact(dist, a, n);
    }
  }

  // Build [T, Tend) record by record, starting at record k.  Every byte
  // before T must be final.  False if a wait for input gave up.
  __device__ __forceinline__ bool tile_exact(uint32_t T, uint32_t Tend) {
    uint32_t j = k;
    for (;;) {
      uint4 r = rec(j);
      const uint32_t os = r.x, src = r.y, L = r.z, info = r.w;
      const uint32_t re = rec_start(j + 1);
      const uint32_t le = os + L;
      uint32_t a = os > T ? os : T, e = le < Tend ? le : Tend;
      if (a < e) {
        if (!need_input(src + (e - os))) return false;
        if (e - a <= 64)
          lit_lanes(src + (a - os), a, e - a);
        else
          copy_exact<IMASK>(sm.inr, src + (a - os), a, e - a);
      }
      a = le > T ? le : T;
      e = re < Tend ? re : Tend;
      if (a < e) match_exact(info, a, e - a);   // LDS ops of one wave stay in order
      if (re >= Tend || j + 1 >= nrec) return true;
      j++;
    }
  }

  // ---- one-pass path

  // One piece of a lane's 16-byte block [P, bend): the bytes that record j's
  // literal run or match puts at [pos, pe), returned as a 16-byte vector
  // aligned to P (the bytes before pos and from pe on are not meaningful).
  // Advances pos to pe, and j past the record when the piece ends it; a lane
  // already at bend stays put.  rve holds each record's end (the next
  // record's start).  Block byte q comes from ring index q + delta: the input
  // ring for literals, the history ring (q - dist) for matches; the 20 bytes
  // that cover the block are read with one 16-byte and one 4-byte LDS load
  // unless they wrap around the ring's end.
  __device__ __forceinline__ uint4 piece(uint4 rv, uint32_t rve, uint32_t T, uint32_t P, uint32_t bend,
                                         uint32_t inr_at, uint32_t hist_at, uint32_t &pos, uint32_t &j) {
    typedef uint32_t u32x4a __attribute__((ext_vector_type(4), aligned(4)));
    const uint32_t j4 = 4 * j;
    const uint32_t os = __builtin_amdgcn_ds_bpermute(j4, rv.x);
    const uint32_t src = __builtin_amdgcn_ds_bpermute(j4, rv.y);
    const uint32_t L = __builtin_amdgcn_ds_bpermute(j4, rv.z);
    const uint32_t info = __builtin_amdgcn_ds_bpermute(j4, rv.w);
    const uint32_t re = __builtin_amdgcn_ds_bpermute(j4, rve);
    const uint32_t le = os + L;
    const bool lit = pos < le;
    const uint32_t pe0 = lit ? le : re;
    const uint32_t pe = pe0 < bend ? pe0 : bend;
    const uint32_t si = P + (lit ? src - os : 0u - rec_dist(info));
    const uint32_t mask = lit ? IMASK : HMASK;
    const uint32_t base = lit ? inr_at : hist_at;
    const uint32_t idx = si & mask & ~3u;
    uint32_t d0, d1, d2, d3, d4;
    if (idx + 20 <= mask + 1) {
      const u32x4a q = *(const __attribute__((address_space(3))) u32x4a *)(uintptr_t)(base + idx);
      d0 = q.x;
      d1 = q.y;
      d2 = q.z;
      d3 = q.w;
      d4 = *(const __attribute__((address_space(3))) uint32_t *)(uintptr_t)(base + idx + 16);
    } else {
      d0 = *(const __attribute__((address_space(3))) uint32_t *)(uintptr_t)(base + idx);
      d1 = *(const __attribute__((address_space(3))) uint32_t *)(uintptr_t)(base + ((idx + 4) & mask));
      d2 = *(const __attribute__((address_space(3))) uint32_t *)(uintptr_t)(base + ((idx + 8) & mask));
      d3 = *(const __attribute__((address_space(3))) uint32_t *)(uintptr_t)(base + ((idx + 12) & mask));
      d4 = *(const __attribute__((address_space(3))) uint32_t *)(uintptr_t)(base + ((idx + 16) & mask));
    }
    const uint32_t sh = si & 3u;
    uint4 v = make_uint4(__builtin_amdgcn_alignbyte(d1, d0, sh), __builtin_amdgcn_alignbyte(d2, d1, sh),
                         __builtin_amdgcn_alignbyte(d3, d2, sh), __builtin_amdgcn_alignbyte(d4, d3, sh));
    if (!lit && (info & F_FILL)) {   // a run of the byte the record carries
      const uint32_t fw = __builtin_amdgcn_perm(0u, info, 0x02020202u);
      v = make_uint4(fw, fw, fw, fw);
    } else if (!lit && rec_dist(info) == 1) {
      // a run of the byte before the run's part in this tile (the byte
      // before the run, or the tile's previous byte, itself of the run)
      const uint32_t at = (le > T ? le : T) - 1;
      const uint32_t fw = (uint32_t)*(const __attribute__((address_space(3))) uint8_t *)(uintptr_t)(
                              hist_at + (at & HMASK)) * 0x01010101u;
      v = make_uint4(fw, fw, fw, fw);
    }
    const bool active = pos < bend;
    j = (active && pe >= re) ? j + 1 : j;
    pos = active ? pe : pos;
    return v;
  }

  // keep the low clamp(s, 0, 32) bits of acc, the rest from v
  __device__ __forceinline__ static uint32_t keep_low(uint32_t acc, uint32_t v, int s) {
    int c;
    asm("v_med3_i32 %0, %1, 0, 32" : "=v"(c) : "v"(s));
    const uint32_t keep = ~(uint32_t)(~0ull << c);
    return (acc & keep) | (v & ~keep);
  }

  // The copies of a tile built before their sources were all final, made
  // again in record order now that they are: record i's copy is the part of
  // its match in [T, Tend) that is not a run of a known byte (rv and rve as
  // for tile_bulk; a tile built this way has no overlapping copy other than
  // distance-1 runs, and every source lies before the bytes it fills).
  __device__ __forceinline__ void redo_copies(uint32_t T, uint32_t Tend, uint4 rv, uint32_t rve, uint32_t m) {
    const uint32_t le = rv.x + rv.z;
    const uint32_t base = le > T ? le : T;
    const uint32_t pend = rve < Tend ? rve : Tend;
    uint64_t cps = __ballot(lane < m && base < pend && !(rv.w & F_FILL));
    while (cps) {
      const uint32_t i = (uint32_t)__builtin_ctzll(cps);
      cps &= cps - 1;
      const uint32_t a = __builtin_amdgcn_readlane(base, i), n = __builtin_amdgcn_readlane(pend, i) - a;
      const uint32_t dist = rec_dist(__builtin_amdgcn_readlane(rv.w, i));
      if (n <= 64) {
        match_lanes(dist, a, n);
      } else if (dist == 1) {   // a run of the byte before it
        fill_exact(a, __builtin_amdgcn_readfirstlane(sm.hist[(a - 1) & HMASK]), n);
      } else {
        copy_exact<HMASK>(sm.hist, a - dist, a, n);   // dist >= n: no source among the bytes written
      }
    }
  }

  // the record (of the m in lanes 0 .. m - 1 of rv) under the first byte of
  // this lane's block of the tile at T
  __device__ __forceinline__ uint32_t first_rec(uint32_t T, uint4 rv, uint32_t m) const {
    const uint32_t P = T + 16 * lane;
    uint32_t j0 = 0;
    for (uint32_t i = 1; i < m; i++) {
      const uint32_t xi = __builtin_amdgcn_readlane(rv.x, i);
      j0 = (xi <= P) ? i : j0;
    }
    return j0;
  }

  // Build [T, Tend) from the m records k .. k + m - 1 held in lanes 0 .. m - 1
  // of rv (lane m holds the end of the last one; rve holds each record's end,
  // the start of the next), in 1 + extra passes.  Each lane builds its 16
  // bytes from the pieces that meet them, in order, from record j0 (the one
  // under the block's first byte).
  __device__ __forceinline__ void tile_bulk(uint32_t T, uint32_t Tend, uint4 rv, uint32_t rve, uint32_t j0,
                                            uint32_t extra) {
    const uint32_t P = T + 16 * lane;
    const uint32_t bend = P + 16 < Tend ? P + 16 : Tend;
    const uint32_t inr_at = lds_addr(sm.inr), hist_at = lds_addr(sm.hist);
    for (uint32_t pass = 0; pass <= extra; pass++) {
      uint32_t pos = P, j = j0;
      uint4 acc = piece(rv, rve, T, P, bend, inr_at, hist_at, pos, j);
      while (__ballot(pos < bend)) {
        const int c8 = (int)(8 * (pos - P));   // bytes before pos are kept
        const uint4 v = piece(rv, rve, T, P, bend, inr_at, hist_at, pos, j);
        acc.x = keep_low(acc.x, v.x, c8);
        acc.y = keep_low(acc.y, v.y, c8 - 32);
        acc.z = keep_low(acc.z, v.z, c8 - 64);
        acc.w = keep_low(acc.w, v.w, c8 - 96);
      }
      // the last block of a chunk's last tile is stored only up to the end:
      // its ring slot beyond holds bytes that a later pass may still read
      if (P + 16 <= Tend) *(uint4 *)(sm.hist + (P & HMASK)) = acc;
      else if (P < Tend) st_block(sm.hist + (P & HMASK), acc, 0, Tend - P);
    }
  }

  __device__ __forceinline__ void run() {
    const uint32_t ntiles = (N + TILE - 1) / TILE;
    constexpr bool G = MODE == MODE_INT4G || MODE == MODE_GEMV;
    const bool fast = G || (MODE == MODE_INT4 && P.group_shift < 64 && P.group >= 8);
    // Each tile's scales and zero points are fetched one tile ahead, so their
    // latency overlaps the build of the tile before.
    // Tiles are taken in increasing order from a shared counter (builder b
    // starts with tile b), each builder taking its next one when it starts
    // the current, so a slow tile holds up only the builder that has it.
    // Every tile below the smallest of the builders' current tiles is final.
    const bool few = fast && P.group_shift >= 7;
    const uint32_t lane31 = lane & 31u;
    const uint64_t ng = G ? (2 * P.total + P.group - 1) >> P.group_shift : 0;
    // the loads of the next tile's scales and zero points are issued once
    // the current tile's write-out has used them: loading into registers
    // that a copy still has to read would make the compiler wait for every
    // load and store in flight, the previous tile's stores included
    Meta4 cur{};
    MetaG cug{};
    MetaG gm{};
    float4_t gacc[2] = {};
    if constexpr (MODE == MODE_GEMM) {
      if (b < ntiles) gm = gemm_meta(P, dst0, b, lane);
    } else if constexpr (G) {
      if (b < ntiles) cug = int4g_meta(P, dst0, b, lane31, ng);
    } else {
      if (fast && b < ntiles) cur = int4_meta(P, dst0, b, lane, N, few);
    }
    uint32_t u;
    for (uint32_t t = b; t < ntiles; t = u) {
      // MODE_GEMM assigns tiles statically (builder b takes b, b + nbs, ...):
      // each builder's partial products then cover a fixed set of tiles,
      // summed in a fixed order, so the product is the same bits every call
      if constexpr (LPF) prio_by_progress(t, ntiles);
      const uint32_t uv = MODE == MODE_GEMM ? 0u : grab_issue();
      const uint32_t T = t * TILE;
      const uint32_t Tend = T + TILE < N ? T + TILE : N;
      if (!wait_cov(T, Tend)) break;
      find_k(T);
      // records k .. k + 63 in lanes, missing ones read as {cov, 0, 0, 0};
      // lane i also reads where record k + i ends (the next one's start)
      const uint32_t jr = k + lane;
      uint4 rv = make_uint4(cov, 0u, 0u, 0u);
      uint32_t re = cov;
      if (jr < nrec) rv = sm.recs[ridx_lane(k, lane)];
      if (jr + 1 < nrec) re = sm.recs[ridx_lane(k + 1, lane)].x;
      announce_rec(T, __builtin_amdgcn_readfirstlane(rv.x), __builtin_amdgcn_readfirstlane(rv.y),
                   __builtin_amdgcn_readfirstlane(rv.z));
      const uint32_t m = __builtin_popcountll(__ballot(jr < nrec && rv.x < Tend));
      // classify: one pass possible?  how many passes?  which input and
      // which earlier tiles are read?
      // (the sources' bound also serves hard tiles; a tile of 64 records or
      // more takes it from a scan of all its records)
      const bool seen = m < 64;
      bool hard = !seen;
      uint32_t extra = 0, src_need = 0, in_end = 0;
      if (seen) {   // lane i looks at record i
        const bool mine = lane < m;
        const uint32_t le = rv.x + rv.z;
        const bool lit = mine && le > T;   // literals in this tile
        const uint32_t base = le > T ? le : T;
        const uint32_t pend = re < Tend ? re : Tend;
        const bool copy = mine && base < pend && !(rv.w & F_FILL);
        const uint32_t dist = rec_dist(rv.w);
        // the copy's sources end here; a distance-1 run without its byte
        // reads the one byte before base
        const uint32_t s_hi = dist == 1 ? base : pend - dist;
        if (__ballot(copy && dist > 1 && (dist < 16 || dist < pend - base))) hard = true;   // overlapping copy
        extra = (uint32_t)__builtin_popcountll(__ballot(copy && s_hi > T));        // reads this tile
        if (m > BULK_RECS && BULK_RATIO * (1 + extra) > m) hard = true;
        const uint64_t lits = __ballot(lit);
        if (lits) {   // the last literal run in the tile ends the input it reads
          const uint32_t li = 63 - __builtin_clzll(lits);
          const uint32_t e = le < Tend ? le : Tend;
          in_end = __builtin_amdgcn_readlane(rv.y + (e - rv.x), li);
        }
        uint64_t cps = __ballot(copy);
        const uint32_t s_fin = s_hi < T ? s_hi : T;
        while (cps) {   // earlier tiles read by copies
          const uint32_t ci = __builtin_ctzll(cps);
          cps &= cps - 1;
          const uint32_t v = __builtin_amdgcn_readlane(s_fin, ci);
          src_need = v > src_need ? v : src_need;
        }
      } else {
        // 64 records or more: built record by record, after the earlier
        // tiles its copies read (every record of the tile is in the ring)
        for (uint32_t w = 0;; w += 64) {
          const uint32_t jw = k + w + lane;
          uint4 r2 = make_uint4(cov, 0u, 0u, 0u);
          uint32_t re2 = cov;
          if (jw < nrec) r2 = sm.recs[ridx_lane(k + w, lane)];
          if (jw + 1 < nrec) re2 = sm.recs[ridx_lane(k + w + 1, lane)].x;
          const bool mine = jw < nrec && r2.x < Tend;
          const uint32_t le = r2.x + r2.z;
          const uint32_t base = le > T ? le : T;
          const uint32_t pend = re2 < Tend ? re2 : Tend;
          const bool copy = mine && base < pend && !(r2.w & F_FILL);
          const uint32_t s_hi = rec_dist(r2.w) == 1 ? base : pend - rec_dist(r2.w);
          const uint32_t s_fin = copy ? (s_hi < T ? s_hi : T) : 0u;
          uint32_t v = s_fin;
          for (int o = 32; o >= 1; o >>= 1) {
            const uint32_t x = (uint32_t)__shfl_xor((int)v, o);
            v = x > v ? x : v;
          }
          v = __builtin_amdgcn_readfirstlane(v);
          src_need = v > src_need ? v : src_need;
          if (__ballot(mine) != ~0ull) break;
        }
      }
      u = MODE == MODE_GEMM ? t + nbs : grab_take(uv);
      // tiles before this one that are read
      uint32_t need_tiles = (src_need + TILE - 1) / TILE;
      uint32_t slot_tiles = 0;   // the tiles the slot rule alone waits for
      uint32_t written = 0;
      if (t >= HTILES) {
        // This tile overwrites the ring slot of tile t - HTILES, whose
        // write-out reads it and whose bytes only tiles up to
        // t - HTILES + reach read (a match reaches at most reach tiles
        // back): the first must be written out and those built first.  When
        // that bound does not stay short of this tile, wait for every
        // earlier tile;
        // and since sources up to a ring length back then share this tile's
        // own slot, build it sequence by sequence (every such source lies
        // ahead of the bytes written so far) rather than in passes that
        // would read their own stores.
        const uint32_t reach = (P.dmax + TILE - 1) / TILE;
        if (reach < HTILES) {
          const uint32_t fin = t - HTILES + reach + 1;
          need_tiles = need_tiles > fin ? need_tiles : fin;
          slot_tiles = fin;
        } else {
          if (extra) hard = true;
          need_tiles = t;
          slot_tiles = t;
        }
      }
      if (t >= HTILES) written = t - HTILES + 1;
      // The tiles after this one wait for it, so while its sources are not
      // all built it is built at once from whatever the history holds
      // (literals and runs of a known byte are final then), and after the
      // wait only its copies are made again, in record order: the wait ends
      // in a few copies instead of a whole build.  (Only when no source can
      // share this tile's own slot: slot_tiles < need_tiles then.)  The
      // record under each lane's first byte is found before the wait too.
      uint32_t j0 = 0;
      if constexpr (SPEC) {
        if (!hard) j0 = first_rec(T, rv, m);
      }
      const bool spec = SPEC && !hard && slot_tiles < need_tiles && !ready(need_tiles, written);
      if (!wait_done(spec ? slot_tiles : need_tiles, written)) break;
      if (hard) {
        if (!tile_exact(T, Tend)) break;
      } else {
        if (!need_input(in_end)) break;
        if constexpr (!SPEC) j0 = first_rec(T, rv, m);
        tile_bulk(T, Tend, rv, re, j0, spec ? 0u : extra);
        if (spec) {
          if (!wait_done(need_tiles, written)) break;
          redo_copies(T, Tend, rv, re, m);
        }
      }
      // the tile's history bytes are final: tiles that copy from it may
      // start while it is written out
      lds_set(&ctl.built[b], u, lane);
      if constexpr (MODE == MODE_GEMM) {
        gemm_tile<HLOG>(sm, lane, P, dst0, T, gm, gacc);
      } else {
        if constexpr (G) {
          cur.s[0] = cug.s;
          cur.z[0] = cug.z;
          cur.g0 = (uint32_t)((2 * (dst0 + T)) >> P.group_shift);
        }
        if (few && Tend - T == TILE) {
          meta_pack_few(cur, P.zp != nullptr);
          flush_int4_few<MODE, HLOG>(sm, lane, P, dst0, T, cur);
        } else {
          if (fast) meta_ready(cur, P.zp != nullptr, P, dst0, t, lane, N, few);
          flush_tile<MODE, HLOG>(sm, lane, P, dst0, t, N, cur, fast);
        }
      }
      lds_set(&ctl.next_tile[b], u, lane);
      if constexpr (MODE == MODE_GEMM) {
        if (u < ntiles) gm = gemm_meta(P, dst0, u, lane);
      } else if constexpr (G) {
        if (u < ntiles) cug = int4g_meta(P, dst0, u, lane31, ng);
      } else {
        if (fast && u < ntiles) cur = int4_meta(P, dst0, u, lane, N, few);
      }
    }
    if constexpr (MODE == MODE_GEMM) gemm_store(P, chunk, b, lane, gacc);
    lds_set(&ctl.need[1 + b], 0xFFFFFFFFu, lane);
    lds_set(&ctl.bk[b], 0xFFFFFFFFu, lane);
    lds_set(&ctl.built[b], 0xFFFFFFFFu, lane);
    lds_set(&ctl.next_tile[b], 0xFFFFFFFFu, lane);
    if (lane == 0) __hip_atomic_fetch_add(&ctl.nfinished, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  }
};

// -------------------------------------------------------------- kernel

template <int MODE, int HLOG, bool SPEC, bool LPF>
__global__ void __launch_bounds__(NTHREADS) __attribute__((amdgpu_waves_per_eu(8, 8))) chunk_kernel(ChunkParams P) {
  __shared__ __attribute__((aligned(16))) Smem<HLOG> sm;
  __shared__ Ctl ctl;
  uint32_t i = blockIdx.x;
  if (P.order) {
    i = __builtin_amdgcn_readfirstlane(P.order[i]);
    if (i >= P.n) return;   // the whole workgroup, before any barrier
  }
  const uint32_t tid = threadIdx.x;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid / 64);
  const uint32_t lane = tid & 63;

  uint64_t c0 = P.comp_off[i], c1 = P.comp_off[i + 1];
  uint64_t d0 = P.dst_off[i], d1 = P.dst_off[i + 1];
  bool bad = c0 < P.comp_base || c0 > c1 || c1 - P.comp_base > P.comp_bytes || d0 > d1 || d1 > P.total ||
             d0 < P.d_first || d1 > P.d_last || (i == 0 && d0 != P.d_first) ||
             (i == P.n - 1 && d1 != P.d_last) || (d0 & 15) != 0 ||
             (MODE == MODE_GEMV && ((d0 | d1) & (TILE - 1)) != 0) ||
             (MODE == MODE_GEMM && (((d0 | d1) & (TILE - 1)) != 0 || d1 == d0 ||
                                    d0 / TILE / P.gemm_tpr != (d1 - 1) / TILE / P.gemm_tpr)) ||
             d1 - d0 > (uint64_t)P.max_chunk || c1 - c0 > (uint64_t)LEN_CAP;
  c0 -= P.comp_base;
  c1 -= P.comp_base;
  uint64_t s0 = 0, s1 = 0;
  if (P.seq_off) {
    s0 = P.seq_off[i];
    s1 = P.seq_off[i + 1];
    bad = bad || s0 > s1 || s1 > P.n_seq || s1 - s0 > (uint64_t)LEN_CAP;
  }
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

  // with a sequence index the walker makes the records itself and wave 1
  // becomes one more builder
  const bool direct = P.seq_pos != nullptr && s1 > s0;
  // With checksums one builder wave hashes instead: wave 1 with an index
  // (six builders become five), wave 7 without (five become four).
  const bool check = P.xxh != nullptr;
  const uint32_t nb = (uint32_t)NB + (direct ? 1u : 0u) - (check ? 1u : 0u);
  const uint32_t hwave = check ? (direct ? 1u : 7u) : 0xFFFFFFFFu;
  if (tid < NSLOT) {
    ctl.need[tid] = (tid <= nb || (check && tid == HSLOT)) ? 0u : 0xFFFFFFFFu;
    ctl.bk[tid] = tid < nb ? 0u : 0xFFFFFFFFu;
    ctl.next_tile[tid] = tid < nb ? tid : 0xFFFFFFFFu;
    ctl.built[tid] = tid < nb ? tid : 0xFFFFFFFFu;
  }
  if (tid == 0) {
    ctl.in_avail = 0;
    ctl.nrec = 0;
    ctl.cov = 0;
    ctl.pstate = ST_RUN;
    ctl.wcnt = 0;
    ctl.rcons = 0;
    ctl.nfinished = 0;
    ctl.tile_ctr = nb;
    ctl.status = 0;
    ctl.stall = 0;
    ctl.xbad = 0;
  }
  __syncthreads();

  if (wave == 0) {
    // INT8 tiles write half the fp16 bytes of INT4 tiles per decoded byte,
    // so their builders have slack and the walk sets the pace: the walker
    // then issues ahead of them (11% faster on an 8192 x 8192 matrix; with
    // INT4 or bytes output the same priority measured 1-3% slower).
    // Sequence-dense tables take prio_by_progress instead.
    if constexpr (MODE == MODE_INT8 && !LPF) __builtin_amdgcn_s_setprio(1);
    Walker<Smem<HLOG>, LPF> W{sm, ctl, lane, head, y_end, N, 0, 0xFFFFFF00u, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0, 0,
                         direct ? P.seq_pos + s0 : nullptr, direct ? (uint32_t)(s1 - s0) : 0u, 0, head, 0, 0, 0,
                         Rec<Smem<HLOG>>{sm, P.dmax, ctl, lane, N, 0, 0, 0, 0, 0, 0}, direct ? 1u : 0u, -1};
    W.spin = P.spin;
    W.rec.spin = P.spin;
    W.run();
    if (direct) {
      // every walk ends with a final status (the last sequence or an error)
      const int32_t st = W.fin >= 0 ? W.fin : C_TABLE;
      if (lane == 0) ctl.status = st;
      lds_set(&ctl.pstate, st == C_OK ? ST_DONE : ST_FAIL, lane);
    }
    if constexpr (MODE == MODE_GEMM) {   // the slots of builders this chunk does not have
      const float4_t zero[2] = {};
      for (uint32_t slot = nb; slot < GEMM_SLOTS; slot++) gemm_store(P, i, slot, lane, zero);
    }
  } else if (wave == 1 && !direct) {
    Rec<Smem<HLOG>> R{sm, P.dmax, ctl, lane, N, 0, 0, 0, 0, 0, 0};
    R.spin = P.spin;
    const int32_t st = recorder(R, sm, ctl, lane);
    if (lane == 0) ctl.status = st;
    lds_set(&ctl.pstate, st == C_OK ? ST_DONE : ST_FAIL, lane);
  } else if (wave == 2) {
    feeder<Smem<HLOG>, LPF>(sm, ctl, lane, S, y_end, nb, P.spin, check);
  } else if (wave == hwave) {
    hasher(sm, ctl, lane, head, y_end, P.xxh[i], P.spin);
  } else {   // waves 3 .. 7 are builders 0 .. 4; with an index wave 1 is builder 5
    Builder<MODE, HLOG, SPEC, LPF> B{sm, ctl, P, d0, lane, wave == 1 ? (uint32_t)NB : wave - 3, N, 0, 0, 0, 0, 0, 0, 0};
    B.chunk = i;
    B.nbs = nb;
    B.run();
  }
  __syncthreads();
  // a stall first, then a checksum mismatch (the stored bytes are wrong,
  // whatever their decode gave), then the decode's own status
  if (tid == 0 && P.status) P.status[i] = ctl.stall ? C_STALL : ctl.xbad ? C_CHECKSUM : ctl.status;
}

}  // namespace lt
