// lt_api.hip -- liblt's C ABI: argument checks and kernel launches.
//
// Entry points follow the calls the roadmap page sketches ("GPU Compression
// Pipeline - TDD Roadmap": INT4 dequantization in Phase 1.1, INT8 in Phase
// 1.2, fused LZ4 + INT4 in Phase 2.1, parallel LZ4 decode in Phase 3.1),
// reshaped for a chunk table of independent LZ4 blocks and caller-owned
// device buffers.  Everything runs on the caller's stream; nothing here
// allocates, synchronizes or keeps state.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <unistd.h>

#include <algorithm>
#include <atomic>
#include <mutex>
#include <thread>
#include <vector>

#include "lt.h"
#include "lt_device.hpp"
#include "lt_lz4.hpp"
#include "lt_verify.hpp"
#include "lt_zr.hpp"

namespace lt {

// ------------------------------------------------- raw (uncompressed) dequant

struct RawParams {
  const uint8_t *src;        // packed int4 or int8 codes
  const uint16_t *scales;
  const int8_t *zp;
  uint64_t n_bytes;          // bytes of src
  uint64_t group;
  uint32_t group_shift;      // log2(group) if group is a power of two, else 64
  uint16_t *out;
  uint64_t e_base;           // element index of src's first code (groups count from 0)
};

constexpr int RAW_THREADS = 256;
constexpr int RAW_UNROLL = 4;   // dwords per thread

__device__ __forceinline__ uint64_t grp(uint64_t e, const RawParams &P) {
  e += P.e_base;
  return P.group_shift < 64 ? (e >> P.group_shift) : e / P.group;
}

// INT4 with groups that are a power of two of at least 64 codes, in tiles of
// 1 KiB of packed codes (2048 codes, at most 33 groups): one wave per tile.
// Lane l reads dword k = bytes 256 k + 4 l (each load instruction reads 256
// contiguous bytes) and writes codes 512 k + 8 l .. + 7 as 16 bytes of fp16
// (each store instruction writes 1 KiB contiguously).  Lanes 0 .. 63 fetch
// the scale and zero point of groups g0 .. g0 + 63 once per tile, as the two
// packed constants of deq8_int4_dual, and every lane takes its group's from
// the lane that holds it (ds_bpermute).
constexpr int RAWT_THREADS = 512;
__global__ void __launch_bounds__(RAWT_THREADS) dequant_int4_tiles(RawParams P, uint64_t ntiles) {
  const uint32_t lane = threadIdx.x & 63u;
  const uint64_t nwaves = (uint64_t)gridDim.x * (RAWT_THREADS / 64);
  const uint64_t ng = (2 * P.n_bytes + P.group - 1) >> P.group_shift;
  // without zero points, read any valid byte and discard it (no branch)
  const int8_t *zsrc = P.zp ? P.zp : (const int8_t *)P.scales;
  const bool has_zp = P.zp != nullptr;
  for (uint64_t w = (uint64_t)blockIdx.x * (RAWT_THREADS / 64) + (threadIdx.x >> 6); w < ntiles; w += nwaves) {
    const uint8_t *src = P.src + 1024 * w + 4 * lane;
    uint32_t d[4];
#pragma unroll
    for (int k = 0; k < 4; k++) d[k] = *(const uint32_t *)(src + 256 * k);
    const uint64_t e = 2048 * w;   // the tile's first code
    const uint64_t g0 = e >> P.group_shift;
    const uint64_t left = ng - g0;   // >= 1
    const uint32_t li = lane < left ? lane : (uint32_t)left - 1;
    const uint32_t sv = P.scales[g0 + li];
    const int z = has_zp ? (int)zsrc[g0 + li] : 0;
    const uint32_t s2 = (sv & 0xFFFFu) * 0x10001u;
    const uint32_t c2 = f16_bits_int(1024 + z) | (f16_bits_int(64 + z) << 16);
    const uint32_t off = (uint32_t)(e & (P.group - 1)) + 8 * lane;
    uint4 *out = (uint4 *)(P.out + e) + lane;
#pragma unroll
    for (int k = 0; k < 4; k++) {
      const uint32_t i = (off + 512 * k) >> P.group_shift;
      const h2 c = as_h2((uint32_t)__builtin_amdgcn_ds_bpermute(4 * i, c2));
      const h2 sc = as_h2((uint32_t)__builtin_amdgcn_ds_bpermute(4 * i, s2));
      out[64 * k] = deq8_int4_dual(d[k], c, sc);
    }
  }
}

// Codebook INT4 (a 16-entry fp16 table per group of at least 16 codes):
// element e is entry q(e) of its group's table.  A workgroup takes 8192
// codes, one 2048-code tile per wave in the lane layout above (each load
// instruction reads 256 contiguous bytes, each store writes 1 KiB), and
// first stages the at most 513 tables its codes use in LDS.
struct LutParams {
  const uint8_t *src;
  const uint16_t *lut;
  uint64_t n;                // codes
  uint64_t group;
  uint32_t group_shift;      // log2(group) if a power of two, else 64
  uint16_t *out;
};
constexpr int LUT_THREADS = 256;
constexpr uint32_t LUT_CODES = 2048 * (LUT_THREADS / 64);
constexpr uint32_t LUT_ROWS = LUT_CODES / 16 + 2;

__device__ __forceinline__ uint64_t lut_group(const LutParams &P, uint64_t e) {
  return P.group_shift < 64 ? e >> P.group_shift : e / P.group;
}

__global__ void __launch_bounds__(LUT_THREADS) dequant_int4_lut_kernel(LutParams P) {
  __shared__ __attribute__((aligned(16))) uint16_t tab[LUT_ROWS * 16];
  const uint32_t lane = threadIdx.x & 63u, wave = threadIdx.x >> 6;
  const uint64_t e0 = (uint64_t)blockIdx.x * LUT_CODES;
  const uint64_t e1 = e0 + LUT_CODES < P.n ? e0 + LUT_CODES : P.n;
  const uint64_t g0 = lut_group(P, e0);
  const uint32_t rows = (uint32_t)(lut_group(P, e1 - 1) - g0 + 1);
  const uint4 *lsrc = (const uint4 *)(P.lut + 16 * g0);
  for (uint32_t i = threadIdx.x; i < 2 * rows; i += LUT_THREADS) ((uint4 *)tab)[i] = lsrc[i];
  __syncthreads();
  const uint64_t te = e0 + 2048 * wave;
#pragma unroll
  for (int k = 0; k < 4; k++) {
    const uint64_t eb = te + 512 * k + 8 * lane;   // this lane's 8 codes
    if (eb >= P.n) break;
    const bool whole = eb + 8 <= P.n;
    uint32_t d = 0;
    if (whole) {
      d = *(const uint32_t *)(P.src + eb / 2);
    } else {
      for (uint32_t j = 0; 2 * j < P.n - eb; j++) d |= (uint32_t)P.src[eb / 2 + j] << (8 * j);
    }
    uint64_t g = lut_group(P, eb);
    uint64_t next = (g + 1) * P.group;
    uint32_t v[8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
      if (eb + i >= next) {   // groups of 16 or more: at most one step per 8 codes
        g++;
        next += P.group;
      }
      v[i] = tab[16 * (uint32_t)(g - g0) + ((d >> (4 * i)) & 15u)];
    }
    if (whole) {
      *(uint4 *)(P.out + eb) = make_uint4(v[0] | v[1] << 16, v[2] | v[3] << 16, v[4] | v[5] << 16, v[6] | v[7] << 16);
    } else {
      for (int i = 0; i < 8; i++)
        if (eb + i < P.n) P.out[eb + i] = (uint16_t)v[i];
    }
  }
}

__global__ void __launch_bounds__(256) zero_f32(float *y, uint64_t n) {
  for (uint64_t i = (uint64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (uint64_t)gridDim.x * 256) y[i] = 0.0f;
}

// Each thread takes RAW_UNROLL dwords spaced a workgroup-width apart, so each
// load instruction reads 1 KiB and each store instruction writes 4 KiB (int4)
// contiguously across the workgroup.
__global__ void __launch_bounds__(RAW_THREADS) dequant_int4_kernel(RawParams P) {
  const uint64_t n_dw = P.n_bytes / 4;
  const uint64_t base = (uint64_t)blockIdx.x * RAW_THREADS * RAW_UNROLL + threadIdx.x;
  uint32_t w[RAW_UNROLL];
#pragma unroll
  for (int k = 0; k < RAW_UNROLL; k++) {
    uint64_t d = base + (uint64_t)k * RAW_THREADS;
    if (d < n_dw) __builtin_memcpy(&w[k], P.src + 4 * d, 4);
  }
#pragma unroll
  for (int k = 0; k < RAW_UNROLL; k++) {
    uint64_t d = base + (uint64_t)k * RAW_THREADS;
    if (d < n_dw) {
      uint64_t e0 = 8 * d;
      uint64_t g0 = grp(e0, P), g1 = grp(e0 + 7, P);
      if (g0 == g1) {
        int z = P.zp ? (int)P.zp[g0] : 0;
        uint4 r = deq8_int4(w[k], splat_h2((uint16_t)f16_bits_1024_plus(z)), splat_h2(P.scales[g0]));
        *(uint4 *)(P.out + e0) = r;
      } else {
        for (int c = 0; c < 8; c++) {
          uint64_t g = grp(e0 + c, P);
          int z = P.zp ? (int)P.zp[g] : 0;
          P.out[e0 + c] = deq1((w[k] >> (4 * c)) & 15, z, P.scales[g]);
        }
      }
    }
  }
  // trailing bytes (n_bytes % 4) go to the first thread of the grid
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    for (uint64_t b = n_dw * 4; b < P.n_bytes; b++) {
      uint32_t v = P.src[b];
      for (int c = 0; c < 2; c++) {
        uint64_t e = 2 * b + c;
        uint64_t g = grp(e, P);
        int z = P.zp ? (int)P.zp[g] : 0;
        P.out[e] = deq1((v >> (4 * c)) & 15, z, P.scales[g]);
      }
    }
  }
}

__global__ void __launch_bounds__(RAW_THREADS) dequant_int8_kernel(RawParams P) {
  // each thread: RAW_UNROLL pairs of dwords (8 codes -> 16 output bytes)
  const uint64_t n_q = P.n_bytes / 8;
  const uint64_t base = (uint64_t)blockIdx.x * RAW_THREADS * RAW_UNROLL + threadIdx.x;
  uint2 w[RAW_UNROLL];
#pragma unroll
  for (int k = 0; k < RAW_UNROLL; k++) {
    uint64_t d = base + (uint64_t)k * RAW_THREADS;
    if (d < n_q) __builtin_memcpy(&w[k], P.src + 8 * d, 8);
  }
#pragma unroll
  for (int k = 0; k < RAW_UNROLL; k++) {
    uint64_t d = base + (uint64_t)k * RAW_THREADS;
    if (d < n_q) {
      uint64_t e0 = 8 * d;
      uint64_t g0 = grp(e0, P), g1 = grp(e0 + 7, P);
      if (g0 == g1) {
        int z = P.zp ? (int)P.zp[g0] : 0;
        h2 c2 = splat_h2((uint16_t)f16_bits_1024_plus(128 + z)), s2 = splat_h2(P.scales[g0]);
        uint2 a = deq4_int8(w[k].x, c2, s2), b = deq4_int8(w[k].y, c2, s2);
        *(uint4 *)(P.out + e0) = make_uint4(a.x, a.y, b.x, b.y);
      } else {
        for (int c = 0; c < 8; c++) {
          uint64_t g = grp(e0 + c, P);
          int z = P.zp ? (int)P.zp[g] : 0;
          uint32_t word = (c < 4) ? w[k].x : w[k].y;
          P.out[e0 + c] = deq1((int)(int8_t)(word >> ((c & 3) * 8)), z, P.scales[g]);
        }
      }
    }
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    for (uint64_t e = n_q * 8; e < P.n_bytes; e++) {
      uint64_t g = grp(e, P);
      int z = P.zp ? (int)P.zp[g] : 0;
      P.out[e] = deq1((int)(int8_t)P.src[e], z, P.scales[g]);
    }
  }
}

}  // namespace lt

// ---------------------------------------------------------------- C ABI

namespace {

bool aligned16(const void *p) { return ((uintptr_t)p & 15) == 0; }

// rows*cols elements in groups of `group`; see lt.h for the rule.
bool shape_ok(uint64_t rows, uint64_t cols, uint64_t group) {
  if (rows == 0 || cols == 0 || group == 0) return false;
  if (rows > (~0ull) / cols) return false;
  uint64_t n = rows * cols;
  if (n > (1ull << 48)) return false;
  if (cols % group != 0 && group % cols != 0) return false;
  if (n % group != 0) return false;
  return true;
}

uint32_t shift_of(uint64_t g) {
  return (g & (g - 1)) == 0 ? (uint32_t)__builtin_ctzll(g) : 64u;
}

template <int MODE, bool SPEC, bool LPF = false>
void launch_kernel(bool small, hipStream_t s, const lt::ChunkParams &P) {
  if (small) {
    hipLaunchKernelGGL((lt::chunk_kernel<MODE, 14, SPEC, LPF>), dim3(P.n), dim3(lt::NTHREADS), 0, s, P);
  } else {
    hipLaunchKernelGGL((lt::chunk_kernel<MODE, 16, SPEC, LPF>), dim3(P.n), dim3(lt::NTHREADS), 0, s, P);
  }
}

// the kernel for a table that takes the speculative build: with progress
// priority too when its index shows it sequence-dense (lt::prio_by_progress)
template <int MODE>
void launch_spec(bool dense, bool small, hipStream_t s, const lt::ChunkParams &P) {
  dense ? launch_kernel<MODE, true, true>(small, s, P) : launch_kernel<MODE, true, false>(small, s, P);
}

lt_status launch_params(int mode, lt::ChunkParams &P, void *stream) {
  hipStream_t s = (hipStream_t)stream;
  // a declared short window lets each chunk keep a 16 KiB history, so more
  // chunks share a CU
  const bool small = P.dmax <= LT_SMALL_WINDOW;
  if (mode == lt::MODE_INT4 && P.group_shift < 64 && P.group >= 128) mode = lt::MODE_INT4G;
  // Speculative tile builds pay where tiles wait on the tiles just before
  // them: general-purpose LZ4 parses (about 4.5 sequences per KiB on INT4
  // weights, twice as fast with them) and activations (decode-only always
  // takes them).  On the host packer's weight blocks (about 2.6 per KiB)
  // they cost 1-2.5%, so a table whose index counts fewer than 3.5
  // sequences per KiB goes without; a table without an index takes them.
  // The sequence-dense tables (index present, 3.5 or more per KiB) also take
  // progress priority; without an index the density is unknown and the
  // weight tables the packer writes are not dense, so those keep the
  // default (oldest waves first).
  const bool dense = P.seq_off && P.n_seq * 2048 >= 7 * P.total;
  const bool spec = !P.seq_off || dense;
  switch (mode) {
    case lt::MODE_BYTES: launch_spec<lt::MODE_BYTES>(dense, small, s, P); break;
    case lt::MODE_INT4:
      spec ? launch_spec<lt::MODE_INT4>(dense, small, s, P) : launch_kernel<lt::MODE_INT4, false>(small, s, P);
      break;
    case lt::MODE_INT8:
      spec ? launch_spec<lt::MODE_INT8>(dense, small, s, P) : launch_kernel<lt::MODE_INT8, false>(small, s, P);
      break;
    case lt::MODE_INT4G:
      spec ? launch_spec<lt::MODE_INT4G>(dense, small, s, P) : launch_kernel<lt::MODE_INT4G, false>(small, s, P);
      break;
    case lt::MODE_GEMV: launch_kernel<lt::MODE_GEMV, false>(small, s, P); break;
    case lt::MODE_GEMM: launch_kernel<lt::MODE_GEMM, false>(small, s, P); break;
    default: return LT_ERR_UNSUPPORTED;
  }
  return hipGetLastError() == hipSuccess ? LT_OK : LT_ERR_LAUNCH;
}

lt::ChunkParams make_params(const lt_chunk_table *t, void *out, int32_t *chunk_status, const uint16_t *scales,
                            const int8_t *zp, uint64_t group) {
  lt::ChunkParams P;
  P.comp = t->comp;
  P.comp_off = t->comp_off;
  P.dst_off = t->dst_off;
  P.comp_bytes = t->comp_bytes;
  P.total = t->total_bytes;
  P.n = t->n_chunks;
  P.max_chunk = t->max_chunk_bytes;
  P.out = out;
  P.status = chunk_status;
  P.scales = scales;
  P.zp = zp;
  P.group = group;
  P.group_shift = shift_of(group);
  P.dmax = t->max_dist ? t->max_dist : 65535u;
  P.seq_off = t->seq_off;
  P.seq_pos = t->seq_pos;
  P.n_seq = t->seq_off ? t->n_seq : 0;
  P.comp_base = 0;
  P.d_first = 0;
  P.d_last = t->total_bytes;
  P.gemv_x = nullptr;
  P.gemv_y = nullptr;
  P.cols = 0;
  P.gemm_part = nullptr;
  P.gemm_nbt = 0;
  P.gemm_tpr = 1;
  P.spin = t->spin_limit ? t->spin_limit : lt::SPIN_DEFAULT;
  P.order = t->order;
  P.xxh = t->xxh;
  return P;
}

lt_status launch_chunks(int mode, const lt_chunk_table *t, void *out, int32_t *chunk_status,
                        const uint16_t *scales, const int8_t *zp, uint64_t group, void *stream) {
  lt::ChunkParams P = make_params(t, out, chunk_status, scales, zp, group);
  return launch_params(mode, P, stream);
}

// ------------------------------------------------------------ streaming

constexpr uint64_t kAlign = 256;
uint64_t up(uint64_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

// Staging layout for a host table t: first the whole table's offsets,
// checksums and sequence index (copied once, before the first batch), then
// two halves that take the compressed bytes of alternate batches.  Every piece starts
// on a 256-byte boundary.
uint64_t meta_bytes(const lt_chunk_table *t) {
  const uint64_t n = t->n_chunks;
  uint64_t b = 2 * up(8 * (n + 1));
  if (t->xxh) b += up(8 * n);
  if (t->seq_off) b += up(8 * (n + 1)) + up(4 * t->seq_off[n]);
  return b;
}

// Bytes a half needs for the compressed bytes of chunks [c, e), plus one
// 16-byte block the decoder may read past the last chunk.
uint64_t batch_bytes(const lt_chunk_table *t, uint64_t c, uint64_t e) {
  return up(t->comp_off[e] - t->comp_off[c] + 16);
}

// Where a streamed batch's compressed bytes come from when they are not in
// host memory: a file, read with pread into the two halves of a pinned host
// buffer in turn.  The calling thread reads batch b while the copy and the
// decode of the batches before it run on the streams; a half is read into
// again only once the copy that last read it has finished.
struct FileSource {
  int fd;
  uint64_t offset;    // file offset of compressed byte 0
  uint8_t *pinned;    // pinned host memory, two halves of `half` bytes
  uint64_t half;
  int threads;        // reader threads per batch
};

// Read len bytes at file offset off into dst, in up to `threads` pieces
// read side by side; false on an error or an early end of file.
bool read_range(int fd, uint64_t off, uint64_t len, uint8_t *dst, int threads) {
  auto rd = [&](uint64_t a, uint64_t b) {
    while (a < b) {
      const ssize_t r = pread(fd, dst + a, (size_t)std::min<uint64_t>(b - a, 1ull << 30), (off_t)(off + a));
      if (r <= 0) return false;
      a += (uint64_t)r;
    }
    return true;
  };
  constexpr uint64_t kPiece = 1ull << 20;   // no thread reads less
  const uint64_t pieces = (len + kPiece - 1) / kPiece;
  const int T = (int)std::min<uint64_t>(std::max(threads, 1), std::max<uint64_t>(pieces, 1));
  if (T <= 1) return rd(0, len);
  const uint64_t per = (len + T - 1) / T;
  std::atomic<bool> ok{true};
  std::vector<std::thread> pool;
  for (int k = 1; k < T; k++)
    pool.emplace_back([&, k] {
      const uint64_t a = k * per, b = std::min(len, a + per);
      if (a < b && !rd(a, b)) ok = false;
    });
  if (!rd(0, std::min(len, per))) ok = false;
  for (auto &th : pool) th.join();
  return ok;
}

// Copy-and-decode of a table whose arrays are in host memory: batches of
// chunks go to the two halves of a device staging buffer in turn, the
// copies on copy_stream and the decode on stream, each half reused once the
// decode of the batch before it in that half has finished.  The offsets and
// the index travel once, ahead of the first batch: many small copies per
// batch cost more than the batch's compressed bytes.
lt_status stream_common(int mode, const lt_chunk_table *t, void *out, int32_t *chunk_status,
                        const uint16_t *scales, const int8_t *zp, uint64_t group, uint8_t *staging,
                        uint64_t staging_bytes, void *copy_stream, void *stream, const FileSource *fs = nullptr) {
  if (t->n_chunks == 0) return LT_OK;
  if (!staging || ((uintptr_t)staging & (kAlign - 1)) != 0) return LT_ERR_INVALID_ARG;
  // host-side checks of what the batching relies on (the device checks the rest)
  const uint64_t n = t->n_chunks;
  if (t->comp_off[0] != 0 || t->comp_off[n] > t->comp_bytes) return LT_ERR_INVALID_ARG;
  if (t->seq_off && (t->seq_off[0] != 0 || t->seq_off[n] > t->n_seq)) return LT_ERR_INVALID_ARG;
  for (uint64_t i = 0; i < n; i++) {
    if (t->comp_off[i + 1] < t->comp_off[i] || t->dst_off[i + 1] < t->dst_off[i]) return LT_ERR_INVALID_ARG;
    if (t->seq_off && t->seq_off[i + 1] < t->seq_off[i]) return LT_ERR_INVALID_ARG;
  }
  const uint64_t mb = meta_bytes(t);
  if (staging_bytes < mb + 2 * kAlign) return LT_ERR_INVALID_ARG;
  const uint64_t half = ((staging_bytes - mb) / 2) & ~(kAlign - 1);
  for (uint64_t i = 0; i < n; i++) {
    if (batch_bytes(t, i, i + 1) > half) return LT_ERR_INVALID_ARG;   // a chunk must fit a half
    if (fs && t->comp_off[i + 1] - t->comp_off[i] > fs->half) return LT_ERR_INVALID_ARG;
  }
  hipStream_t cs = (hipStream_t)copy_stream, ds = (hipStream_t)stream;
  // on one stream the copies and decodes are ordered by the stream itself,
  // and no event is needed (nor created); a file source needs the copy
  // events to know when a pinned half is free
  const bool one = cs == ds && !fs;
  uint64_t *m_coff = (uint64_t *)staging;
  uint64_t *m_doff = (uint64_t *)(staging + up(8 * (n + 1)));
  uint8_t *m_rest = staging + 2 * up(8 * (n + 1));
  uint64_t *m_xxh = t->xxh ? (uint64_t *)m_rest : nullptr;
  if (t->xxh) m_rest += up(8 * n);
  uint64_t *m_soff = (uint64_t *)m_rest;
  uint32_t *m_spos = (uint32_t *)(m_rest + up(8 * (n + 1)));
  const uint64_t ns = t->seq_off ? t->seq_off[n] : 0;
  hipEvent_t copied[2] = {nullptr, nullptr}, done[2] = {nullptr, nullptr}, start = nullptr;
  lt_status st = LT_OK;
  for (int h = 0; h < 2 && st == LT_OK && !one; h++) {
    if (hipEventCreateWithFlags(&copied[h], hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&done[h], hipEventDisableTiming) != hipSuccess)
      st = LT_ERR_DEVICE;
  }
  // the first copy waits for the work already on stream, so a staging
  // buffer reused by consecutive calls is not overwritten under a decode
  if (st == LT_OK && !one &&
      (hipEventCreateWithFlags(&start, hipEventDisableTiming) != hipSuccess || hipEventRecord(start, ds) != hipSuccess ||
       hipStreamWaitEvent(cs, start, 0) != hipSuccess))
    st = LT_ERR_DEVICE;
  if (st == LT_OK) {
    bool ok = hipMemcpyAsync(m_coff, t->comp_off, 8 * (n + 1), hipMemcpyHostToDevice, cs) == hipSuccess &&
              hipMemcpyAsync(m_doff, t->dst_off, 8 * (n + 1), hipMemcpyHostToDevice, cs) == hipSuccess;
    if (ok && t->xxh) ok = hipMemcpyAsync(m_xxh, t->xxh, 8 * n, hipMemcpyHostToDevice, cs) == hipSuccess;
    if (ok && t->seq_off)
      ok = hipMemcpyAsync(m_soff, t->seq_off, 8 * (n + 1), hipMemcpyHostToDevice, cs) == hipSuccess &&
           (ns == 0 || hipMemcpyAsync(m_spos, t->seq_pos, 4 * ns, hipMemcpyHostToDevice, cs) == hipSuccess);
    if (!ok) st = LT_ERR_DEVICE;
  }
  uint64_t c = 0;
  for (uint64_t batch = 0; st == LT_OK && c < n; batch++) {
    // the batch: as many chunks as the half holds
    uint64_t e = c + 1;
    while (e < n && batch_bytes(t, c, e + 1) <= half && (!fs || t->comp_off[e + 1] - t->comp_off[c] <= fs->half)) e++;
    const int h = (int)(batch & 1);
    uint8_t *p_comp = staging + mb + h * half;
    const uint64_t cb = t->comp_off[e] - t->comp_off[c];
    // copies into this half wait for the decode that last read it
    if (!one && batch >= 2 && hipStreamWaitEvent(cs, done[h], 0) != hipSuccess) { st = LT_ERR_DEVICE; break; }
    const uint8_t *src = t->comp + t->comp_off[c];
    if (fs) {
      // the pinned half was last read by the copy of batch - 2
      uint8_t *pin = fs->pinned + h * fs->half;
      if (batch >= 2 && hipEventSynchronize(copied[h]) != hipSuccess) { st = LT_ERR_DEVICE; break; }
      if (!read_range(fs->fd, fs->offset + t->comp_off[c], cb, pin, fs->threads)) { st = LT_ERR_IO; break; }
      src = pin;
    }
    if (hipMemcpyAsync(p_comp, src, cb, hipMemcpyHostToDevice, cs) != hipSuccess ||
        (!one && (hipEventRecord(copied[h], cs) != hipSuccess || hipStreamWaitEvent(ds, copied[h], 0) != hipSuccess))) {
      st = LT_ERR_DEVICE;
      break;
    }
    // the kernel sees chunks c .. e-1 as 0 .. e-c-1: the offset arrays are
    // the device copies from chunk c on, compressed offsets counted from
    // the batch's first byte
    lt::ChunkParams P = make_params(t, out, chunk_status ? chunk_status + c : nullptr, scales, zp, group);
    P.order = nullptr;   // batches are decoded in table order
    P.xxh = m_xxh ? m_xxh + c : nullptr;
    P.comp = p_comp;
    P.comp_off = m_coff + c;
    P.dst_off = m_doff + c;
    P.comp_bytes = cb;
    P.comp_base = t->comp_off[c];
    P.n = (uint32_t)(e - c);
    P.d_first = t->dst_off[c];
    P.d_last = t->dst_off[e];
    if (t->seq_off) {
      P.seq_off = m_soff + c;
      P.seq_pos = m_spos;
      P.n_seq = ns;
    }
    st = launch_params(mode, P, stream);
    if (st == LT_OK && !one && hipEventRecord(done[h], ds) != hipSuccess) st = LT_ERR_DEVICE;
    c = e;
  }
  for (int h = 0; h < 2; h++) {   // destruction waits for nothing: pending events are released later
    if (copied[h]) (void)hipEventDestroy(copied[h]);
    if (done[h]) (void)hipEventDestroy(done[h]);
  }
  if (start) (void)hipEventDestroy(start);
  return st;
}

// ------------------------------------------ staging without allocation

// The staging workspace of lt_stream_fused_lz4_int4_static: one array per
// device, in the code object, held until the process ends.  Its name is a
// host-side stand-in; its device address is taken once per device with
// hipGetSymbolAddress, and only that address is used.
constexpr uint64_t kStaticScratch = LT_STATIC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint8_t *g_scratch_ptr[kMaxDevices];

}  // namespace

static __device__ __align__(256) uint8_t scratch[LT_STATIC_SCRATCH_BYTES];

namespace {

// the current device's copy of `scratch`, or NULL when its address cannot
// be taken
uint8_t *static_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    g_scratch_ptr[dev] = (uint8_t *)p;
  }
  return g_scratch_ptr[dev];
}

bool table_ok(const lt_chunk_table *t) {
  if (!t) return false;
  if (t->n_chunks == 0) return t->total_bytes == 0;
  if (!t->comp || !t->comp_off || !t->dst_off) return false;
  if (t->max_chunk_bytes == 0 || t->max_chunk_bytes > LT_MAX_CHUNK_BYTES) return false;
  if (t->max_dist > 65535u) return false;
  if ((t->seq_off == nullptr) != (t->seq_pos == nullptr)) return false;
  if (t->n_chunks > 0x7FFFFFFFu) return false;
  return true;
}

lt_status fused_common(int mode, const lt_chunk_table *t, const uint16_t *scales, const int8_t *zp,
                       uint64_t rows, uint64_t cols, uint64_t group, uint16_t *out,
                       int32_t *chunk_status, void *stream) {
  if (!table_ok(t) || !scales || !out || !aligned16(out)) return LT_ERR_INVALID_ARG;
  if (!shape_ok(rows, cols, group)) return LT_ERR_INVALID_ARG;
  uint64_t n = rows * cols;
  if (mode == lt::MODE_INT4) {
    if (n % 2 != 0 || t->total_bytes != n / 2) return LT_ERR_INVALID_ARG;
  } else {
    if (t->total_bytes != n) return LT_ERR_INVALID_ARG;
  }
  if (t->n_chunks == 0) return LT_OK;
  return launch_chunks(mode, t, out, chunk_status, scales, zp, group, stream);
}

// A chunk range [first, first + count) of a device-resident table, decoded
// into a buffer that holds only the range's output: the kernel addresses
// output by global position, so the base pointer is moved back by the
// range's first position (address arithmetic only; every write lands in
// [out, out + range size), which the per-chunk bounds check guarantees).
lt_status range_common(int mode, const lt_chunk_table *t, const uint16_t *scales, const int8_t *zp,
                       uint64_t rows, uint64_t cols, uint64_t group, uint32_t first, uint32_t count,
                       uint64_t dst_first, uint64_t dst_last, void *out, int32_t *chunk_status, void *stream) {
  if (!table_ok(t) || !out || !aligned16(out)) return LT_ERR_INVALID_ARG;
  if ((uint64_t)first + count > t->n_chunks) return LT_ERR_INVALID_ARG;
  if (dst_first > dst_last || dst_last > t->total_bytes || (dst_first & 15) != 0) return LT_ERR_INVALID_ARG;
  uint64_t scale = 1;   // output bytes per decoded byte
  if (mode != lt::MODE_BYTES) {
    if (!scales || !shape_ok(rows, cols, group)) return LT_ERR_INVALID_ARG;
    const uint64_t n = rows * cols;
    if (mode == lt::MODE_INT4) {
      if (n % 2 != 0 || t->total_bytes != n / 2) return LT_ERR_INVALID_ARG;
      scale = 4;
    } else {
      if (t->total_bytes != n) return LT_ERR_INVALID_ARG;
      scale = 2;
    }
  }
  if (count == 0) return LT_OK;
  lt::ChunkParams P = make_params(t, (void *)((uintptr_t)out - scale * dst_first), chunk_status, scales, zp, group);
  P.order = nullptr;   // a range is decoded in table order
  if (t->xxh) P.xxh = t->xxh + first;
  P.comp_off = t->comp_off + first;
  P.dst_off = t->dst_off + first;
  if (t->seq_off) P.seq_off = t->seq_off + first;
  P.n = count;
  P.d_first = dst_first;
  P.d_last = dst_last;
  return launch_params(mode, P, stream);
}

lt_status stream_args(int mode, const lt_chunk_table *t, const uint16_t *scales, uint64_t rows, uint64_t cols,
                      uint64_t group, const void *out) {
  if (!table_ok(t) || !out || !aligned16(out)) return LT_ERR_INVALID_ARG;
  if (mode == lt::MODE_BYTES) return LT_OK;
  if (!scales || !shape_ok(rows, cols, group)) return LT_ERR_INVALID_ARG;
  const uint64_t n = rows * cols;
  if (mode == lt::MODE_INT8) return t->total_bytes == n ? LT_OK : LT_ERR_INVALID_ARG;
  if (n % 2 != 0 || t->total_bytes != n / 2) return LT_ERR_INVALID_ARG;
  return LT_OK;
}

lt_status raw_common(bool int4, const uint8_t *src, const uint16_t *scales, const int8_t *zp,
                     uint64_t rows, uint64_t cols, uint64_t group, uint16_t *out, void *stream) {
  if (!src || !scales || !out || !aligned16(out)) return LT_ERR_INVALID_ARG;
  if (!shape_ok(rows, cols, group)) return LT_ERR_INVALID_ARG;
  uint64_t n = rows * cols;
  if (int4 && n % 2 != 0) return LT_ERR_INVALID_ARG;
  lt::RawParams P;
  P.src = src;
  P.scales = scales;
  P.zp = zp;
  P.n_bytes = int4 ? n / 2 : n;
  P.group = group;
  P.group_shift = shift_of(group);
  P.out = out;
  P.e_base = 0;
  hipStream_t s = (hipStream_t)stream;
  if (int4 && P.group_shift >= 6 && P.group_shift < 64 && P.n_bytes >= 1024) {
    // whole 1 KiB tiles with per-tile group constants; the rest below
    const uint64_t ntiles = P.n_bytes / 1024;
    uint64_t blocks = (ntiles + lt::RAWT_THREADS / 64 - 1) / (lt::RAWT_THREADS / 64);
    // one tile per wave measures fastest (more waves in flight than a
    // grid-strided loop keeps); the loop only serves grids past the limit
    if (blocks > 0x7FFFFFFFull) blocks = 0x7FFFFFFFull;
    hipLaunchKernelGGL(lt::dequant_int4_tiles, dim3((uint32_t)blocks), dim3(lt::RAWT_THREADS), 0, s, P, ntiles);
    const uint64_t done = ntiles * 1024;
    if (done == P.n_bytes) return hipGetLastError() == hipSuccess ? LT_OK : LT_ERR_LAUNCH;
    P.src += done;
    P.out += 2 * done;
    P.e_base = 2 * done;
    P.n_bytes -= done;
  }
  uint64_t units = int4 ? P.n_bytes / 4 : P.n_bytes / 8;
  uint64_t per_block = (uint64_t)lt::RAW_THREADS * lt::RAW_UNROLL;
  uint64_t blocks = (units + per_block - 1) / per_block;
  if (blocks == 0) blocks = 1;
  if (blocks > 0x7FFFFFFFull) return LT_ERR_UNSUPPORTED;
  if (int4)
    hipLaunchKernelGGL(lt::dequant_int4_kernel, dim3((uint32_t)blocks), dim3(lt::RAW_THREADS), 0, s, P);
  else
    hipLaunchKernelGGL(lt::dequant_int8_kernel, dim3((uint32_t)blocks), dim3(lt::RAW_THREADS), 0, s, P);
  return hipGetLastError() == hipSuccess ? LT_OK : LT_ERR_LAUNCH;
}

}  // namespace

extern "C" {

lt_status lt_decode_lz4(const lt_chunk_table *t, uint8_t *dst, int32_t *chunk_status, void *stream) {
  if (!table_ok(t) || !dst || !aligned16(dst)) return LT_ERR_INVALID_ARG;
  if (t->n_chunks == 0) return LT_OK;
  return launch_chunks(lt::MODE_BYTES, t, dst, chunk_status, nullptr, nullptr, 1, stream);
}

lt_status lt_dequant_int4(const uint8_t *packed, const uint16_t *scales, const int8_t *zp,
                          uint64_t rows, uint64_t cols, uint64_t group, uint16_t *out, void *stream) {
  return raw_common(true, packed, scales, zp, rows, cols, group, out, stream);
}

lt_status lt_dequant_int8(const int8_t *q, const uint16_t *scales, const int8_t *zp, uint64_t rows,
                          uint64_t cols, uint64_t group, uint16_t *out, void *stream) {
  return raw_common(false, (const uint8_t *)q, scales, zp, rows, cols, group, out, stream);
}

lt_status lt_dequant_int4_lut(const uint8_t *packed, const uint16_t *lut, uint64_t rows, uint64_t cols,
                              uint64_t group, uint16_t *out, void *stream) {
  if (!packed || !lut || !out || !aligned16(out) || !aligned16(lut) || ((uintptr_t)packed & 3) != 0)
    return LT_ERR_INVALID_ARG;
  if (!shape_ok(rows, cols, group) || group < 16) return LT_ERR_INVALID_ARG;
  const uint64_t n = rows * cols;
  if (n % 2 != 0) return LT_ERR_INVALID_ARG;
  lt::LutParams P;
  P.src = packed;
  P.lut = lut;
  P.n = n;
  P.group = group;
  P.group_shift = shift_of(group);
  P.out = out;
  const uint64_t blocks = (n + lt::LUT_CODES - 1) / lt::LUT_CODES;
  if (blocks > 0x7FFFFFFFull) return LT_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(lt::dequant_int4_lut_kernel, dim3((uint32_t)blocks), dim3(lt::LUT_THREADS), 0,
                     (hipStream_t)stream, P);
  return hipGetLastError() == hipSuccess ? LT_OK : LT_ERR_LAUNCH;
}

lt_status lt_fused_lz4_int4_gemv(const lt_chunk_table *t, const uint16_t *scales, const int8_t *zp,
                                 uint64_t rows, uint64_t cols, uint64_t group, const uint16_t *x, float *y,
                                 int32_t *chunk_status, void *stream) {
  if (!table_ok(t) || !scales || !x || !y || !aligned16(x) || ((uintptr_t)y & 3) != 0) return LT_ERR_INVALID_ARG;
  if (!shape_ok(rows, cols, group)) return LT_ERR_INVALID_ARG;
  const uint64_t n = rows * cols;
  if (t->total_bytes != n / 2) return LT_ERR_INVALID_ARG;
  if (cols % 512 != 0 || shift_of(group) >= 64 || group < 128) return LT_ERR_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  uint64_t zb = (rows + 255) / 256;
  zb = zb < 4096 ? zb : 4096;
  hipLaunchKernelGGL(lt::zero_f32, dim3((uint32_t)zb), dim3(256), 0, s, y, rows);
  if (hipGetLastError() != hipSuccess) return LT_ERR_LAUNCH;
  if (t->n_chunks == 0) return LT_OK;
  lt::ChunkParams P = make_params(t, nullptr, chunk_status, scales, zp, group);
  P.gemv_x = x;
  P.gemv_y = y;
  P.cols = cols;
  return launch_params(lt::MODE_GEMV, P, stream);
}

}  // extern "C"

namespace lt {

// The GEMM's second pass: y[b][16 rb + w] = the sum, over the chunks of row
// block rb in table order and their GEMM_SLOTS slots in order, of the
// partial products D[w][b].  One workgroup per 16-row block, one thread per
// (row, vector); the chunks of a block are found by binary search on
// dst_off (chunks hold whole tiles of one block, in order).
__global__ void __launch_bounds__(512) gemm_reduce(const float *part, const uint64_t *dst_off, uint32_t n,
                                                   uint32_t nbt, uint64_t rows, uint64_t cols, float *y) {
  const uint64_t rb = blockIdx.x, rb_bytes = 8 * cols;   // 16 rows of cols 4-bit codes
  auto first_at = [&](uint64_t pos) {   // first chunk starting at or after pos
    uint32_t lo = 0, hi = n;
    while (lo < hi) {
      const uint32_t mid = (lo + hi) / 2;
      if (dst_off[mid] < pos) lo = mid + 1;
      else hi = mid;
    }
    return lo;
  };
  const uint32_t c0 = first_at(rb * rb_bytes), c1 = first_at((rb + 1) * rb_bytes);
  const uint32_t tid = threadIdx.x, w = tid & 15, b = tid >> 4, bt = b >> 4, bc = b & 15;
  if (b >= 16 * nbt) return;
  float sum = 0.0f;
  for (uint32_t c = c0; c < c1; c++)
    for (uint32_t slot = 0; slot < GEMM_SLOTS; slot++)
      sum += part[(((uint64_t)c * GEMM_SLOTS + slot) * nbt + bt) * 256 + w * 16 + bc];
  y[(uint64_t)b * rows + 16 * rb + w] = sum;
}

}  // namespace lt

extern "C" {

uint64_t lt_gemm_workspace_bytes(uint32_t n_chunks, uint32_t batch) {
  return (uint64_t)n_chunks * lt::GEMM_SLOTS * batch * 16 * sizeof(float);
}

lt_status lt_fused_lz4_int4_gemm(const lt_chunk_table *t, const uint16_t *scales, const int8_t *zp, uint64_t rows,
                                 uint64_t cols, uint64_t group, const uint16_t *x, uint32_t batch, float *y,
                                 float *workspace, uint64_t workspace_bytes, int32_t *chunk_status, void *stream) {
  if (!table_ok(t) || !scales || !x || !y || !workspace || !aligned16(x) || ((uintptr_t)y & 3) != 0 ||
      ((uintptr_t)workspace & 15) != 0)
    return LT_ERR_INVALID_ARG;
  if (!shape_ok(rows, cols, group)) return LT_ERR_INVALID_ARG;
  if (t->total_bytes != rows * cols / 2) return LT_ERR_INVALID_ARG;
  if (rows % 16 != 0 || cols % 128 != 0 || shift_of(group) >= 64 || group < 128) return LT_ERR_UNSUPPORTED;
  if (batch != 16 && batch != 32) return LT_ERR_UNSUPPORTED;
  if (workspace_bytes < lt_gemm_workspace_bytes(t->n_chunks, batch)) return LT_ERR_INVALID_ARG;
  if (rows / 16 > 0x7FFFFFFFull) return LT_ERR_UNSUPPORTED;
  lt::ChunkParams P = make_params(t, nullptr, chunk_status, scales, zp, group);
  P.gemv_x = x;
  P.cols = cols;
  P.gemm_part = workspace;
  P.gemm_nbt = batch / 16;
  P.gemm_tpr = cols / 128;
  const lt_status st = launch_params(lt::MODE_GEMM, P, stream);
  if (st != LT_OK) return st;
  hipLaunchKernelGGL(lt::gemm_reduce, dim3((uint32_t)(rows / 16)), dim3(16 * batch), 0, (hipStream_t)stream,
                     workspace, t->dst_off, t->n_chunks, batch / 16, rows, cols, y);
  return hipGetLastError() == hipSuccess ? LT_OK : LT_ERR_LAUNCH;
}

lt_status lt_fused_lz4_int4(const lt_chunk_table *t, const uint16_t *scales, const int8_t *zp,
                            uint64_t rows, uint64_t cols, uint64_t group, uint16_t *out,
                            int32_t *chunk_status, void *stream) {
  return fused_common(lt::MODE_INT4, t, scales, zp, rows, cols, group, out, chunk_status, stream);
}

lt_status lt_fused_lz4_int8(const lt_chunk_table *t, const uint16_t *scales, const int8_t *zp,
                            uint64_t rows, uint64_t cols, uint64_t group, uint16_t *out,
                            int32_t *chunk_status, void *stream) {
  return fused_common(lt::MODE_INT8, t, scales, zp, rows, cols, group, out, chunk_status, stream);
}

lt_status lt_decode_lz4_range(const lt_chunk_table *t, uint32_t first, uint32_t count, uint64_t dst_first,
                              uint64_t dst_last, uint8_t *dst, int32_t *chunk_status, void *stream) {
  return range_common(lt::MODE_BYTES, t, nullptr, nullptr, 0, 0, 0, first, count, dst_first, dst_last, dst,
                      chunk_status, stream);
}

lt_status lt_fused_lz4_int4_range(const lt_chunk_table *t, const uint16_t *scales, const int8_t *zp,
                                  uint64_t rows, uint64_t cols, uint64_t group, uint32_t first, uint32_t count,
                                  uint64_t dst_first, uint64_t dst_last, uint16_t *out, int32_t *chunk_status,
                                  void *stream) {
  return range_common(lt::MODE_INT4, t, scales, zp, rows, cols, group, first, count, dst_first, dst_last, out,
                      chunk_status, stream);
}

lt_status lt_fused_lz4_int8_range(const lt_chunk_table *t, const uint16_t *scales, const int8_t *zp,
                                  uint64_t rows, uint64_t cols, uint64_t group, uint32_t first, uint32_t count,
                                  uint64_t dst_first, uint64_t dst_last, uint16_t *out, int32_t *chunk_status,
                                  void *stream) {
  return range_common(lt::MODE_INT8, t, scales, zp, rows, cols, group, first, count, dst_first, dst_last, out,
                      chunk_status, stream);
}

lt_status lt_decode_zero_runs(const lt_zr_tensor *z, uint16_t *out, int32_t *block_status, void *stream) {
  static_assert(lt::ZR_BLOCK == LT_ZR_BLOCK, "block size");
  if (!z || !out || !aligned16(out)) return LT_ERR_INVALID_ARG;
  if (z->n_elem == 0) return LT_OK;
  if (!z->bitmap || !z->val_off || (!z->vals && z->n_vals)) return LT_ERR_INVALID_ARG;
  if (z->n_elem > (1ull << 48)) return LT_ERR_INVALID_ARG;
  lt::ZrParams P;
  P.bitmap = z->bitmap;
  P.val_off = z->val_off;
  P.vals = z->vals;
  P.n = z->n_elem;
  P.n_vals = z->n_vals;
  P.nb = (z->n_elem + LT_ZR_BLOCK - 1) / LT_ZR_BLOCK;
  P.out = out;
  P.status = block_status;
  const uint64_t grid = (P.nb + lt::ZR_WAVES - 1) / lt::ZR_WAVES;
  if (grid > 0x7FFFFFFFull) return LT_ERR_UNSUPPORTED;
  hipLaunchKernelGGL(lt::zr_decode_kernel, dim3((uint32_t)grid), dim3(64 * lt::ZR_WAVES), 0, (hipStream_t)stream, P);
  return hipGetLastError() == hipSuccess ? LT_OK : LT_ERR_LAUNCH;
}

lt_status lt_verify_chunks(const lt_chunk_table *t, const uint64_t *expect, uint64_t *got, int32_t *chunk_status,
                           void *stream) {
  if (!table_ok(t)) return LT_ERR_INVALID_ARG;
  if (!got && !chunk_status) return LT_ERR_INVALID_ARG;   // nothing to report into
  if (expect && !chunk_status) return LT_ERR_INVALID_ARG;
  if (t->n_chunks == 0) return LT_OK;
  lt::XxhParams P;
  P.comp = t->comp;
  P.comp_off = t->comp_off;
  P.comp_bytes = t->comp_bytes;
  P.n = t->n_chunks;
  P.expect = expect;
  P.got = got;
  P.status = chunk_status;
  const uint32_t grid = (t->n_chunks + lt::XXH_WAVES - 1) / lt::XXH_WAVES;
  hipLaunchKernelGGL(lt::xxh_kernel, dim3(grid), dim3(64 * lt::XXH_WAVES), 0, (hipStream_t)stream, P);
  return hipGetLastError() == hipSuccess ? LT_OK : LT_ERR_LAUNCH;
}

lt_status lt_stream_decode_lz4(const lt_chunk_table *host_table, uint8_t *dst, int32_t *chunk_status,
                               uint8_t *staging, uint64_t staging_bytes, void *copy_stream, void *stream) {
  const lt_status a = stream_args(lt::MODE_BYTES, host_table, nullptr, 0, 0, 0, dst);
  if (a != LT_OK) return a;
  return stream_common(lt::MODE_BYTES, host_table, dst, chunk_status, nullptr, nullptr, 1, staging, staging_bytes,
                       copy_stream, stream);
}

lt_status lt_stream_fused_lz4_int4(const lt_chunk_table *host_table, const uint16_t *scales, const int8_t *zp,
                                   uint64_t rows, uint64_t cols, uint64_t group, uint16_t *out,
                                   int32_t *chunk_status, uint8_t *staging, uint64_t staging_bytes,
                                   void *copy_stream, void *stream) {
  const lt_status a = stream_args(lt::MODE_INT4, host_table, scales, rows, cols, group, out);
  if (a != LT_OK) return a;
  return stream_common(lt::MODE_INT4, host_table, out, chunk_status, scales, zp, group, staging, staging_bytes,
                       copy_stream, stream);
}

lt_status lt_stream_fused_lz4_int8(const lt_chunk_table *host_table, const uint16_t *scales, const int8_t *zp,
                                   uint64_t rows, uint64_t cols, uint64_t group, uint16_t *out,
                                   int32_t *chunk_status, uint8_t *staging, uint64_t staging_bytes,
                                   void *copy_stream, void *stream) {
  const lt_status a = stream_args(lt::MODE_INT8, host_table, scales, rows, cols, group, out);
  if (a != LT_OK) return a;
  return stream_common(lt::MODE_INT8, host_table, out, chunk_status, scales, zp, group, staging, staging_bytes,
                       copy_stream, stream);
}

}  // extern "C"

namespace {

// The streamed calls with the compressed bytes in a file: the table's comp
// array is not read (chunk i's bytes are at file_offset + comp_off[i]).
lt_status file_common(int mode, int fd, uint64_t file_offset, const lt_chunk_table *host_table,
                      const uint16_t *scales, const int8_t *zp, uint64_t rows, uint64_t cols, uint64_t group,
                      void *out, int32_t *chunk_status, uint8_t *pinned, uint64_t pinned_bytes, int read_threads,
                      uint8_t *staging, uint64_t staging_bytes, void *copy_stream, void *stream) {
  if (!host_table || fd < 0 || !pinned || pinned_bytes < 2 * kAlign) return LT_ERR_INVALID_ARG;
  lt_chunk_table t = *host_table;
  t.comp = pinned;   // any host pointer: only checked against NULL
  const lt_status a = stream_args(mode, &t, scales, rows, cols, group, out);
  if (a != LT_OK) return a;
  const FileSource fs{fd, file_offset, pinned, (pinned_bytes / 2) & ~(kAlign - 1), read_threads};
  return stream_common(mode, &t, out, chunk_status, scales, zp, group, staging, staging_bytes, copy_stream, stream,
                       &fs);
}

}  // namespace

extern "C" {

lt_status lt_stream_file_decode_lz4(int fd, uint64_t file_offset, const lt_chunk_table *host_table, uint8_t *dst,
                                    int32_t *chunk_status, uint8_t *pinned, uint64_t pinned_bytes, int read_threads,
                                    uint8_t *staging, uint64_t staging_bytes, void *copy_stream, void *stream) {
  return file_common(lt::MODE_BYTES, fd, file_offset, host_table, nullptr, nullptr, 0, 0, 1, dst, chunk_status, pinned,
                     pinned_bytes, read_threads, staging, staging_bytes, copy_stream, stream);
}

lt_status lt_stream_file_fused_lz4_int4(int fd, uint64_t file_offset, const lt_chunk_table *host_table,
                                        const uint16_t *scales, const int8_t *zp, uint64_t rows, uint64_t cols,
                                        uint64_t group, uint16_t *out, int32_t *chunk_status, uint8_t *pinned,
                                        uint64_t pinned_bytes, int read_threads, uint8_t *staging,
                                        uint64_t staging_bytes, void *copy_stream, void *stream) {
  return file_common(lt::MODE_INT4, fd, file_offset, host_table, scales, zp, rows, cols, group, out, chunk_status,
                     pinned, pinned_bytes, read_threads, staging, staging_bytes, copy_stream, stream);
}

lt_status lt_stream_file_fused_lz4_int8(int fd, uint64_t file_offset, const lt_chunk_table *host_table,
                                        const uint16_t *scales, const int8_t *zp, uint64_t rows, uint64_t cols,
                                        uint64_t group, uint16_t *out, int32_t *chunk_status, uint8_t *pinned,
                                        uint64_t pinned_bytes, int read_threads, uint8_t *staging,
                                        uint64_t staging_bytes, void *copy_stream, void *stream) {
  return file_common(lt::MODE_INT8, fd, file_offset, host_table, scales, zp, rows, cols, group, out, chunk_status,
                     pinned, pinned_bytes, read_threads, staging, staging_bytes, copy_stream, stream);
}

lt_status lt_stream_fused_lz4_int4_static(const lt_chunk_table *host_table, const uint16_t *scales,
                                          const int8_t *zp, uint64_t rows, uint64_t cols, uint64_t group,
                                          uint16_t *out, int32_t *chunk_status, void *stream) {
  const lt_status a = stream_args(lt::MODE_INT4, host_table, scales, rows, cols, group, out);
  if (a != LT_OK) return a;
  const lt_chunk_table *t = host_table;
  if (t->n_chunks == 0) return LT_OK;
  // the table's offsets and index, and two halves that each hold the
  // largest chunk's compressed bytes, must fit the static workspace
  uint64_t big = 0;
  for (uint64_t i = 0; i < t->n_chunks; i++) {
    if (t->comp_off[i + 1] < t->comp_off[i]) return LT_ERR_INVALID_ARG;
    const uint64_t c = t->comp_off[i + 1] - t->comp_off[i];
    big = c > big ? c : big;
  }
  if (t->seq_off && t->seq_off[t->n_chunks] > t->n_seq) return LT_ERR_INVALID_ARG;
  if (meta_bytes(t) + 2 * up(big + 16) > kStaticScratch) return LT_ERR_TOO_LARGE;
  uint8_t *ws = static_scratch();
  if (!ws) return LT_ERR_DEVICE;
  return stream_common(lt::MODE_INT4, t, out, chunk_status, scales, zp, group, ws, kStaticScratch, stream, stream);
}

const char *lt_status_str(lt_status s) {
  switch (s) {
    case LT_OK: return "ok";
    case LT_ERR_INVALID_ARG: return "invalid argument";
    case LT_ERR_UNSUPPORTED: return "unsupported";
    case LT_ERR_LAUNCH: return "kernel launch failed";
    case LT_ERR_DEVICE: return "no usable device";
    case LT_ERR_TOO_LARGE: return "request exceeds the static workspace";
    case LT_ERR_IO: return "a file read failed or ended early";
  }
  return "unknown status";
}

int lt_abi_version(void) { return LT_ABI_VERSION; }

}  // extern "C"

#ifdef LT_DEBUG
namespace lt {
// Two calls that break the uniformity rule on purpose (lane 0 inactive; a
// value that differs between lanes), each a harmless store to a local LDS
// word: the debug counter must count both.
__global__ void debug_selftest_kernel(uint32_t *sink) {
  __shared__ uint32_t x;
  const uint32_t lane = threadIdx.x & 63;
  if (lane >= 32) lds_set(&x, 7u);
  lds_set(&x, lane);
  __syncthreads();
  if (threadIdx.x == 0) sink[0] = x;
}
}  // namespace lt
#endif

extern "C" {

lt_status lt_debug_selftest(uint32_t *sink, void *stream) {
#ifdef LT_DEBUG
  if (!sink) return LT_ERR_INVALID_ARG;
  hipLaunchKernelGGL(lt::debug_selftest_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream, sink);
  return hipGetLastError() == hipSuccess ? LT_OK : LT_ERR_LAUNCH;
#else
  (void)sink;
  (void)stream;
  return LT_ERR_UNSUPPORTED;
#endif
}

lt_status lt_debug_violations(uint32_t *count, uint32_t *first_line, int reset) {
#ifdef LT_DEBUG
  if (!count || !first_line) return LT_ERR_INVALID_ARG;
  if (hipMemcpyFromSymbol(count, HIP_SYMBOL(lt::g_debug_count), sizeof(uint32_t)) != hipSuccess ||
      hipMemcpyFromSymbol(first_line, HIP_SYMBOL(lt::g_debug_line), sizeof(uint32_t)) != hipSuccess)
    return LT_ERR_DEVICE;
  if (reset) {
    const uint32_t zero = 0;
    if (hipMemcpyToSymbol(HIP_SYMBOL(lt::g_debug_count), &zero, sizeof zero) != hipSuccess ||
        hipMemcpyToSymbol(HIP_SYMBOL(lt::g_debug_line), &zero, sizeof zero) != hipSuccess)
      return LT_ERR_DEVICE;
  }
  return LT_OK;
#else
  (void)count;
  (void)first_line;
  (void)reset;
  return LT_ERR_UNSUPPORTED;
#endif
}

}  // extern "C"
