/*
 * lt.h -- C ABI of liblt, just-in-time decompression of compressed tensors in
 * MI355X (gfx950) device memory.
 *
 * The method: tensors stay resident in device memory in compressed form and
 * are expanded into a working buffer right before use (page "Openai/692db884
 * ..." (section 28), the five-step decode description: a compact blob plus a
 * small metadata record per tensor, decoded into a temporary buffer whose
 * pointer is handed to the consumer).  For weights the compressed form is
 * INT4 or INT8 codes with fp16 scales and int8 zero points, LZ4-compressed in
 * independent blocks, expanded on the GPU straight to fp16 ("GPU Compression
 * Pipeline - TDD Roadmap", Phase 1.1, Phase 1.2, Phase 2.1, Phase 3.1; the
 * 64 KiB block size from Phase 6.1).  For zero-heavy ReLU activations it is
 * plain LZ4, decoded to bytes (page "Openai/691a41cd ..." (section 38), the
 * list of what wastes GPU memory: zeros after ReLU).
 *
 * Conventions shared by every entry point
 *   - Pointers marked DEVICE point to device memory; HOST to host memory.
 *   - Every device entry point is asynchronous on `stream` (a hipStream_t
 *     passed as void*, NULL = the null stream).  It checks its arguments
 *     synchronously, launches, and returns; it never synchronizes, allocates,
 *     or keeps state.  The caller owns every buffer; device buffers must stay
 *     alive until the stream work completes.  Calls are reentrant.
 *   - Tensors are row-major [rows, cols]; element e = r*cols + c.
 *   - INT4 codes are unsigned 0..15, two per byte, element 2k in the low
 *     nibble of byte k and element 2k+1 in the high nibble.  INT8 codes are
 *     signed bytes.
 *   - Groups are `group` consecutive elements in element order: element e
 *     uses scale and zero point number e / group.  Per-row (per-channel)
 *     scaling is group = cols, per-tensor is group = rows*cols.  Either
 *     cols % group == 0 or group % cols == 0, and (rows*cols) % group == 0.
 *   - Scales are fp16 bit patterns (uint16).  Zero points are int8; zp = NULL
 *     means every zero point is 0.
 *   - Dequantization: out[e] = fp16_rne( (q[e] - zp[g]) * scale[g] ).  The
 *     product is exact before the single rounding, so results are bit-exact.
 *   - The return value reports argument and launch errors only.  Decode errors
 *     are reported per chunk on the device in `chunk_status` (may be NULL).
 *     A failed chunk's own output range holds unspecified bytes afterwards;
 *     nothing outside the chunk's range is ever written.
 */
#ifndef LT_H
#define LT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LT_ABI_VERSION 15

typedef enum lt_status {
  LT_OK = 0,
  LT_ERR_INVALID_ARG = 1, /* a pointer, size, shape or alignment is invalid */
  LT_ERR_UNSUPPORTED = 2, /* valid request this build cannot serve */
  LT_ERR_LAUNCH = 3,      /* the HIP runtime refused the launch */
  LT_ERR_DEVICE = 4,      /* no usable gfx950 device for the current context */
  LT_ERR_TOO_LARGE = 5,   /* the request does not fit a fixed-size workspace */
  LT_ERR_IO = 6           /* a read from a file failed or ended early */
} lt_status;

/* Per-chunk codes written to chunk_status[i] (DEVICE, int32). */
enum {
  LT_CHUNK_OK = 0,
  LT_CHUNK_TRUNCATED = 1,     /* block ended inside a sequence, or is empty */
  LT_CHUNK_BAD_OFFSET = 2,    /* match distance 0, or before the chunk start */
  LT_CHUNK_OVERRUN = 3,       /* a sequence would write past the chunk end */
  LT_CHUNK_SIZE_MISMATCH = 4, /* block decoded to fewer bytes than the chunk */
  LT_CHUNK_BAD_TABLE = 5,     /* the chunk's table entries are inconsistent */
  LT_CHUNK_CHECKSUM = 6,      /* the stored bytes do not match their XXH3-64 (see xxh, lt_verify_chunks) */
  LT_CHUNK_STALLED = 7        /* a wait inside the decoder polled past its bound (see spin_limit) */
};

/* Largest decoded chunk the device decoder accepts (bytes).  It bounds a
 * sequence's length-extension run (about size / 255 bytes) so that the
 * decoder's compressed-input ring (8 KiB, or 16 KiB for short-window
 * tables) always holds what is being parsed. */
#define LT_MAX_CHUNK_BYTES (1u << 20)

/* Tables whose max_dist is at most this (bytes) are decoded with a 16 KiB
 * history per chunk instead of 64 KiB, which lets more chunks share a CU.
 * lt_compress_chunks produces such tables when asked for this window. */
#define LT_SMALL_WINDOW 11264u

/*
 * Chunk table (HOST struct; its members point to DEVICE memory).
 * A tensor's byte stream (packed INT4 codes, INT8 codes or raw bytes) of
 * total_bytes bytes is cut into n_chunks consecutive chunks; chunk i holds
 * decoded bytes [dst_off[i], dst_off[i+1]) and is stored as one raw LZ4 block
 * (no frame, no size prefix, no dictionary) at comp[comp_off[i] ..
 * comp_off[i+1]).  The blocks are independent: a match never reaches before
 * its own chunk's start.  So one table may also cover several tensors laid
 * end to end (say the projections of one model layer, with their scales and
 * zero points end to end too, each tensor's groups ending where it ends):
 * one call then decodes all of them, and the chunks of every tensor share
 * one launch.
 *   comp       DEVICE uint8[comp_bytes]
 *   comp_off   DEVICE uint64[n_chunks + 1], non-decreasing, comp_off[n] <= comp_bytes
 *   dst_off    DEVICE uint64[n_chunks + 1], dst_off[0] = 0, non-decreasing,
 *              dst_off[n] = total_bytes, dst_off[i] % 16 == 0 for i < n
 *   max_chunk_bytes  host-known max(dst_off[i+1] - dst_off[i]),
 *              1 <= max_chunk_bytes <= LT_MAX_CHUNK_BYTES (ignored if n_chunks == 0)
 *   max_dist   the largest match distance in any block, 1..65535, or 0 when
 *              not known (any distance).  It is a promise about the blocks:
 *              a match farther back makes its chunk fail with
 *              LT_CHUNK_BAD_OFFSET.  LZ4 blocks may use distances up to
 *              65535; a compressor that keeps them shorter lets the decoder
 *              keep less history (see LT_SMALL_WINDOW).
 *   spin_limit the number of polls each wave of the decoder may make while
 *              it waits for another (for input, records, ring space or
 *              earlier tiles) before it gives up and fails the chunk with
 *              LT_CHUNK_STALLED; 0 means the library's default (2^24, far
 *              above any legitimate wait: a protocol mistake then ends as a
 *              failed chunk instead of a hung GPU).  Small values exist to
 *              test that failure path; every wave still exits normally.
 *   seq_off    DEVICE uint64[n_chunks + 1] or NULL: an optional sequence
 *              index.  Chunk i's LZ4 sequences start at the block offsets
 *              seq_pos[seq_off[i] .. seq_off[i+1]), in order (the first is
 *              0); seq_off is non-decreasing and seq_off[n_chunks] <= n_seq.
 *   seq_pos    DEVICE uint32[n_seq] or NULL (given exactly when seq_off is).
 *   n_seq      entries in seq_pos (0 without an index).
 *   order      DEVICE uint32[n_chunks] or NULL: the order in which the
 *              chunks are started, the k-th workgroup of a launch taking
 *              chunk order[k] (NULL: chunk k).  It should be a permutation
 *              of 0 .. n_chunks-1; an entry >= n_chunks is skipped, a chunk
 *              listed twice is decoded twice (the same bytes), and a chunk
 *              not listed is neither decoded nor given a status.  A launch
 *              lasts at least as long as its slowest chunk, so tables whose
 *              chunks differ in size start the largest first
 *              (lt_order_chunks), and sequence-dense tables also the chunks
 *              with the most sequences (lt_order_chunks_by_sequences).
 *              Chunk-range and streamed calls decode in
 *              table order and ignore it.
 *   xxh        DEVICE uint64[n_chunks] or NULL: the expected XXH3-64 (seed 0)
 *              of each chunk's compressed bytes comp[comp_off[i] ..
 *              comp_off[i+1]), as lt_checksum_chunks computes it (the block
 *              checksum of page "GPU Compression Pipeline - TDD Roadmap",
 *              Phase 6.1).  When given, every decode call hashes each chunk's
 *              bytes as it stages them for the decoder (no second pass over
 *              HBM), streams every chunk whole, and reports
 *              LT_CHUNK_CHECKSUM for a chunk whose hash differs, whatever its
 *              decode gave; that chunk's output range then holds unspecified
 *              bytes.  Range and streamed calls check their chunks too (the
 *              streamed calls copy xxh with the offsets).
 * The index lets a chunk's sequences be parsed side by side instead of one
 * after another (lt_index_chunks builds it from the blocks).  It is checked
 * against the blocks: a listed sequence that does not end where the next
 * listed one starts, or a block that goes on past its last listed
 * sequence, makes the chunk fail with LT_CHUNK_BAD_TABLE.  Entries listed
 * after a block's last sequence are not read.  A chunk with no entries is
 * decoded without the index.
 * Entries that break these rules make that chunk fail with LT_CHUNK_BAD_TABLE
 * (checked on the device); the struct itself is read only during the call.
 */
typedef struct lt_chunk_table {
  const uint8_t *comp;
  const uint64_t *comp_off;
  const uint64_t *dst_off;
  uint32_t n_chunks;
  uint32_t max_chunk_bytes;
  uint64_t total_bytes;
  uint64_t comp_bytes;
  uint32_t max_dist;
  uint32_t spin_limit;
  const uint64_t *seq_off;
  const uint32_t *seq_pos;
  uint64_t n_seq;
  const uint32_t *order;
  const uint64_t *xxh;
} lt_chunk_table;

/*
 * lt_decode_lz4 -- decode-only mode (zero-heavy activations, or any bytes):
 * the chunk-parallel LZ4 block decompression of page "GPU Compression
 * Pipeline - TDD Roadmap", Phase 3.1, with nothing fused after it; the
 * activations it serves are the mostly-zero ReLU outputs that page
 * "Openai/691a41cd-... (section 38)" lists among the compression targets.
 * dst: DEVICE uint8[t->total_bytes], 16-byte aligned.
 * chunk_status: DEVICE int32[t->n_chunks] or NULL.
 * Decodes every chunk of the table into dst.  One workgroup per chunk.
 */
lt_status lt_decode_lz4(const lt_chunk_table *t, uint8_t *dst, int32_t *chunk_status,
                        void *stream);

/*
 * lt_dequant_int4 -- packed INT4 -> fp16 (roadmap Phase 1.1).
 * packed: DEVICE uint8[rows*cols/2]; scales: DEVICE uint16[rows*cols/group];
 * zp: DEVICE int8[rows*cols/group] or NULL; out: DEVICE uint16 (fp16)
 * [rows*cols], 16-byte aligned.  rows*cols must be even and > 0.
 */
lt_status lt_dequant_int4(const uint8_t *packed, const uint16_t *scales, const int8_t *zp,
                          uint64_t rows, uint64_t cols, uint64_t group, uint16_t *out,
                          void *stream);

/*
 * lt_dequant_int8 -- INT8 -> fp16, per-tensor or per-channel (roadmap Phase
 * 1.2).  q: DEVICE int8[rows*cols]; other arguments as lt_dequant_int4.
 */
lt_status lt_dequant_int8(const int8_t *q, const uint16_t *scales, const int8_t *zp,
                          uint64_t rows, uint64_t cols, uint64_t group, uint16_t *out,
                          void *stream);

/*
 * lt_dequant_int4_lut -- codebook dequantization of packed INT4 codes (the
 * value dictionaries of page "Openai/692db884-... (section 28)": small
 * integer codes plus a tiny lookup table, in place of the affine rule).
 * Element e (row-major, low nibble first as lt_dequant_int4) becomes entry
 * q(e) of the table of its group e / group:
 *   lut    DEVICE uint16 [rows*cols/group][16] fp16 bits, 16-byte aligned;
 *          group = rows*cols gives one dictionary for the whole tensor
 *   packed DEVICE, 4-byte aligned; out DEVICE uint16 [rows*cols], 16-byte
 *          aligned
 * group must be at least 16 (a table per fewer codes outweighs the codes)
 * and follow the shape rule of lt_dequant_int4.
 */
lt_status lt_dequant_int4_lut(const uint8_t *packed, const uint16_t *lut, uint64_t rows, uint64_t cols,
                              uint64_t group, uint16_t *out, void *stream);

/*
 * lt_fused_lz4_int4 -- LZ4 decode fused with INT4 unpack and dequantization
 * (roadmap Phase 2.1: decompress and dequantize in one kernel, no
 * intermediate buffer).  The table's decoded stream is the packed INT4 codes:
 * t->total_bytes must equal rows*cols/2.  out: DEVICE uint16 (fp16)
 * [rows*cols], 16-byte aligned; other arguments as lt_dequant_int4.
 * Result equals lt_dequant_int4 applied to lt_decode_lz4's output.
 */
lt_status lt_fused_lz4_int4(const lt_chunk_table *t, const uint16_t *scales, const int8_t *zp,
                            uint64_t rows, uint64_t cols, uint64_t group, uint16_t *out,
                            int32_t *chunk_status, void *stream);

/*
 * lt_fused_lz4_int4_gemv -- LZ4 decode and INT4 dequantization fused with a
 * matrix-vector product, y = W x, W the rows x cols fp16 matrix that
 * lt_fused_lz4_int4 would write (decompress-then-multiply, the decode plus
 * GEMM benchmarks of page "Openai/691a41cd-... (section 38)"; a decoded
 * tensor used in a matmul, "GPU Compression Pipeline - TDD Roadmap",
 * Phase 4.1): each decoded tile of 2048 codes is dotted with x where it
 * lies and never stored, so the fp16 matrix costs no memory traffic.
 *   x  DEVICE fp16 [cols], 16-byte aligned
 *   y  DEVICE fp32 [rows], 4-byte aligned: zeroed on `stream`, then each
 *      tile adds its dot products (fp16 x fp16 products exact in fp32, fp32
 *      sums: per lane, across the wave, then one atomic add per tile and
 *      row, so
 *      the order of the sums, and the last bits of y, vary between calls)
 * Requires group a power of two of at least 128 and cols a multiple of
 * 512 (LT_ERR_UNSUPPORTED otherwise); chunks whose decoded bytes do not
 * start and end on 1 KiB boundaries fail with LT_CHUNK_BAD_TABLE and add
 * nothing.  Other arguments as lt_fused_lz4_int4.
 */
lt_status lt_fused_lz4_int4_gemv(const lt_chunk_table *t, const uint16_t *scales, const int8_t *zp,
                                 uint64_t rows, uint64_t cols, uint64_t group, const uint16_t *x, float *y,
                                 int32_t *chunk_status, void *stream);

/*
 * lt_fused_lz4_int4_gemm -- Y = X W^T with W never stored: the decode feeds
 * dequantized tiles straight into a product on the matrix cores (the decode
 * plus GEMM benchmark of page "Openai/691a41cd-... (section 38)"; the
 * roadmap's decoded tensor used in a matmul, Phase 4.1).  W [rows, cols] is
 * the fp16 matrix lt_fused_lz4_int4 would write from the same codes, scales
 * and zero points, but the table's decoded bytes hold its codes in the GEMM
 * layout: tiles of 16 rows x 128 columns (1 KiB), the 16-row blocks in
 * order, each block's column tiles in order, each tile's 16 rows of 64
 * bytes in turn, two codes per byte, low nibble first.  Every chunk holds
 * whole tiles of one 16-row block (others fail with LT_CHUNK_BAD_TABLE and
 * leave their rows of Y unspecified).
 *   x          DEVICE fp16 [batch][cols], 16-byte aligned; batch 16 or 32
 *   y          DEVICE fp32 [batch][rows], receives Y
 *   workspace  DEVICE fp32 scratch of at least lt_gemm_workspace_bytes(
 *              n_chunks, batch) bytes, 16-byte aligned, owned by the caller:
 *              each chunk's builders leave their partial products there and
 *              a second kernel sums them per row block in a fixed order, so
 *              Y is the same bits on every call
 * rows % 16 == 0, cols % 128 == 0, group a power of two >= 128
 * (LT_ERR_UNSUPPORTED otherwise); the fp16 products are exact in fp32 and
 * the sums are fp32.
 */
lt_status lt_fused_lz4_int4_gemm(const lt_chunk_table *t, const uint16_t *scales, const int8_t *zp, uint64_t rows,
                                 uint64_t cols, uint64_t group, const uint16_t *x, uint32_t batch, float *y,
                                 float *workspace, uint64_t workspace_bytes, int32_t *chunk_status, void *stream);
/* Bytes of workspace lt_fused_lz4_int4_gemm needs for n_chunks and batch. */
uint64_t lt_gemm_workspace_bytes(uint32_t n_chunks, uint32_t batch);

/*
 * lt_fused_lz4_int8 -- LZ4 decode fused with INT8 dequantization; the
 * table's decoded stream is the int8 codes: t->total_bytes == rows*cols.
 */
lt_status lt_fused_lz4_int8(const lt_chunk_table *t, const uint16_t *scales, const int8_t *zp,
                            uint64_t rows, uint64_t cols, uint64_t group, uint16_t *out,
                            int32_t *chunk_status, void *stream);

/*
 * Chunk-range (partial) decode: only chunks [first, first + count) of a
 * device-resident table, into a buffer that holds only their output
 * (page "Openai/692db884-... (section 28)", the comparison with generic
 * compressors: decode only the part an operation needs and skip the chunks
 * it does not touch; here the chunk table is the index that makes a range
 * addressable).
 *   first, count      the range; first + count <= t->n_chunks; count 0 is
 *                     a no-op
 *   dst_first,        the range's bounds in the decoded stream: the values
 *   dst_last          of dst_off[first] and dst_off[first + count], which the
 *                     caller knows from building the table; dst_first a
 *                     multiple of 16, dst_last <= t->total_bytes
 *   dst / out         receives decoded bytes [dst_first, dst_last) at
 *                     offset 0 (fused: the fp16 elements of those bytes, 2
 *                     per byte for INT4, 1 for INT8); 16-byte aligned
 *   chunk_status      count entries: entry k is chunk first + k
 * rows, cols, group, scales, zp describe the WHOLE tensor, as for the
 * full-table call; each element keeps its own group's scale.  The device
 * checks every chunk of the range against dst_first / dst_last (the first
 * chunk must start at dst_first, the last end at dst_last, none reach
 * outside): a chunk that does not is LT_CHUNK_BAD_TABLE and writes nothing,
 * so the output buffer is never overrun.  Output and statuses equal the
 * corresponding part of the full-table call's.
 */
lt_status lt_decode_lz4_range(const lt_chunk_table *t, uint32_t first, uint32_t count, uint64_t dst_first,
                              uint64_t dst_last, uint8_t *dst, int32_t *chunk_status, void *stream);
lt_status lt_fused_lz4_int4_range(const lt_chunk_table *t, const uint16_t *scales, const int8_t *zp,
                                  uint64_t rows, uint64_t cols, uint64_t group, uint32_t first, uint32_t count,
                                  uint64_t dst_first, uint64_t dst_last, uint16_t *out, int32_t *chunk_status,
                                  void *stream);
lt_status lt_fused_lz4_int8_range(const lt_chunk_table *t, const uint16_t *scales, const int8_t *zp,
                                  uint64_t rows, uint64_t cols, uint64_t group, uint32_t first, uint32_t count,
                                  uint64_t dst_first, uint64_t dst_last, uint16_t *out, int32_t *chunk_status,
                                  void *stream);

/*
 * Zero-run coding of fp16 activations (page "Openai/692db884-...
 * (section 28)", zero-run encoding: the zero slices of ReLU outputs stored
 * as runs of zeros instead of full arrays), in a block form every GPU wave
 * decodes on its own: the tensor of n_elem fp16 elements is cut into blocks
 * of LT_ZR_BLOCK elements (the last may be partial).
 *   bitmap   uint32 [32 per block]: bit k of word w of block b is 1 when
 *            element LT_ZR_BLOCK*b + 32w + k is nonzero (its 16 bits are
 *            not all zero, so -0.0 is kept); bits past n_elem are 0
 *   val_off  uint64 [blocks + 1]: nonzero elements before block b
 *   vals     uint16 [n_vals]: the nonzero elements in order (fp16 bits)
 */
#define LT_ZR_BLOCK 1024
typedef struct lt_zr_tensor {
  const uint32_t *bitmap;
  const uint64_t *val_off;
  const uint16_t *vals;     /* may be NULL when n_vals == 0 */
  uint64_t n_elem;
  uint64_t n_vals;
} lt_zr_tensor;

/*
 * lt_decode_zero_runs -- expand a zero-run coded tensor on the device.  All
 * arrays of *z are DEVICE memory; out: DEVICE uint16 [n_elem], 16-byte
 * aligned.  block_status (optional, DEVICE int32 [blocks]): LT_CHUNK_OK, or
 * LT_CHUNK_BAD_TABLE when a block's bit count differs from its val_off
 * span, val_off leaves [0, n_vals] or a bit past n_elem is set; such a
 * block writes nothing.  Output equals the input of lt_encode_zero_runs.
 */
lt_status lt_decode_zero_runs(const lt_zr_tensor *z, uint16_t *out, int32_t *block_status, void *stream);

/*
 * lt_verify_chunks -- per-chunk XXH3-64 (seed 0, the default secret) of the
 * compressed bytes on the device, without decoding (the container check of
 * page "GPU Compression Pipeline - TDD Roadmap", Phase 6.1: a changed stored
 * byte must be reported as a checksum mismatch); chunk i covers
 * t->comp[comp_off[i] .. comp_off[i+1]).  Decode calls check the same value
 * on the fly when the table carries xxh; this call checks a table without
 * decoding it.
 *   expect        DEVICE uint64 [n_chunks] stored checksums, or NULL
 *                 (compute only)
 *   got           DEVICE uint64 [n_chunks], receives the computed values, or
 *                 NULL
 *   chunk_status  DEVICE int32 [n_chunks]: LT_CHUNK_OK, LT_CHUNK_CHECKSUM
 *                 when expect[i] differs, LT_CHUNK_BAD_TABLE for offsets
 *                 outside comp_bytes or decreasing (required with expect)
 * Only comp, comp_off and comp_bytes of the table are read.  The host
 * packer's lt_checksum_chunks computes the stored values.
 */
lt_status lt_verify_chunks(const lt_chunk_table *t, const uint64_t *expect, uint64_t *got, int32_t *chunk_status,
                           void *stream);

/*
 * Streamed decode ("GPU Compression Pipeline - TDD Roadmap", Phase 5.1: the
 * transfer of one part overlaps the decompression of the part before, and
 * the result equals the sequential one).  The table's arrays -- comp,
 * comp_off, dst_off and, when present, seq_off and seq_pos -- are HOST
 * arrays; for the copies to overlap the decode they must be pinned
 * (hipHostMalloc, or torch's pin_memory).  comp_off[0] must be 0, and
 * comp_off, dst_off and seq_off must not decrease (checked on the host).  The
 * staging buffer holds, in order, the table's offset arrays and sequence
 * index (copied once, ahead of the first batch), then two halves for
 * compressed bytes.  The chunks are cut into batches, each as large as a
 * half holds; batch b is copied into half b % 2 on copy_stream, then
 * decoded on stream, and half b % 2 is copied into again only after that
 * decode has finished.  Output, chunk statuses and the validity rules are
 * those of lt_decode_lz4 / lt_fused_lz4_int4 on the same table.
 *   staging        DEVICE scratch owned by the caller, 256-byte aligned
 *   staging_bytes  its size: with u(x) = x rounded up to 256, at least
 *                  2*u(8(n+1)) [+ u(8 n) with checksums] [+ u(8(n+1)) +
 *                  u(4 n_seq) with an index] for the table, plus two
 *                  halves each holding
 *                  u(largest chunk's compressed bytes + 16);
 *                  LT_ERR_INVALID_ARG otherwise
 *   copy_stream    the stream the host-to-device copies run on (it may
 *                  equal stream, which then serializes copy and decode);
 *                  its first copy waits for the work already on `stream`,
 *                  so consecutive calls may share one staging buffer
 * Calls return once everything is enqueued.  The host arrays and the
 * staging buffer must stay untouched until the work on `stream` finishes.
 * Events are created and destroyed within the call; nothing else is
 * allocated.  LT_ERR_DEVICE if a copy or an event could not be enqueued.
 */
lt_status lt_stream_decode_lz4(const lt_chunk_table *host_table, uint8_t *dst, int32_t *chunk_status,
                               uint8_t *staging, uint64_t staging_bytes, void *copy_stream, void *stream);
lt_status lt_stream_fused_lz4_int4(const lt_chunk_table *host_table, const uint16_t *scales, const int8_t *zp,
                                   uint64_t rows, uint64_t cols, uint64_t group, uint16_t *out,
                                   int32_t *chunk_status, uint8_t *staging, uint64_t staging_bytes,
                                   void *copy_stream, void *stream);
/* INT8 codes (t->total_bytes == rows*cols), as lt_fused_lz4_int8. */
lt_status lt_stream_fused_lz4_int8(const lt_chunk_table *host_table, const uint16_t *scales, const int8_t *zp,
                                   uint64_t rows, uint64_t cols, uint64_t group, uint16_t *out,
                                   int32_t *chunk_status, uint8_t *staging, uint64_t staging_bytes,
                                   void *copy_stream, void *stream);

/*
 * The streamed calls with the compressed bytes in a file, the roadmap's
 * three stages ("GPU Compression Pipeline - TDD Roadmap", Phase 5.1: read
 * part N+1 while part N is transferred and part N-1 decompressed).  Chunk
 * i's compressed bytes are the file's bytes at file_offset + comp_off[i]
 * (the table's comp array is not read and may be NULL); the table's other
 * arrays are HOST arrays as for lt_stream_decode_lz4.  The calling thread
 * reads each batch with pread (read_threads threads side by side, pieces
 * of at least 1 MiB) into half b % 2 of `pinned`, then enqueues its copy
 * and decode as lt_stream_decode_lz4 does; it reads the next batch while
 * those run, and reads into a half again only after the copy that last
 * read it has finished.  Batches are as large as both a staging half and a
 * pinned half hold.
 *   fd            a file descriptor open for reading (pread: the file
 *                 position is not used or moved)
 *   pinned        HOST pinned memory (hipHostMalloc, torch's pin_memory)
 *                 owned by the caller, split into two halves of
 *                 (pinned_bytes / 2) rounded down to 256 bytes, each at
 *                 least the largest chunk's compressed bytes
 * Output, statuses and errors are those of the memory-resident streamed
 * calls, plus LT_ERR_IO when a read fails or the file ends early (the
 * batches before it stay enqueued).  The call returns once every batch has
 * been read and its copy and decode enqueued; the copies still read
 * `pinned`, so it and the staging buffer must stay untouched until the
 * work on `stream` finishes.
 */
lt_status lt_stream_file_decode_lz4(int fd, uint64_t file_offset, const lt_chunk_table *host_table, uint8_t *dst,
                                    int32_t *chunk_status, uint8_t *pinned, uint64_t pinned_bytes, int read_threads,
                                    uint8_t *staging, uint64_t staging_bytes, void *copy_stream, void *stream);
lt_status lt_stream_file_fused_lz4_int4(int fd, uint64_t file_offset, const lt_chunk_table *host_table,
                                        const uint16_t *scales, const int8_t *zp, uint64_t rows, uint64_t cols,
                                        uint64_t group, uint16_t *out, int32_t *chunk_status, uint8_t *pinned,
                                        uint64_t pinned_bytes, int read_threads, uint8_t *staging,
                                        uint64_t staging_bytes, void *copy_stream, void *stream);
lt_status lt_stream_file_fused_lz4_int8(int fd, uint64_t file_offset, const lt_chunk_table *host_table,
                                        const uint16_t *scales, const int8_t *zp, uint64_t rows, uint64_t cols,
                                        uint64_t group, uint16_t *out, int32_t *chunk_status, uint8_t *pinned,
                                        uint64_t pinned_bytes, int read_threads, uint8_t *staging,
                                        uint64_t staging_bytes, void *copy_stream, void *stream);

/*
 * lt_stream_fused_lz4_int4_static -- lt_stream_fused_lz4_int4 for callers
 * that cannot allocate: code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc.  It takes no staging argument and calls
 * no allocating routine (no hipMalloc, hipFree or event creation): its
 * staging workspace is a static device array of LT_STATIC_SCRATCH_BYTES
 * that every GPU the library runs on holds until the process ends (its
 * address is taken on each device's first call), and the copies and the
 * decodes run in order on `stream` alone, so copy and decode do not overlap.
 * Arguments, validity rules, output and chunk statuses are those of
 * lt_stream_fused_lz4_int4 (host table, pinned for asynchronous copies).
 * Returns LT_ERR_TOO_LARGE when the table's offsets and index plus twice the
 * largest chunk's compressed bytes (each rounded up to 256 bytes, plus 16)
 * exceed the workspace.  Every call on one GPU uses that GPU's one array, so
 * calls that overlap on one GPU (on different streams, or from different
 * threads without ordering between them) race and give wrong results; calls
 * in order on one stream are safe.  LT_ERR_DEVICE if the workspace's address
 * cannot be taken or a copy cannot be enqueued.
 */
#define LT_STATIC_SCRATCH_BYTES (32u << 20)
lt_status lt_stream_fused_lz4_int4_static(const lt_chunk_table *host_table, const uint16_t *scales,
                                          const int8_t *zp, uint64_t rows, uint64_t cols, uint64_t group,
                                          uint16_t *out, int32_t *chunk_status, void *stream);

/* ---- host-side packer: builds the inputs above (no device work) ---- */

/* Zero-run coding on the host (HOST arrays): bitmap [32 per block] and
 * val_off [blocks + 1] are always written; vals (capacity vals_cap) only
 * when not NULL, so a first call with vals NULL gives the size in
 * val_off[blocks].  LT_ERR_INVALID_ARG when vals_cap is too small. */
lt_status lt_encode_zero_runs(const uint16_t *x, uint64_t n, uint32_t *bitmap, uint64_t *val_off, uint16_t *vals,
                              uint64_t vals_cap, int threads);

/* XXH3-64 (seed 0, the default secret) of each chunk's compressed bytes, as
 * lt_verify_chunks and the decode calls compute them on the device, on up
 * to `threads` host threads (0: all).  xxh has n_chunks entries. */
lt_status lt_checksum_chunks(const uint8_t *comp, const uint64_t *comp_off, uint32_t n_chunks, uint64_t *xxh,
                             int threads);

/* The order field of a table (HOST arrays): order (uint32[n_chunks])
 * receives 0 .. n_chunks-1 sorted by decreasing decoded size
 * (dst_off[i+1] - dst_off[i]); chunks of one size keep table order.
 * LT_ERR_INVALID_ARG for a non-monotone dst_off. */
lt_status lt_order_chunks(const uint64_t *dst_off, uint32_t n_chunks, uint32_t *order);

/* The order field of a sequence-dense table (HOST arrays): like
 * lt_order_chunks, and chunks of one size by decreasing sequence count
 * (seq_off[i+1] - seq_off[i], the table's sequence index offsets); equal
 * counts keep table order.  A chunk with many short sequences lives longer
 * than one of the same size with few, and a launch lasts as long as its
 * slowest chunk, so those start first.  LT_ERR_INVALID_ARG for a NULL
 * array or a non-monotone dst_off or seq_off. */
lt_status lt_order_chunks_by_sequences(const uint64_t *dst_off, const uint64_t *seq_off, uint32_t n_chunks,
                                       uint32_t *order);

/*
 * lt_debug_violations -- only in the LT_DEBUG build (liblt_debug.so): the
 * number of calls of the decoder's exec-narrowing LDS stores that were not
 * wave-uniform (HOST *count) and the source line of the first (HOST
 * *first_line, 0 if none), since the library was loaded or last reset;
 * reset != 0 clears both afterwards.  Synchronous with the device.  The
 * release build returns LT_ERR_UNSUPPORTED.
 */
lt_status lt_debug_violations(uint32_t *count, uint32_t *first_line, int reset);
/* lt_debug_selftest -- LT_DEBUG build only: one wave on `stream` makes two
 * calls that break the uniformity rule on purpose (harmless LDS stores; sink
 * is DEVICE uint32[1] scratch), so that lt_debug_violations then counts 2.
 * The release build returns LT_ERR_UNSUPPORTED. */
lt_status lt_debug_selftest(uint32_t *sink, void *stream);

/* Worst-case size of one LZ4 block holding n bytes. */
uint64_t lt_lz4_bound(uint64_t n);

/*
 * lt_pack_int4 -- HOST.  codes: uint8[n_codes] (values 0..15, higher bits
 * ignored), n_codes even; packed: uint8[n_codes/2].  Low nibble first.
 */
lt_status lt_pack_int4(const uint8_t *codes, uint64_t n_codes, uint8_t *packed);

/*
 * lt_compress_chunks -- HOST.  Compresses src[dst_off[i] .. dst_off[i+1]) for
 * each of n_chunks chunks as an independent LZ4 block (the public block
 * format, which the pages name without defining) and concatenates them
 * into comp (capacity comp_cap); comp_off (uint64[n_chunks+1]) receives the
 * prefix sums.  threads <= 0 means one per host core.  Matches reach at most
 * max_dist bytes back (0 or anything above 65535 means 65535); the table
 * built from the result may declare that window.  Returns
 * LT_ERR_INVALID_ARG for a non-monotone table or too small a buffer
 * (sum of lt_lz4_bound over the chunks always suffices).
 */
lt_status lt_compress_chunks(const uint8_t *src, const uint64_t *dst_off, uint32_t n_chunks,
                             uint8_t *comp, uint64_t comp_cap, uint64_t *comp_off, int threads,
                             uint32_t max_dist);

/*
 * lt_compress_chunks_greedy -- HOST.  As lt_compress_chunks (same arguments,
 * layout and errors), with the plain greedy LZ4 parse of a general-purpose
 * block compressor: every hashed match of 4 bytes or more at any distance
 * from 1 to max_dist is taken and extended.  lt_compress_chunks accepts
 * hashed matches of 8 bytes or more and prefers runs of one byte, which
 * gives the device decoder longer sequences to work on; this form gives
 * the blocks a standard compressor would write, for tables not made here.
 */
lt_status lt_compress_chunks_greedy(const uint8_t *src, const uint64_t *dst_off, uint32_t n_chunks,
                                    uint8_t *comp, uint64_t comp_cap, uint64_t *comp_off, int threads,
                                    uint32_t max_dist);

/*
 * lt_index_chunks -- HOST.  Builds the sequence index of a chunk table from
 * its blocks (comp, comp_off as in lt_chunk_table): walks each block's
 * sequences and lists where each one starts, relative to the block.
 * seq_off (uint64[n_chunks+1]) always receives the prefix sums of the
 * per-chunk counts; seq_pos (uint32[seq_cap]) receives the offsets when it
 * is not NULL.  A block that breaks the format is listed up to the sequence
 * that breaks it (the device then fails that chunk).  threads <= 0 means one
 * per host core.  Returns LT_ERR_INVALID_ARG for NULL arrays, a
 * non-monotone comp_off, or seq_pos given with seq_cap < seq_off[n_chunks]
 * (seq_off is filled either way, so a first call with seq_pos NULL sizes
 * the second).
 */
lt_status lt_index_chunks(const uint8_t *comp, const uint64_t *comp_off, uint32_t n_chunks,
                          uint64_t *seq_off, uint32_t *seq_pos, uint64_t seq_cap, int threads);

const char *lt_status_str(lt_status s);
int lt_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* LT_H */
