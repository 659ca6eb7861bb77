/*
 * ltref.c -- CPU oracle for just-in-time tensor decompression.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load or call this library.  The product
 * path (the HIP library and its Python binding) never does, and this file
 * shares no code, header, table or helper with it.
 *
 * Everything here is plain, slow and written to be checked by eye:
 *   - fp16 <-> fp64 conversion from the IEEE 754 binary16/binary64 bit fields
 *     (round to nearest, ties to even);
 *   - the LZ4 *block* format (a public format that the pages name but never
 *     spell out): a block is a list of sequences; each sequence is a token
 *     byte whose high nibble is the literal count and low nibble is the match
 *     length minus 4 (value 15 in either nibble means "more length follows in
 *     bytes of 255 ended by a byte < 255"), then the literals, then a 2-byte
 *     little-endian back-reference distance, then the match length's extra
 *     bytes.  The last sequence carries literals only.  A match copies byte by
 *     byte from `distance` bytes back, so it may overlap its own output;
 *   - a greedy LZ4 block compressor and an all-literal "store" encoder;
 *   - nibble packing, INT4/INT8 dequantization (q - zp) * scale -> fp16, as the
 *     roadmap page ("GPU Compression Pipeline - TDD Roadmap", Phase 1.1 INT4
 *     Dequantization and Phase 1.2 INT8 Dequantization) defines it;
 *   - the fused path as the composition decode-then-dequantize, which is the
 *     roadmap's own CPU reference for its fused kernel (Phase 2.1 LZ4 + INT4
 *     Fused Kernel);
 *   - a random LZ4 sequence generator that builds a stream and its expected
 *     output side by side, independent of the compressor;
 *   - codebook dequantization of INT4 codes: each group of `group` elements
 *     has a 16-entry table of fp16 values and element e is entry q(e) of its
 *     group's table (the pages' value dictionaries: small integer codes plus
 *     a tiny lookup table);
 *   - zero-run coding of fp16 activations (the pages' zero-run encoding for
 *     ReLU outputs, "runs of zeros" stored instead of full arrays): per block
 *     of 1024 elements a bitmap marks the nonzero elements, and the nonzero
 *     values follow in element order; element bits are compared, so -0.0
 *     counts as nonzero and the round trip is exact;
 *   - XXH3-64 (seed 0, default secret) of each chunk's compressed bytes: the
 *     per-block checksum the roadmap's container format names ("GPU
 *     Compression Pipeline - TDD Roadmap", Phase 6.1), written from the
 *     hash's public definition, one input-length class at a time.
 *
 * Floating point: the product (q - zp) * s has at most 19 significant bits, so
 * it is exact in fp64 (and in fp32); the only rounding is the final one to
 * fp16, done here from the bit fields.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ fp16 */

/* binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * Normal value (1 + f/1024) * 2^(e-15); subnormal (e = 0) f * 2^-24. */
double ltref_f64_from_f16(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 31;
  int f = h & 1023;
  double v;
  if (e == 0) {
    v = ldexp((double)f, -24);
  } else if (e == 31) {
    v = (f == 0) ? INFINITY : NAN;
  } else {
    v = ldexp((double)(1024 + f), e - 25);
  }
  return sign ? -v : v;
}

/* Round a binary64 value to binary16, nearest-even.  The value is taken as an
 * integer significand M times 2^E, the fp16 quantum 2^qe for its binade is
 * found, and M is shifted right by (qe - E) bits with a guard/sticky
 * comparison against half a quantum. */
uint16_t ltref_f16_from_f64(double x) {
  uint64_t bits;
  memcpy(&bits, &x, 8);
  uint16_t sign = (uint16_t)((bits >> 48) & 0x8000u);
  int be = (int)((bits >> 52) & 0x7FF);
  uint64_t frac = bits & ((1ull << 52) - 1);
  if (be == 0x7FF) return frac ? (uint16_t)(sign | 0x7E00u) : (uint16_t)(sign | 0x7C00u);
  if (be == 0 && frac == 0) return sign;
  uint64_t M;
  int E;
  if (be == 0) { M = frac; E = -1074; }              /* binary64 subnormal */
  else { M = frac | (1ull << 52); E = be - 1075; }   /* binary64 normal */
  int bitlen = 64 - __builtin_clzll(M);
  int p = bitlen - 1 + E;                             /* floor(log2|x|) */
  int qe = (p < -14) ? -24 : p - 10;                  /* fp16 quantum exponent */
  int s = qe - E;                                     /* bits to drop */
  uint64_t n;
  if (s <= 0) {
    n = M << (-s);                                     /* exact (never for valid doubles) */
  } else if (s >= 64) {
    n = 0;                                             /* below a quarter quantum */
  } else {
    n = M >> s;
    uint64_t rem = M & ((1ull << s) - 1);
    uint64_t half = 1ull << (s - 1);
    if (rem > half || (rem == half && (n & 1))) n += 1;
  }
  if (qe == -24) {
    /* subnormal range: n in [0, 1024]; n == 1024 is the smallest normal and
     * its encoding (exponent field 1, fraction 0) equals n itself */
    return (uint16_t)(sign | (uint16_t)n);
  }
  if (n == 2048) { n = 1024; p += 1; }                /* rounding carried into the exponent */
  if (p + 15 >= 31) return (uint16_t)(sign | 0x7C00u); /* overflow to infinity */
  return (uint16_t)(sign | (uint16_t)((p + 15) << 10) | (uint16_t)(n - 1024));
}

void ltref_f16_from_f64_array(const double *x, uint64_t n, uint16_t *out) {
  for (uint64_t i = 0; i < n; i++) out[i] = ltref_f16_from_f64(x[i]);
}

/* fp32 bit patterns -> fp16 via an exact widening to binary64 */
void ltref_f16_from_f32bits_array(const uint32_t *b, uint64_t n, uint16_t *out) {
  for (uint64_t i = 0; i < n; i++) {
    float f;
    memcpy(&f, &b[i], 4);
    out[i] = ltref_f16_from_f64((double)f);
  }
}

void ltref_f64_from_f16_array(const uint16_t *h, uint64_t n, double *out) {
  for (uint64_t i = 0; i < n; i++) out[i] = ltref_f64_from_f16(h[i]);
}

/* ------------------------------------------------------------ LZ4 decode */

enum {
  LTREF_OK = 0,
  LTREF_TRUNCATED = 1,       /* input ended inside a sequence, or is empty */
  LTREF_BAD_OFFSET = 2,      /* distance 0, or reaching before the chunk start */
  LTREF_OVERRUN = 3,         /* a sequence would write past the chunk's size */
  LTREF_SIZE_MISMATCH = 4,   /* block ended with fewer bytes than the chunk's size */
  LTREF_BAD_TABLE = 5        /* offset table inconsistent for this chunk */
};

#define LTREF_LEN_CAP (1ull << 31)

/* Decode one LZ4 block in[0..m) into out[0..cap).  *produced gets the number
 * of bytes written.  Returns LTREF_OK only if the block parses completely and
 * produces exactly `cap` bytes. */
int ltref_lz4_decode_block(const uint8_t *in, uint64_t m, uint8_t *out, uint64_t cap,
                           uint64_t *produced) {
  uint64_t ip = 0, op = 0;
  int st = LTREF_OK;
  for (;;) {
    if (ip >= m) { st = LTREF_TRUNCATED; break; }
    uint8_t token = in[ip++];
    uint64_t lit = token >> 4;
    if (lit == 15) {
      uint8_t b;
      do {
        if (ip >= m) { st = LTREF_TRUNCATED; goto done; }
        b = in[ip++];
        lit += b;
        if (lit > LTREF_LEN_CAP) { st = LTREF_OVERRUN; goto done; }
      } while (b == 255);
    }
    if (lit > m - ip) { st = LTREF_TRUNCATED; break; }
    if (lit > cap - op) { st = LTREF_OVERRUN; break; }
    for (uint64_t k = 0; k < lit; k++) out[op + k] = in[ip + k];
    ip += lit;
    op += lit;
    if (ip == m) break;                               /* last sequence: literals only */
    if (m - ip < 2) { st = LTREF_TRUNCATED; break; }
    uint64_t dist = (uint64_t)in[ip] | ((uint64_t)in[ip + 1] << 8);
    ip += 2;
    if (dist == 0 || dist > op) { st = LTREF_BAD_OFFSET; break; }
    uint64_t mlen = (uint64_t)(token & 15) + 4;
    if ((token & 15) == 15) {
      uint8_t b;
      do {
        if (ip >= m) { st = LTREF_TRUNCATED; goto done; }
        b = in[ip++];
        mlen += b;
        if (mlen > LTREF_LEN_CAP) { st = LTREF_OVERRUN; goto done; }
      } while (b == 255);
    }
    if (mlen > cap - op) { st = LTREF_OVERRUN; break; }
    for (uint64_t k = 0; k < mlen; k++) out[op + k] = out[op - dist + k];  /* byte-serial */
    op += mlen;
  }
done:
  if (st == LTREF_OK && op != cap) st = LTREF_SIZE_MISMATCH;
  if (produced) *produced = op;
  return st;
}

/* ---------------------------------------------------------- LZ4 encoders */

static uint64_t put_len(uint8_t *out, uint64_t o, uint64_t v) {
  /* extra length bytes for a nibble that saturated at 15: v = total - 15 */
  while (v >= 255) { out[o++] = 255; v -= 255; }
  out[o++] = (uint8_t)v;
  return o;
}

static uint64_t put_sequence(uint8_t *out, uint64_t o, const uint8_t *lit, uint64_t nlit,
                             int has_match, uint64_t dist, uint64_t mlen) {
  uint64_t mcode = has_match ? mlen - 4 : 0;
  uint8_t token = (uint8_t)(((nlit >= 15 ? 15 : nlit) << 4) | (mcode >= 15 ? 15 : mcode));
  out[o++] = token;
  if (nlit >= 15) o = put_len(out, o, nlit - 15);
  memcpy(out + o, lit, nlit);
  o += nlit;
  if (has_match) {
    out[o++] = (uint8_t)(dist & 255);
    out[o++] = (uint8_t)(dist >> 8);
    if (mcode >= 15) o = put_len(out, o, mcode - 15);
  }
  return o;
}

/* Worst-case encoded size: every byte a literal. */
uint64_t ltref_lz4_bound(uint64_t n) { return n + n / 255 + 16; }

/* All-literal block: one literal-only sequence. */
uint64_t ltref_lz4_store(const uint8_t *in, uint64_t n, uint8_t *out) {
  return put_sequence(out, 0, in, n, 0, 0, 0);
}

static uint32_t le32(const uint8_t *p) {
  return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}

static uint32_t hash4(uint32_t v) { return (uint32_t)(v * 2654435761u) >> 16; }

/* Greedy compressor: one most-recent-position hash table over 4-byte values,
 * the format's end-of-block rules (the last 5 bytes are literals, no match
 * starts within the last 12 bytes), distances up to 65535. */
uint64_t ltref_lz4_compress(const uint8_t *x, uint64_t n, uint8_t *out) {
  const uint64_t MINMATCH = 4, LASTLITERALS = 5, MFLIMIT = 12, MAXDIST = 65535;
  if (n < MFLIMIT + 1) return put_sequence(out, 0, x, n, 0, 0, 0);
  int64_t *H = (int64_t *)malloc(sizeof(int64_t) * 65536);
  for (int k = 0; k < 65536; k++) H[k] = -1;
  uint64_t o = 0, anchor = 0, i = 0;
  while (i + MFLIMIT <= n) {
    uint32_t h = hash4(le32(x + i));
    int64_t c = H[h];
    H[h] = (int64_t)i;
    if (c >= 0 && i - (uint64_t)c <= MAXDIST && le32(x + c) == le32(x + i)) {
      uint64_t len = MINMATCH;
      while (i + len < n - LASTLITERALS && x[c + len] == x[i + len]) len++;
      o = put_sequence(out, o, x + anchor, i - anchor, 1, i - (uint64_t)c, len);
      for (uint64_t j = i + 1; j < i + len && j + MFLIMIT <= n; j++) H[hash4(le32(x + j))] = (int64_t)j;
      i += len;
      anchor = i;
    } else {
      i += 1;
    }
  }
  o = put_sequence(out, o, x + anchor, n - anchor, 0, 0, 0);
  free(H);
  return o;
}

/* ----------------------------------------------------------- INT4 / INT8 */

/* Two 4-bit codes per byte, the even element in the low nibble. */
void ltref_pack_int4(const uint8_t *codes, uint64_t n_codes, uint8_t *packed) {
  for (uint64_t k = 0; k < n_codes / 2; k++)
    packed[k] = (uint8_t)((codes[2 * k] & 15) | ((codes[2 * k + 1] & 15) << 4));
}

void ltref_unpack_int4(const uint8_t *packed, uint64_t n_codes, uint8_t *codes) {
  for (uint64_t e = 0; e < n_codes; e++) {
    uint8_t b = packed[e / 2];
    codes[e] = (e % 2 == 0) ? (uint8_t)(b & 15) : (uint8_t)(b >> 4);
  }
}

/* out[e] = fp16( (q[e] - zp[e / group]) * scale[e / group] ), zp = 0 when absent. */
void ltref_dequant_int4(const uint8_t *packed, uint64_t n_elem, const uint16_t *scales,
                        const int8_t *zp, uint64_t group, uint16_t *out) {
  for (uint64_t e = 0; e < n_elem; e++) {
    uint8_t b = packed[e / 2];
    int q = (e % 2 == 0) ? (b & 15) : (b >> 4);
    uint64_t g = e / group;
    int z = zp ? zp[g] : 0;
    double v = (double)(q - z) * ltref_f64_from_f16(scales[g]);
    out[e] = ltref_f16_from_f64(v);
  }
}

void ltref_dequant_int8(const int8_t *q, uint64_t n_elem, const uint16_t *scales,
                        const int8_t *zp, uint64_t group, uint16_t *out) {
  for (uint64_t e = 0; e < n_elem; e++) {
    uint64_t g = e / group;
    int z = zp ? zp[g] : 0;
    double v = (double)((int)q[e] - z) * ltref_f64_from_f16(scales[g]);
    out[e] = ltref_f16_from_f64(v);
  }
}

/* ----------------------------------------------------------- chunk tables */

/* Check chunk i's table entries: offsets in range and non-decreasing, the
 * first chunk starting at 0, the last ending at total. */
static int chunk_ok(uint64_t comp_bytes, const uint64_t *comp_off, const uint64_t *dst_off,
                    uint32_t n, uint64_t total, uint32_t i) {
  uint64_t c0 = comp_off[i], c1 = comp_off[i + 1], d0 = dst_off[i], d1 = dst_off[i + 1];
  if (c0 > c1 || c1 > comp_bytes || d0 > d1 || d1 > total) return 0;
  if (i == 0 && d0 != 0) return 0;
  if (i == n - 1 && d1 != total) return 0;
  return 1;
}

/* Decode chunk i of a table into out (the chunk's own bytes, dst_off[i+1] -
 * dst_off[i] of them); returns its status. */
static int decode_chunk(const uint8_t *comp, uint64_t comp_bytes, const uint64_t *comp_off,
                        const uint64_t *dst_off, uint32_t n, uint64_t total, uint32_t i,
                        uint8_t *out) {
  if (!chunk_ok(comp_bytes, comp_off, dst_off, n, total, i)) return LTREF_BAD_TABLE;
  return ltref_lz4_decode_block(comp + comp_off[i], comp_off[i + 1] - comp_off[i], out,
                                dst_off[i + 1] - dst_off[i], NULL);
}

typedef struct {
  const uint8_t *comp; uint64_t comp_bytes; const uint64_t *comp_off; const uint64_t *dst_off;
  uint32_t n; uint64_t total; uint8_t *dst; int32_t *status;
  uint32_t begin, step;
} decode_job;

static void *decode_worker(void *arg) {
  decode_job *j = (decode_job *)arg;
  for (uint32_t i = j->begin; i < j->n; i += j->step) {
    int st = LTREF_BAD_TABLE;
    if (chunk_ok(j->comp_bytes, j->comp_off, j->dst_off, j->n, j->total, i))
      st = decode_chunk(j->comp, j->comp_bytes, j->comp_off, j->dst_off, j->n, j->total, i,
                        j->dst + j->dst_off[i]);
    if (j->status) j->status[i] = st;
  }
  return NULL;
}

/* Decode every chunk of a table; chunks are independent, so `threads` workers
 * take every threads-th chunk.  Returns the number of chunks not OK. */
uint32_t ltref_decode_table(const uint8_t *comp, uint64_t comp_bytes, const uint64_t *comp_off,
                            const uint64_t *dst_off, uint32_t n, uint64_t total, uint8_t *dst,
                            int32_t *status, int threads) {
  if (threads < 1) threads = 1;
  if (threads > 256) threads = 256;
  int32_t *st = status ? status : (int32_t *)malloc(sizeof(int32_t) * (n ? n : 1));
  decode_job jobs[256];
  pthread_t tid[256];
  for (int t = 0; t < threads; t++) {
    jobs[t] = (decode_job){comp, comp_bytes, comp_off, dst_off, n, total, dst, st, (uint32_t)t, (uint32_t)threads};
    if (threads > 1) pthread_create(&tid[t], NULL, decode_worker, &jobs[t]);
  }
  if (threads == 1) decode_worker(&jobs[0]);
  else for (int t = 0; t < threads; t++) pthread_join(tid[t], NULL);
  uint32_t bad = 0;
  for (uint32_t i = 0; i < n; i++) bad += (st[i] != LTREF_OK);
  if (!status) free(st);
  return bad;
}

typedef struct {
  const uint8_t *src; const uint64_t *dst_off; uint32_t n; uint8_t **bufs; uint64_t *sizes;
  uint32_t begin, step;
} compress_job;

static void *compress_worker(void *arg) {
  compress_job *j = (compress_job *)arg;
  for (uint32_t i = j->begin; i < j->n; i += j->step) {
    uint64_t a = j->dst_off[i], b = j->dst_off[i + 1];
    j->bufs[i] = (uint8_t *)malloc(ltref_lz4_bound(b - a));
    j->sizes[i] = ltref_lz4_compress(j->src + a, b - a, j->bufs[i]);
  }
  return NULL;
}

/* Compress each chunk [dst_off[i], dst_off[i+1]) of src independently and
 * concatenate the blocks into comp (capacity comp_cap); comp_off gets the
 * prefix sums (n+1 entries).  Returns the total size, or 0 if comp_cap is too
 * small. */
uint64_t ltref_compress_table(const uint8_t *src, const uint64_t *dst_off, uint32_t n,
                              uint8_t *comp, uint64_t comp_cap, uint64_t *comp_off, int threads) {
  if (threads < 1) threads = 1;
  if (threads > 256) threads = 256;
  uint8_t **bufs = (uint8_t **)calloc(n ? n : 1, sizeof(uint8_t *));
  uint64_t *sizes = (uint64_t *)calloc(n ? n : 1, sizeof(uint64_t));
  compress_job jobs[256];
  pthread_t tid[256];
  for (int t = 0; t < threads; t++) {
    jobs[t] = (compress_job){src, dst_off, n, bufs, sizes, (uint32_t)t, (uint32_t)threads};
    if (threads > 1) pthread_create(&tid[t], NULL, compress_worker, &jobs[t]);
  }
  if (threads == 1) compress_worker(&jobs[0]);
  else for (int t = 0; t < threads; t++) pthread_join(tid[t], NULL);
  uint64_t pos = 0, ok = 1;
  comp_off[0] = 0;
  for (uint32_t i = 0; i < n; i++) {
    if (pos + sizes[i] > comp_cap) ok = 0;
    if (ok) memcpy(comp + pos, bufs[i], sizes[i]);
    pos += sizes[i];
    comp_off[i + 1] = pos;
    free(bufs[i]);
  }
  free(bufs);
  free(sizes);
  return ok ? pos : 0;
}

/* Fused reference: decode the whole table, then dequantize (the composition
 * the roadmap uses as the CPU reference for its fused kernel). */
uint32_t ltref_fused_int4(const uint8_t *comp, uint64_t comp_bytes, const uint64_t *comp_off,
                          const uint64_t *dst_off, uint32_t n, uint64_t total,
                          const uint16_t *scales, const int8_t *zp, uint64_t n_elem,
                          uint64_t group, uint16_t *out, int32_t *status, int threads) {
  uint8_t *tmp = (uint8_t *)calloc(total ? total : 1, 1);
  uint32_t bad = ltref_decode_table(comp, comp_bytes, comp_off, dst_off, n, total, tmp, status, threads);
  ltref_dequant_int4(tmp, n_elem, scales, zp, group, out);
  free(tmp);
  return bad;
}

uint32_t ltref_fused_int8(const uint8_t *comp, uint64_t comp_bytes, const uint64_t *comp_off,
                          const uint64_t *dst_off, uint32_t n, uint64_t total,
                          const uint16_t *scales, const int8_t *zp, uint64_t n_elem,
                          uint64_t group, uint16_t *out, int32_t *status, int threads) {
  uint8_t *tmp = (uint8_t *)calloc(total ? total : 1, 1);
  uint32_t bad = ltref_decode_table(comp, comp_bytes, comp_off, dst_off, n, total, tmp, status, threads);
  ltref_dequant_int8((const int8_t *)tmp, n_elem, scales, zp, group, out);
  free(tmp);
  return bad;
}

typedef struct {
  const uint8_t *comp; uint64_t comp_bytes; const uint64_t *comp_off; const uint64_t *dst_off;
  uint32_t n; uint64_t total; const uint16_t *scales; const int8_t *zp; uint64_t group;
  uint16_t *out; int32_t *status; uint32_t begin, step;
} fused_job;

static void *fused_worker(void *arg) {
  fused_job *j = (fused_job *)arg;
  uint8_t *tmp = NULL;
  uint64_t tmp_cap = 0;
  for (uint32_t i = j->begin; i < j->n; i += j->step) {
    uint64_t d0 = j->dst_off[i], d1 = j->dst_off[i + 1];
    int st = LTREF_BAD_TABLE;
    if (chunk_ok(j->comp_bytes, j->comp_off, j->dst_off, j->n, j->total, i)) {
      if (d1 - d0 > tmp_cap || !tmp) { free(tmp); tmp_cap = d1 - d0; tmp = (uint8_t *)malloc(tmp_cap + 1); }
      st = decode_chunk(j->comp, j->comp_bytes, j->comp_off, j->dst_off, j->n, j->total, i, tmp);
      if (st == LTREF_OK) {
        /* chunk i holds packed bytes [d0, d1), i.e. elements [2*d0, 2*d1) */
        for (uint64_t e = 2 * d0; e < 2 * d1; e++) {
          uint8_t b = tmp[e / 2 - d0];
          int q = (e % 2 == 0) ? (b & 15) : (b >> 4);
          uint64_t g = e / j->group;
          int z = j->zp ? j->zp[g] : 0;
          j->out[e] = ltref_f16_from_f64((double)(q - z) * ltref_f64_from_f16(j->scales[g]));
        }
      }
    }
    if (j->status) j->status[i] = st;
  }
  free(tmp);
  return NULL;
}

/* Chunk-parallel fused reference for timing: per chunk, decode into a private
 * buffer, then dequantize that chunk's elements.  Same arithmetic as
 * ltref_fused_int4, with threads over chunks. */
uint32_t ltref_fused_int4_chunked(const uint8_t *comp, uint64_t comp_bytes, const uint64_t *comp_off,
                                  const uint64_t *dst_off, uint32_t n, uint64_t total,
                                  const uint16_t *scales, const int8_t *zp, uint64_t group,
                                  uint16_t *out, int32_t *status, int threads) {
  if (threads < 1) threads = 1;
  if (threads > 256) threads = 256;
  int32_t *st = status ? status : (int32_t *)malloc(sizeof(int32_t) * (n ? n : 1));
  fused_job jobs[256];
  pthread_t tid[256];
  for (int t = 0; t < threads; t++) {
    jobs[t] = (fused_job){comp, comp_bytes, comp_off, dst_off, n, total, scales, zp, group, out, st,
                          (uint32_t)t, (uint32_t)threads};
    if (threads > 1) pthread_create(&tid[t], NULL, fused_worker, &jobs[t]);
  }
  if (threads == 1) fused_worker(&jobs[0]);
  else for (int t = 0; t < threads; t++) pthread_join(tid[t], NULL);
  uint32_t bad = 0;
  for (uint32_t i = 0; i < n; i++) bad += (st[i] != LTREF_OK);
  if (!status) free(st);
  return bad;
}

/* ------------------------------------------------------ sequence generator */

/* splitmix64 (Steele, Lea, Flood, "Fast splittable pseudorandom number
 * generators", 2014): state += 0x9E3779B97F4A7C15, then two xor-shift-multiply
 * rounds. */
static uint64_t sm64(uint64_t *s) {
  uint64_t z = (*s += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

static uint64_t rnd_below(uint64_t *s, uint64_t n) { return n ? sm64(s) % n : 0; }

static uint64_t pick_len(uint64_t *s, uint64_t lo, uint64_t hi, const uint64_t *special, int ns) {
  /* half the time a boundary value, otherwise uniform in [lo, hi] */
  if (sm64(s) & 1) return special[rnd_below(s, (uint64_t)ns)];
  return lo + rnd_below(s, hi - lo + 1);
}

/* Build a random valid LZ4 block and the bytes it must decode to, side by
 * side, without using the compressor: literal lengths biased to the nibble /
 * extra-byte boundaries, match lengths likewise, distances biased to small and
 * extreme values (1, 2, 3, 4, 7, 8, 63, 64, 65, 65535).  Once the next match
 * would pass `target` output bytes, a literal-only last sequence fills the
 * output to exactly `target` bytes.  Returns the stream length (0 if a capacity is too small);
 * *out_len gets the output length.  Needs stream_cap >= 2*target + 64 and
 * out_cap >= target. */
uint64_t ltref_seqgen(uint64_t seed, uint64_t target, uint8_t *stream, uint64_t stream_cap,
                      uint8_t *expected, uint64_t out_cap, uint64_t *out_len) {
  static const uint64_t LSP[] = {0, 1, 14, 15, 16, 269, 270, 271, 524, 525, 526};
  static const uint64_t MSP[] = {4, 5, 18, 19, 20, 273, 274, 275, 528, 529, 530};
  static const uint64_t DSP[] = {1, 2, 3, 4, 7, 8, 63, 64, 65, 65535};
  *out_len = 0;
  if (stream_cap < 2 * target + 64 || out_cap < target) return 0;
  uint64_t s = seed;
  uint64_t o = 0, op = 0;
  uint8_t *lit = (uint8_t *)malloc(target + 1);
  for (;;) {
    uint64_t nl = pick_len(&s, 0, 300, LSP, 11);
    if (op == 0 && nl == 0 && target > 0) nl = 1;
    if (nl > target - op) nl = target - op;
    for (uint64_t k = 0; k < nl; k++) {
      /* literals: mostly a small alphabet so later matches against them are common */
      uint64_t r = sm64(&s);
      lit[k] = (r & 3) ? (uint8_t)((r >> 8) & 7) : (uint8_t)(r >> 16);
    }
    uint64_t after = op + nl;
    uint64_t ml = pick_len(&s, 4, 300, MSP, 11);
    if (after == 0 || ml > target - after) {
      /* last sequence: literals only, filling the output to exactly target */
      nl = target - op;
      for (uint64_t k = 0; k < nl; k++) {
        uint64_t r = sm64(&s);
        lit[k] = (r & 3) ? (uint8_t)((r >> 8) & 7) : (uint8_t)(r >> 16);
      }
      o = put_sequence(stream, o, lit, nl, 0, 0, 0);
      memcpy(expected + op, lit, nl);
      op += nl;
      break;
    }
    uint64_t maxd = after < 65535 ? after : 65535;
    uint64_t d = DSP[rnd_below(&s, 10)];
    if ((sm64(&s) & 1) || d > maxd) d = 1 + rnd_below(&s, maxd);
    o = put_sequence(stream, o, lit, nl, 1, d, ml);
    memcpy(expected + op, lit, nl);
    op += nl;
    for (uint64_t k = 0; k < ml; k++) expected[op + k] = expected[op - d + k];
    op += ml;
  }
  free(lit);
  *out_len = op;
  return o;
}

/* ---------------------------------------------------------------- XXH3-64 */

/* XXH3, 64-bit result, seed 0, the default 192-byte secret: the block
 * checksum named by the roadmap's container format (page "GPU Compression
 * Pipeline - TDD Roadmap", Phase 6.1 HCT Format V2).  The pages only name
 * it; the steps below follow the public XXH3 definition, one input-length
 * class at a time, with arithmetic modulo 2^64 and the 128-bit products
 * taken whole. */
static const uint8_t XXH_SECRET[192] = {
  0xb8, 0xfe, 0x6c, 0x39, 0x23, 0xa4, 0x4b, 0xbe, 0x7c, 0x01, 0x81, 0x2c, 0xf7, 0x21, 0xad, 0x1c,
  0xde, 0xd4, 0x6d, 0xe9, 0x83, 0x90, 0x97, 0xdb, 0x72, 0x40, 0xa4, 0xa4, 0xb7, 0xb3, 0x67, 0x1f,
  0xcb, 0x79, 0xe6, 0x4e, 0xcc, 0xc0, 0xe5, 0x78, 0x82, 0x5a, 0xd0, 0x7d, 0xcc, 0xff, 0x72, 0x21,
  0xb8, 0x08, 0x46, 0x74, 0xf7, 0x43, 0x24, 0x8e, 0xe0, 0x35, 0x90, 0xe6, 0x81, 0x3a, 0x26, 0x4c,
  0x3c, 0x28, 0x52, 0xbb, 0x91, 0xc3, 0x00, 0xcb, 0x88, 0xd0, 0x65, 0x8b, 0x1b, 0x53, 0x2e, 0xa3,
  0x71, 0x64, 0x48, 0x97, 0xa2, 0x0d, 0xf9, 0x4e, 0x38, 0x19, 0xef, 0x46, 0xa9, 0xde, 0xac, 0xd8,
  0xa8, 0xfa, 0x76, 0x3f, 0xe3, 0x9c, 0x34, 0x3f, 0xf9, 0xdc, 0xbb, 0xc7, 0xc7, 0x0b, 0x4f, 0x1d,
  0x8a, 0x51, 0xe0, 0x4b, 0xcd, 0xb4, 0x59, 0x31, 0xc8, 0x9f, 0x7e, 0xc9, 0xd9, 0x78, 0x73, 0x64,
  0xea, 0xc5, 0xac, 0x83, 0x34, 0xd3, 0xeb, 0xc3, 0xc5, 0x81, 0xa0, 0xff, 0xfa, 0x13, 0x63, 0xeb,
  0x17, 0x0d, 0xdd, 0x51, 0xb7, 0xf0, 0xda, 0x49, 0xd3, 0x16, 0x55, 0x26, 0x29, 0xd4, 0x68, 0x9e,
  0x2b, 0x16, 0xbe, 0x58, 0x7d, 0x47, 0xa1, 0xfc, 0x8f, 0xf8, 0xb8, 0xd1, 0x7a, 0xd0, 0x31, 0xce,
  0x45, 0xcb, 0x3a, 0x8f, 0x95, 0x16, 0x04, 0x28, 0xaf, 0xd7, 0xfb, 0xca, 0xbb, 0x4b, 0x40, 0x7e,
};
static const uint64_t XP32_1 = 0x9E3779B1u, XP32_2 = 0x85EBCA77u, XP32_3 = 0xC2B2AE3Du;
static const uint64_t XP64_1 = 0x9E3779B185EBCA87ull, XP64_2 = 0xC2B2AE3D27D4EB4Full,
                      XP64_3 = 0x165667B19E3779F9ull, XP64_4 = 0x85EBCA77C2B2AE63ull,
                      XP64_5 = 0x27D4EB2F165667C5ull;

static uint64_t x_rd64(const uint8_t *p) {
  uint64_t v = 0;
  for (int k = 7; k >= 0; k--) v = (v << 8) | p[k];
  return v;
}
static uint32_t x_rd32(const uint8_t *p) { return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24); }
static uint64_t x_rotl(uint64_t v, int r) { return (v << r) | (v >> (64 - r)); }
static uint64_t x_swap64(uint64_t v) {
  uint64_t r = 0;
  for (int k = 0; k < 8; k++) r = (r << 8) | ((v >> (8 * k)) & 0xFF);
  return r;
}
/* the 128-bit product of a and b, its two halves XORed together */
static uint64_t x_fold(uint64_t a, uint64_t b) {
  const unsigned __int128 m = (unsigned __int128)a * b;
  return (uint64_t)m ^ (uint64_t)(m >> 64);
}
/* final mixes: the one XXH64 ends with, and XXH3's own */
static uint64_t x_avalanche64(uint64_t h) {
  h ^= h >> 33;
  h *= XP64_2;
  h ^= h >> 29;
  h *= XP64_3;
  return h ^ (h >> 32);
}
static uint64_t x_avalanche3(uint64_t h) {
  h ^= h >> 37;
  h *= 0x165667919E3779F9ull;
  return h ^ (h >> 32);
}
static uint64_t x_mix16(const uint8_t *in, const uint8_t *sec) {
  return x_fold(x_rd64(in) ^ x_rd64(sec), x_rd64(in + 8) ^ x_rd64(sec + 8));
}

/* one 64-byte stripe into the eight accumulators */
static void x_stripe(uint64_t acc[8], const uint8_t *in, const uint8_t *sec) {
  for (int i = 0; i < 8; i++) {
    const uint64_t v = x_rd64(in + 8 * i);
    const uint64_t k = v ^ x_rd64(sec + 8 * i);
    acc[i ^ 1] += v;
    acc[i] += (k & 0xFFFFFFFFu) * (k >> 32);
  }
}
static void x_scramble(uint64_t acc[8], const uint8_t *sec) {
  for (int i = 0; i < 8; i++) {
    uint64_t a = acc[i];
    a ^= a >> 47;
    a ^= x_rd64(sec + 8 * i);
    acc[i] = a * XP32_1;
  }
}

uint64_t ltref_xxh3_64(const uint8_t *in, uint64_t n) {
  const uint8_t *sec = XXH_SECRET;
  if (n == 0) return x_avalanche64(x_rd64(sec + 56) ^ x_rd64(sec + 64));
  if (n <= 3) {
    const uint32_t c = ((uint32_t)in[0] << 16) | ((uint32_t)in[n >> 1] << 24) | (uint32_t)in[n - 1] | ((uint32_t)n << 8);
    const uint64_t flip = (uint64_t)(x_rd32(sec) ^ x_rd32(sec + 4));
    return x_avalanche64((uint64_t)c ^ flip);
  }
  if (n <= 8) {
    const uint64_t flip = x_rd64(sec + 8) ^ x_rd64(sec + 16);
    const uint64_t v = (uint64_t)x_rd32(in + n - 4) + ((uint64_t)x_rd32(in) << 32);
    uint64_t h = v ^ flip;
    h ^= x_rotl(h, 49) ^ x_rotl(h, 24);
    h *= 0x9FB21C651E98DF25ull;
    h ^= (h >> 35) + n;
    h *= 0x9FB21C651E98DF25ull;
    return h ^ (h >> 28);
  }
  if (n <= 16) {
    const uint64_t lo = x_rd64(in) ^ (x_rd64(sec + 24) ^ x_rd64(sec + 32));
    const uint64_t hi = x_rd64(in + n - 8) ^ (x_rd64(sec + 40) ^ x_rd64(sec + 48));
    return x_avalanche3(n + x_swap64(lo) + hi + x_fold(lo, hi));
  }
  if (n <= 128) {
    uint64_t acc = n * XP64_1;
    /* pairs of 16-byte pieces from both ends, inward */
    const uint64_t pairs = (n - 1) / 32;   /* 0 .. 3: how many extra pairs */
    for (uint64_t j = pairs + 1; j-- > 0;) {
      acc += x_mix16(in + 16 * j, sec + 32 * j);
      acc += x_mix16(in + n - 16 * (j + 1), sec + 32 * j + 16);
    }
    return x_avalanche3(acc);
  }
  if (n <= 240) {
    uint64_t acc = n * XP64_1;
    for (uint64_t j = 0; j < 8; j++) acc += x_mix16(in + 16 * j, sec + 16 * j);
    acc = x_avalanche3(acc);
    for (uint64_t j = 8; j < n / 16; j++) acc += x_mix16(in + 16 * j, sec + 16 * (j - 8) + 3);
    acc += x_mix16(in + n - 16, sec + 136 - 17);
    return x_avalanche3(acc);
  }
  /* long inputs: blocks of 16 stripes (1024 bytes), each followed by a
   * scramble; then the last block's whole stripes, the input's last 64
   * bytes as one more stripe, and the merge of the accumulators */
  uint64_t acc[8] = {XP32_3, XP64_1, XP64_2, XP64_3, XP64_4, XP32_2, XP64_5, XP32_1};
  const uint64_t nblocks = (n - 1) / 1024;
  for (uint64_t b = 0; b < nblocks; b++) {
    for (uint64_t s = 0; s < 16; s++) x_stripe(acc, in + 1024 * b + 64 * s, sec + 8 * s);
    x_scramble(acc, sec + 192 - 64);
  }
  const uint64_t nstripes = ((n - 1) - 1024 * nblocks) / 64;
  for (uint64_t s = 0; s < nstripes; s++) x_stripe(acc, in + 1024 * nblocks + 64 * s, sec + 8 * s);
  x_stripe(acc, in + n - 64, sec + 192 - 64 - 7);
  uint64_t h = n * XP64_1;
  for (int i = 0; i < 4; i++) h += x_fold(acc[2 * i] ^ x_rd64(sec + 11 + 16 * i), acc[2 * i + 1] ^ x_rd64(sec + 11 + 16 * i + 8));
  return x_avalanche3(h);
}

/* One XXH3-64 per chunk over comp[comp_off[i] .. comp_off[i+1]). */
void ltref_xxh3_chunks(const uint8_t *comp, const uint64_t *comp_off, uint32_t n, uint64_t *h) {
  for (uint32_t i = 0; i < n; i++) h[i] = ltref_xxh3_64(comp + comp_off[i], comp_off[i + 1] - comp_off[i]);
}

/* ------------------------------------------------------------ zero runs */

/* Block b covers elements [1024 b, min(1024 (b + 1), n)).  Bit k of bitmap
 * word w stands for element 32 w + k and is 1 when that element's bits are
 * not all zero.  val_off[b] counts the nonzero elements before block b;
 * vals lists the nonzero elements in order.  Returns the nonzero count. */
uint64_t ltref_zr_encode(const uint16_t *x, uint64_t n, uint32_t *bitmap, uint64_t *val_off, uint16_t *vals) {
  const uint64_t nb = (n + 1023) / 1024;
  uint64_t m = 0;
  for (uint64_t b = 0; b < nb; b++) {
    val_off[b] = m;
    for (uint64_t w = 0; w < 32; w++) bitmap[32 * b + w] = 0;
    for (uint64_t e = 1024 * b; e < n && e < 1024 * (b + 1); e++) {
      if (x[e] != 0) {
        bitmap[e / 32] |= 1u << (e % 32);
        vals[m++] = x[e];
      }
    }
  }
  val_off[nb] = m;
  return m;
}

/* Inverse of the above: each element is its next listed value when its bit
 * is set, else zero.  Block status 0 when the block's bit count equals its
 * val_off span within n_vals and no bit is set past n; otherwise 5 (the
 * table's entries are inconsistent) and the block's output is left as it
 * was. */
void ltref_zr_decode(const uint32_t *bitmap, const uint64_t *val_off, const uint16_t *vals, uint64_t n,
                     uint64_t n_vals, uint16_t *out, int32_t *status) {
  const uint64_t nb = (n + 1023) / 1024;
  for (uint64_t b = 0; b < nb; b++) {
    uint64_t bits = 0, past = 0;
    for (uint64_t e = 1024 * b; e < 1024 * (b + 1); e++) {
      const int set = (bitmap[e / 32] >> (e % 32)) & 1u;
      bits += set;
      if (set && e >= n) past = 1;
    }
    if (past || val_off[b] > val_off[b + 1] || val_off[b + 1] > n_vals || val_off[b + 1] - val_off[b] != bits) {
      if (status) status[b] = 5;
      continue;
    }
    uint64_t m = val_off[b];
    for (uint64_t e = 1024 * b; e < n && e < 1024 * (b + 1); e++)
      out[e] = ((bitmap[e / 32] >> (e % 32)) & 1u) ? vals[m++] : 0;
    if (status) status[b] = 0;
  }
}

/* ------------------------------------------------------------ codebooks */

/* out[e] = lut[16 * (e / group) + q(e)], q(e) the 4-bit code of element e
 * (low nibble first). */
void ltref_dequant_int4_lut(const uint8_t *packed, uint64_t n_elem, const uint16_t *lut, uint64_t group,
                            uint16_t *out) {
  for (uint64_t e = 0; e < n_elem; e++) {
    const uint8_t b = packed[e / 2];
    const uint32_t q = (e % 2 == 0) ? (b & 15u) : (b >> 4);
    out[e] = lut[16 * (e / group) + q];
  }
}
