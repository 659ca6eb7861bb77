// lt_pack.cpp -- host-side packer for liblt: nibble packing and an LZ4 block
// compressor that builds the chunk tables the device entry points consume
// (the pages' packing tool and compressor, "Openai/691a41cd ..." (section 38),
// the list of shipped tools; block size 64 KiB from "GPU Compression Pipeline
// - TDD Roadmap", Phase 6.1).
//
// The compressor is greedy.  At each position it tries two candidates and
// keeps the longer match:
//   * a run check at distance 1 (runs of one byte: pruned rows, zero groups,
//     ReLU zeros), accepted from 4 bytes;
//   * the most recent earlier position with the same 4-byte hash (distance up
//     to 65535), accepted from 8 bytes, so isolated 4-byte coincidences in
//     near-random code bytes do not split long literal runs.
// A hashed match is passed over when a run starting at the next byte covers
// nearly as much (within kRunSlack bytes; a zero group after a nonzero byte,
// say, which an earlier zero group followed by the same byte would match one
// byte longer): the run costs a few more bytes, but the device decoder
// builds it without reading earlier output, so the tiles of the decoded
// stream stay independent.
// It keeps the format's end-of-block rules (the last 5 bytes are literals and
// no match starts within the last 12 bytes), so standard LZ4 block decoders
// accept its output.
#include <stdint.h>
#include <string.h>

#include <algorithm>
#include <thread>
#include <vector>

#include "lt.h"
#include "lt_xxh_secret.h"

namespace {

constexpr uint32_t kMinRun = 4;       // accepted length for distance-1 runs
constexpr uint32_t kRunSlack = 4;     // a run is preferred to a match at most this much longer
constexpr uint32_t kMinMatch = 8;     // accepted length for hashed matches
constexpr uint32_t kLastLiterals = 5;
constexpr uint32_t kMatchLimit = 12;  // no match may start in the last 12 bytes
constexpr uint32_t kMaxDist = 65535;   // the format's limit; callers may ask for less
constexpr int kHashBits = 15;

inline uint32_t rd32(const uint8_t *p) {
  uint32_t v;
  memcpy(&v, p, 4);
  return v;
}

inline uint32_t hash32(uint32_t v) { return (v * 2654435761u) >> (32 - kHashBits); }

struct Writer {
  uint8_t *out;
  uint64_t pos;
  void len_bytes(uint64_t v) {  // v = length - 15
    while (v >= 255) {
      out[pos++] = 255;
      v -= 255;
    }
    out[pos++] = (uint8_t)v;
  }
  void sequence(const uint8_t *lit, uint64_t nlit, uint64_t dist, uint64_t mlen) {
    uint64_t mc = mlen ? mlen - 4 : 0;
    out[pos++] = (uint8_t)((std::min<uint64_t>(nlit, 15) << 4) | std::min<uint64_t>(mc, 15));
    if (nlit >= 15) len_bytes(nlit - 15);
    memcpy(out + pos, lit, nlit);
    pos += nlit;
    if (mlen) {
      out[pos++] = (uint8_t)(dist & 255);
      out[pos++] = (uint8_t)(dist >> 8);
      if (mc >= 15) len_bytes(mc - 15);
    }
  }
};

// Compress src[0, n) into out (capacity >= lt_lz4_bound(n)); returns size.
// Greedy is the plain LZ4 parse: at each position the hashed candidate is
// taken when its first 4 bytes match (any distance from 1 to max_dist),
// extended forward, every position inside it is indexed, and the scan
// resumes after it.  The default parse
// instead accepts hashed matches of 8 bytes or more and prefers runs
// (distance 1), which a decoder builds without reading earlier output.
template <bool Greedy>
uint64_t compress_block(const uint8_t *src, uint64_t n, uint8_t *out, std::vector<int32_t> &table,
                        uint64_t max_dist) {
  Writer w{out, 0};
  if (n < kMatchLimit + 1) {
    w.sequence(src, n, 0, 0);
    return w.pos;
  }
  std::fill(table.begin(), table.end(), -1);
  const uint64_t match_end = n - kLastLiterals;  // matches must stop before this
  uint64_t anchor = 0, i = 0;
  while (i + kMatchLimit <= n) {
    uint64_t best_len = 0, best_dist = 0;
    // distance-1 run
    if (!Greedy && i > 0 && src[i] == src[i - 1]) {
      uint64_t len = 0;
      while (i + len < match_end && src[i + len] == src[i - 1]) len++;
      if (len >= kMinRun) {
        best_len = len;
        best_dist = 1;
      }
    }
    uint32_t h = hash32(rd32(src + i));
    int64_t c = table[h];
    table[h] = (int32_t)i;
    if (c >= 0 && i - (uint64_t)c <= max_dist && i - (uint64_t)c > (Greedy ? 0u : 1u) &&
        rd32(src + c) == rd32(src + i)) {
      uint64_t len = 4;
      while (i + len < match_end && src[c + len] == src[i + len]) len++;
      if (len >= (Greedy ? 4u : kMinMatch) && len > best_len) {
        best_len = len;
        best_dist = i - (uint64_t)c;
      }
    }
    if (!Greedy && best_dist > 1 && i + 2 + kMatchLimit <= n) {
      // A run starting at i + 1 (of src[i]) or at i + 2 (of src[i + 1]) that
      // covers nearly as much as the hashed match, with the bytes before it
      // as literals, is taken instead: a run decodes without reading earlier
      // output.
      for (uint64_t s0 = 1; s0 <= 2 && best_len; s0++) {
        const uint8_t v = src[i + s0 - 1];
        uint64_t r = 0;
        while (i + s0 + r < match_end && src[i + s0 + r] == v) r++;
        if (r >= kMinRun && r + s0 + kRunSlack >= best_len) best_len = 0;
      }
    }
    if (best_len) {
      w.sequence(src + anchor, i - anchor, best_dist, best_len);
      uint64_t stop = i + best_len;
      // index positions inside the match so later repeats find it (the
      // greedy parse indexes all of them, the default only the last two)
      const uint64_t j0 = Greedy ? i + 1 : std::max<uint64_t>(i + 1, stop > 2 ? stop - 2 : 0);
      for (uint64_t j = j0; j < stop && j + kMatchLimit <= n; j++) table[hash32(rd32(src + j))] = (int32_t)j;
      i = stop;
      anchor = i;
    } else {
      i++;
    }
  }
  w.sequence(src + anchor, n - anchor, 0, 0);
  return w.pos;
}

// Calls visit(p) for the offset p of each sequence of the block b[0 .. n),
// in order.  The walk ends after the literal-only last sequence, or at the
// sequence that breaks the format (that one is still visited).
template <class F>
void walk_block(const uint8_t *b, uint64_t n, F &&visit) {
  uint64_t p = 0;
  while (p < n) {
    visit(p);
    const uint8_t token = b[p++];
    uint64_t lit = token >> 4;
    if (lit == 15) {
      for (;;) {
        if (p >= n) return;
        const uint8_t v = b[p++];
        lit += v;
        if (v != 255) break;
      }
    }
    if (lit > n - p) return;
    p += lit;
    if (p == n || n - p < 2) return;
    p += 2;   // the distance
    if ((token & 15) == 15) {
      for (;;) {
        if (p >= n) return;
        if (b[p++] != 255) break;
      }
    }
  }
}

// runs fn(i) for i in [0, n) on up to `threads` host threads
template <class F>
void parallel_chunks(uint32_t n, int threads, F &&fn) {
  if (threads <= 0) threads = (int)std::max(1u, std::thread::hardware_concurrency());
  threads = std::min<int>(threads, (int)n);
  threads = std::min(threads, 256);
  auto work = [&](int t) {
    for (uint32_t i = (uint32_t)t; i < n; i += (uint32_t)threads) fn(i);
  };
  std::vector<std::thread> pool;
  for (int t = 1; t < threads; t++) pool.emplace_back(work, t);
  work(0);
  for (auto &th : pool) th.join();
}

// XXH3-64 with seed 0 and the default secret (the hash's public
// definition): the per-chunk checksum the device verifies.
constexpr uint64_t kXSec[24] = {LT_XXH_SECRET_WORDS};
constexpr uint64_t kXP64_1 = 0x9E3779B185EBCA87ull, kXP64_2 = 0xC2B2AE3D27D4EB4Full, kXP64_3 = 0x165667B19E3779F9ull;

inline uint64_t ld64(const uint8_t *p) {
  uint64_t v;
  memcpy(&v, p, 8);
  return v;
}
inline uint32_t ld32(const uint8_t *p) { return rd32(p); }
// secret bytes off .. off + 7
inline uint64_t xsec(uint32_t off) {
  const uint32_t w = off / 8, sh = (off % 8) * 8;
  return sh ? (kXSec[w] >> sh) | (kXSec[w + 1] << (64 - sh)) : kXSec[w];
}
inline uint64_t xfold(uint64_t a, uint64_t b) {
  const unsigned __int128 m = (unsigned __int128)a * b;
  return (uint64_t)m ^ (uint64_t)(m >> 64);
}
inline uint64_t xfinish3(uint64_t h) {
  h ^= h >> 37;
  h *= 0x165667919E3779F9ull;
  return h ^ (h >> 32);
}
inline uint64_t xfinish64(uint64_t h) {
  h ^= h >> 33;
  h *= kXP64_2;
  h ^= h >> 29;
  h *= kXP64_3;
  return h ^ (h >> 32);
}
inline uint64_t xmix16(const uint8_t *p, uint32_t s) { return xfold(ld64(p) ^ xsec(s), ld64(p + 8) ^ xsec(s + 8)); }

uint64_t xxh3_bytes(const uint8_t *p, uint64_t n) {
  if (n == 0) return xfinish64(xsec(56) ^ xsec(64));
  if (n <= 3) {
    const uint64_t c = ((uint64_t)p[0] << 16) | ((uint64_t)p[n / 2] << 24) | p[n - 1] | (n << 8);
    return xfinish64(c ^ (uint64_t)((uint32_t)xsec(0) ^ (uint32_t)xsec(4)));
  }
  if (n <= 8) {
    uint64_t h = ((uint64_t)ld32(p + n - 4) | ((uint64_t)ld32(p) << 32)) ^ xsec(8) ^ xsec(16);
    h ^= ((h << 49) | (h >> 15)) ^ ((h << 24) | (h >> 40));
    h *= 0x9FB21C651E98DF25ull;
    h ^= (h >> 35) + n;
    h *= 0x9FB21C651E98DF25ull;
    return h ^ (h >> 28);
  }
  if (n <= 16) {
    const uint64_t lo = ld64(p) ^ xsec(24) ^ xsec(32), hi = ld64(p + n - 8) ^ xsec(40) ^ xsec(48);
    return xfinish3(n + __builtin_bswap64(lo) + hi + xfold(lo, hi));
  }
  uint64_t acc = n * kXP64_1;
  if (n <= 128) {
    for (uint64_t j = 0; 32 * j < n; j++) acc += xmix16(p + 16 * j, 32 * j) + xmix16(p + n - 16 * (j + 1), 32 * j + 16);
    return xfinish3(acc);
  }
  if (n <= 240) {
    for (uint64_t j = 0; j < 8; j++) acc += xmix16(p + 16 * j, 16 * j);
    acc = xfinish3(acc);
    for (uint64_t j = 8; j < n / 16; j++) acc += xmix16(p + 16 * j, 16 * (j - 8) + 3);
    return xfinish3(acc + xmix16(p + n - 16, 119));
  }
  uint64_t a[8] = {0xC2B2AE3Dull, kXP64_1, kXP64_2, kXP64_3, 0x85EBCA77C2B2AE63ull, 0x85EBCA77ull,
                   0x27D4EB2F165667C5ull, 0x9E3779B1ull};
  // stripe at q with secret words starting at byte s8
  auto stripe = [&](const uint8_t *q, uint32_t s8) {
    for (int i = 0; i < 8; i++) {
      const uint64_t v = ld64(q + 8 * i), k = v ^ xsec(s8 + 8 * i);
      a[i ^ 1] += v;
      a[i] += (k & 0xFFFFFFFFull) * (k >> 32);
    }
  };
  const uint64_t nblocks = (n - 1) / 1024;
  for (uint64_t b = 0; b < nblocks; b++) {
    for (uint32_t s = 0; s < 16; s++) stripe(p + 1024 * b + 64 * s, 8 * s);
    for (int i = 0; i < 8; i++) a[i] = (a[i] ^ (a[i] >> 47) ^ kXSec[16 + i]) * 0x9E3779B1ull;
  }
  const uint64_t tail = 1024 * nblocks;
  for (uint32_t s = 0; s < ((n - 1) - tail) / 64; s++) stripe(p + tail + 64 * s, 8 * s);
  stripe(p + n - 64, 121);
  uint64_t h = n * kXP64_1;
  for (int i = 0; i < 4; i++) h += xfold(a[2 * i] ^ xsec(11 + 16 * i), a[2 * i + 1] ^ xsec(19 + 16 * i));
  return xfinish3(h);
}

}  // namespace

extern "C" {

uint64_t lt_lz4_bound(uint64_t n) { return n + n / 255 + 16; }

lt_status lt_pack_int4(const uint8_t *codes, uint64_t n_codes, uint8_t *packed) {
  if ((!codes || !packed) && n_codes) return LT_ERR_INVALID_ARG;
  if (n_codes % 2) return LT_ERR_INVALID_ARG;
  for (uint64_t k = 0; k < n_codes / 2; k++)
    packed[k] = (uint8_t)((codes[2 * k] & 15) | ((codes[2 * k + 1] & 15) << 4));
  return LT_OK;
}

}  // extern "C"

namespace {

template <bool Greedy>
lt_status compress_chunks(const uint8_t *src, const uint64_t *dst_off, uint32_t n_chunks, uint8_t *comp,
                          uint64_t comp_cap, uint64_t *comp_off, int threads, uint32_t max_dist) {
  if (!dst_off || !comp_off) return LT_ERR_INVALID_ARG;
  const uint64_t window = (max_dist == 0 || max_dist > kMaxDist) ? kMaxDist : max_dist;
  if (n_chunks == 0) {
    comp_off[0] = 0;
    return LT_OK;
  }
  if (!src || !comp || dst_off[0] != 0) return LT_ERR_INVALID_ARG;
  uint64_t need = 0;
  for (uint32_t i = 0; i < n_chunks; i++) {
    if (dst_off[i + 1] < dst_off[i]) return LT_ERR_INVALID_ARG;
    need += lt_lz4_bound(dst_off[i + 1] - dst_off[i]);
  }
  if (threads <= 0) threads = (int)std::max(1u, std::thread::hardware_concurrency());
  threads = std::min<int>(threads, (int)n_chunks);
  threads = std::min(threads, 256);
  // compress each chunk into its own slot of a scratch buffer, then pack
  std::vector<uint64_t> slot(n_chunks + 1, 0), size(n_chunks, 0);
  for (uint32_t i = 0; i < n_chunks; i++) slot[i + 1] = slot[i] + lt_lz4_bound(dst_off[i + 1] - dst_off[i]);
  std::vector<uint8_t> scratch(need);
  auto work = [&](int t) {
    std::vector<int32_t> table(1u << kHashBits);
    for (uint32_t i = (uint32_t)t; i < n_chunks; i += (uint32_t)threads)
      size[i] = compress_block<Greedy>(src + dst_off[i], dst_off[i + 1] - dst_off[i], scratch.data() + slot[i],
                                       table, window);
  };
  std::vector<std::thread> pool;
  for (int t = 1; t < threads; t++) pool.emplace_back(work, t);
  work(0);
  for (auto &th : pool) th.join();
  uint64_t pos = 0;
  comp_off[0] = 0;
  for (uint32_t i = 0; i < n_chunks; i++) {
    if (pos + size[i] > comp_cap) return LT_ERR_INVALID_ARG;
    memcpy(comp + pos, scratch.data() + slot[i], size[i]);
    pos += size[i];
    comp_off[i + 1] = pos;
  }
  return LT_OK;
}

}  // namespace

extern "C" {

lt_status lt_compress_chunks(const uint8_t *src, const uint64_t *dst_off, uint32_t n_chunks,
                             uint8_t *comp, uint64_t comp_cap, uint64_t *comp_off, int threads,
                             uint32_t max_dist) {
  return compress_chunks<false>(src, dst_off, n_chunks, comp, comp_cap, comp_off, threads, max_dist);
}

lt_status lt_compress_chunks_greedy(const uint8_t *src, const uint64_t *dst_off, uint32_t n_chunks,
                                    uint8_t *comp, uint64_t comp_cap, uint64_t *comp_off, int threads,
                                    uint32_t max_dist) {
  return compress_chunks<true>(src, dst_off, n_chunks, comp, comp_cap, comp_off, threads, max_dist);
}

lt_status lt_order_chunks(const uint64_t *dst_off, uint32_t n_chunks, uint32_t *order) {
  if (n_chunks == 0) return LT_OK;
  if (!dst_off || !order) return LT_ERR_INVALID_ARG;
  for (uint32_t i = 0; i < n_chunks; i++)
    if (dst_off[i + 1] < dst_off[i]) return LT_ERR_INVALID_ARG;
  // largest decoded size first; equal sizes keep table order (neighbouring
  // chunks then run side by side, as without an order)
  for (uint32_t i = 0; i < n_chunks; i++) order[i] = i;
  std::stable_sort(order, order + n_chunks, [&](uint32_t a, uint32_t b) {
    return dst_off[a + 1] - dst_off[a] > dst_off[b + 1] - dst_off[b];
  });
  return LT_OK;
}

lt_status lt_order_chunks_by_sequences(const uint64_t *dst_off, const uint64_t *seq_off, uint32_t n_chunks,
                                       uint32_t *order) {
  if (n_chunks == 0) return LT_OK;
  if (!dst_off || !seq_off || !order) return LT_ERR_INVALID_ARG;
  for (uint32_t i = 0; i < n_chunks; i++)
    if (dst_off[i + 1] < dst_off[i] || seq_off[i + 1] < seq_off[i]) return LT_ERR_INVALID_ARG;
  // largest decoded size first, then the most sequences: on sequence-dense
  // tables a chunk's life grows with its sequences, and a launch ends with
  // its slowest chunk
  for (uint32_t i = 0; i < n_chunks; i++) order[i] = i;
  std::stable_sort(order, order + n_chunks, [&](uint32_t a, uint32_t b) {
    const uint64_t sa = dst_off[a + 1] - dst_off[a], sb = dst_off[b + 1] - dst_off[b];
    if (sa != sb) return sa > sb;
    return seq_off[a + 1] - seq_off[a] > seq_off[b + 1] - seq_off[b];
  });
  return LT_OK;
}

lt_status lt_index_chunks(const uint8_t *comp, const uint64_t *comp_off, uint32_t n_chunks,
                          uint64_t *seq_off, uint32_t *seq_pos, uint64_t seq_cap, int threads) {
  if (!comp_off || !seq_off) return LT_ERR_INVALID_ARG;
  seq_off[0] = 0;
  if (n_chunks == 0) return LT_OK;
  if (!comp) return LT_ERR_INVALID_ARG;
  for (uint32_t i = 0; i < n_chunks; i++)
    if (comp_off[i + 1] < comp_off[i] || comp_off[i + 1] - comp_off[i] > 0xFFFFFFFFull)
      return LT_ERR_INVALID_ARG;
  std::vector<uint64_t> count(n_chunks, 0);
  parallel_chunks(n_chunks, threads, [&](uint32_t i) {
    uint64_t c = 0;
    walk_block(comp + comp_off[i], comp_off[i + 1] - comp_off[i], [&](uint64_t) { c++; });
    count[i] = c;
  });
  for (uint32_t i = 0; i < n_chunks; i++) seq_off[i + 1] = seq_off[i] + count[i];
  if (!seq_pos) return LT_OK;
  if (seq_cap < seq_off[n_chunks]) return LT_ERR_INVALID_ARG;
  parallel_chunks(n_chunks, threads, [&](uint32_t i) {
    uint32_t *out = seq_pos + seq_off[i];
    walk_block(comp + comp_off[i], comp_off[i + 1] - comp_off[i], [&](uint64_t p) { *out++ = (uint32_t)p; });
  });
  return LT_OK;
}

lt_status lt_encode_zero_runs(const uint16_t *x, uint64_t n, uint32_t *bitmap, uint64_t *val_off, uint16_t *vals,
                              uint64_t vals_cap, int threads) {
  if (!val_off || (n && (!x || !bitmap))) return LT_ERR_INVALID_ARG;
  const uint64_t nb = (n + LT_ZR_BLOCK - 1) / LT_ZR_BLOCK;
  if (nb > 0xFFFFFFFFull) return LT_ERR_INVALID_ARG;
  val_off[0] = 0;
  if (nb == 0) return LT_OK;
  std::vector<uint32_t> count(nb);
  parallel_chunks((uint32_t)nb, threads, [&](uint32_t b) {
    const uint64_t e0 = (uint64_t)b * LT_ZR_BLOCK, e1 = std::min<uint64_t>(e0 + LT_ZR_BLOCK, n);
    uint32_t *w = bitmap + (uint64_t)b * (LT_ZR_BLOCK / 32);
    for (int k = 0; k < LT_ZR_BLOCK / 32; k++) w[k] = 0;
    uint32_t c = 0;
    for (uint64_t e = e0; e < e1; e++)
      if (x[e]) {
        w[(e - e0) >> 5] |= 1u << ((e - e0) & 31);
        c++;
      }
    count[b] = c;
  });
  for (uint64_t b = 0; b < nb; b++) val_off[b + 1] = val_off[b] + count[b];
  if (!vals) return LT_OK;
  if (vals_cap < val_off[nb]) return LT_ERR_INVALID_ARG;
  parallel_chunks((uint32_t)nb, threads, [&](uint32_t b) {
    const uint64_t e0 = (uint64_t)b * LT_ZR_BLOCK, e1 = std::min<uint64_t>(e0 + LT_ZR_BLOCK, n);
    uint16_t *o = vals + val_off[b];
    for (uint64_t e = e0; e < e1; e++)
      if (x[e]) *o++ = x[e];
  });
  return LT_OK;
}

lt_status lt_checksum_chunks(const uint8_t *comp, const uint64_t *comp_off, uint32_t n_chunks, uint64_t *xxh,
                             int threads) {
  if (!comp_off || !xxh) return LT_ERR_INVALID_ARG;
  if (n_chunks == 0) return LT_OK;
  if (!comp) return LT_ERR_INVALID_ARG;
  for (uint32_t i = 0; i < n_chunks; i++)
    if (comp_off[i + 1] < comp_off[i]) return LT_ERR_INVALID_ARG;
  parallel_chunks(n_chunks, threads, [&](uint32_t i) {
    xxh[i] = xxh3_bytes(comp + comp_off[i], comp_off[i + 1] - comp_off[i]);
  });
  return LT_OK;
}

}  // extern "C"
