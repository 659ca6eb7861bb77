// Host code under AddressSanitizer and UndefinedBehaviorSanitizer: the
// oracle's C (oracle/ltref.c) and the library's host packer (lt_pack.cpp),
// built into one program with the sanitizers by tests/test_sanitizers.py and
// run on generated inputs, damaged blocks included.  It prints "ok" at the
// end; any out-of-bounds access, overflow or other undefined behaviour ends
// it earlier with the sanitizer's report.  Test infrastructure: it checks
// that the two sides agree, it is not part of either.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "lt.h"

extern "C" {
int ltref_lz4_decode_block(const uint8_t *in, uint64_t m, uint8_t *out, uint64_t cap, uint64_t *produced);
uint64_t ltref_lz4_bound(uint64_t n);
uint64_t ltref_lz4_compress(const uint8_t *x, uint64_t n, uint8_t *out);
uint32_t ltref_decode_table(const uint8_t *comp, uint64_t comp_bytes, const uint64_t *comp_off,
                            const uint64_t *dst_off, uint32_t n, uint64_t total, uint8_t *dst, int32_t *status,
                            int threads);
uint64_t ltref_seqgen(uint64_t seed, uint64_t target, uint8_t *stream, uint64_t stream_cap, uint8_t *expected,
                      uint64_t out_cap, uint64_t *out_len);
uint64_t ltref_xxh3_64(const uint8_t *in, uint64_t n);
void ltref_pack_int4(const uint8_t *codes, uint64_t n_codes, uint8_t *packed);
uint64_t ltref_zr_encode(const uint16_t *x, uint64_t n, uint32_t *bitmap, uint64_t *val_off, uint16_t *vals);
void ltref_zr_decode(const uint32_t *bitmap, const uint64_t *val_off, const uint16_t *vals, uint64_t n,
                     uint64_t n_vals, uint16_t *out, int32_t *status);
}

static int failures = 0;
#define CHECK(c, ...)                      \
  do {                                     \
    if (!(c)) {                            \
      std::fprintf(stderr, __VA_ARGS__);   \
      std::fprintf(stderr, "\n");          \
      failures++;                          \
    }                                      \
  } while (0)

static std::vector<uint8_t> make_input(std::mt19937_64 &rng, size_t n, int kind) {
  std::vector<uint8_t> v(n);
  for (size_t i = 0; i < n; i++) {
    switch (kind) {
      case 0: v[i] = (uint8_t)rng(); break;                                   // incompressible
      case 1: v[i] = 0; break;                                                // one long run
      case 2: v[i] = (rng() % 8 == 0) ? (uint8_t)rng() : 0; break;            // sparse, short runs
      case 3: v[i] = (uint8_t)((rng() % 3) * 0x11); break;                    // few symbols
      default: v[i] = (uint8_t)((i / 37) % 5 == 0 ? rng() : (i % 251)); break; // periodic pieces
    }
  }
  return v;
}

static std::vector<uint64_t> chunking(size_t n, size_t chunk) {
  std::vector<uint64_t> d;
  for (size_t o = 0; o < n; o += chunk) d.push_back(o);
  d.push_back(n);
  return d;
}

// the packer's table for src (both parses, both windows) decodes through the
// oracle to src; its index, launch orders and checksums are consistent
static void packer_tables(const std::vector<uint8_t> &src, size_t chunk) {
  const std::vector<uint64_t> dst_off = chunking(src.size(), chunk);
  const uint32_t n = (uint32_t)(dst_off.size() - 1);
  for (int greedy = 0; greedy < 2; greedy++) {
    for (uint32_t md : {4096u, 0u}) {
      uint64_t cap = 16;
      for (uint32_t i = 0; i < n; i++) cap += lt_lz4_bound(dst_off[i + 1] - dst_off[i]);
      std::vector<uint8_t> comp(cap);
      std::vector<uint64_t> comp_off(n + 1);
      lt_status st = greedy ? lt_compress_chunks_greedy(src.data(), dst_off.data(), n, comp.data(), cap,
                                                        comp_off.data(), 2, md)
                            : lt_compress_chunks(src.data(), dst_off.data(), n, comp.data(), cap, comp_off.data(),
                                                 2, md);
      CHECK(st == LT_OK, "compress status %d", (int)st);
      if (st != LT_OK) continue;
      std::vector<uint8_t> out(src.size() + 1);
      std::vector<int32_t> status(n + 1);
      uint32_t bad = ltref_decode_table(comp.data(), comp_off[n], comp_off.data(), dst_off.data(), n, src.size(),
                                        out.data(), status.data(), 2);
      CHECK(bad == 0 && std::memcmp(out.data(), src.data(), src.size()) == 0, "packer table does not round-trip");
      std::vector<uint64_t> seq_off(n + 1);
      st = lt_index_chunks(comp.data(), comp_off.data(), n, seq_off.data(), nullptr, 0, 2);
      CHECK(st == LT_OK, "index size status %d", (int)st);
      std::vector<uint32_t> seq_pos(seq_off[n] + 1);
      st = lt_index_chunks(comp.data(), comp_off.data(), n, seq_off.data(), seq_pos.data(), seq_off[n], 2);
      CHECK(st == LT_OK, "index status %d", (int)st);
      std::vector<uint32_t> order(n + 1);
      CHECK(lt_order_chunks(dst_off.data(), n, order.data()) == LT_OK, "order");
      CHECK(lt_order_chunks_by_sequences(dst_off.data(), seq_off.data(), n, order.data()) == LT_OK, "order by seq");
      std::vector<uint64_t> xxh(n + 1);
      CHECK(lt_checksum_chunks(comp.data(), comp_off.data(), n, xxh.data(), 2) == LT_OK, "checksums");
      for (uint32_t i = 0; i < n; i++)
        CHECK(xxh[i] == ltref_xxh3_64(comp.data() + comp_off[i], comp_off[i + 1] - comp_off[i]),
              "checksum of chunk %u", i);
    }
  }
}

// damaged blocks: every decoder and the indexer must stay inside their
// buffers whatever they are given (their statuses are checked elsewhere)
static void damaged_blocks(std::mt19937_64 &rng, const std::vector<uint8_t> &src) {
  std::vector<uint8_t> comp(ltref_lz4_bound(src.size()));
  const uint64_t m = ltref_lz4_compress(src.data(), src.size(), comp.data());
  comp.resize(m);
  for (int t = 0; t < 300; t++) {
    std::vector<uint8_t> b(comp);
    const int how = (int)(rng() % 4);
    if (how == 0 && !b.empty()) b.resize(rng() % b.size());
    if (how == 1 && !b.empty()) b[rng() % b.size()] ^= (uint8_t)(1u << (rng() % 8));
    if (how == 2) b.insert(b.begin() + (b.empty() ? 0 : rng() % b.size()), (uint8_t)rng());
    if (how == 3 && !b.empty()) b[rng() % b.size()] = (uint8_t)rng();
    uint64_t produced = 0;
    // exact-size buffers, so an overrun is the sanitizer's to find
    std::vector<uint8_t> in(b);
    std::vector<uint8_t> dst(src.size());
    (void)ltref_lz4_decode_block(in.data(), in.size(), dst.data(), dst.size(), &produced);
    CHECK(produced <= dst.size(), "decoder claims more bytes than its buffer");
    uint64_t comp_off[2] = {0, in.size()};
    uint64_t seq_off[2];
    (void)lt_index_chunks(in.data(), comp_off, 1, seq_off, nullptr, 0, 1);
  }
}

int main() {
  std::mt19937_64 rng(20261204);
  for (size_t n : {1u, 15u, 16u, 17u, 100u, 4095u, 4096u, 65536u, 200003u}) {
    for (int kind = 0; kind < 5; kind++) {
      const std::vector<uint8_t> src = make_input(rng, n, kind);
      std::vector<uint8_t> comp(ltref_lz4_bound(n));
      const uint64_t m = ltref_lz4_compress(src.data(), n, comp.data());
      std::vector<uint8_t> out(n);
      uint64_t produced = 0;
      const int st = ltref_lz4_decode_block(comp.data(), m, out.data(), n, &produced);
      CHECK(st == 0 && produced == n && std::memcmp(out.data(), src.data(), n) == 0,
            "oracle round trip n=%zu kind=%d", n, kind);
      packer_tables(src, n > 20000 ? 16384 : 4096);
      if (n <= 4096) damaged_blocks(rng, src);
    }
  }
  for (uint64_t seed = 1; seed <= 200; seed++) {   // generated streams, every length class
    const uint64_t target = 64 + seed * 97 % 20000;
    std::vector<uint8_t> stream(2 * target + 64), expected(target), out(target);
    uint64_t len = 0;
    const uint64_t m = ltref_seqgen(seed, target, stream.data(), stream.size(), expected.data(), target, &len);
    uint64_t produced = 0;
    const int st = ltref_lz4_decode_block(stream.data(), m, out.data(), len, &produced);
    CHECK(st == 0 && produced == len && std::memcmp(out.data(), expected.data(), len) == 0, "seqgen %lu",
          (unsigned long)seed);
  }
  {  // INT4 packing and zero runs: the packer's and the oracle's agree
    const size_t n = 70002;   // an even count of codes (two per byte)
    std::vector<uint8_t> codes(n);
    for (auto &c : codes) c = (uint8_t)(rng() % 16);
    std::vector<uint8_t> a((n + 1) / 2), b((n + 1) / 2);
    CHECK(lt_pack_int4(codes.data(), n, a.data()) == LT_OK, "pack");
    ltref_pack_int4(codes.data(), n, b.data());
    CHECK(a == b, "INT4 packing differs");
    std::vector<uint16_t> x(n);
    for (auto &v : x) v = (rng() % 10 == 0) ? (uint16_t)(rng() | 1) : 0;
    const uint64_t nb = (n + 1023) / 1024;
    std::vector<uint32_t> bm1(32 * nb), bm2(32 * nb);
    std::vector<uint64_t> vo1(nb + 1), vo2(nb + 1);
    std::vector<uint16_t> v1(n), v2(n);
    CHECK(lt_encode_zero_runs(x.data(), n, bm1.data(), vo1.data(), v1.data(), n, 2) == LT_OK, "zr encode");
    const uint64_t nv = ltref_zr_encode(x.data(), n, bm2.data(), vo2.data(), v2.data());
    CHECK(bm1 == bm2 && vo1 == vo2 && vo1[nb] == nv && std::memcmp(v1.data(), v2.data(), 2 * nv) == 0,
          "zero-run coding differs");
    std::vector<uint16_t> y(n);
    std::vector<int32_t> st(nb);
    ltref_zr_decode(bm2.data(), vo2.data(), v2.data(), n, nv, y.data(), st.data());
    CHECK(y == x, "zero-run round trip");
  }
  if (failures) {
    std::fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  std::printf("ok\n");
  return 0;
}
