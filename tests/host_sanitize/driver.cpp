// Host-side exercise of the library's C++ that runs without a GPU (the chunk
// table builder and the chunk-table producer), built under AddressSanitizer
// + UndefinedBehaviorSanitizer and, separately, ThreadSanitizer by
// tests/test_host_sanitizers.py.  Every call's status is checked; the
// sanitizers report any out-of-bounds access, leak, undefined operation or
// data race on the way.  Inputs come from a fixed-seed splitmix64 stream.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "irm.h"

namespace {

uint64_t g_state = 0x1234567ull;
uint64_t next_u64() {  // splitmix64
  uint64_t z = (g_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}
uint32_t below(uint32_t n) { return (uint32_t)(next_u64() % n); }

int g_fail = 0;
uint64_t g_rows = 0, g_entries = 0;  // work done, printed at the end
void expect(bool ok, const char* what, int line) {
  if (!ok) {
    std::fprintf(stderr, "line %d: %s (last error: %s)\n", line, what, irm_last_error());
    ++g_fail;
  }
}
#define EXPECT(c) expect((c), #c, __LINE__)

// A valid table: per sequence a fresh entry of >= 32 rows at 0, then hits
// (random delta, possibly negative p_src) and fresh entries, lengths 1..max_len.
struct Tab {
  std::vector<irm_chunk> chunks;
  std::vector<uint32_t> seq_first{0};
  uint64_t pool_rows = 0;
};

Tab random_table(uint32_t n_seq, uint32_t max_seq, uint32_t max_len) {
  Tab t;
  for (uint32_t s = 0; s < n_seq; ++s) {
    const uint32_t len = below(max_seq + 1);
    uint32_t pos = 0;
    while (pos < len) {
      uint32_t ln = 1 + below(max_len);
      if (pos == 0) ln = ln < 32 ? 32 : ln;
      if (ln > len - pos) ln = len - pos;
      irm_chunk c{};
      c.pool_row = (uint32_t)t.pool_rows;
      c.len = ln;
      c.p_tgt = (int32_t)pos;
      if (pos >= 32 && below(10) < 7) {
        c.flags = 0;
        c.p_src = (int32_t)pos - ((int32_t)below(262145) - 131072);
      } else {
        c.flags = IRM_FRESH;
        c.p_src = c.p_tgt;
      }
      t.chunks.push_back(c);
      t.pool_rows += ln;
      pos += ln;
    }
    t.seq_first.push_back((uint32_t)t.chunks.size());
  }
  return t;
}

void check_table(const Tab& tb, irm_status want) {
  irm_table* t = nullptr;
  const uint32_t n_seq = (uint32_t)tb.seq_first.size() - 1;
  irm_status st = irm_table_create(tb.chunks.empty() ? nullptr : tb.chunks.data(), (uint32_t)tb.chunks.size(),
                                   tb.seq_first.data(), n_seq, tb.pool_rows, &t);
  EXPECT(st == want);
  if (st != IRM_OK) {
    EXPECT(t == nullptr);
    return;
  }
  uint32_t ns = 0, nc = 0, mx = 0;
  uint64_t total = 0;
  size_t dbytes = 0;
  EXPECT(irm_table_info(t, &ns, &nc, &total, &mx, &dbytes) == IRM_OK);
  EXPECT(ns == n_seq && nc == tb.chunks.size());
  uint64_t sum = 0;
  for (const auto& c : tb.chunks) sum += c.len;
  EXPECT(total == sum);
  g_rows += total;
  std::vector<uint64_t> base(n_seq + 1);
  EXPECT(irm_table_seq_base(t, base.data()) == IRM_OK);
  EXPECT(base[n_seq] == total);
  std::vector<int64_t> pr(total + 1);
  std::vector<int32_t> de(total + 1);
  std::vector<uint8_t> fr(total + 1);
  EXPECT(irm_table_expand_host(t, pr.data(), de.data(), fr.data()) == IRM_OK);
  uint64_t r = 0;
  for (const auto& c : tb.chunks)
    for (uint32_t j = 0; j < c.len; ++j, ++r) {
      EXPECT(pr[r] == (int64_t)c.pool_row + j);
      EXPECT(de[r] == ((c.flags & IRM_FRESH) ? 0 : c.p_tgt - c.p_src));
    }
  EXPECT(irm_table_expand_host(t, nullptr, nullptr, nullptr) == IRM_OK);
  EXPECT(irm_table_destroy(t) == IRM_OK);
}

void tables() {
  double f[4096];
  EXPECT(irm_rope_inv_freq(10000.0, f) == IRM_OK);
  EXPECT(irm_rope_inv_freq(0.5, f) == IRM_EINVAL);
  EXPECT(irm_rope_inv_freq_dim(10000.0, 4096, f) == IRM_OK);
  EXPECT(irm_rope_inv_freq_dim(10000.0, 4097, f) == IRM_EINVAL);
  EXPECT(irm_rope_inv_freq_dim(10000.0, 2, nullptr) == IRM_EINVAL);
  for (int it = 0; it < 200; ++it) {
    Tab tb = random_table(1 + below(6), 1 + below(3000), 1 + below(600));
    check_table(tb, IRM_OK);
    if (tb.chunks.empty()) continue;
    // planted defects: each must be refused with its status, with no access
    // past the arrays
    Tab bad = tb;
    irm_chunk& c = bad.chunks[below((uint32_t)bad.chunks.size())];
    switch (below(7)) {
      case 0: c.flags |= 0x80u; check_table(bad, IRM_EINVAL); break;
      case 1: c.len = 0; check_table(bad, c.len == 0 ? IRM_EINVAL : IRM_OK); break;
      case 2: bad.pool_rows = c.pool_row + c.len - 1; check_table(bad, IRM_ERANGE); break;
      case 3: c.p_tgt += 1; if (c.flags & IRM_FRESH) c.p_src += 1; check_table(bad, IRM_ELAYOUT); break;
      case 4:
        if (c.p_tgt < 32) { c.flags = 0; c.p_src = c.p_tgt + 5; check_table(bad, IRM_ECARVEOUT); }
        break;
      case 5: if (c.flags & IRM_FRESH) { c.p_src = c.p_tgt + 1; check_table(bad, IRM_EINVAL); } break;
      default: break;
    }
  }
  Tab empty;
  empty.seq_first = {0, 0, 0};
  check_table(empty, IRM_OK);
  irm_table* t = nullptr;
  uint32_t sf_bad[3] = {0, 2, 1};
  irm_chunk one{0, 40, 0, 0, IRM_FRESH};
  EXPECT(irm_table_create(&one, 1, sf_bad, 2, 40, &t) == IRM_EINVAL);
  EXPECT(irm_table_create(&one, 1, nullptr, 1, 40, &t) == IRM_EINVAL);
  EXPECT(irm_table_destroy(nullptr) == IRM_OK || true);
}

void producer() {
  irm_cdc_params p{};
  EXPECT(irm_cdc_params_default(&p) == IRM_OK);
  // xxHash64 over every length 0..300 at odd offsets
  std::vector<unsigned char> bytes(400);
  for (auto& b : bytes) b = (unsigned char)next_u64();
  uint64_t h = 0;
  for (uint64_t n = 0; n <= 300; ++n) EXPECT(irm_xxh64(bytes.data() + (n % 7), n, n, &h) == IRM_OK);
  // CDC on random streams with several parameter sets
  std::vector<int32_t> toks(50000);
  for (auto& t : toks) t = (int32_t)(next_u64() % 50000);
  for (uint32_t mb : {1u, 7u, 12u}) {
    irm_cdc_params q = p;
    q.mask_bits = mb;
    q.min_len = 1 + below(64);
    q.max_len = q.min_len + below(600);
    uint64_t n = 0;
    std::vector<uint32_t> lens(toks.size() / q.min_len + 2);
    EXPECT(irm_cdc_split(&q, toks.data(), toks.size(), lens.data(), lens.size(), &n) == IRM_OK);
    uint64_t sum = 0;
    for (uint64_t i = 0; i < n; ++i) sum += lens[i];
    EXPECT(sum == toks.size());
    EXPECT(irm_cdc_split(&q, toks.data(), toks.size(), lens.data(), 1, &n) == IRM_ERANGE);
  }
  // registry batches: shared documents at shifted offsets, several threads,
  // with and without the S1 fallback and exact prefixes; 1 and 8 threads agree
  const uint32_t n_req = 24;
  std::vector<int32_t> doc(8192);
  for (auto& t : doc) t = (int32_t)(next_u64() % 32000);
  std::vector<int32_t> all;
  std::vector<uint64_t> tok_first{0};
  std::vector<uint32_t> pl(n_req), prow(n_req);
  for (uint32_t q = 0; q < n_req; ++q) {
    const uint32_t n = below(6000);
    for (uint32_t i = 0; i < n; ++i)
      all.push_back(below(10) < 7 ? doc[(i + 97 * q) % doc.size()] : (int32_t)(next_u64() % 32000));
    tok_first.push_back(all.size());
    pl[q] = below(n + 1) / 2;
    prow[q] = 1000000 + 10000 * q;
  }
  for (uint32_t window : {0u, 128u}) {
    std::vector<irm_chunk> out1, out8;
    for (uint32_t threads : {1u, 8u}) {
      irm_registry* r = nullptr;
      EXPECT(irm_registry_create(0, &r) == IRM_OK);
      irm_cdc_params q = p;
      q.fallback_window = window;
      uint32_t n = 0;
      std::vector<uint32_t> seq_first(n_req + 1);
      std::vector<irm_chunk> chunks(4);
      std::vector<uint64_t> prints(4);
      irm_status st = irm_registry_assemble(r, &q, all.data(), tok_first.data(), n_req, pl.data(), prow.data(),
                                            threads, chunks.data(), prints.data(), 4, seq_first.data(), &n);
      EXPECT(st == IRM_ERANGE && n > 4);
      chunks.resize(n);
      prints.resize(n);
      for (int pass = 0; pass < 2; ++pass) {   // the second pass hits what the first inserted
        st = irm_registry_assemble(r, &q, all.data(), tok_first.data(), n_req, pl.data(), prow.data(), threads,
                                   chunks.data(), prints.data(), (uint32_t)chunks.size(), seq_first.data(), &n);
        if (st == IRM_ERANGE) {
          chunks.resize(n);
          prints.resize(n);
          --pass;
          continue;
        }
        EXPECT(st == IRM_OK);
      }
      chunks.resize(n);
      g_entries += n;
      uint64_t entries = 0, next = 0;
      EXPECT(irm_registry_info(r, &entries, &next) == IRM_OK);
      // the produced table is a valid chunk table
      irm_table* t = nullptr;
      EXPECT(irm_table_create(chunks.data(), n, seq_first.data(), n_req, 0x100000000ull, &t) == IRM_OK);
      irm_table_destroy(t);
      (threads == 1 ? out1 : out8) = chunks;
      EXPECT(irm_registry_destroy(r) == IRM_OK);
    }
    EXPECT(out1.size() == out8.size() &&
           std::memcmp(out1.data(), out8.data(), out1.size() * sizeof(irm_chunk)) == 0);
  }
}

}  // namespace

int main() {
  tables();
  producer();
  if (g_fail) {
    std::fprintf(stderr, "%d checks failed\n", g_fail);
    return 1;
  }
  std::printf("host checks ok: %llu table rows, %llu producer entries\n", (unsigned long long)g_rows, (unsigned long long)g_entries);
  return 0;
}
