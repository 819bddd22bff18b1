// Host chunk-table producer: content-defined chunking of a request's tokens,
// chunk fingerprints and the registry lookup that turns them into chunk-table
// entries.  No HIP call is made here.
//
// Irminsul pages: the serve path splits the unmatched tail by content-defined
// chunking, fingerprints every chunk with xxHash64 and looks it up in a
// content registry; a hit at target position p is reused with delta =
// p - p_src, a miss is prefilled and inserted as (c_KV, k_r_base, p), and a
// segment starting below position 32 is always prefilled (gentlecold.top
// article, section 5 pseudocode).  The chunker is a rolling Gear hash over a
// 64-token window that emits a boundary when its low 7 bits meet the mask,
// for chunks of about 128 tokens clamped to [32, 512] (gentlecold.top
// section 6; gist.science summary, section 2.2).
//
// Choices where the pages are silent: the Gear state is 64 bits wide and
// rolls as h = (h << 1) + gear(token), so a token leaves it after 64 steps;
// it starts at 0 at the tail and rolls on across chunk boundaries; gear(t) is
// the splitmix64 output for the state seed + t * 0x9E3779B97F4A7C15; a
// boundary follows token i when the chunk holds at least min_len tokens and
// the low mask bits are zero, or when it holds max_len tokens; the
// fingerprint is xxHash64 (seed 0) of the token ids as 4-byte little-endian
// integers; a registry entry of another length counts as a miss.

#include <algorithm>
#include <atomic>
#include <cstring>
#include <new>
#include <string>
#include <thread>
#include <unordered_map>
#include <vector>

#include "irm_internal.h"

using irm::fail;

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ull;

inline uint64_t gear(int32_t token, uint64_t seed) {
  // splitmix64 (Steele, Lea, Flood 2014): output for the state below
  uint64_t z = seed + (uint64_t)(int64_t)token * kGamma + kGamma;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// ---------------------------------------------------------------------------
// xxHash64 (algorithm as described in the xxHash specification)
// ---------------------------------------------------------------------------
constexpr uint64_t kP1 = 0x9E3779B185EBCA87ull, kP2 = 0xC2B2AE3D27D4EB4Full, kP3 = 0x165667B19E3779F9ull,
                   kP4 = 0x85EBCA77C2B2AE63ull, kP5 = 0x27D4EB2F165667C5ull;

inline uint64_t rotl(uint64_t x, int r) { return (x << r) | (x >> (64 - r)); }
inline uint64_t rd64(const unsigned char* p) {
  uint64_t v;
  std::memcpy(&v, p, 8);
  return v;  // little-endian host
}
inline uint32_t rd32(const unsigned char* p) {
  uint32_t v;
  std::memcpy(&v, p, 4);
  return v;
}
inline uint64_t xround(uint64_t acc, uint64_t lane) { return rotl(acc + lane * kP2, 31) * kP1; }
inline uint64_t xmerge(uint64_t acc, uint64_t v) { return (acc ^ xround(0, v)) * kP1 + kP4; }

uint64_t xxh64(const void* data, uint64_t n, uint64_t seed) {
  const unsigned char* p = static_cast<const unsigned char*>(data);
  const unsigned char* const end = p + n;
  uint64_t acc;
  if (n >= 32) {
    uint64_t v1 = seed + kP1 + kP2, v2 = seed + kP2, v3 = seed, v4 = seed - kP1;
    const unsigned char* const limit = end - 32;
    do {
      v1 = xround(v1, rd64(p));
      v2 = xround(v2, rd64(p + 8));
      v3 = xround(v3, rd64(p + 16));
      v4 = xround(v4, rd64(p + 24));
      p += 32;
    } while (p <= limit);
    acc = rotl(v1, 1) + rotl(v2, 7) + rotl(v3, 12) + rotl(v4, 18);
    acc = xmerge(acc, v1);
    acc = xmerge(acc, v2);
    acc = xmerge(acc, v3);
    acc = xmerge(acc, v4);
  } else {
    acc = seed + kP5;
  }
  acc += n;
  for (; p + 8 <= end; p += 8) acc = rotl(acc ^ xround(0, rd64(p)), 27) * kP1 + kP4;
  if (p + 4 <= end) {
    acc = rotl(acc ^ ((uint64_t)rd32(p) * kP1), 23) * kP2 + kP3;
    p += 4;
  }
  for (; p < end; ++p) acc = rotl(acc ^ ((uint64_t)*p * kP5), 11) * kP1;
  acc ^= acc >> 33;
  acc *= kP2;
  acc ^= acc >> 29;
  acc *= kP3;
  acc ^= acc >> 32;
  return acc;
}

irm_status check_params(const irm_cdc_params* p, const char* fn) {
  if (!p) return fail(IRM_EINVAL, std::string(fn) + ": params is NULL");
  if (p->mask_bits < 1 || p->mask_bits > 63) return fail(IRM_EINVAL, std::string(fn) + ": mask_bits must be in [1, 63]");
  if (p->min_len < 1 || p->max_len < p->min_len)
    return fail(IRM_EINVAL, std::string(fn) + ": need 1 <= min_len <= max_len");
  return IRM_OK;
}

// Chunk lengths of tokens[0, n) appended to out.
void cdc(const irm_cdc_params& p, const int32_t* tokens, uint64_t n, std::vector<uint32_t>& out) {
  const uint64_t mask = (1ull << p.mask_bits) - 1;
  uint64_t h = 0, start = 0;
  for (uint64_t i = 0; i < n; ++i) {
    h = (h << 1) + gear(tokens[i], p.seed);
    const uint64_t len = i - start + 1;
    if ((len >= p.min_len && (h & mask) == 0) || len == p.max_len) {
      out.push_back((uint32_t)len);
      start = i + 1;
    }
  }
  if (start < n) out.push_back((uint32_t)(n - start));
}

inline uint64_t fingerprint(const int32_t* tokens, uint32_t len) {
  static_assert(sizeof(int32_t) == 4, "token ids are 4-byte integers");
  return xxh64(tokens, (uint64_t)len * 4, 0);  // little-endian host: the ids' bytes as stored
}

}  // namespace

struct irm_registry {
  struct Entry {
    uint32_t pool_row, len;
    int32_t p_src;
  };
  std::unordered_map<uint64_t, Entry> map;
  uint64_t next_row = 0;
};

extern "C" irm_status irm_cdc_params_default(irm_cdc_params* p) {
  if (!p) return fail(IRM_EINVAL, "irm_cdc_params_default: params is NULL");
  p->seed = 0;
  p->mask_bits = 7;
  p->min_len = 32;
  p->max_len = 512;
  p->fallback_window = 0;
  return IRM_OK;
}

extern "C" irm_status irm_xxh64(const void* data, uint64_t bytes, uint64_t seed, uint64_t* out) {
  if (!out) return fail(IRM_EINVAL, "irm_xxh64: out is NULL");
  if (bytes && !data) return fail(IRM_EINVAL, "irm_xxh64: data is NULL");
  *out = xxh64(data, bytes, seed);
  return IRM_OK;
}

extern "C" irm_status irm_cdc_split(const irm_cdc_params* p, const int32_t* tokens, uint64_t n, uint32_t* lens,
                                    uint64_t max_chunks, uint64_t* n_chunks) {
  irm_status st = check_params(p, "irm_cdc_split");
  if (st != IRM_OK) return st;
  if (!n_chunks) return fail(IRM_EINVAL, "irm_cdc_split: n_chunks is NULL");
  if (n && !tokens) return fail(IRM_EINVAL, "irm_cdc_split: tokens is NULL");
  std::vector<uint32_t> v;
  try {
    v.reserve(n / p->min_len + 1);
    cdc(*p, tokens, n, v);
  } catch (const std::bad_alloc&) {
    return fail(IRM_EINVAL, "irm_cdc_split: out of host memory");
  }
  *n_chunks = v.size();
  if (v.size() > max_chunks) return fail(IRM_ERANGE, "irm_cdc_split: more chunks than max_chunks");
  if (!v.empty()) {
    if (!lens) return fail(IRM_EINVAL, "irm_cdc_split: lens is NULL");
    std::memcpy(lens, v.data(), v.size() * sizeof(uint32_t));
  }
  return IRM_OK;
}

extern "C" irm_status irm_registry_create(uint64_t first_free_row, irm_registry** out) {
  if (!out) return fail(IRM_EINVAL, "irm_registry_create: out is NULL");
  *out = new (std::nothrow) irm_registry;
  if (!*out) return fail(IRM_EINVAL, "irm_registry_create: out of host memory");
  (*out)->next_row = first_free_row;
  return IRM_OK;
}

extern "C" irm_status irm_registry_destroy(irm_registry* r) {
  delete r;
  return IRM_OK;
}

extern "C" irm_status irm_registry_info(const irm_registry* r, uint64_t* n_entries, uint64_t* next_free_row) {
  if (!r) return fail(IRM_EINVAL, "irm_registry_info: registry is NULL");
  if (n_entries) *n_entries = r->map.size();
  if (next_free_row) *next_free_row = r->next_row;
  return IRM_OK;
}

extern "C" irm_status irm_registry_assemble(irm_registry* r, const irm_cdc_params* p, const int32_t* tokens,
                                            const uint64_t* tok_first, uint32_t n_req, const uint32_t* prefix_len,
                                            const uint32_t* prefix_row, uint32_t n_threads, irm_chunk* chunks,
                                            uint64_t* fingerprints, uint32_t max_chunks, uint32_t* seq_first,
                                            uint32_t* n_chunks) {
  static const char* fn = "irm_registry_assemble";
  if (!r) return fail(IRM_EINVAL, std::string(fn) + ": registry is NULL");
  irm_status st = check_params(p, fn);
  if (st != IRM_OK) return st;
  if (!tok_first || !seq_first || !n_chunks) return fail(IRM_EINVAL, std::string(fn) + ": NULL argument");
  if (tok_first[0] != 0) return fail(IRM_EINVAL, std::string(fn) + ": tok_first[0] must be 0");
  for (uint32_t q = 0; q < n_req; ++q) {
    if (tok_first[q + 1] < tok_first[q]) return fail(IRM_EINVAL, std::string(fn) + ": tok_first must be nondecreasing");
    const uint64_t n = tok_first[q + 1] - tok_first[q];
    const uint32_t pl = prefix_len ? prefix_len[q] : 0;
    if (pl > n) return fail(IRM_EINVAL, std::string(fn) + ": prefix longer than its request");
    if (n > 0x7fffffffull) return fail(IRM_ERANGE, std::string(fn) + ": request longer than 2^31 - 1 tokens");
    if (pl && prefix_row && (uint64_t)prefix_row[q] + pl > 0x100000000ull)
      return fail(IRM_ERANGE, std::string(fn) + ": prefix rows beyond 2^32");
  }
  if (tok_first[n_req] && !tokens) return fail(IRM_EINVAL, std::string(fn) + ": tokens is NULL");

  // 1. chunk boundaries and fingerprints of every tail, in parallel
  std::vector<std::vector<uint32_t>> lens(n_req);
  std::vector<std::vector<uint64_t>> prints(n_req);
  try {
    auto work = [&](uint32_t q) {
      const uint32_t pl = prefix_len ? prefix_len[q] : 0;
      const int32_t* t = tokens + tok_first[q] + pl;
      cdc(*p, t, tok_first[q + 1] - tok_first[q] - pl, lens[q]);
      prints[q].resize(lens[q].size());
      uint64_t off = 0;
      for (size_t c = 0; c < lens[q].size(); ++c) {
        prints[q][c] = fingerprint(t + off, lens[q][c]);
        off += lens[q][c];
      }
    };
    unsigned nt = n_threads ? n_threads : std::max(1u, std::thread::hardware_concurrency());
    nt = std::min<unsigned>(nt, std::max<uint32_t>(n_req, 1));
    if (nt <= 1) {
      for (uint32_t q = 0; q < n_req; ++q) work(q);
    } else {
      std::atomic<uint32_t> next{0};
      std::vector<std::thread> pool;
      for (unsigned k = 0; k < nt; ++k)
        pool.emplace_back([&] {
          for (uint32_t q; (q = next.fetch_add(1)) < n_req;) work(q);
        });
      for (auto& th : pool) th.join();
    }
  } catch (const std::exception&) {
    return fail(IRM_EINVAL, std::string(fn) + ": out of host memory or threads");
  }

  // 2. capacity check before the registry changes (with the fallback on, a
  // missed chunk may become one entry per window: counted as such)
  const uint32_t W = p->fallback_window;
  uint64_t total = 0;
  for (uint32_t q = 0; q < n_req; ++q) {
    const uint32_t pl = prefix_len ? prefix_len[q] : 0;
    total += (pl ? (pl > (uint32_t)IRM_CARVE_OUT ? 2 : 1) : 0);
    if (W == 0)
      total += lens[q].size();
    else
      for (uint32_t n : lens[q]) total += (n + W - 1) / W;
  }
  *n_chunks = (uint32_t)std::min<uint64_t>(total, 0xffffffffull);
  if (total > max_chunks) return fail(IRM_ERANGE, std::string(fn) + ": more entries than max_chunks");
  if (total && !chunks) return fail(IRM_EINVAL, std::string(fn) + ": chunks is NULL");
  uint64_t fresh_rows = 0;
  for (uint32_t q = 0; q < n_req; ++q)
    fresh_rows += tok_first[q + 1] - tok_first[q] - (prefix_len ? prefix_len[q] : 0);
  if (r->next_row + fresh_rows > 0x100000000ull)
    return fail(IRM_ERANGE, std::string(fn) + ": fresh rows would pass pool row 2^32");

  // 3. registry lookups and inserts, in request order
  try {
    uint32_t k = 0;
    std::vector<uint64_t> wfp;
    std::vector<char> whit;
    std::vector<irm_registry::Entry> went;
    auto lookup = [&](uint64_t f, uint32_t len) -> const irm_registry::Entry* {
      auto it = r->map.find(f);
      return (it != r->map.end() && it->second.len == len) ? &it->second : nullptr;
    };
    auto put = [&](uint32_t row, uint32_t len, int32_t p_src, int32_t p_tgt, uint32_t flags, uint64_t fp) {
      chunks[k] = irm_chunk{row, len, p_src, p_tgt, flags};
      if (fingerprints) fingerprints[k] = fp;
      ++k;
    };
    for (uint32_t q = 0; q < n_req; ++q) {
      seq_first[q] = k;
      const uint32_t pl = prefix_len ? prefix_len[q] : 0;
      if (pl) {
        const uint32_t row = prefix_row ? prefix_row[q] : 0;
        const uint32_t head = std::min<uint32_t>(pl, IRM_CARVE_OUT);
        put(row, head, 0, 0, IRM_FRESH, 0);
        if (pl > head) put(row + head, pl - head, (int32_t)head, (int32_t)head, 0, 0);
      }
      int32_t pos = (int32_t)pl;
      for (size_t c = 0; c < lens[q].size(); ++c) {
        const uint32_t n = lens[q][c];
        const uint64_t fp = prints[q][c];
        if (pos < IRM_CARVE_OUT) {
          put((uint32_t)r->next_row, n, pos, pos, IRM_FRESH, fp);
          r->next_row += n;
        } else if (const irm_registry::Entry* e = lookup(fp, n)) {
          put(e->pool_row, n, e->p_src, pos, 0, fp);
        } else if (W == 0) {
          const uint32_t row = (uint32_t)r->next_row;
          r->next_row += n;
          r->map[fp] = irm_registry::Entry{row, n, pos};
          put(row, n, pos, pos, IRM_FRESH, fp);
        } else {
          // S1: look the chunk's W-token windows up again
          const int32_t* seg = tokens + tok_first[q] + pos;
          const uint32_t n_win = (n + W - 1) / W;
          wfp.resize(n_win);
          whit.resize(n_win);
          went.resize(n_win);
          bool any = false;
          for (uint32_t k = 0; k < n_win; ++k) {  // every window looked up before any insert
            const uint32_t o = k * W, len = std::min(W, n - o);
            wfp[k] = fingerprint(seg + o, len);
            const irm_registry::Entry* e = lookup(wfp[k], len);
            whit[k] = e != nullptr;
            if (e) went[k] = *e;
            any = any || whit[k];
          }
          if (!any) {
            const uint32_t row = (uint32_t)r->next_row;
            r->next_row += n;
            r->map[fp] = irm_registry::Entry{row, n, pos};
            for (uint32_t k = 0; k < n_win; ++k) {
              const uint32_t o = k * W;
              r->map[wfp[k]] = irm_registry::Entry{row + o, std::min(W, n - o), pos + (int32_t)o};
            }
            put(row, n, pos, pos, IRM_FRESH, fp);
          } else {
            for (uint32_t k = 0; k < n_win; ++k) {
              const uint32_t o = k * W, len = std::min(W, n - o);
              const int32_t pw = pos + (int32_t)o;
              if (whit[k]) {
                put(went[k].pool_row, len, went[k].p_src, pw, 0, wfp[k]);
              } else {
                const uint32_t row = (uint32_t)r->next_row;
                r->next_row += len;
                r->map[wfp[k]] = irm_registry::Entry{row, len, pw};
                put(row, len, pw, pw, IRM_FRESH, wfp[k]);
              }
            }
          }
        }
        pos += (int32_t)n;
      }
    }
    seq_first[n_req] = k;
    *n_chunks = k;
  } catch (const std::bad_alloc&) {
    return fail(IRM_EINVAL, std::string(fn) + ": out of host memory (the registry keeps the inserts made so far)");
  }
  return IRM_OK;
}
