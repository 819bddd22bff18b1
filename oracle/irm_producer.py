"""CPU oracle for the host chunk-table producer: content-defined chunking,
chunk fingerprints and the registry lookup that turns a request's tokens into
chunk-table entries.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  It shares
no code with the library (each side implements the Gear table generator and
xxHash64 from their published definitions) and imports nothing from it.

Plain, slow, single-threaded Python integers.  What the pages fix and where:

* gentlecold.top article, section 5 (serve-path pseudocode): the unmatched
  tail is split by CDC; each segment at target position p is freshly
  prefilled when p < 32, served from the registry when its xxhash hits
  (delta = p - p_src), else prefilled and inserted as (c_KV, k_r_base, p);
  segments are appended in target order.
* gentlecold.top, section 6: a rolling Gear hash emits a boundary when its
  low 7 bits meet the mask, expected chunk size about 128 tokens, chunk
  lengths clamped to [32, 512]; each emitted chunk is fingerprinted with
  xxHash64.  gist.science summary, section 2.2: the Gear hash rolls over
  64-token windows.

Readings where the pages are silent:

* Gear state: 64-bit, h <- (h << 1) + gear(token) mod 2^64, so a token's
  contribution leaves the state after 64 steps (the 64-token window).  The
  state rolls on across chunk boundaries and starts at 0 at the tail start.
* gear(t) = splitmix64 output for the state seed + t * 0x9E3779B97F4A7C15
  (our own seeded table; the pages give none).
* Boundary after token i when the chunk holds at least min_len tokens and
  (h & (2^mask_bits - 1)) == 0 (the low 7 bits are zero), or when it holds
  max_len tokens; the last chunk takes what remains.
* Fingerprint: xxHash64, seed 0, of the chunk's token ids as 4-byte
  little-endian signed integers.
* Registry: keyed by fingerprint; a stored entry of another length counts as
  a miss and is replaced.  Fresh rows (carve-out and misses) get consecutive
  pool rows from the registry's allocation counter; carve-out segments are
  not inserted.
* Exact prefix (RadixCache match, outside the method): the caller states its
  length and first pool row; its first 32 rows are emitted as a fresh entry
  and the rest as an exact-prefix entry (delta 0), as the validator of the
  chunk table wants rows below 32 to be fresh.
* S1 fallback (gist.science summary, section 2.2; gentlecold.top section 6:
  a CDC miss is re-split into fixed 128-token windows that are looked up
  again), when enabled: the windows start at the chunk start (the last one
  may be shorter); if none hits, the chunk is prefilled on consecutive rows
  and registered together with each of its windows (pointing into those
  rows); otherwise every window becomes its own entry, a hit from the
  registry or a miss on new rows that is registered as a window (the chunk
  itself, no longer on consecutive rows, is not registered).
"""
from __future__ import annotations

from typing import Dict, List, Optional, Tuple

MASK64 = (1 << 64) - 1
CARVE_OUT = 32
FLAG_FRESH = 1
GOLDEN_GAMMA = 0x9E3779B97F4A7C15

# CDC parameters the pages fix: 7 mask bits, chunk lengths in [32, 512]
CDC_MASK_BITS = 7
CDC_MIN = 32
CDC_MAX = 512


# ---------------------------------------------------------------------------
# splitmix64 (Steele, Lea and Flood, "Fast splittable pseudorandom number
# generators", OOPSLA 2014; the 64-bit finaliser constants as published with
# Vigna's splitmix64.c): one output for a given state.
# ---------------------------------------------------------------------------
def splitmix64(state: int) -> int:
    z = (state + GOLDEN_GAMMA) & MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def gear(token: int, seed: int) -> int:
    """Gear table entry of a token id (our own seeded table)."""
    return splitmix64((seed + (token & MASK64) * GOLDEN_GAMMA) & MASK64)


def gear_hash_at(tokens, i: int, seed: int) -> int:
    """Gear state after token i, from its definition: the sum of the window's
    gear values, token i - k shifted left by k (k = 0..63), mod 2^64."""
    h = 0
    for k in range(64):
        if i - k < 0:
            break
        h = (h + (gear(int(tokens[i - k]), seed) << k)) & MASK64
    return h


def cdc_split(tokens, seed: int = 0, mask_bits: int = CDC_MASK_BITS, min_len: int = CDC_MIN,
              max_len: int = CDC_MAX) -> List[int]:
    """Chunk lengths of a token stream (gentlecold.top section 6): rolling
    Gear state, boundary at the first position where the chunk has min_len
    tokens and the low mask_bits bits are zero, forced at max_len."""
    mask = (1 << mask_bits) - 1
    lens: List[int] = []
    h = 0
    start = 0
    for i in range(len(tokens)):
        h = ((h << 1) + gear(int(tokens[i]), seed)) & MASK64
        n = i - start + 1
        if (n >= min_len and (h & mask) == 0) or n == max_len:
            lens.append(n)
            start = i + 1
    if start < len(tokens):
        lens.append(len(tokens) - start)
    return lens


# ---------------------------------------------------------------------------
# xxHash64, from the algorithm description of the xxHash specification
# (Yann Collet, xxhash_spec.md, "XXH64 algorithm description").
# ---------------------------------------------------------------------------
P1 = 0x9E3779B185EBCA87
P2 = 0xC2B2AE3D27D4EB4F
P3 = 0x165667B19E3779F9
P4 = 0x85EBCA77C2B2AE63
P5 = 0x27D4EB2F165667C5


def _rotl(x: int, r: int) -> int:
    return ((x << r) | (x >> (64 - r))) & MASK64


def _round(acc: int, lane: int) -> int:
    acc = (acc + lane * P2) & MASK64
    acc = _rotl(acc, 31)
    return (acc * P1) & MASK64


def _merge(acc: int, v: int) -> int:
    acc ^= _round(0, v)
    return (acc * P1 + P4) & MASK64


def xxh64(data: bytes, seed: int = 0) -> int:
    n = len(data)
    p = 0
    if n >= 32:
        v = [(seed + P1 + P2) & MASK64, (seed + P2) & MASK64, seed & MASK64, (seed - P1) & MASK64]
        while p + 32 <= n:
            for j in range(4):
                v[j] = _round(v[j], int.from_bytes(data[p + 8 * j:p + 8 * j + 8], "little"))
            p += 32
        acc = (_rotl(v[0], 1) + _rotl(v[1], 7) + _rotl(v[2], 12) + _rotl(v[3], 18)) & MASK64
        for j in range(4):
            acc = _merge(acc, v[j])
    else:
        acc = (seed + P5) & MASK64
    acc = (acc + n) & MASK64
    while p + 8 <= n:
        acc ^= _round(0, int.from_bytes(data[p:p + 8], "little"))
        acc = (_rotl(acc, 27) * P1 + P4) & MASK64
        p += 8
    if p + 4 <= n:
        acc ^= (int.from_bytes(data[p:p + 4], "little") * P1) & MASK64
        acc = (_rotl(acc, 23) * P2 + P3) & MASK64
        p += 4
    while p < n:
        acc ^= (data[p] * P5) & MASK64
        acc = (_rotl(acc, 11) * P1) & MASK64
        p += 1
    acc ^= acc >> 33
    acc = (acc * P2) & MASK64
    acc ^= acc >> 29
    acc = (acc * P3) & MASK64
    acc ^= acc >> 32
    return acc


def chunk_fingerprint(tokens) -> int:
    """xxHash64 (seed 0) of token ids as 4-byte little-endian integers."""
    return xxh64(b"".join(int(t).to_bytes(4, "little", signed=True) for t in tokens), 0)


# ---------------------------------------------------------------------------
# Registry and request assembly (gentlecold.top section 5 pseudocode)
# ---------------------------------------------------------------------------
class Registry:
    """fingerprint -> (pool_row, len, p_src), plus the pool-row allocation
    counter for freshly prefilled rows."""

    def __init__(self, first_free_row: int = 0):
        self.map: Dict[int, Tuple[int, int, int]] = {}
        self.next_row = first_free_row

    def _alloc(self, n: int) -> int:
        r = self.next_row
        self.next_row += n
        return r

    def _lookup(self, fp: int, n: int):
        hit = self.map.get(fp)
        return hit if hit is not None and hit[1] == n else None

    def assemble(self, tokens, prefix_len: int = 0, prefix_row: int = 0, seed: int = 0,
                 mask_bits: int = CDC_MASK_BITS, min_len: int = CDC_MIN, max_len: int = CDC_MAX,
                 fallback_window: int = 0
                 ) -> Tuple[List[Tuple[int, int, int, int, int]], List[Optional[int]]]:
        """Chunk-table entries (pool_row, len, p_src, p_tgt, flags) of one
        request and the fingerprint of each entry's tokens (None for prefix
        entries).  fallback_window > 0 turns on the S1 fallback with windows
        of that many tokens."""
        entries: List[Tuple[int, int, int, int, int]] = []
        prints: List[Optional[int]] = []
        if prefix_len > 0:
            head = min(prefix_len, CARVE_OUT)
            entries.append((prefix_row, head, 0, 0, FLAG_FRESH))
            prints.append(None)
            if prefix_len > head:
                entries.append((prefix_row + head, prefix_len - head, head, head, 0))
                prints.append(None)
        tail = list(tokens[prefix_len:])
        p = prefix_len
        off = 0
        for n in cdc_split(tail, seed, mask_bits, min_len, max_len):
            seg = tail[off:off + n]
            fp = chunk_fingerprint(seg)
            hit = None if p < CARVE_OUT else self._lookup(fp, n)
            if p < CARVE_OUT:
                entries.append((self._alloc(n), n, p, p, FLAG_FRESH))
                prints.append(fp)
            elif hit is not None:
                entries.append((hit[0], n, hit[2], p, 0))
                prints.append(fp)
            elif fallback_window <= 0:
                row = self._alloc(n)
                self.map[fp] = (row, n, p)
                entries.append((row, n, p, p, FLAG_FRESH))
                prints.append(fp)
            else:
                wins = [(o, min(fallback_window, n - o)) for o in range(0, n, fallback_window)]
                wfps = [chunk_fingerprint(seg[o:o + k]) for o, k in wins]
                whits = [self._lookup(f, k) for f, (o, k) in zip(wfps, wins)]
                if all(h is None for h in whits):
                    row = self._alloc(n)
                    self.map[fp] = (row, n, p)
                    for f, (o, k) in zip(wfps, wins):
                        self.map[f] = (row + o, k, p + o)
                    entries.append((row, n, p, p, FLAG_FRESH))
                    prints.append(fp)
                else:
                    for f, h, (o, k) in zip(wfps, whits, wins):
                        if h is not None:
                            entries.append((h[0], k, h[2], p + o, 0))
                        else:
                            row = self._alloc(k)
                            self.map[f] = (row, k, p + o)
                            entries.append((row, k, p + o, p + o, FLAG_FRESH))
                        prints.append(f)
            p += n
            off += n
        return entries, prints
