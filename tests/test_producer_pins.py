"""Pins of the chunk-table producer oracle (oracle/irm_producer.py).

xxHash64 is checked against the xxhash library, splitmix64 against its
published first output, the rolling Gear state against its definition as a
window sum, the chunk boundaries against the boundary rule evaluated from that
definition, and the registry assembly against the serve-path pseudocode of
the pages (gentlecold.top section 5): repeated content hits with the right
delta, the carve-out stays fresh, and every table it builds passes the path's
own validator.
"""
import numpy as np
import pytest
import xxhash

import oracle
from oracle import irm_producer as P
from synth import CHUNK_DTYPE


def test_xxh64_matches_library():
    rng = np.random.default_rng(0)
    for n in list(range(0, 70)) + [127, 128, 129, 1000, 4099]:
        for seed in (0, 1, 0xDEADBEEF, 2**64 - 1):
            d = rng.integers(0, 256, size=n, dtype=np.uint8).tobytes()
            assert P.xxh64(d, seed) == xxhash.xxh64_intdigest(d, seed), (n, seed)


def test_chunk_fingerprint_is_xxh64_of_le_int32():
    toks = [0, 1, -1, 2**31 - 1, -2**31, 123456]
    assert P.chunk_fingerprint(toks) == xxhash.xxh64_intdigest(np.array(toks, "<i4").tobytes(), 0)


def test_splitmix64_first_output():
    """splitmix64 seeded with 0: first output 0xE220A8397B1DCDAF."""
    assert P.splitmix64(0) == 0xE220A8397B1DCDAF


def test_gear_rolling_equals_window_sum():
    rng = np.random.default_rng(1)
    toks = rng.integers(0, 1000, size=200)
    h = 0
    for i in range(len(toks)):
        h = ((h << 1) + P.gear(int(toks[i]), 7)) & P.MASK64
        assert h == P.gear_hash_at(toks, i, 7), i


def _check_rule(toks, lens, seed, mask_bits, lo, hi):
    mask = (1 << mask_bits) - 1
    assert sum(lens) == len(toks)
    start = 0
    for c, n in enumerate(lens):
        last = c == len(lens) - 1
        assert 1 <= n <= hi
        if not last:
            assert n >= lo
        hits = [i for i in range(start + lo - 1, start + n)
                if (P.gear_hash_at(toks, i, seed) & mask) == 0]
        if not last or n >= lo:
            if hits and hits[0] < start + n - 1:
                raise AssertionError(f"chunk {c} skipped an earlier boundary at {hits[0]}")
            if not last:
                assert (hits and hits[0] == start + n - 1) or n == hi, c
        start += n


@pytest.mark.parametrize("seed,mask_bits,lo,hi", [(0, 7, 32, 512), (3, 4, 8, 40), (9, 2, 1, 6)])
def test_cdc_boundary_rule(seed, mask_bits, lo, hi):
    rng = np.random.default_rng(seed)
    toks = rng.integers(0, 30000, size=1500)
    lens = P.cdc_split(toks, seed, mask_bits, lo, hi)
    _check_rule(toks, lens, seed, mask_bits, lo, hi)


def test_cdc_forced_cuts_on_repetitive_content():
    """A constant stream never meets the mask (unless its Gear value does), so
    every chunk is cut at the maximum length."""
    toks = [5] * 2000
    lens = P.cdc_split(toks, 0)
    g = P.gear(5, 0)
    if all(((g * ((1 << min(k + 1, 64)) - 1)) & 127) != 0 for k in range(64)):
        assert lens[:-1] == [512] * (len(lens) - 1)
    _check_rule(toks, lens, 0, 7, 32, 512)


def test_cdc_boundaries_follow_content():
    """The same region after two different prefixes: once a boundary falls at
    the same content position in both, every later boundary does too."""
    rng = np.random.default_rng(4)
    shared = list(rng.integers(0, 30000, size=6000))
    a = list(rng.integers(0, 30000, size=333)) + shared
    b = list(rng.integers(0, 30000, size=1017)) + shared
    def cuts(toks, off):
        pos, out = 0, set()
        for n in P.cdc_split(toks, 0):
            pos += n
            if pos > off:
                out.add(pos - off)
        return sorted(out)
    ca, cb = cuts(a, 333), cuts(b, 1017)
    common = sorted(set(ca) & set(cb))
    assert common, "no common boundary"
    first = common[0]
    assert [x for x in ca if x >= first] == [x for x in cb if x >= first]
    assert first < 2000


def _table_ok(entries, pool_rows):
    chunks = np.array(entries, dtype=CHUNK_DTYPE)
    oracle.expand_table(chunks, np.array([0, len(entries)]), pool_rows)   # raises on an invalid table


def test_registry_serve_path():
    rng = np.random.default_rng(5)
    doc = list(rng.integers(0, 30000, size=4000))
    reg = P.Registry(first_free_row=100)
    e1, f1 = reg.assemble(doc)
    assert all(e[4] == P.FLAG_FRESH and e[2] == e[3] for e in e1)   # cold registry: all prefilled
    assert e1[0][3] == 0 and e1[0][0] == 100
    _table_ok(e1, reg.next_row)
    # the same request again: every segment past the carve-out hits, delta 0
    e2, f2 = reg.assemble(doc)
    assert f2 == f1
    assert e2[0][4] == P.FLAG_FRESH and e2[0][0] != e1[0][0]   # carve-out stays fresh, new rows
    for x, y in zip(e1[1:], e2[1:]):
        assert y[4] == 0 and y[0] == x[0] and y[1] == x[1] and y[2] == x[3] and y[3] == x[3]
    _table_ok(e2, reg.next_row)
    # the document behind a new 700-token preamble: hits carry delta = shift
    pre = list(rng.integers(0, 30000, size=700))
    e3, _ = reg.assemble(pre + doc)
    hits = [e for e in e3 if e[4] == 0]
    assert len(hits) >= 10
    assert all(e[3] - e[2] == 700 for e in hits)
    _table_ok(e3, reg.next_row)


def test_registry_exact_prefix_and_carve_out():
    rng = np.random.default_rng(6)
    toks = list(rng.integers(0, 30000, size=900))
    reg = P.Registry(first_free_row=5000)
    e, f = reg.assemble(toks, prefix_len=300, prefix_row=40)
    assert e[0] == (40, 32, 0, 0, P.FLAG_FRESH)
    assert e[1] == (72, 268, 32, 32, 0)
    assert f[:2] == [None, None]
    assert e[2][3] == 300
    _table_ok(e, reg.next_row)
    # a short exact prefix: the first tail segment still starts below 32 and is fresh
    reg2 = P.Registry()
    e, _ = reg2.assemble(toks, prefix_len=10, prefix_row=0)
    assert e[0] == (0, 10, 0, 0, P.FLAG_FRESH)
    assert e[1][3] == 10 and e[1][4] == P.FLAG_FRESH
    _table_ok(e, max(reg2.next_row, 10))


def test_registry_length_mismatch_is_a_miss():
    reg = P.Registry()
    toks = list(range(1000, 1200))
    fp = P.chunk_fingerprint(toks[40:80])
    reg.map[fp] = (7, 39, 3)            # same fingerprint, other length
    e, f = reg.assemble(toks[:40] + toks[40:80], seed=0, min_len=40, max_len=40)
    assert f[1] == fp and e[1][4] == P.FLAG_FRESH
    assert reg.map[fp][1] == 40


def test_s1_fallback_recovers_windows_of_a_missed_chunk():
    """gist.science 2.2 / gentlecold.top 6: a CDC miss is re-split into fixed
    128-token windows and looked up again.  One token changed inside a long
    chunk: that chunk misses, but its windows that do not hold the change hit
    at their own positions, and the chunks after it hit whole."""
    rng = np.random.default_rng(7)
    doc = list(rng.integers(0, 30000, size=6000))
    lens = P.cdc_split(doc)
    starts = np.cumsum([0] + lens[:-1])
    c = next(i for i in range(1, len(lens)) if lens[i] >= 400 and starts[i] >= 32)
    x = int(starts[c]) + 200                      # inside window 1 of chunk c, far from its end
    reg = P.Registry()
    e1, _ = reg.assemble(doc, fallback_window=128)
    assert all(e[4] == P.FLAG_FRESH for e in e1)
    doc2 = list(doc)
    doc2[x] = (doc2[x] + 1) % 30000
    assert P.cdc_split(doc2) == lens                 # the change moves no boundary here
    e2, f2 = reg.assemble(doc2, fallback_window=128)
    by_pos = {e[3]: e for e in e2}
    s = int(starts[c])
    for o in range(0, lens[c], 128):
        e = by_pos[s + o]
        assert e[1] == min(128, lens[c] - o)
        if o <= x - s < o + e[1]:
            assert e[4] == P.FLAG_FRESH                # the changed window is prefilled
        else:
            assert e[4] == 0 and e[2] == e[3]          # the others come back at delta 0
    for i in range(c + 1, len(lens)):
        e = by_pos[int(starts[i])]
        assert e[4] == 0 and e[1] == lens[i]
    _table_ok(e2, reg.next_row)
    # without the fallback the whole chunk is prefilled again
    reg0 = P.Registry()
    reg0.assemble(doc)
    e3, _ = reg0.assemble(doc2)
    assert {e[3]: e for e in e3}[s][1] == lens[c] and {e[3]: e for e in e3}[s][4] == P.FLAG_FRESH
