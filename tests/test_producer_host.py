"""The library's chunk-table producer (host C++, through the C ABI) against the
producer oracle: chunk lengths, fingerprints and assembled tables bit for
bit, registry state after each batch, error codes.  No GPU needed."""
import numpy as np
import pytest

import mla_position_independent_amd as irm
import oracle
from oracle import irm_producer as P
from synth import CHUNK_DTYPE


def _toks(rng, n, hi=60000, lo=0):
    return rng.integers(lo, hi, size=n).astype(np.int32)


@pytest.mark.parametrize("seed,mask_bits,lo,hi", [
    (0, 7, 32, 512), (1, 7, 32, 512), (5, 3, 4, 20), (7, 1, 1, 1), (9, 63, 10, 64), (11, 5, 50, 50),
])
def test_cdc_split_matches_oracle(seed, mask_bits, lo, hi):
    rng = np.random.default_rng(seed)
    for n in (0, 1, 2, 31, 32, 33, 511, 512, 513, 3000):
        t = _toks(rng, n, lo=-2**31, hi=2**31 - 1)
        got = irm.cdc_split(t, irm.cdc_params(seed * 977, mask_bits, lo, hi))
        assert list(got) == P.cdc_split(t, seed * 977, mask_bits, lo, hi), n


def test_cdc_split_long_stream():
    rng = np.random.default_rng(3)
    t = _toks(rng, 60000)
    got = irm.cdc_split(t)
    ref = P.cdc_split(t)
    assert list(got) == ref
    assert min(ref[:-1]) >= 32 and max(ref) <= 512


def test_xxh64_matches_oracle():
    rng = np.random.default_rng(4)
    for n in list(range(0, 100)) + [1000, 4097]:
        d = rng.integers(0, 256, size=n, dtype=np.uint8).tobytes()
        for s in (0, 12345, 2**64 - 7):
            assert irm.xxh64(d, s) == P.xxh64(d, s), (n, s)


def _oracle_batch(reg, reqs, prefix_len=None, prefix_row=None, window=0):
    entries, prints, seq_first = [], [], [0]
    for q, r in enumerate(reqs):
        pl = 0 if prefix_len is None else int(prefix_len[q])
        pr = 0 if prefix_row is None else int(prefix_row[q])
        e, f = reg.assemble(list(r), pl, pr, fallback_window=window)
        entries += e
        prints += [0 if x is None else x for x in f]
        seq_first.append(len(entries))
    return entries, prints, seq_first


def _same(lib_out, ref):
    chunks, seq_first, prints = lib_out
    entries, ref_prints, ref_sf = ref
    assert [tuple(int(v) for v in row) for row in chunks] == entries
    assert list(prints) == ref_prints
    assert list(seq_first) == ref_sf


@pytest.mark.parametrize("window", [0, 128, 50])
def test_registry_batches_match_oracle(window):
    rng = np.random.default_rng(5 + window)
    docs = [list(_toks(rng, int(rng.integers(200, 3000)))) for _ in range(12)]
    lib_reg, ref_reg = irm.Registry(1000), P.Registry(1000)
    for batch in range(4):
        reqs, pls, prs = [], [], []
        for q in range(int(rng.integers(1, 7))):
            parts = []
            for _ in range(int(rng.integers(1, 4))):
                if rng.random() < 0.7:
                    parts += docs[int(rng.integers(0, len(docs)))]
                else:
                    parts += list(_toks(rng, int(rng.integers(1, 600))))
            reqs.append(np.array(parts, dtype=np.int32))
            pls.append(int(rng.choice([0, 0, 10, 31, 32, 33, min(300, len(parts))])) if parts else 0)
            prs.append(int(rng.integers(0, 100)))
        pls = [min(p, len(r)) for p, r in zip(pls, reqs)]
        got = lib_reg.assemble(reqs, pls, prs, params=irm.cdc_params(fallback_window=window), n_threads=1 + batch % 3)
        ref = _oracle_batch(ref_reg, reqs, pls, prs, window)
        _same(got, ref)
        assert lib_reg.info() == (len(ref_reg.map), ref_reg.next_row)
        # the table is valid for the path's own validator (library and oracle)
        pool_rows = max(lib_reg.info()[1], 400)
        irm.Table(got[0], got[1], pool_rows)
        oracle.expand_table(np.asarray(got[0], CHUNK_DTYPE), got[1], pool_rows)
    n_hits = int(np.sum(got[0]["flags"] == 0))
    assert n_hits > 0


def test_registry_edge_requests():
    rng = np.random.default_rng(6)
    reqs = [np.zeros(0, np.int32), _toks(rng, 1), _toks(rng, 31), _toks(rng, 32), _toks(rng, 40)]
    lib_reg, ref_reg = irm.Registry(), P.Registry()
    _same(lib_reg.assemble(reqs), _oracle_batch(ref_reg, reqs))
    # an exact prefix covering the whole request, and one of 1 token
    reqs2 = [_toks(rng, 50), _toks(rng, 500)]
    _same(lib_reg.assemble(reqs2, [50, 1], [7, 9]), _oracle_batch(ref_reg, reqs2, [50, 1], [7, 9]))
    assert lib_reg.info() == (len(ref_reg.map), ref_reg.next_row)


def test_registry_threads_do_not_change_results():
    rng = np.random.default_rng(8)
    doc = list(_toks(rng, 5000))
    reqs = [np.array(list(_toks(rng, int(rng.integers(0, 900)))) + doc, np.int32) for _ in range(9)]
    outs = []
    for nt in (1, 2, 0):
        outs.append(irm.Registry(3).assemble(reqs, n_threads=nt))
    for o in outs[1:]:
        for a, b in zip(outs[0], o):
            assert np.array_equal(a, b)


def test_registry_capacity_error_leaves_registry_unchanged():
    import ctypes
    rng = np.random.default_rng(9)
    t = _toks(rng, 3000)
    reg = irm.Registry(0)
    L = irm.lib()
    p = irm.cdc_params()
    tok_first = np.array([0, t.size], np.uint64)
    chunks = np.zeros(2, CHUNK_DTYPE)
    sf = np.zeros(2, np.uint32)
    n = ctypes.c_uint32()
    st = L.irm_registry_assemble(reg._h, ctypes.byref(p), t.ctypes.data, tok_first.ctypes.data, 1, None, None, 1,
                                 chunks.ctypes.data, None, 2, sf.ctypes.data, ctypes.byref(n))
    assert irm.STATUS[st] == "ERANGE" and n.value == len(P.cdc_split(list(t)))
    assert reg.info() == (0, 0)


def test_producer_error_codes():
    with pytest.raises(irm.IrmError) as e:
        irm.cdc_split(np.arange(10, dtype=np.int32), irm.cdc_params(0, 0, 32, 512))
    assert e.value.code == "EINVAL"
    with pytest.raises(irm.IrmError) as e:
        irm.cdc_split(np.arange(10, dtype=np.int32), irm.cdc_params(0, 7, 40, 39))
    assert e.value.code == "EINVAL"
    with pytest.raises(irm.IrmError) as e:
        irm.Registry().assemble([np.arange(10, dtype=np.int32)], prefix_len=[11])
    assert e.value.code == "EINVAL"


def test_s1_fallback_edge_cases_match_oracle():
    """Edits inside shared documents (chunks miss, some windows hit), windows
    repeated inside one chunk, and windows longer than the chunk."""
    rng = np.random.default_rng(12)
    doc = list(_toks(rng, 5000))
    rep = list(_toks(rng, 64)) * 12 + list(_toks(rng, 300))
    edits = []
    for k in range(6):
        d = list(doc)
        for _ in range(k + 1):
            d[int(rng.integers(100, 5000))] += 1
        edits.append(np.array(d, np.int32))
    for window in (128, 64, 1000):
        lib_reg, ref_reg = irm.Registry(0), P.Registry(0)
        for reqs in ([np.array(doc, np.int32), np.array(rep, np.int32)], edits, [np.array(rep[7:], np.int32)]):
            got = lib_reg.assemble(reqs, params=irm.cdc_params(fallback_window=window))
            _same(got, _oracle_batch(ref_reg, reqs, window=window))
            assert lib_reg.info() == (len(ref_reg.map), ref_reg.next_row)
            irm.Table(got[0], got[1], max(lib_reg.info()[1], 1))

