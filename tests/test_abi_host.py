"""Host-side checks of the C ABI (no GPU): the library loads and exports every
symbol the header declares, and the chunk-table builder agrees bit for bit
with the oracle's table expansion, including every failure code."""
import os
import re

import numpy as np
import pytest

import mla_position_independent_amd as irm
import oracle
from synth import CHUNK_DTYPE, FRESH, random_table, tiny_decode, batched_decode, tail_prefill

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "irm.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(irm_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = irm.lib()
    names = _declared()
    assert len(names) >= 13
    for n in names:
        assert hasattr(L, n), n
    assert sorted(irm.EXPORTS) == names


def test_rope_inv_freq_matches_oracle():
    got = irm.rope_inv_freq(10000.0)
    want = oracle.rope_inv_freq(10000.0)
    assert np.allclose(got, want, rtol=1e-15, atol=0)   # a few ulp between libm pow and numpy power
    with pytest.raises(irm.IrmError) as e:
        irm.rope_inv_freq(0.5)
    assert e.value.code == "EINVAL"


def _compare_with_oracle(chunks, seq_first, pool_rows):
    t = irm.Table(chunks, seq_first, pool_rows)
    pr, de, fr = t.expand_host()
    ref = oracle.expand_table(chunks, seq_first, pool_rows)
    base = t.seq_base()
    assert base[0] == 0
    for s, (g, d, f) in enumerate(ref):
        sl = slice(int(base[s]), int(base[s + 1]))
        assert np.array_equal(pr[sl], g)
        assert np.array_equal(de[sl].astype(np.int64), d)
        assert np.array_equal(fr[sl].astype(bool), f)
    assert t.total_rows == sum(len(g) for g, _, _ in ref)
    assert t.n_seq == len(ref)
    assert t.max_seq_len == max([len(g) for g, _, _ in ref], default=0)
    return t


@pytest.mark.parametrize("seed", range(12))
def test_table_matches_oracle_random(seed):
    rng = np.random.default_rng(500 + seed)
    n_seq = int(rng.integers(1, 6))
    lens = [int(x) for x in rng.integers(1, 700, size=n_seq)]
    w = random_table(seed, lens, p_hit=0.7, prefix_frac=float(rng.random()) * 0.5,
                     len_fn=lambda r: int(r.integers(1, 80)))
    _compare_with_oracle(w.chunks, w.seq_first, w.pool.shape[0])


def test_table_matches_oracle_workloads():
    for w in (tiny_decode(), batched_decode(batch=3, ctx=3000), tail_prefill(n_q=64, prefix_end=1000,
                                                                           hits_end=4000, total=6000)):
        _compare_with_oracle(w.chunks, w.seq_first, w.pool.shape[0])


def test_table_empty_sequences():
    t = _compare_with_oracle(np.zeros(0, CHUNK_DTYPE), np.array([0, 0, 0], np.uint32), 0)
    assert t.total_rows == 0 and t.n_seq == 2
    c = np.array([(0, 40, 0, 0, FRESH)], dtype=CHUNK_DTYPE)
    _compare_with_oracle(c, np.array([0, 0, 1, 1], np.uint32), 40)


CASES = [
    ([(0, 32, 0, 0, FRESH | 4)], "EINVAL"),
    ([(0, 0, 0, 0, FRESH)], "EINVAL"),
    ([(990, 32, 0, 0, FRESH)], "ERANGE"),
    ([(0, 32, 5, 5, FRESH)], "ELAYOUT"),
    ([(0, 32, 0, 0, FRESH), (40, 8, 7, 33, 0)], "ELAYOUT"),
    ([(0, 32, 3, 0, FRESH)], "EINVAL"),
    ([(0, 16, 0, 0, FRESH), (40, 8, 500, 16, 0)], "ECARVEOUT"),
    ([(0, 32, 0, 0, FRESH), (40, 8, -2**31, 32, 0)], "ERANGE"),
    ([(0, 32, 0, 0, FRESH), (40, 8, 2**31 - 1, 32, 0)], "OK"),
    ([(0, 31, 0, 0, FRESH), (40, 8, 31, 31, 0)], "ECARVEOUT"),   # exact prefix below 32 still rejected
]


@pytest.mark.parametrize("rows,code", CASES)
def test_table_error_codes_match_oracle(rows, code):
    c = np.array(rows, dtype=CHUNK_DTYPE)
    sf = np.array([0, len(rows)], dtype=np.uint32)
    try:
        oracle.expand_table(c, sf, 1000)
        ocode = "OK"
    except oracle.TableError as e:
        ocode = e.code
    assert ocode == code
    if code == "OK":
        _compare_with_oracle(c, sf, 1000)
    else:
        with pytest.raises(irm.IrmError) as e:
            irm.Table(c, sf, 1000)
        assert e.value.code == code
        assert len(str(e.value)) > 20


def test_bad_seq_first():
    c = np.array([(0, 32, 0, 0, FRESH)], dtype=CHUNK_DTYPE)
    for sf in ([1, 1], [0, 2], [0, 1, 0, 1]):
        with pytest.raises(irm.IrmError) as e:
            irm.Table(c, np.array(sf, np.uint32), 1000)
        assert e.value.code == "EINVAL"


def test_seq_base_is_prefix_sum():
    w = random_table(3, [100, 1, 257, 64])
    t = irm.Table(w.chunks, w.seq_first, w.pool.shape[0])
    assert t.seq_base().tolist() == [0, 100, 101, 358, 422]
    assert t.device_bytes % 256 == 0 and t.device_bytes >= 32 * t.n_chunks + 256 * t.n_chunks


def test_prefill_assembled_validation_errors():
    """Argument checks of irm_mla_prefill_assembled come before any HIP call."""
    import ctypes
    L = irm.lib()
    A = 4096  # an aligned stand-in address; validation fails before any use
    f = L.irm_mla_prefill_assembled
    def st(q_pos0=0, n_q=1, kv=A, kv_rows=64, heads=16, scale=0.1, q=A, out=A):
        return irm.STATUS[f(q, q, q_pos0, n_q, kv, kv_rows, heads, ctypes.c_float(scale), out, None, None)]
    assert st(heads=24) == "EUNSUPPORTED"
    assert st(heads=256) == "EUNSUPPORTED"
    assert st(scale=0.0) == "EINVAL"
    assert st(q_pos0=-1) == "ERANGE"
    assert st(n_q=0) == "ERANGE"
    assert st(q_pos0=60, n_q=5) == "ERANGE"
    assert st(kv=None) == "EINVAL"
    assert st(kv=A + 8) == "EINVAL"
    assert st(out=A + 2) == "EINVAL"


def test_nonabsorbed_validation_errors():
    """Argument checks of irm_mla_kv_upproj and irm_mla_prefill_nonabsorbed
    come before any HIP call."""
    import ctypes
    L = irm.lib()
    A = 4096
    def up(kv=A, rows=64, w=A, heads=16, out=A):
        return irm.STATUS[L.irm_mla_kv_upproj(kv, rows, w, w, heads, out, None)]
    assert up(heads=0) == "EUNSUPPORTED" and up(heads=129) == "EUNSUPPORTED"
    assert up(rows=2**32) == "EUNSUPPORTED"
    assert up(kv=None) == "EINVAL" and up(w=A + 4) == "EINVAL" and up(out=A + 8) == "EINVAL"
    def pf(q_pos0=0, n_q=1, kv=A, kvh=A, rows=64, heads=16, scale=0.1, q=A, out=A):
        return irm.STATUS[L.irm_mla_prefill_nonabsorbed(q, q, q_pos0, n_q, kv, kvh, rows, heads,
                                                        ctypes.c_float(scale), out, None, None)]
    assert pf(heads=0) == "EUNSUPPORTED" and pf(heads=200) == "EUNSUPPORTED"
    assert pf(rows=2**32) == "EUNSUPPORTED"
    assert pf(scale=float("inf")) == "EINVAL" and pf(scale=-1.0) == "EINVAL"
    assert pf(q_pos0=-1) == "ERANGE" and pf(n_q=0) == "ERANGE" and pf(q_pos0=60, n_q=5) == "ERANGE"
    assert pf(kvh=None) == "EINVAL" and pf(kv=A + 2) == "EINVAL" and pf(q=A + 8) == "EINVAL"



# ---------------------------------------------------------------- property-based
from hypothesis import HealthCheck, given, settings, strategies as st

_POOL = 5000


@st.composite
def _tables(draw):
    """Chunk tables that are valid by construction (contiguous p_tgt from 0,
    fresh rows below 32 and fresh entries with p_src == p_tgt) with, now and
    then, one planted defect: a pool row past the end, an unknown flag bit, a
    gap or overlap in p_tgt, a hit below position 32, a fresh entry with
    p_src != p_tgt, a zero length, or an extreme delta."""
    n_seq = draw(st.integers(1, 4))
    rows, seq_first = [], [0]
    for _ in range(n_seq):
        pos = 0
        for _ in range(draw(st.integers(0, 6))):
            ln = draw(st.integers(1, 120))
            fresh = pos < 32 or draw(st.booleans())
            if pos < 32 and pos + ln > 32 and draw(st.booleans()):
                ln = 32 - pos                    # fresh entry ending exactly at the carve-out
            p_src = pos if fresh else draw(st.integers(-(2 ** 20), 2 ** 20))
            pool_row = draw(st.integers(0, _POOL - ln))
            rows.append([pool_row, ln, p_src, pos, FRESH if fresh else 0])
            pos += ln
        seq_first.append(len(rows))
    if rows and draw(st.integers(0, 3)) == 0:     # plant one defect
        i = draw(st.integers(0, len(rows) - 1))
        kind = draw(st.integers(0, 6))
        r = rows[i]
        if kind == 0:
            r[0] = _POOL - r[1] + draw(st.integers(1, 50))
        elif kind == 1:
            r[4] |= 1 << draw(st.integers(1, 31))
        elif kind == 2:
            r[3] += draw(st.sampled_from([-1, 1, 7]))
        elif kind == 3:
            r[4] = 0
            r[2] = r[3] + 5
        elif kind == 4:
            r[4] = FRESH
            r[2] = r[3] + draw(st.integers(1, 9))
        elif kind == 5:
            r[1] = 0
        else:
            r[2] = r[3] - draw(st.sampled_from([2 ** 31 - 1, -(2 ** 31) + r[3] + 1]))
            r[4] = 0
    return rows, seq_first


@settings(max_examples=400, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(_tables())
def test_table_builder_agrees_with_oracle_on_generated_tables(case):
    rows, seq_first = case
    c = np.array([tuple(int(x) for x in r) for r in rows], dtype=CHUNK_DTYPE) if rows else np.zeros(0, CHUNK_DTYPE)
    sf = np.array(seq_first, dtype=np.uint32)
    try:
        oracle.expand_table(c, sf, _POOL)
        ocode = "OK"
    except oracle.TableError as e:
        ocode = e.code
    if ocode == "OK":
        _compare_with_oracle(c, sf, _POOL)
    else:
        with pytest.raises(irm.IrmError) as e:
            irm.Table(c, sf, _POOL)
        assert e.value.code == ocode


def test_rope_inv_freq_dim_matches_oracle():
    from oracle import irm_gqa
    for d in (2, 16, 48, 64, 128, 256):
        got = irm.gqa_inv_freq(10000.0, d)        # the library's irm_rope_inv_freq_dim
        want = irm_gqa.gqa_inv_freq(10000.0, d)
        assert got.shape == (d // 2,)
        assert np.allclose(got, want, rtol=1e-15, atol=0)
    # the 64-wide form is the k_r frequencies of irm_rope_inv_freq, bit for bit
    assert np.array_equal(irm.gqa_inv_freq(10000.0, 64), irm.rope_inv_freq(10000.0))
    for theta, d in ((0.5, 64), (10000.0, 63), (10000.0, 0), (float("inf"), 64), (10000.0, 8192)):
        with pytest.raises(irm.IrmError) as e:
            irm.gqa_inv_freq(theta, d)
        assert e.value.code == "EINVAL"


def test_decode_workspace_of_an_empty_batch():
    # a table without sequences is legal; asking for its decode workspace must
    # not divide by the sequence count (run apart: a host fault would end the run)
    import subprocess
    import sys
    code = ("import numpy as np, mla_position_independent_amd as irm\n"
            "t = irm.Table(np.zeros(0, irm.CHUNK_DTYPE), np.array([0], np.uint32), 0)\n"
            "assert t.n_seq == 0\n"
            "for h in (16, 64, 128):\n"
            "    assert irm.decode_workspace_bytes(t, h) <= 512\n"
            "print('ok')\n")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    res = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stderr
    assert res.stdout.strip() == "ok"


def test_default_split_count_keeps_64_rows_per_split():
    # the library's split count when n_splits == 0: enough (sequence, split)
    # workgroups for the 256 CUs, each split at least 64 rows long; the
    # workspace of the default equals the workspace of that explicit count
    def default_splits(t, heads):
        ws = irm.decode_workspace_bytes(t, heads, 0)
        return [s for s in range(1, 65) if irm.decode_workspace_bytes(t, heads, s) == ws]

    w = tiny_decode()  # 1 sequence of 1024 rows: 16 splits of 64 rows
    t = irm.Table(w.chunks, w.seq_first, w.pool.shape[0])
    assert default_splits(t, 16) == [16]
    w = batched_decode()  # 64 sequences of 8192 rows: 4 splits fill 256 CUs
    t = irm.Table(w.chunks, w.seq_first, w.pool.shape[0])
    assert default_splits(t, 16) == [4]


def test_check_out_refuses_outputs_the_kernels_could_overrun():
    import torch
    good = torch.empty((3, 4), dtype=torch.bfloat16)
    irm.check_out(good, (3, 4), "cpu")
    with pytest.raises(ValueError):
        irm.check_out(torch.empty((3, 5), dtype=torch.bfloat16), (3, 4), "cpu")
    with pytest.raises(ValueError):
        irm.check_out(torch.empty((12,), dtype=torch.bfloat16), (3, 4), "cpu")
    with pytest.raises(TypeError):
        irm.check_out(torch.empty((3, 4), dtype=torch.float32), (3, 4), "cpu")
    with pytest.raises(TypeError):
        irm.check_out(torch.empty((3, 4), dtype=torch.int16), (3, 4), "cpu")
    with pytest.raises(ValueError):
        irm.check_out(torch.empty((4, 3), dtype=torch.bfloat16).t(), (3, 4), "cpu")
    with pytest.raises(ValueError):
        irm.check_out(good, (3, 4), "meta")
    with pytest.raises(TypeError):
        irm.check_out(np.zeros((3, 4)), (3, 4), "cpu")
    irm.check_out(torch.empty(10, dtype=torch.uint8), (10,), "cpu", "workspace", torch.uint8)


def test_table_gather_stats_counts_shared_runs():
    """Entries that start at the same pool row are read once by the
    rotate-gather.  Groups of the table below, counted by hand: pool row 0
    (two fresh placements of 40 rows) 40 rows, 5 items; pool row 100 (600,
    300, 257, 600 and 1 rows) 600 rows in records of 256, 256 and 88 rows,
    32 + 32 + 11 items; pool row 800 (50, 10, 50) 50 rows, 7 items; pool row
    900 (1, 1) 1 row, 1 item; pool row 1000 (32) 4 items; pool row 150 (100,
    a run starting inside the 600-row chunk: its own group) 13 items."""
    rng = np.random.default_rng(41)
    src = lambda: int(rng.integers(0, 131072))
    s0 = [(0, 40, 0, 0, FRESH), (100, 600, src(), 40, 0), (800, 50, src(), 640, 0), (100, 300, src(), 690, 0),
          (900, 1, src(), 990, 0)]
    s1 = [(1000, 32, 0, 0, FRESH), (100, 257, src(), 32, 0), (900, 1, src(), 289, 0), (800, 10, src(), 290, 0),
          (150, 100, src(), 300, 0), (800, 50, src(), 400, 0)]
    s2 = [(0, 40, 0, 0, FRESH), (100, 600, src(), 40, 0), (100, 1, src(), 640, 0)]
    chunks = np.array(s0 + s1 + s2, dtype=CHUNK_DTYPE)
    t = irm.Table(chunks, np.array([0, len(s0), len(s0) + len(s1), len(chunks)], np.uint32), 1100)
    st = t.gather_stats()
    assert st["n_groups"] == 8
    assert st["n_items"] == 5 + 75 + 7 + 1 + 4 + 13
    assert st["read_rows"] == 40 + 600 + 50 + 1 + 32 + 100
    assert t.total_rows == 991 + 450 + 641
    assert 32 * len(chunks) < st["host_bytes"] < t.device_bytes
    # no shared starts: every assembled row is read once
    u = irm.Table(np.array([(0, 40, 0, 0, FRESH), (40, 300, 9, 40, 0)], dtype=CHUNK_DTYPE),
                  np.array([0, 2], np.uint32), 400)
    su = u.gather_stats()
    assert su["read_rows"] == u.total_rows == 340 and su["n_groups"] == 1 + 2 and su["n_items"] == 5 + 32 + 6


def test_table_gather_stats_caps_placements_per_record():
    """A run placed by 20 entries (a prompt every request shares) is read once
    per 8 placements: records of 8, 8 and 4 members; the 4-row tail of the
    40-row run placed by the longest members only is read by their record."""
    seq_first = [0]
    chunks = []
    for s in range(20):
        n = 40 if s < 3 else 36          # the first record's first three members are longer
        chunks += [(1000 + 40 * s, 32, 0, 0, FRESH), (0, n, 5, 32, 0)]
        seq_first.append(len(chunks))
    t = irm.Table(np.array(chunks, dtype=CHUNK_DTYPE), np.array(seq_first, np.uint32), 2000)
    st = t.gather_stats()
    # 20 fresh runs of 32 rows (own groups, 4 items each) + the shared run: members 0-7 (40 rows,
    # 5 items), 8-15 (36 rows, 5 items), 16-19 (36 rows, 5 items)
    assert st["n_groups"] == 20 + 3
    assert st["n_items"] == 20 * 4 + 5 + 5 + 5
    assert st["read_rows"] == 20 * 32 + 40 + 36 + 36
