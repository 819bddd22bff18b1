"""irm_mla_decode_noalloc: the decode entry point that allocates nothing,
its partial states in the library's per-device scratch array, against
irm_mla_decode with a caller workspace (same kernels, so the same bits)."""
import ctypes

import numpy as np
import pytest

import mla_position_independent_amd as irm
from synth import long_decode, random_table

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    irm.lib()
    yield
    torch.cuda.synchronize()


def _inputs(w):
    pool = irm.to_device_bf16(w.pool)
    t = irm.Table(w.chunks, w.seq_first, w.pool.shape[0]).upload()
    return pool, t, irm.to_device_bf16(w.q_lat), irm.to_device_bf16(w.q_rope)


def _noalloc(ql, qr, t, pool, H, S, scale):
    """The call through the C ABI, into outputs allocated beforehand."""
    import torch
    B = t.n_seq
    out = torch.full((B, H, 512), 7.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, H), 7.0, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()
    st = irm.lib().irm_mla_decode_noalloc(ql.data_ptr(), qr.data_ptr(), t.handle, pool.data_ptr(), pool.shape[0],
                                          H, S, ctypes.c_float(scale), out.data_ptr(), lse.data_ptr(), None)
    assert st == 0, irm.lib().irm_last_error().decode()
    torch.cuda.synchronize()
    return out, lse


def _same(a, b):
    import torch
    return torch.equal(a[0].view(torch.int16), b[0].view(torch.int16)) and torch.equal(a[1], b[1])


def test_noalloc_equals_workspace_decode_twice_in_a_row():
    """A large call (the 32 x 32768 x 128-head decode, 16 splits: about 34 MB
    of partial states) and then a smaller one (ragged 16-head batch), each
    bit-identical to irm_mla_decode with a caller workspace."""
    w = long_decode()
    pool, t, ql, qr = _inputs(w)
    got = _noalloc(ql, qr, t, pool, w.n_heads, w.n_splits, w.scale)
    ref = irm.mla_decode(ql, qr, t, pool, n_splits=w.n_splits, scale=w.scale, want_lse=True)
    assert _same(got, ref)
    del pool, t, ql, qr
    w2 = random_table(401, [1, 33, 700, 2100, 5], heads=16, p_hit=0.7, prefix_frac=0.3)
    pool, t, ql, qr = _inputs(w2)
    got = _noalloc(ql, qr, t, pool, 16, 0, w2.scale)
    ref = irm.mla_decode(ql, qr, t, pool, n_splits=0, scale=w2.scale, want_lse=True)
    assert _same(got, ref)


@pytest.mark.parametrize("seed,heads,lens,splits", [
    (402, 64, [5, 1200, 64], 16),
    (403, 128, [900] * 40, 16),      # runs of splits: fewer partial states than splits
    (404, 32, [3000, 1], 7),
])
def test_noalloc_equals_workspace_decode(seed, heads, lens, splits):
    w = random_table(seed, lens, heads=heads, p_hit=0.7, prefix_frac=0.3)
    pool, t, ql, qr = _inputs(w)
    for _ in range(2):   # the scratch keeps the last call's contents: a repeat must not depend on them
        got = _noalloc(ql, qr, t, pool, heads, splits, w.scale)
        ref = irm.mla_decode(ql, qr, t, pool, n_splits=splits, scale=w.scale, want_lse=True)
        assert _same(got, ref)


def test_noalloc_refuses_batches_beyond_its_scratch():
    """40 sequences x 64 splits x 16 heads need 84 MB of partial states, more
    than the 64 MiB array: EWORKSPACE before any launch, outputs untouched."""
    import torch
    w = random_table(405, [1] * 40, heads=16)
    pool, t, ql, qr = _inputs(w)
    out = torch.full((40, 16, 512), 3.0, dtype=torch.bfloat16, device="cuda")
    torch.cuda.synchronize()
    st = irm.lib().irm_mla_decode_noalloc(ql.data_ptr(), qr.data_ptr(), t.handle, pool.data_ptr(), pool.shape[0],
                                          16, 64, ctypes.c_float(w.scale), out.data_ptr(), None, None)
    assert irm.STATUS[st] == "EWORKSPACE"
    torch.cuda.synchronize()
    assert bool(torch.all(out == 3.0))
    # the same batch with fewer splits fits
    got = _noalloc(ql, qr, t, pool, 16, 4, w.scale)
    ref = irm.mla_decode(ql, qr, t, pool, n_splits=4, scale=w.scale, want_lse=True)
    assert _same(got, ref)


def test_noalloc_binding_allocates_nothing():
    """The binding's wrapper takes the outputs from the caller and allocates
    no device memory (torch's allocator statistics do not move)."""
    import torch
    w = random_table(406, [2000, 900], heads=64, p_hit=0.7)
    pool, t, ql, qr = _inputs(w)
    out = torch.empty((2, 64, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((2, 64), dtype=torch.float32, device="cuda")
    irm.mla_decode_noalloc(ql, qr, t, pool, out, lse=lse, n_splits=4, scale=w.scale)
    torch.cuda.synchronize()
    before = torch.cuda.memory_stats()["allocation.all.allocated"]
    irm.mla_decode_noalloc(ql, qr, t, pool, out, lse=lse, n_splits=4, scale=w.scale)
    torch.cuda.synchronize()
    assert torch.cuda.memory_stats()["allocation.all.allocated"] == before
    ref = irm.mla_decode(ql, qr, t, pool, n_splits=4, scale=w.scale, want_lse=True)
    assert _same((out, lse), ref)


def test_noalloc_graph_replay():
    """Captured in a HIP graph (code under capture is what the entry point is
    for) and replayed, with eager calls of it between the replays and new
    query values in the captured buffers, the no-alloc decode matches the
    workspace decode bit for bit on every replay."""
    import torch
    from synth import randn_bf16
    w = random_table(407, [1500, 900, 2600], heads=16, p_hit=0.7, prefix_frac=0.3)
    pool, t, ql, qr = _inputs(w)
    out = torch.empty((w.n_seq, 16, 512), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((w.n_seq, 16), dtype=torch.float32, device="cuda")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # the first call on the device, outside the capture
        irm.mla_decode_noalloc(ql, qr, t, pool, out, lse=lse, n_splits=4, scale=w.scale)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        irm.mla_decode_noalloc(ql, qr, t, pool, out, lse=lse, n_splits=4, scale=w.scale)
    rng = np.random.default_rng(408)
    for rep in range(4):
        if rep >= 2:
            ql.copy_(irm.to_device_bf16(randn_bf16(rng, tuple(ql.shape))))
            qr.copy_(irm.to_device_bf16(randn_bf16(rng, tuple(qr.shape))))
        graph.replay()
        torch.cuda.synchronize()
        got = (out.clone(), lse.clone())
        ref = irm.mla_decode(ql, qr, t, pool, n_splits=4, scale=w.scale, want_lse=True)
        torch.cuda.synchronize()
        assert _same(got, ref), rep
        # an eager call on the same scratch between replays
        assert _same(_noalloc(ql, qr, t, pool, 16, 4, w.scale), ref), rep
