"""Guard bands around every buffer the kernels write.

Each output (assembled rows, the float k_r side output, gather indices,
decode output / lse / workspace, prefill output / lse, the non-absorbed
per-head cache and output, the GQA rows and trig workspace, and the table's
device image) is placed in the middle of a larger allocation whose head and
tail hold a byte pattern; the call goes straight through the C ABI with
pointers to the middle, and the pattern must come back untouched.  A write
past either end of an output would otherwise go unnoticed by the parity
tests, which read only the output itself.  The middle is also compared with
the same call made through the binding, so the pointers were the right ones.
"""
import ctypes

import numpy as np
import pytest

import mla_position_independent_amd as irm
from synth import random_table, nonabsorbed_inputs

pytestmark = pytest.mark.gpu

GUARD = 64 * 1024          # bytes on each side (a multiple of 256: keeps the middle aligned)
PATTERN = 0xA5


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a ROCm GPU")
    irm.lib()
    yield
    torch.cuda.synchronize()


class Guarded:
    """n bytes in the middle of a pattern-filled allocation."""

    def __init__(self, n_bytes: int, fill_middle: int = 0):
        import torch
        self.n = int(n_bytes)
        self.buf = torch.full((self.n + 2 * GUARD,), PATTERN, dtype=torch.uint8, device="cuda")
        self.mid = self.buf[GUARD:GUARD + self.n]
        if self.n:
            self.mid.fill_(fill_middle)

    @property
    def ptr(self) -> int:
        return self.mid.data_ptr()

    def view(self, dtype, shape):
        return self.mid.view(dtype).view(shape)

    def check(self, what: str):
        import torch
        torch.cuda.synchronize()
        head = self.buf[:GUARD].cpu().numpy()
        tail = self.buf[GUARD + self.n:].cpu().numpy()
        bad_h = np.flatnonzero(head != PATTERN)
        bad_t = np.flatnonzero(tail != PATTERN)
        assert bad_h.size == 0, f"{what}: {bad_h.size} bytes written before the buffer (last at -{GUARD - bad_h[-1]})"
        assert bad_t.size == 0, f"{what}: {bad_t.size} bytes written after the buffer (first at +{bad_t[0]})"


def _ok(st, fn):
    assert st == 0, f"{fn}: {irm.STATUS.get(st, st)}: {irm.lib().irm_last_error().decode()}"


def _table_guarded(w):
    """Upload the table's device image into a guarded buffer."""
    t = irm.Table(w.chunks, w.seq_first, w.pool.shape[0])
    img = Guarded(t.device_bytes, fill_middle=0x3C)
    inv = np.ascontiguousarray(irm.rope_inv_freq(w.theta))
    _ok(irm.lib().irm_table_upload(t.handle, inv.ctypes.data, img.ptr, img.n, None), "irm_table_upload")
    t._dev = img.buf
    t._inv = inv
    return t, img


@pytest.mark.parametrize("seed,lens,short", [(301, [1, 31, 33, 700], False), (302, [1500, 64, 5], True)])
def test_rotate_gather_and_gather_index_stay_inside(seed, lens, short):
    import torch
    len_fn = (lambda r: int(r.integers(1, 9))) if short else None
    kw = {"len_fn": len_fn} if short else {}
    w = random_table(seed, lens, p_hit=0.7, prefix_frac=0.2, **kw)
    pool = irm.to_device_bf16(w.pool)
    t, img = _table_guarded(w)
    n = t.total_rows
    out = Guarded(n * 576 * 2, 0x11)
    kr = Guarded(n * 64 * 4, 0x22)
    pr = Guarded(n * 8, 0x33)
    de = Guarded(n * 4, 0x44)
    L = irm.lib()
    _ok(L.irm_rotate_gather(t.handle, pool.data_ptr(), pool.shape[0], out.ptr, kr.ptr, None), "irm_rotate_gather")
    _ok(L.irm_table_gather_index(t.handle, pr.ptr, de.ptr, None), "irm_table_gather_index")
    for g, name in ((img, "table image"), (out, "out_kv"), (kr, "kr_f32"), (pr, "pool_row"), (de, "delta")):
        g.check(name)
    ref, ref_kr = irm.rotate_gather(t, pool, kr_f32=True)
    ref_pr, ref_de = t.gather_index()
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16, (n, 576)), ref.view(torch.int16))
    assert torch.equal(kr.view(torch.float32, (n, 64)), ref_kr)
    assert torch.equal(pr.view(torch.int64, (n,)), ref_pr)
    assert torch.equal(de.view(torch.int32, (n,)), ref_de)


@pytest.mark.parametrize("seed,heads,lens,splits", [
    (311, 16, [1, 33, 700, 2100], 0),     # 16-head groups, ragged
    (312, 64, [5, 1200, 64], 16),         # 64-head blocks, empty splits
    (313, 128, [3000, 40], 0),            # 128 heads, default splits
    (314, 128, [1] * 3 + [900] * 37, 16),  # enough sequences for runs of splits
])
def test_decode_stays_inside(seed, heads, lens, splits):
    import torch
    w = random_table(seed, lens, heads=heads, p_hit=0.7, prefix_frac=0.3)
    pool = irm.to_device_bf16(w.pool)
    t, img = _table_guarded(w)
    ql, qr = irm.to_device_bf16(w.q_lat), irm.to_device_bf16(w.q_rope)
    B, H = w.n_seq, heads
    need = irm.decode_workspace_bytes(t, H, splits)
    out = Guarded(B * H * 512 * 2, 0x55)
    lse = Guarded(B * H * 4, 0x66)
    ws = Guarded(need, 0x77)
    L = irm.lib()
    _ok(L.irm_mla_decode(ql.data_ptr(), qr.data_ptr(), t.handle, pool.data_ptr(), pool.shape[0], H, splits,
                         ctypes.c_float(w.scale), out.ptr, lse.ptr, ws.ptr, ws.n, None), "irm_mla_decode")
    for g, name in ((img, "table image"), (out, "out"), (lse, "lse"), (ws, "workspace")):
        g.check(name)
    ref, ref_l = irm.mla_decode(ql, qr, t, pool, n_splits=splits, scale=w.scale, want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16, (B, H, 512)), ref.view(torch.int16))
    assert torch.equal(lse.view(torch.float32, (B, H)), ref_l)


@pytest.mark.parametrize("seed,heads,N,nq", [(321, 16, 700, 130), (322, 64, 95, 33), (323, 128, 300, 9)])
def test_prefill_stays_inside(seed, heads, N, nq):
    import torch
    w = random_table(seed, [N], heads=heads, p_hit=0.7, prefix_frac=0.25, n_q=nq, kind="prefill")
    pool = irm.to_device_bf16(w.pool)
    t, img = _table_guarded(w)
    ql, qr = irm.to_device_bf16(w.q_lat), irm.to_device_bf16(w.q_rope)
    L = irm.lib()
    out = Guarded(nq * heads * 512 * 2, 0x12)
    lse = Guarded(nq * heads * 4, 0x13)
    _ok(L.irm_mla_prefill_tail(ql.data_ptr(), qr.data_ptr(), w.q_pos0, nq, t.handle, pool.data_ptr(),
                               pool.shape[0], heads, ctypes.c_float(w.scale), out.ptr, lse.ptr, None),
        "irm_mla_prefill_tail")
    kv = irm.rotate_gather(t, pool)
    out2 = Guarded(nq * heads * 512 * 2, 0x14)
    lse2 = Guarded(nq * heads * 4, 0x15)
    _ok(L.irm_mla_prefill_assembled(ql.data_ptr(), qr.data_ptr(), w.q_pos0, nq, kv.data_ptr(), kv.shape[0], heads,
                                    ctypes.c_float(w.scale), out2.ptr, lse2.ptr, None), "irm_mla_prefill_assembled")
    for g, name in ((img, "table image"), (out, "tail out"), (lse, "tail lse"), (out2, "assembled out"),
                    (lse2, "assembled lse")):
        g.check(name)
    ref, ref_l = irm.mla_prefill_tail(ql, qr, w.q_pos0, t, pool, scale=w.scale, want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16, (nq, heads, 512)), ref.view(torch.int16))
    assert torch.equal(out2.view(torch.int16, (nq, heads, 512)), ref.view(torch.int16))
    assert torch.equal(lse.view(torch.float32, (nq, heads)), ref_l)


def test_nonabsorbed_stays_inside():
    import torch
    w = random_table(331, [300], heads=3, p_hit=0.7, n_q=37, kind="prefill")
    pool = irm.to_device_bf16(w.pool)
    t = irm.Table(w.chunks, w.seq_first, w.pool.shape[0]).upload()
    kv = irm.rotate_gather(t, pool)
    q_nope, wk, wv = nonabsorbed_inputs(331, 37, 3)
    qn, qr = irm.to_device_bf16(q_nope), irm.to_device_bf16(w.q_rope)
    wk, wv = irm.to_device_bf16(wk), irm.to_device_bf16(wv)
    H, rows, nq = 3, kv.shape[0], 37
    L = irm.lib()
    kvh = Guarded(H * rows * 256 * 2, 0x21)
    _ok(L.irm_mla_kv_upproj(kv.data_ptr(), rows, wk.data_ptr(), wv.data_ptr(), H, kvh.ptr, None), "irm_mla_kv_upproj")
    out = Guarded(nq * H * 128 * 2, 0x23)
    lse = Guarded(nq * H * 4, 0x24)
    kvh_t = kvh.view(torch.bfloat16, (H, rows, 256))
    _ok(L.irm_mla_prefill_nonabsorbed(qn.data_ptr(), qr.data_ptr(), w.q_pos0, nq, kv.data_ptr(), kvh.ptr, rows, H,
                                      ctypes.c_float(w.scale), out.ptr, lse.ptr, None), "irm_mla_prefill_nonabsorbed")
    for g, name in ((kvh, "per-head cache"), (out, "out"), (lse, "lse")):
        g.check(name)
    ref_kvh = irm.mla_kv_upproj(kv, wk, wv)
    ref, ref_l = irm.mla_prefill_nonabsorbed(qn, qr, w.q_pos0, kv, kvh_t, scale=w.scale, want_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(kvh_t.view(torch.int16), ref_kvh.view(torch.int16))
    assert torch.equal(out.view(torch.int16, (nq, H, 128)), ref.view(torch.int16))
    assert torch.equal(lse.view(torch.float32, (nq, H)), ref_l)


def test_gqa_rotate_gather_stays_inside():
    import torch
    from synth import randn_bf16
    w = random_table(341, [400, 77], p_hit=0.8)
    n_kv, d = 2, 48
    width = 2 * n_kv * d
    rng = np.random.default_rng(341)
    pool = irm.to_device_bf16(randn_bf16(rng, (w.pool.shape[0], width)))
    t = irm.Table(w.chunks, w.seq_first, w.pool.shape[0]).upload()
    inv = np.ascontiguousarray(irm.gqa_inv_freq(w.theta, d))
    nb = ctypes.c_size_t()
    _ok(irm.lib().irm_gqa_workspace(t.handle, d, ctypes.byref(nb)), "irm_gqa_workspace")
    ws = Guarded(nb.value, 0x31)
    out = Guarded(t.total_rows * width * 2, 0x32)
    _ok(irm.lib().irm_gqa_rotate_gather(t.handle, pool.data_ptr(), pool.shape[0], n_kv, d, inv.ctypes.data, ws.ptr,
                                        ws.n, out.ptr, None), "irm_gqa_rotate_gather")
    ws.check("trig workspace")
    out.check("out")
    ref = irm.gqa_rotate_gather(t, pool, n_kv, d, inv)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16, (t.total_rows, width)), ref.view(torch.int16))


def test_binding_refuses_outputs_of_the_wrong_shape():
    """The binding checks a caller's output before any launch (the C ABI takes
    no output size)."""
    import torch
    w = random_table(351, [200, 90], heads=16, p_hit=0.7)
    pool = irm.to_device_bf16(w.pool)
    t = irm.Table(w.chunks, w.seq_first, w.pool.shape[0]).upload()
    ql, qr = irm.to_device_bf16(w.q_lat), irm.to_device_bf16(w.q_rope)
    short = torch.empty((t.total_rows - 1, 576), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        irm.rotate_gather(t, pool, out=short)
    with pytest.raises(TypeError):
        irm.rotate_gather(t, pool, out=torch.empty((t.total_rows, 576), dtype=torch.float16, device="cuda"))
    with pytest.raises(ValueError):
        irm.mla_decode(ql, qr, t, pool, out=torch.empty((2, 16, 511), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        irm.mla_decode(ql, qr, t, pool, out=torch.empty((2, 512, 16), dtype=torch.bfloat16,
                                                        device="cuda").transpose(1, 2))
    wp = random_table(352, [300], heads=16, n_q=5, kind="prefill")
    pp = irm.to_device_bf16(wp.pool)
    tp = irm.Table(wp.chunks, wp.seq_first, wp.pool.shape[0]).upload()
    qpl, qpr = irm.to_device_bf16(wp.q_lat), irm.to_device_bf16(wp.q_rope)
    with pytest.raises(ValueError):
        irm.mla_prefill_tail(qpl, qpr, wp.q_pos0, tp, pp, out=torch.empty((4, 16, 512), dtype=torch.bfloat16,
                                                                          device="cuda"))
    kv = irm.rotate_gather(tp, pp)
    with pytest.raises(ValueError):
        irm.mla_prefill_assembled(qpl, qpr, wp.q_pos0, kv, out=torch.empty((5, 16, 256), dtype=torch.bfloat16,
                                                                           device="cuda"))
    torch.cuda.synchronize()


def test_side_stream_allocations():
    """Calls on a stream other than the current one allocate their
    temporaries (workspace, lse, outputs) on that stream and give the same
    results as on the current stream."""
    import torch
    w = random_table(361, [2000, 900, 33], heads=64, p_hit=0.7)
    pool = irm.to_device_bf16(w.pool)
    ql, qr = irm.to_device_bf16(w.q_lat), irm.to_device_bf16(w.q_rope)
    t = irm.Table(w.chunks, w.seq_first, w.pool.shape[0]).upload()
    ref, ref_l = irm.mla_decode(ql, qr, t, pool, n_splits=4, scale=w.scale, want_lse=True)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    outs = []
    for k in range(3):
        # the binding's workspace is freed on return each time; allocated on
        # `side`, its block is reused only by work ordered after these kernels
        outs.append(irm.mla_decode(ql, qr, t, pool, n_splits=4, scale=w.scale, want_lse=True, stream=side))
        junk = torch.empty(1 << 20, dtype=torch.uint8, device="cuda")
        junk.fill_(k)
    side.synchronize()
    torch.cuda.synchronize()
    for o, l in outs:
        assert torch.equal(o.view(torch.int16), ref.view(torch.int16))
        assert torch.equal(l, ref_l)
