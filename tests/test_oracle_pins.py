"""Pins of the CPU oracle to facts fixed outside itself.

Each test checks the oracle against what the Irminsul pages or mathematics fix:
the worked delta example, textbook trigonometric values, the complex-number
form of RoPE, the composition law R(delta) R(p_src) = R(p_tgt), an independent
library attention (torch scaled_dot_product_attention on the non-absorbed MLA
form, with explicit up-projections), scipy's logsumexp, closed-form special
cases and brute force on tiny tables.  A dropped term, a wrong sign, a swapped
pair layout or a transposed operand in the oracle fails at least one of them.
"""
import json
import os

import numpy as np
import pytest
import scipy.special
import torch

import oracle
from oracle.irm_oracle import CARVE_OUT, D_LATENT, D_ROPE
from synth import CHUNK_DTYPE, FRESH, bf16_bits_from_f32, random_table

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
OMEGA = oracle.rope_inv_freq(10000.0)
SCALE = 1.0 / np.sqrt(192.0)


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- positions
def test_worked_example_delta():
    """gentlecold.top section 15: 100 -> 350 is +250, 360 -> 110 is -250."""
    for case in _load("delta_worked_example.json")["cases"]:
        p_src, p_tgt = case["p_src"], case["p_tgt"]
        chunks = np.array([(0, p_tgt, 0, 0, FRESH), (1000, 7, p_src, p_tgt, 0)], dtype=CHUNK_DTYPE)
        (gather, delta, fresh), = oracle.expand_table(chunks, np.array([0, 2]), 2000)
        assert np.all(delta[p_tgt:] == case["delta"])
        assert np.all(delta[:p_tgt] == 0)
        assert np.array_equal(gather[p_tgt:], 1000 + np.arange(7))
        assert fresh[:p_tgt].all() and not fresh[p_tgt:].any()


# ---------------------------------------------------------------- rotation
def test_inv_freq_closed_forms():
    assert OMEGA.shape == (32,)
    assert OMEGA[0] == 1.0
    assert abs(OMEGA[16] - 0.01) < 1e-17          # 10000^(-1/2)
    ratio = OMEGA[1:] / OMEGA[:-1]
    assert np.allclose(ratio, 10000.0 ** (-1.0 / 32.0), rtol=1e-14, atol=0)
    assert abs(OMEGA[31] - 10000.0 ** (-31.0 / 32.0)) < 1e-18


def test_rotation_unit_vectors_golden():
    g = _load("rope_unit_vectors.json")

    def val(name):
        return -g[name[1:]] if name.startswith("-") else g[name]

    for case in g["cases"]:
        e = np.zeros(D_ROPE)
        e[case["basis"]] = 1.0
        r = oracle.rotate(e, case["pos"], OMEGA)
        want = np.zeros(D_ROPE)
        for idx, name in case["expect"].items():
            want[int(idx)] = val(name)
        assert np.allclose(r, want, rtol=0, atol=1e-15), case["note"]


def test_rotation_is_complex_multiplication():
    """Pair (x, y) as z = x + iy turns into z * exp(i p omega)."""
    rng = np.random.default_rng(0)
    k = rng.standard_normal((200, D_ROPE))
    pos = rng.integers(-131072, 131073, size=200)
    z = k[:, 0::2] + 1j * k[:, 1::2]
    zr = z * np.exp(1j * (pos[:, None].astype(np.float64) * OMEGA[None, :]))
    r = oracle.rotate(k, pos, OMEGA)
    assert np.allclose(r[:, 0::2], zr.real, rtol=0, atol=1e-12)
    assert np.allclose(r[:, 1::2], zr.imag, rtol=0, atol=1e-12)


def test_composition_law():
    """R(delta) R(p_src) = R(p_tgt) with delta = p_tgt - p_src (gentlecold.top section 4)."""
    rng = np.random.default_rng(1)
    k = rng.standard_normal((500, D_ROPE))
    p_src = rng.integers(-131072, 131073, size=500)
    p_tgt = rng.integers(0, 131073, size=500)
    two_step = oracle.delta_rotate(oracle.rotate(k, p_src, OMEGA), p_tgt - p_src, OMEGA)
    direct = oracle.rotate(k, p_tgt, OMEGA)
    rel = np.linalg.norm(two_step - direct) / np.linalg.norm(direct)
    assert rel < 1e-10


def test_identity_inverse_and_norm():
    rng = np.random.default_rng(2)
    k = rng.standard_normal((100, D_ROPE))
    assert np.array_equal(oracle.delta_rotate(k, 0, OMEGA), k)            # R(0) = I, bit for bit
    d = rng.integers(-131072, 131073, size=100)
    back = oracle.delta_rotate(oracle.delta_rotate(k, d, OMEGA), -d, OMEGA)
    assert np.allclose(back, k, rtol=0, atol=1e-10)
    r = oracle.delta_rotate(k, d, OMEGA)
    n0 = k[:, 0::2] ** 2 + k[:, 1::2] ** 2
    n1 = r[:, 0::2] ** 2 + r[:, 1::2] ** 2
    assert np.allclose(n0, n1, rtol=1e-12, atol=0)


def test_relative_position_invariance():
    """<R(a) q, R(b) k> depends on b - a only."""
    rng = np.random.default_rng(3)
    q = rng.standard_normal(D_ROPE)
    k = rng.standard_normal(D_ROPE)
    a = rng.integers(0, 50000, size=20)
    b = rng.integers(0, 50000, size=20)
    lhs = np.einsum("nd,nd->n", oracle.rotate(q, a, OMEGA), oracle.rotate(k, b, OMEGA))
    rhs = oracle.rotate(k, b - a, OMEGA) @ q
    assert np.allclose(lhs, rhs, rtol=0, atol=1e-9)


def test_bf16_storage_error_within_pages_bound():
    """Rotating a bf16-stored k_r_base reaches the freshly positioned key within the
    bf16 storage error, below the 4.7e-3 relative L2 figure the pages quote for
    bf16 (gist.science summary section 3; gentlecold.top section 11)."""
    rng = np.random.default_rng(4)
    k_pre = rng.standard_normal((4096, D_ROPE))
    p_src = rng.integers(0, 131073, size=4096)
    p_tgt = rng.integers(0, 131073, size=4096)
    base = oracle.rotate(k_pre, p_src, OMEGA)
    base_bf16 = oracle.bf16_to_f64(bf16_bits_from_f32(base.astype(np.float32)))
    got = oracle.delta_rotate(base_bf16, p_tgt - p_src, OMEGA)
    want = oracle.rotate(k_pre, p_tgt, OMEGA)
    rel = np.linalg.norm(got - want) / np.linalg.norm(want)
    assert rel < 4.7e-3
    # the rotation is orthogonal, so the error equals the bf16 storage error exactly
    store = np.linalg.norm(base_bf16 - base) / np.linalg.norm(base)
    assert abs(rel - store) < 1e-9


# ---------------------------------------------------------------- table
def _brute_force_expand(chunks, seq_first):
    """Per output position, search the entry that covers it."""
    out = []
    for s in range(len(seq_first) - 1):
        ents = chunks[seq_first[s]:seq_first[s + 1]]
        L = int(sum(int(e["len"]) for e in ents))
        g, d, f = [], [], []
        for r in range(L):
            hit = [e for e in ents if int(e["p_tgt"]) <= r < int(e["p_tgt"]) + int(e["len"])]
            assert len(hit) == 1
            e = hit[0]
            g.append(int(e["pool_row"]) + r - int(e["p_tgt"]))
            fr = bool(int(e["flags"]) & FRESH)
            f.append(fr)
            d.append(0 if fr else int(e["p_tgt"]) - int(e["p_src"]))
        out.append((g, d, f))
    return out


@pytest.mark.parametrize("seed", range(8))
def test_table_expand_matches_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    lens = [int(x) for x in rng.integers(1, 300, size=rng.integers(1, 5))]
    w = random_table(seed, lens, p_hit=0.6, prefix_frac=0.3, len_fn=lambda r: int(r.integers(1, 40)))
    got = oracle.expand_table(w.chunks, w.seq_first, w.pool.shape[0])
    want = _brute_force_expand(w.chunks, w.seq_first)
    for (g, d, f), (g2, d2, f2) in zip(got, want):
        assert g.tolist() == g2 and d.tolist() == d2 and f.tolist() == f2


def _table(rows, seq_first=None):
    c = np.array(rows, dtype=CHUNK_DTYPE)
    sf = np.array([0, len(rows)] if seq_first is None else seq_first)
    return c, sf


@pytest.mark.parametrize("rows,code", [
    ([(0, 32, 0, 0, FRESH | 4)], "EINVAL"),                     # unknown flag bit
    ([(0, 0, 0, 0, FRESH)], "EINVAL"),                          # zero length
    ([(990, 32, 0, 0, FRESH)], "ERANGE"),                       # pool overflow
    ([(0, 32, 5, 5, FRESH)], "ELAYOUT"),                        # does not start at 0
    ([(0, 32, 0, 0, FRESH), (40, 8, 7, 33, 0)], "ELAYOUT"),     # gap in p_tgt
    ([(0, 32, 3, 0, FRESH)], "EINVAL"),                         # fresh with p_src != p_tgt
    ([(0, 16, 0, 0, FRESH), (40, 8, 500, 16, 0)], "ECARVEOUT"),  # hit below position 32
    ([(0, 32, 0, 0, FRESH), (40, 8, -2**31, 32, 0)], "ERANGE"),  # delta beyond int32
])
def test_table_errors(rows, code):
    c, sf = _table(rows)
    with pytest.raises(oracle.TableError) as ei:
        oracle.expand_table(c, sf, 1000)
    assert ei.value.code == code


def test_table_bad_seq_first_and_empty():
    c, _ = _table([(0, 32, 0, 0, FRESH)])
    for sf in ([1, 1], [0, 2], [0]):
        with pytest.raises(oracle.TableError):
            oracle.expand_table(c, np.array(sf), 1000)
    # empty sequences are valid tables with no rows
    out = oracle.expand_table(np.zeros(0, CHUNK_DTYPE), np.array([0, 0, 0]), 0)
    assert len(out) == 2 and all(len(g) == 0 for g, _, _ in out)


def test_rotate_gather_assembly():
    w = random_table(7, [300, 77, 1], p_hit=0.7, prefix_frac=0.2,
                     len_fn=lambda r: int(r.integers(1, 60)))
    seqs = oracle.rotate_gather(w.pool, w.chunks, w.seq_first, OMEGA)
    for s, (c_kv, k_r) in enumerate(seqs):
        ents = w.chunks[w.seq_first[s]:w.seq_first[s + 1]]
        for e in ents:
            sl = slice(int(e["p_tgt"]), int(e["p_tgt"]) + int(e["len"]))
            src = w.pool[int(e["pool_row"]):int(e["pool_row"]) + int(e["len"])]
            # c_KV is the stored latent, bit for bit
            assert np.array_equal(c_kv[sl], oracle.bf16_to_f64(src[:, :D_LATENT]))
            base = oracle.bf16_to_f64(src[:, D_LATENT:])
            delta = int(e["p_tgt"]) - int(e["p_src"])
            if int(e["flags"]) & FRESH or delta == 0:
                assert np.array_equal(k_r[sl], base)
            else:
                z = (base[:, 0::2] + 1j * base[:, 1::2]) * np.exp(1j * delta * OMEGA)
                assert np.allclose(k_r[sl][:, 0::2], z.real, atol=1e-12, rtol=0)
                assert np.allclose(k_r[sl][:, 1::2], z.imag, atol=1e-12, rtol=0)


# ---------------------------------------------------------------- attention
def _sdpa_nonabsorbed(rng, H, N, q_nope_dim=128, v_dim=128):
    """Non-absorbed MLA with explicit random up-projections, run through torch's
    scaled_dot_product_attention (float64, CPU).  The absorbed query is
    q_lat = W_UK^T q_nope and the latent output maps back through W_UV."""
    c_kv = rng.standard_normal((N, D_LATENT))
    k_r = rng.standard_normal((N, D_ROPE))
    w_uk = rng.standard_normal((H, q_nope_dim, D_LATENT)) / np.sqrt(D_LATENT)
    w_uv = rng.standard_normal((H, v_dim, D_LATENT)) / np.sqrt(D_LATENT)
    q_nope = rng.standard_normal((H, q_nope_dim))
    q_rope = rng.standard_normal((H, D_ROPE))
    k_full = np.concatenate([np.einsum("hdc,nc->hnd", w_uk, c_kv), np.broadcast_to(k_r, (H, N, D_ROPE))], -1)
    v_full = np.einsum("hdc,nc->hnd", w_uv, c_kv)
    q_full = np.concatenate([q_nope, q_rope], -1)[:, None, :]          # [H, 1, 192]
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    o = torch.nn.functional.scaled_dot_product_attention(t(q_full), t(k_full), t(v_full)).numpy()[:, 0]
    scores = (t(q_full) @ t(k_full).transpose(1, 2)).numpy()[:, 0] / np.sqrt(q_full.shape[-1])
    q_lat = np.einsum("hdc,hd->hc", w_uk, q_nope)
    return c_kv, k_r, q_lat, q_rope, w_uv, o, scores


@pytest.mark.parametrize("H,N", [(1, 1), (2, 7), (16, 300)])
def test_decode_matches_library_attention(H, N):
    rng = np.random.default_rng(10 + N)
    c_kv, k_r, q_lat, q_rope, w_uv, o_ref, scores = _sdpa_nonabsorbed(rng, H, N)
    o_lat, lse = oracle.mla_decode(q_lat, q_rope, c_kv, k_r, SCALE)
    o = np.einsum("hdc,hc->hd", w_uv, o_lat)
    assert np.allclose(o, o_ref, rtol=1e-10, atol=1e-12)
    assert np.allclose(lse, scipy.special.logsumexp(scores, axis=-1), rtol=0, atol=1e-10)


def test_decode_special_cases():
    rng = np.random.default_rng(11)
    c_kv = rng.standard_normal((1, D_LATENT))
    k_r = rng.standard_normal((1, D_ROPE))
    q_lat = rng.standard_normal((3, D_LATENT))
    q_rope = rng.standard_normal((3, D_ROPE))
    o, lse = oracle.mla_decode(q_lat, q_rope, c_kv, k_r, SCALE)
    assert np.allclose(o, np.broadcast_to(c_kv[0], o.shape), rtol=0, atol=1e-14)   # one key
    assert np.allclose(lse, SCALE * (q_lat @ c_kv[0] + q_rope @ k_r[0]), rtol=0, atol=1e-12)
    c_kv = rng.standard_normal((50, D_LATENT))
    k_r = rng.standard_normal((50, D_ROPE))
    o, lse = oracle.mla_decode(np.zeros((2, D_LATENT)), np.zeros((2, D_ROPE)), c_kv, k_r, SCALE)
    assert np.allclose(o, np.broadcast_to(c_kv.mean(0), o.shape), rtol=0, atol=1e-13)  # equal scores
    assert np.allclose(lse, np.log(50.0), rtol=0, atol=1e-13)
    # two keys whose scores differ by exactly 1: weights are sigmoid(+-1)
    c2 = np.zeros((2, D_LATENT)); c2[0, 0] = 1.0; c2[1, 1] = 1.0
    q = np.zeros((1, D_LATENT)); q[0, 0] = 1.0 / SCALE
    o, _ = oracle.mla_decode(q, np.zeros((1, D_ROPE)), c2, np.zeros((2, D_ROPE)), SCALE)
    assert abs(o[0, 0] - scipy.special.expit(1.0)) < 1e-14 and abs(o[0, 1] - scipy.special.expit(-1.0)) < 1e-14
    # huge scores stay finite
    o, lse = oracle.mla_decode(1e4 * q_lat[:1], q_rope[:1], c_kv, k_r, SCALE)
    assert np.all(np.isfinite(o)) and np.isfinite(lse).all()


def test_rotated_cache_attention_equals_fresh_cache():
    """Attention over rows rotated from p_src equals attention over rows freshly
    RoPE'd at p_tgt (composition law; gentlecold.top sections 4-5)."""
    rng = np.random.default_rng(12)
    N, H = 256, 4
    c_kv = rng.standard_normal((N, D_LATENT))
    k_pre = rng.standard_normal((N, D_ROPE))
    p_tgt = np.arange(N)
    p_src = p_tgt - rng.integers(-131072, 131073, size=N)
    base = oracle.rotate(k_pre, p_src, OMEGA)
    rotated = oracle.delta_rotate(base, p_tgt - p_src, OMEGA)
    fresh = oracle.rotate(k_pre, p_tgt, OMEGA)
    q_lat = rng.standard_normal((H, D_LATENT))
    q_rope = rng.standard_normal((H, D_ROPE))
    o1, l1 = oracle.mla_decode(q_lat, q_rope, c_kv, rotated, SCALE)
    o2, l2 = oracle.mla_decode(q_lat, q_rope, c_kv, fresh, SCALE)
    assert np.allclose(o1, o2, rtol=0, atol=1e-9) and np.allclose(l1, l2, rtol=0, atol=1e-9)


def test_prefill_matches_library_causal_attention():
    rng = np.random.default_rng(13)
    N, nq, H = 96, 40, 2
    q_pos0 = N - nq
    c_kv = rng.standard_normal((N, D_LATENT))
    k_r = rng.standard_normal((N, D_ROPE))
    q_lat = rng.standard_normal((nq, H, D_LATENT))
    q_rope = rng.standard_normal((nq, H, D_ROPE))
    o, lse = oracle.mla_prefill_tail(q_lat, q_rope, c_kv, k_r, q_pos0, SCALE)
    t = torch.from_numpy
    q = t(np.concatenate([q_lat, q_rope], -1).transpose(1, 0, 2).copy())        # [H, nq, 576]
    k = t(np.concatenate([c_kv, k_r], -1))[None].expand(H, N, 576)
    v = t(c_kv)[None].expand(H, N, D_LATENT)
    mask = t(np.arange(N)[None, :] <= (q_pos0 + np.arange(nq))[:, None])
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=SCALE).numpy()
    assert np.allclose(o, ref.transpose(1, 0, 2), rtol=1e-10, atol=1e-12)
    # last query sees the whole cache: equals decode
    od, ld = oracle.mla_decode(q_lat[-1], q_rope[-1], c_kv, k_r, SCALE)
    assert np.allclose(o[-1], od, rtol=0, atol=1e-13) and np.allclose(lse[-1], ld, rtol=0, atol=1e-13)


def test_prefill_mask_boundary_is_inclusive():
    rng = np.random.default_rng(14)
    N, nq, H = 64, 8, 1
    q_pos0 = N - nq
    c_kv = rng.standard_normal((N, D_LATENT))
    k_r = rng.standard_normal((N, D_ROPE))
    q_lat = rng.standard_normal((nq, H, D_LATENT))
    q_rope = rng.standard_normal((nq, H, D_ROPE))
    o, _ = oracle.mla_prefill_tail(q_lat, q_rope, c_kv, k_r, q_pos0, SCALE)
    i = 3
    own = q_pos0 + i
    c2 = c_kv.copy(); c2[own + 1] += 5.0          # a row after query i: no effect on it
    o2, _ = oracle.mla_prefill_tail(q_lat, q_rope, c2, k_r, q_pos0, SCALE, query_ids=[i])
    assert np.array_equal(o2[0], o[i])
    c3 = c_kv.copy(); c3[own] += 5.0              # its own row: changes it
    o3, _ = oracle.mla_prefill_tail(q_lat, q_rope, c3, k_r, q_pos0, SCALE, query_ids=[i])
    assert not np.allclose(o3[0], o[i])


def test_carve_out_constant():
    assert CARVE_OUT == 32     # gist.science section 2.2; gentlecold.top section 7
