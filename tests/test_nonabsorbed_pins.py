"""Pins of the non-absorbed MLA prefill oracle (oracle/irm_nonabsorbed.py).

The up-projection is checked against a per-row matrix-vector product with
weights laid out [head][feature][latent]; the attention against torch's
scaled_dot_product_attention (float64, CPU) on the full 192-wide keys with an
explicit causal mask; and the whole prefill against the absorbed oracle with
the query folded through W_UK and the latent output mapped through W_UV
(gentlecold.top section 4: the two forms give the same attention).  Special
cases: one visible key returns its value, the last query equals a query that
sees the whole cache, and the inclusive mask boundary.
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import irm_nonabsorbed as NA

SCALE = 1.0 / np.sqrt(192.0)


def _case(rng, N, nq, H):
    c_kv = rng.standard_normal((N, 512))
    k_r = rng.standard_normal((N, 64))
    w_uk = rng.standard_normal((H, 128, 512)) / np.sqrt(512)
    w_uv = rng.standard_normal((H, 128, 512)) / np.sqrt(512)
    q_nope = rng.standard_normal((nq, H, 128))
    q_rope = rng.standard_normal((nq, H, 64))
    return c_kv, k_r, w_uk, w_uv, q_nope, q_rope


def test_up_project_is_per_row_matvec():
    rng = np.random.default_rng(20)
    c_kv, _, w_uk, w_uv, _, _ = _case(rng, 5, 1, 3)
    k, v = NA.up_project(c_kv, w_uk, w_uv)
    assert k.shape == (5, 3, 128) and v.shape == (5, 3, 128)
    for t in range(5):
        for h in range(3):
            assert np.allclose(k[t, h], w_uk[h] @ c_kv[t], rtol=0, atol=1e-12)
            assert np.allclose(v[t, h], w_uv[h] @ c_kv[t], rtol=0, atol=1e-12)
    # features are not transposed: a one-hot latent picks a column of each weight
    e = np.zeros((1, 512)); e[0, 7] = 1.0
    k1, v1 = NA.up_project(e, w_uk, w_uv)
    assert np.array_equal(k1[0], w_uk[:, :, 7]) and np.array_equal(v1[0], w_uv[:, :, 7])


@pytest.mark.parametrize("N,nq,H", [(40, 40, 1), (96, 33, 3)])
def test_matches_library_causal_attention(N, nq, H):
    rng = np.random.default_rng(21 + N)
    c_kv, k_r, w_uk, w_uv, q_nope, q_rope = _case(rng, N, nq, H)
    q_pos0 = N - nq
    o, lse = NA.mla_prefill_nonabsorbed(q_nope, q_rope, c_kv, k_r, w_uk, w_uv, q_pos0, SCALE)
    t = torch.from_numpy
    k_full = np.concatenate([np.einsum("hjc,tc->htj", w_uk, c_kv), np.broadcast_to(k_r, (H, N, 64))], -1)
    v_full = np.einsum("hjc,tc->htj", w_uv, c_kv)
    q_full = np.concatenate([q_nope, q_rope], -1).transpose(1, 0, 2)            # [H, nq, 192]
    mask = t(np.arange(N)[None, :] <= (q_pos0 + np.arange(nq))[:, None])
    ref = torch.nn.functional.scaled_dot_product_attention(
        t(np.ascontiguousarray(q_full)), t(np.ascontiguousarray(k_full)), t(np.ascontiguousarray(v_full)),
        attn_mask=mask).numpy()                                                  # default scale 1/sqrt(192)
    assert np.allclose(o, ref.transpose(1, 0, 2), rtol=1e-10, atol=1e-12)
    s = np.einsum("hqd,htd->hqt", q_full, k_full) * SCALE
    s = np.where(mask.numpy()[None], s, -np.inf)
    m = s.max(-1)
    ref_lse = m + np.log(np.exp(s - m[..., None]).sum(-1))
    assert np.allclose(lse, ref_lse.T, rtol=0, atol=1e-10)


def test_equals_absorbed_form():
    """q_lat = W_UK^T q_nope per head; out = W_UV o_lat; lse unchanged."""
    rng = np.random.default_rng(23)
    N, nq, H = 80, 20, 4
    c_kv, k_r, w_uk, w_uv, q_nope, q_rope = _case(rng, N, nq, H)
    q_pos0 = N - nq
    o, lse = NA.mla_prefill_nonabsorbed(q_nope, q_rope, c_kv, k_r, w_uk, w_uv, q_pos0, SCALE)
    q_lat = np.einsum("hjc,qhj->qhc", w_uk, q_nope)
    o_lat, lse_a = oracle.mla_prefill_tail(q_lat, q_rope, c_kv, k_r, q_pos0, SCALE)
    assert np.allclose(o, np.einsum("hjc,qhc->qhj", w_uv, o_lat), rtol=1e-10, atol=1e-12)
    assert np.allclose(lse, lse_a, rtol=0, atol=1e-10)


def test_special_cases_and_mask_boundary():
    rng = np.random.default_rng(24)
    N, H = 50, 2
    c_kv, k_r, w_uk, w_uv, q_nope, q_rope = _case(rng, N, N, H)
    _, v = NA.up_project(c_kv, w_uk, w_uv)
    # query 0 at position 0 sees only row 0: its output is that row's value
    o, lse = NA.mla_prefill_nonabsorbed(q_nope, q_rope, c_kv, k_r, w_uk, w_uv, 0, SCALE, query_ids=[0, N - 1])
    assert np.allclose(o[0], v[0], rtol=0, atol=1e-13)
    k, _ = NA.up_project(c_kv, w_uk, w_uv)
    assert np.allclose(lse[0], SCALE * (np.einsum("hj,hj->h", k[0], q_nope[0]) + q_rope[0] @ k_r[0]), atol=1e-12)
    # the last query sees every row: a plain softmax over the whole cache
    s = SCALE * (np.einsum("thj,hj->ht", k, q_nope[N - 1]) + q_rope[N - 1] @ k_r.T)
    p = np.exp(s - s.max(-1, keepdims=True))
    ref = np.einsum("ht,thj->hj", p, v) / p.sum(-1)[:, None]
    assert np.allclose(o[1], ref, rtol=1e-11, atol=1e-12)
    # inclusive boundary: row q_pos0 + i changes query i, row q_pos0 + i + 1 does not
    q_pos0, i = 30, 4
    base, _ = NA.mla_prefill_nonabsorbed(q_nope[:10], q_rope[:10], c_kv, k_r, w_uk, w_uv, q_pos0, SCALE)
    c2 = c_kv.copy(); c2[q_pos0 + i] += 1.0
    moved, _ = NA.mla_prefill_nonabsorbed(q_nope[:10], q_rope[:10], c2, k_r, w_uk, w_uv, q_pos0, SCALE)
    assert not np.allclose(moved[i], base[i]) and np.array_equal(moved[i - 1], base[i - 1])
    c3 = c_kv.copy(); c3[q_pos0 + i + 1] += 1.0
    later, _ = NA.mla_prefill_nonabsorbed(q_nope[:10], q_rope[:10], c3, k_r, w_uk, w_uv, q_pos0, SCALE)
    assert np.array_equal(later[i], base[i]) and not np.allclose(later[i + 1], base[i + 1])
