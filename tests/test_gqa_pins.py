"""Pins of the GQA/MHA comparison oracle (oracle/irm_gqa.py): the half-split
rotation against the complex-number form of RoPE, against the MLA oracle's
interleaved rotation after the permutation that interleaves the two halves,
the composition law R(delta) R(p_src) = R(p_tgt), delta 0 as the identity,
and the assembled rows against hand-built rows of a tiny table."""
import numpy as np

import oracle
from oracle import irm_gqa as G
from synth import CHUNK_DTYPE, FRESH


def test_half_split_equals_complex_form():
    rng = np.random.default_rng(0)
    d = 128
    w = G.gqa_inv_freq(1e6, d)
    k = rng.standard_normal((5, 3, d))
    pos = rng.integers(-70000, 70000, size=(5, 3)).astype(np.float64)
    got = G.rotate_half_split(k, pos, w)
    z = (k[..., :d // 2] + 1j * k[..., d // 2:]) * np.exp(1j * pos[..., None] * w)
    assert np.allclose(got, np.concatenate([z.real, z.imag], axis=-1), rtol=0, atol=1e-12)


def test_half_split_is_interleaved_rope_after_permutation():
    """Interleaving the halves (x_0, x_h, x_1, x_{h+1}, ...) turns the
    half-split form into the interleaved form of the MLA path (same
    frequencies for head_dim 64)."""
    rng = np.random.default_rng(1)
    d = 64
    w = G.gqa_inv_freq(10000.0, d)
    assert np.allclose(w, oracle.rope_inv_freq(10000.0), rtol=1e-15)
    k = rng.standard_normal((7, d))
    pos = rng.integers(-100000, 100000, size=7)
    perm = np.stack([np.arange(d // 2), np.arange(d // 2) + d // 2], axis=1).ravel()
    a = G.rotate_half_split(k, pos, w)[:, perm]
    b = oracle.rotate(k[:, perm], pos, oracle.rope_inv_freq(10000.0))
    assert np.allclose(a, b, rtol=0, atol=1e-12)


def test_composition_law_and_identity():
    rng = np.random.default_rng(2)
    d = 128
    w = G.gqa_inv_freq(1e6, d)
    k = rng.standard_normal((9, 8, d))
    p_src = rng.integers(0, 131072, size=(9, 1))
    p_tgt = rng.integers(0, 131072, size=(9, 1))
    at_src = G.rotate_half_split(k, p_src, w)
    moved = G.rotate_half_split(at_src, p_tgt - p_src, w)
    assert np.allclose(moved, G.rotate_half_split(k, p_tgt, w), rtol=0, atol=1e-9)
    assert np.array_equal(G.rotate_half_split(k, 0, w), k)


def test_tiny_table_by_hand():
    """Two entries: a fresh run and a hit moved by +100; K rotated by delta,
    V copied, rows in target order."""
    H, d = 2, 8
    rng = np.random.default_rng(3)
    pool = rng.integers(0x3C00, 0x4100, size=(50, 2 * H * d), dtype=np.uint16)  # finite bf16 values
    chunks = np.array([(10, 40, 0, 0, FRESH), (3, 5, -60, 40, 0)], dtype=CHUNK_DTYPE)
    w = G.gqa_inv_freq(10000.0, d)
    k, v, gather, delta = G.gqa_rotate_gather(pool, chunks, np.array([0, 2]), H, d, w)
    assert list(gather) == list(range(10, 50)) + list(range(3, 8))
    assert np.array_equal(v, pool[gather][:, H * d:])
    kb = oracle.bf16_to_f64(pool[gather][:, :H * d]).reshape(-1, H, d)
    assert np.array_equal(k[:40], kb[:40])
    for r in range(40, 45):
        for h in range(H):
            x = kb[r, h]
            ang = 100.0 * w
            exp = np.concatenate([x[:4] * np.cos(ang) - x[4:] * np.sin(ang), x[:4] * np.sin(ang) + x[4:] * np.cos(ang)])
            assert np.allclose(k[r, h], exp, rtol=0, atol=1e-12)
