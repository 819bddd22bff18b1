"""CPU oracle for the GQA/MHA comparison path: position-independent reuse of a
grouped-query KV cache, where the whole key of every KV head is rotated.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  It shares
no code with the library and imports nothing from it.

What the pages fix (gist.science summary, section 1; gentlecold.top article,
sections 3 and 4): in GQA/MHA the position is folded into the full key,
K(p) = R(p) K_content over all d_K dimensions of every KV head, so earlier
position-independent caching systems correct the full key of each reused
token, an O(N d_K) correction per KV head, while MLA corrects only the
64-wide k_r slice (O(64 N)); values carry no position and are reused as
they are.  The same delta rotation applies: R(p_tgt - p_src) R(p_src) =
R(p_tgt).

Readings where the pages are silent: a row is
[K of n_kv_heads heads | V of n_kv_heads heads], each head head_dim wide, bf16;
the rotation covers the whole head_dim with the half-split pairing of
GQA models (element i turns with element i + head_dim/2, frequency
omega_i = theta^(-2i/head_dim)); the chunk table, its validation and the
per-entry delta are those of the MLA path.
"""
from __future__ import annotations

import numpy as np

from .irm_oracle import bf16_to_f64, expand_table


def gqa_inv_freq(theta: float, head_dim: int) -> np.ndarray:
    """omega_i = theta^(-2i/head_dim), i < head_dim/2, float64."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return theta ** (-2.0 * i / head_dim)


def rotate_half_split(k: np.ndarray, pos, inv_freq: np.ndarray) -> np.ndarray:
    """R(pos) on the last axis (head_dim): (x_i, x_{i+h}) -> (x_i cos - x_{i+h}
    sin, x_i sin + x_{i+h} cos), angle pos * omega_i, h = head_dim / 2.
    pos broadcasts to k's leading axes (k.shape[:-1])."""
    k = np.asarray(k, dtype=np.float64)
    h = k.shape[-1] // 2
    ang = np.broadcast_to(np.asarray(pos, dtype=np.float64), k.shape[:-1])[..., None] * inv_freq
    c, s = np.cos(ang), np.sin(ang)
    x, y = k[..., :h], k[..., h:]
    return np.concatenate([x * c - y * s, x * s + y * c], axis=-1)


def gqa_rotate_gather(pool_bits: np.ndarray, chunks: np.ndarray, seq_first: np.ndarray, n_kv_heads: int,
                      head_dim: int, inv_freq: np.ndarray):
    """Assembled GQA rows of every sequence of a chunk table: K as exact
    float64 values [rows][n_kv_heads][head_dim] (rotated by the entry's delta,
    unrotated for fresh / delta-0 rows), V as the pool's bf16 bits."""
    width = 2 * n_kv_heads * head_dim
    assert pool_bits.shape[1] == width
    exp = expand_table(chunks, seq_first, pool_bits.shape[0])
    gather = np.concatenate([g for g, _, _ in exp]) if exp else np.zeros(0, np.int64)
    delta = np.concatenate([d for _, d, _ in exp]) if exp else np.zeros(0, np.int64)
    rows = pool_bits[gather]
    kd = n_kv_heads * head_dim
    k = bf16_to_f64(rows[:, :kd]).reshape(-1, n_kv_heads, head_dim)
    k_rot = rotate_half_split(k, delta[:, None], inv_freq)
    return k_rot, rows[:, kd:], gather, delta
