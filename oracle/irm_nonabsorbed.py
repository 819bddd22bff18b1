"""CPU oracle for the non-absorbed MLA prefill: the latent rows are up-projected
to a full key and value per head before attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  It shares
no code with the library and imports nothing from it.

What the pages fix (gentlecold.top article, section 4, MLA structure; section
13, where a non-absorbed MLA model still has to up-project c_KV into the full
key at run time): the key of row t for head h is [W_UK[h] c_KV[t], k_r[t]],
the value is derived from c_KV alone, and only k_r carries the position, so
the rotated k_r of the assembled cache is used as it is.

Readings where the pages are silent: W_UK[h] and W_UV[h]
are [128][512] per head (output feature, latent input), the nope part of the
key and the value are both 128 wide, the query is [q_nope 128 | q_rope 64]
per head, the score scale is 1/sqrt(192), and the causal mask is the one of
the absorbed tail-prefill (query i at q_pos0 + i sees rows t <= q_pos0 + i).
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

D_NOPE = 128
D_V = 128


def up_project(c_kv: np.ndarray, w_uk: np.ndarray, w_uv: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """k_nope[t][h] = W_UK[h] c_KV[t], v[t][h] = W_UV[h] c_KV[t] (float64).
    c_kv [N][512], w_uk / w_uv [H][128][512].  Returns ([N][H][128], [N][H][128])."""
    c = np.asarray(c_kv, dtype=np.float64)
    k = np.matmul(c, np.asarray(w_uk, dtype=np.float64).transpose(0, 2, 1))   # [H][N][128]
    v = np.matmul(c, np.asarray(w_uv, dtype=np.float64).transpose(0, 2, 1))
    return np.ascontiguousarray(k.transpose(1, 0, 2)), np.ascontiguousarray(v.transpose(1, 0, 2))


def _attend(s: np.ndarray, values: np.ndarray) -> Tuple[np.ndarray, float]:
    """Two-pass softmax: m = max s, p = exp(s - m), o = sum p v / sum p,
    lse = m + ln sum p (natural log)."""
    m = np.max(s)
    p = np.exp(s - m)
    z = np.sum(p)
    return (p @ values) / z, float(m + np.log(z))


def mla_prefill_nonabsorbed(q_nope: np.ndarray, q_rope: np.ndarray, c_kv: np.ndarray, k_r: np.ndarray,
                            w_uk: np.ndarray, w_uv: np.ndarray, q_pos0: int, scale: float,
                            query_ids=None) -> Tuple[np.ndarray, np.ndarray]:
    """Causal prefill of queries at q_pos0 + i over an assembled cache, with
    the key and value of every head up-projected from c_KV.

    q_nope [Nq][H][128], q_rope [Nq][H][64], c_kv [N][512], k_r [N][64] (the
    rotated slice of the assembled rows).  ``query_ids`` optionally selects a
    subset of queries.  Returns (o [n][H][128], lse [n][H])."""
    k_nope, v = up_project(c_kv, w_uk, w_uv)
    kr = np.asarray(k_r, dtype=np.float64)
    ids = np.arange(q_nope.shape[0]) if query_ids is None else np.asarray(query_ids)
    H = q_nope.shape[1]
    o = np.empty((len(ids), H, D_V), dtype=np.float64)
    lse = np.empty((len(ids), H), dtype=np.float64)
    for n, i in enumerate(ids):
        lim = int(q_pos0) + int(i) + 1
        for h in range(H):
            s = scale * (k_nope[:lim, h] @ np.asarray(q_nope[i, h], np.float64)
                         + kr[:lim] @ np.asarray(q_rope[i, h], np.float64))
            o[n, h], lse[n, h] = _attend(s, v[:lim, h])
    return o, lse
