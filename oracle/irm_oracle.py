"""CPU oracle for MLA position-independent KV assembly and absorbed MLA attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module.  It shares
no code with the HIP path (no kernels, headers, helpers or constants) and
imports nothing from it; the product path never falls back to it.

Plain, slow, single-threaded numpy in float64.  bf16 inputs arrive as uint16
bit patterns and are widened exactly to float64; nothing here rounds back to
bf16.  Each function cites the passage of the Irminsul pages (arXiv:2605.05696)
it follows:

* gist.science technical summary (French), sections 2.1-2.2;
* gentlecold.top article, sections 3 (K(p) = R(p) K_content), 4 (MLA row
  split, absorbed form, delta = p_tgt - p_src, R(delta) R(p_src) = R(p_tgt)),
  5 (serve-path pseudocode: segments appended in target order, carve-out for
  p < 32, registry value (c_KV, k_r_base, p_src)), 7 (carve-out) and 15
  (worked example of delta).

Readings of points the pages leave open (RoPE pair layout, theta, scale,
masks, carve-out extent, fresh rows), as used here: interleaved RoPE pairs (2i, 2i+1) with omega_i = theta^(-2i/64),
softmax scale 1/sqrt(192), decode attends to every cached row, tail-prefill
query i attends to rows t <= q_pos0 + i, rows at positions < 32 must come
from fresh entries, and fresh entries have p_src == p_tgt.
"""
from __future__ import annotations

from typing import List, Tuple

import numpy as np

D_LATENT = 512
D_ROPE = 64
ROW = D_LATENT + D_ROPE
CARVE_OUT = 32
FLAG_FRESH = 1
INT32_MAX = 2**31 - 1
INT32_MIN = -(2**31)


class TableError(ValueError):
    """Invalid chunk table; ``code`` is one of EINVAL, ERANGE, ELAYOUT, ECARVEOUT."""

    def __init__(self, code: str, msg: str):
        super().__init__(f"{code}: {msg}")
        self.code = code


# ---------------------------------------------------------------------------
# bf16 widening
# ---------------------------------------------------------------------------
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact float64 values."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# RoPE frequencies and the delta rotation
# ---------------------------------------------------------------------------
def rope_inv_freq(theta: float = 10000.0, rope_dim: int = D_ROPE) -> np.ndarray:
    """omega_i = theta ** (-2 i / rope_dim), i = 0 .. rope_dim/2 - 1 (float64).

    Standard RoPE frequencies; the pages say only that the rotary class and its
    inverse frequencies must match the model (gentlecold.top, section 11)."""
    i = np.arange(rope_dim // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * i / rope_dim)


def rotate(k: np.ndarray, pos, inv_freq: np.ndarray) -> np.ndarray:
    """R(pos) applied to RoPE slices k[..., 64] (float64).

    Pair i is (k[2i], k[2i+1]) and turns by the angle pos * omega_i:
    (x, y) -> (x cos - y sin, x sin + y cos).  ``pos`` is a scalar or an array
    broadcasting against k[..., 0].  K(p) = R(p) K_content (gentlecold.top,
    section 3); the delta rotation is this map with pos = delta (section 4)."""
    k = np.asarray(k, dtype=np.float64)
    pos = np.asarray(pos, dtype=np.float64)
    phi = pos[..., None] * inv_freq                     # [..., 32]
    c, s = np.cos(phi), np.sin(phi)
    x, y = k[..., 0::2], k[..., 1::2]
    xr = x * c - y * s
    yr = x * s + y * c
    return np.stack([xr, yr], axis=-1).reshape(xr.shape[:-1] + (2 * xr.shape[-1],))


def delta_rotate(k_r_base: np.ndarray, delta, inv_freq: np.ndarray) -> np.ndarray:
    """k_r = R(delta) k_r_base with delta = p_tgt - p_src (gist.science summary,
    section 2.2; gentlecold.top, sections 4 and 5).  delta == 0 leaves the
    slice untouched (R(0) is the identity)."""
    k = np.asarray(k_r_base, dtype=np.float64)
    d = np.broadcast_to(np.asarray(delta, dtype=np.int64), k.shape[:-1])
    out = rotate(k, d, inv_freq)
    zero = d == 0
    if np.any(zero):
        out[zero] = k[zero]
    return out


# ---------------------------------------------------------------------------
# chunk table
# ---------------------------------------------------------------------------
def expand_table(chunks: np.ndarray, seq_first: np.ndarray, pool_rows: int
                 ) -> List[Tuple[np.ndarray, np.ndarray, np.ndarray]]:
    """Validate a chunk table and expand it row by row.

    The serve path appends segments in target order; every token j of a
    segment placed at p_tgt moves by the same delta = p_tgt - p_src
    (gentlecold.top, section 5 pseudocode; section 15 worked example).
    Positions below 32 are never served from the registry (gist.science
    summary, section 2.2; gentlecold.top, section 7).

    Returns, per sequence, (pool row per output row [int64], delta per output
    row [int64], fresh flag per output row [bool]); output row r of a sequence
    is absolute position r.  Raises TableError on the first violation, checking
    entries in order: flags, len, pool range, target contiguity, position
    range, fresh p_src, carve-out, delta range."""
    chunks = np.asarray(chunks)
    seq_first = np.asarray(seq_first, dtype=np.int64)
    n = chunks.shape[0]
    if seq_first.ndim != 1 or seq_first.shape[0] < 1:
        raise TableError("EINVAL", "seq_first needs n_seq + 1 entries")
    if seq_first[0] != 0 or seq_first[-1] != n or np.any(np.diff(seq_first) < 0):
        raise TableError("EINVAL", "seq_first must run from 0 to n_chunks, nondecreasing")
    out = []
    total = 0
    for s in range(seq_first.shape[0] - 1):
        gathers, deltas, freshes = [], [], []
        expect = 0
        for e in range(int(seq_first[s]), int(seq_first[s + 1])):
            pool_row = int(chunks["pool_row"][e])
            ln = int(chunks["len"][e])
            p_src = int(chunks["p_src"][e])
            p_tgt = int(chunks["p_tgt"][e])
            flags = int(chunks["flags"][e])
            if flags & ~FLAG_FRESH:
                raise TableError("EINVAL", f"entry {e}: unknown flag bits")
            if ln == 0:
                raise TableError("EINVAL", f"entry {e}: zero length")
            if pool_row + ln > pool_rows:
                raise TableError("ERANGE", f"entry {e}: pool rows out of range")
            if p_tgt != expect:
                raise TableError("ELAYOUT", f"entry {e}: p_tgt {p_tgt} != {expect}")
            if p_tgt + ln - 1 > INT32_MAX:
                raise TableError("ERANGE", f"entry {e}: positions exceed int32")
            fresh = bool(flags & FLAG_FRESH)
            if fresh and p_src != p_tgt:
                raise TableError("EINVAL", f"entry {e}: fresh entry with p_src != p_tgt")
            if not fresh and p_tgt < CARVE_OUT:
                raise TableError("ECARVEOUT", f"entry {e}: registry rows below position {CARVE_OUT}")
            delta = p_tgt - p_src
            if delta > INT32_MAX or delta < INT32_MIN:
                raise TableError("ERANGE", f"entry {e}: delta exceeds int32")
            gathers.append(pool_row + np.arange(ln, dtype=np.int64))
            deltas.append(np.full(ln, 0 if fresh else delta, dtype=np.int64))
            freshes.append(np.full(ln, fresh, dtype=bool))
            expect = p_tgt + ln
        total += expect
        if total > INT32_MAX:
            raise TableError("ERANGE", "total assembled rows exceed int32")
        if gathers:
            out.append((np.concatenate(gathers), np.concatenate(deltas), np.concatenate(freshes)))
        else:
            out.append((np.zeros(0, np.int64), np.zeros(0, np.int64), np.zeros(0, bool)))
    return out


# ---------------------------------------------------------------------------
# rotate-gather
# ---------------------------------------------------------------------------
def assemble_rows(pool_bits: np.ndarray, gather: np.ndarray, delta: np.ndarray,
                  inv_freq: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Assembled KV rows for the given gather rows and deltas: c_KV is the
    stored latent unchanged (position free; gist.science summary, section 2.1)
    and k_r = R(delta) k_r_base (gentlecold.top, section 4).  Returns
    (c_kv [n][512], k_r [n][64]) in float64."""
    rows = pool_bits[np.asarray(gather, dtype=np.int64)]
    c_kv = bf16_to_f64(rows[:, :D_LATENT])
    k_r = delta_rotate(bf16_to_f64(rows[:, D_LATENT:]), delta, inv_freq)
    return c_kv, k_r


def rotate_gather(pool_bits: np.ndarray, chunks: np.ndarray, seq_first: np.ndarray,
                  inv_freq: np.ndarray) -> List[Tuple[np.ndarray, np.ndarray]]:
    """Assemble every sequence of the table: the ordered concatenation of
    segments of the serve-path pseudocode (gentlecold.top, section 5)."""
    out = []
    for gather, delta, _fresh in expand_table(chunks, seq_first, pool_bits.shape[0]):
        out.append(assemble_rows(pool_bits, gather, delta, inv_freq))
    return out


# ---------------------------------------------------------------------------
# absorbed MLA attention
# ---------------------------------------------------------------------------
def _softmax_attend(scores: np.ndarray, values: np.ndarray) -> Tuple[np.ndarray, float]:
    """Two-pass softmax: m = max, p = exp(s - m), o = sum p v / sum p,
    lse = m + ln sum p."""
    m = np.max(scores)
    p = np.exp(scores - m)
    l = np.sum(p)
    return (p @ values) / l, float(m + np.log(l))


def mla_decode(q_lat: np.ndarray, q_rope: np.ndarray, c_kv: np.ndarray, k_r: np.ndarray,
               scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """One decode query per head over an assembled cache of N rows.

    Absorbed MLA: the key is [W_UK c_KV, k_r] with W_UK folded into the query,
    so the score of row t is q_lat . c_KV[t] + q_rope . k_r[t] and the value is
    c_KV[t] itself (gentlecold.top, section 4).  The query attends to all N rows.

    q_lat [H][512], q_rope [H][64], c_kv [N][512], k_r [N][64] (float64).
    Returns (o [H][512], lse [H])."""
    H = q_lat.shape[0]
    o = np.empty((H, D_LATENT), dtype=np.float64)
    lse = np.empty(H, dtype=np.float64)
    for h in range(H):
        s = scale * (c_kv @ q_lat[h] + k_r @ q_rope[h])
        o[h], lse[h] = _softmax_attend(s, c_kv)
    return o, lse


def mla_prefill_tail(q_lat: np.ndarray, q_rope: np.ndarray, c_kv: np.ndarray, k_r: np.ndarray,
                     q_pos0: int, scale: float, query_ids=None) -> Tuple[np.ndarray, np.ndarray]:
    """Chunked tail-prefill: query i sits at absolute position q_pos0 + i and
    attends to rows t <= q_pos0 + i of the assembled cache, with the absorbed
    score and value of ``mla_decode``.

    q_lat [Nq][H][512], q_rope [Nq][H][64]; ``query_ids`` optionally selects a
    subset of queries.  Returns (o [n][H][512], lse [n][H])."""
    ids = np.arange(q_lat.shape[0]) if query_ids is None else np.asarray(query_ids)
    H = q_lat.shape[1]
    o = np.empty((len(ids), H, D_LATENT), dtype=np.float64)
    lse = np.empty((len(ids), H), dtype=np.float64)
    for n, i in enumerate(ids):
        lim = int(q_pos0) + int(i) + 1
        o[n], lse[n] = mla_decode(q_lat[i], q_rope[i], c_kv[:lim], k_r[:lim], scale)
    return o, lse
