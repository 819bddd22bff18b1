"""Seeded synthetic workloads for the MLA position-independent KV path.

The shapes follow the Irminsul pages (arXiv:2605.05696):

* a KV row is a 512-wide position-free latent c_KV followed by a 64-wide RoPE
  key slice k_r (gist.science summary, section 2.1; gentlecold.top article,
  section 4), stored here as 576 bf16 values;
* registry chunks come from content-defined chunking with lengths clamped to
  [32, 512] and an expected length near 128 (gentlecold.top, section 6);
* the first 32 absolute positions are always freshly prefilled (gist.science
  summary, section 2.2; gentlecold.top, section 7);
* an exact prefix precedes the position-independent tail (gentlecold.top,
  section 5).

No trained weights, traces or datasets exist here, so every value is drawn
from N(0, 1) and rounded to bf16.  The pool stores the registered RoPE slice
k_r_base directly as an N(0, 1) vector: a RoPE rotation is orthogonal, so an
isotropic Gaussian pre-RoPE key rotated to any p_src is again an isotropic
Gaussian, and drawing k_r_base directly gives the same distribution without
putting any of the method's arithmetic in this module.

A chunk-table entry is (pool_row, len, p_src, p_tgt, flags); entries of a
sequence are listed in target order and ``seq_first[s]:seq_first[s+1]``
selects sequence s.  Pool rows are handed out in a random permutation of the
chunks so that an identity gather cannot pass a test by accident.
"""
from __future__ import annotations

import hashlib
from dataclasses import dataclass, field
from typing import Callable, Dict, List, Optional, Tuple

import numpy as np

D_LATENT = 512
D_ROPE = 64
ROW = D_LATENT + D_ROPE
FRESH = 1
CARVE_OUT = 32

CHUNK_DTYPE = np.dtype(
    [("pool_row", "<u4"), ("len", "<u4"), ("p_src", "<i4"), ("p_tgt", "<i4"), ("flags", "<u4")]
)


# --------------------------------------------------------------------------
# bf16 encoding of random samples (round to nearest, ties to even)
# --------------------------------------------------------------------------
def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = u + np.uint32(0x7FFF) + lsb
    return (r >> np.uint32(16)).astype(np.uint16)


def randn_bf16(rng: np.random.Generator, shape, block_rows: int = 1 << 16) -> np.ndarray:
    """N(0,1) samples rounded to bf16, drawn in row blocks to bound memory."""
    shape = tuple(int(s) for s in shape)
    out = np.empty(shape, dtype=np.uint16)
    if out.size == 0:
        return out
    flat = out.reshape(shape[0], -1)
    for r0 in range(0, shape[0], block_rows):
        r1 = min(shape[0], r0 + block_rows)
        flat[r0:r1] = bf16_bits_from_f32(rng.standard_normal((r1 - r0, flat.shape[1]), dtype=np.float32))
    return out


# --------------------------------------------------------------------------
# workload container
# --------------------------------------------------------------------------
@dataclass
class Workload:
    name: str
    pool: np.ndarray                 # uint16 bf16 bits [n_rows][576]
    chunks: np.ndarray               # CHUNK_DTYPE [n_chunks]
    seq_first: np.ndarray            # uint32 [n_seq + 1]
    n_heads: int = 0
    q_lat: Optional[np.ndarray] = None   # uint16 [B or Nq][H][512]
    q_rope: Optional[np.ndarray] = None  # uint16 [B or Nq][H][64]
    q_pos0: int = -1                 # tail-prefill: absolute position of query 0
    n_splits: int = 0                # decode: split count used by the bench (0 = library choice)
    theta: float = 10000.0
    scale: float = 1.0 / np.sqrt(192.0)
    kind: str = "gather"             # "gather" | "decode" | "prefill"
    meta: Dict[str, object] = field(default_factory=dict)

    @property
    def n_seq(self) -> int:
        return int(self.seq_first.shape[0] - 1)

    def seq_len(self, s: int) -> int:
        c = self.chunks[int(self.seq_first[s]):int(self.seq_first[s + 1])]
        return int(c["len"].astype(np.int64).sum())

    @property
    def total_rows(self) -> int:
        return int(self.chunks["len"].astype(np.int64).sum())


def manifest(w: Workload) -> Dict[str, str]:
    """SHA-256 of every array of a workload (same bytes on both sides)."""
    out = {}
    for k in ("pool", "chunks", "seq_first", "q_lat", "q_rope"):
        a = getattr(w, k)
        if a is not None:
            out[k] = hashlib.sha256(np.ascontiguousarray(a).tobytes()).hexdigest()
    return out


# --------------------------------------------------------------------------
# table layout helpers
# --------------------------------------------------------------------------
def _uniform_len(rng: np.random.Generator) -> int:
    return int(rng.integers(32, 513))


def _cdc_like_len(rng: np.random.Generator) -> int:
    # memoryless boundary after a 32-token minimum, clamped at 512 (mean ~127)
    return int(min(512, 32 + rng.geometric(1.0 / 96.0) - 1))


class _Layout:
    """Collects sequences of (kind, len, p_src, p_tgt) entries, then assigns
    pool rows to distinct chunks in a random permutation."""

    def __init__(self):
        self.seqs: List[List[Tuple[str, int, int, int]]] = []

    def add_sequence(self, entries: List[Tuple[str, int, int, int]]):
        self.seqs.append(entries)

    def finish(self, rng: np.random.Generator) -> Tuple[np.ndarray, np.ndarray, int]:
        flat = [e for s in self.seqs for e in s]
        n = len(flat)
        lens = np.array([e[1] for e in flat], dtype=np.int64)
        order = rng.permutation(n)
        start = np.zeros(n, dtype=np.int64)
        off = 0
        for idx in order:
            start[idx] = off
            off += lens[idx]
        chunks = np.zeros(n, dtype=CHUNK_DTYPE)
        for i, (kind, ln, p_src, p_tgt) in enumerate(flat):
            chunks[i] = (start[i], ln, p_src, p_tgt, FRESH if kind == "fresh" else 0)
        seq_first = np.zeros(len(self.seqs) + 1, dtype=np.uint32)
        seq_first[1:] = np.cumsum([len(s) for s in self.seqs])
        return chunks, seq_first, int(off)


def _decode_sequence(rng, seq_len: int, prefix_end: int, p_hit: float,
                     len_fn: Callable, delta_abs: int) -> List[Tuple[str, int, int, int]]:
    """Fresh rows [0,32), an optional exact prefix [32,prefix_end) with delta 0,
    then registry hits (probability p_hit, delta uniform in [-delta_abs, delta_abs])
    and fresh chunks; the last entry is truncated to fit seq_len."""
    ents = [("fresh", min(CARVE_OUT, seq_len), 0, 0)]
    pos = ents[0][1]
    if prefix_end > pos:
        ents.append(("prefix", prefix_end - pos, pos, pos))
        pos = prefix_end
    while pos < seq_len:
        ln = min(len_fn(rng), seq_len - pos)
        if rng.random() < p_hit:
            delta = int(rng.integers(-delta_abs, delta_abs + 1))
            ents.append(("hit", ln, pos - delta, pos))
        else:
            ents.append(("fresh", ln, pos, pos))
        pos += ln
    return ents


def _queries(rng, n: int, h: int) -> Tuple[np.ndarray, np.ndarray]:
    q_lat = randn_bf16(rng, (n, h, D_LATENT))
    q_rope = randn_bf16(rng, (n, h, D_ROPE))
    return q_lat, q_rope


def nonabsorbed_inputs(seed: int, n_q: int, heads: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Random up-projection weights and nope queries of the non-absorbed MLA
    prefill (no trained weights): q_nope [n_q][H][128] N(0,1), W_UK and W_UV
    [H][128][512] N(0, 1/512) (so that W c_KV is about unit scale for N(0,1)
    latents), all rounded to bf16."""
    rng = np.random.default_rng(seed)
    q_nope = randn_bf16(rng, (n_q, heads, 128))
    w = rng.standard_normal((2, heads, 128, D_LATENT), dtype=np.float32) * np.float32(1.0 / np.sqrt(D_LATENT))
    w_bits = bf16_bits_from_f32(w)
    return q_nope, w_bits[0], w_bits[1]


# --------------------------------------------------------------------------
# the five workloads of the hot path
# --------------------------------------------------------------------------
def tiny_decode(seed: int = 1001) -> Workload:
    """1 sequence, 16 heads, 1024 tokens in 8 chunks of 128: chunk 0 fresh at
    positions 0..127 (covers the 0..31 carve-out), chunks 1..7 registry hits with
    p_src uniform in [0, 16384] and p_tgt contiguous after chunk 0."""
    rng = np.random.default_rng(seed)
    lay = _Layout()
    ents = [("fresh", 128, 0, 0)]
    for k in range(1, 8):
        ents.append(("hit", 128, int(rng.integers(0, 16385)), 128 * k))
    lay.add_sequence(ents)
    chunks, seq_first, n_rows = lay.finish(rng)
    pool = randn_bf16(rng, (n_rows, ROW))
    q_lat, q_rope = _queries(rng, 1, 16)
    return Workload("tiny_decode_h16_n1024", pool, chunks, seq_first, n_heads=16,
                    q_lat=q_lat, q_rope=q_rope, n_splits=4, kind="decode")


def rotate_gather_batch(seed: int = 1002, n_req: int = 64, req_len: int = 32768,
                        n_registry: int = 4096, len_fn: Callable = _uniform_len,
                        p_hit: float = 0.8, p_src_max: int = 131072) -> Workload:
    """A registry of ``n_registry`` chunks (lengths from ``len_fn``, p_src uniform
    in [0, p_src_max]) at permuted pool slots, plus one fresh region per request.
    Each request assembles ``req_len`` tokens: a fresh first chunk (>= 32 rows),
    then hits drawn uniformly from the registry with probability ``p_hit`` and
    fresh chunks otherwise; the last entry is truncated to fit."""
    rng = np.random.default_rng(seed)
    reg_len = np.array([len_fn(rng) for _ in range(n_registry)], dtype=np.int64)
    reg_psrc = rng.integers(0, p_src_max + 1, size=n_registry)
    order = rng.permutation(n_registry)
    reg_row = np.zeros(n_registry, dtype=np.int64)
    off = 0
    for idx in order:
        reg_row[idx] = off
        off += reg_len[idx]
    rows: List[Tuple[int, int, int, int, int]] = []
    seq_first = [0]
    for _ in range(n_req):
        pos = 0
        first = True
        while pos < req_len:
            if first or rng.random() >= p_hit:
                ln = min(max(len_fn(rng), CARVE_OUT if first else 1), req_len - pos)
                rows.append((off, ln, pos, pos, FRESH))
                off += ln
                first = False
            else:
                c = int(rng.integers(0, n_registry))
                ln = int(min(reg_len[c], req_len - pos))
                rows.append((int(reg_row[c]), ln, int(reg_psrc[c]), pos, 0))
            pos += ln
        seq_first.append(len(rows))
    chunks = np.array(rows, dtype=CHUNK_DTYPE)
    pool = randn_bf16(rng, (off, ROW))
    return Workload(f"rotate_gather_{n_req}x{req_len}", pool, chunks,
                    np.array(seq_first, dtype=np.uint32), kind="gather",
                    meta={"n_registry": n_registry, "registry_rows": int(reg_len.sum())})


def rotate_gather_cdc_batch(seed: int = 1012, n_req: int = 64, req_len: int = 32768,
                            n_registry: int = 4096) -> Workload:
    """The rotate-gather batch with CDC-like chunk lengths instead of uniform
    ones: 32 plus a geometric tail (a memoryless content-defined boundary after
    the 32-token minimum), clamped at 512, mean about 127 -- the chunk size the
    pages' CDC targets.  About twice as many entries per request as the
    uniform [32, 512] law (mean 272), so the per-entry work weighs more."""
    w = rotate_gather_batch(seed=seed, n_req=n_req, req_len=req_len, n_registry=n_registry,
                            len_fn=_cdc_like_len)
    w.name = f"rotate_gather_cdc_{n_req}x{req_len}"
    w.meta["chunk_len"] = "32 + Geometric(1/96) - 1, at most 512 (mean ~127)"
    return w


def batched_decode(seed: int = 1003, batch: int = 64, ctx: int = 8192, heads: int = 16,
                   n_splits: int = 0) -> Workload:
    """Per sequence: about 1/3 exact prefix (delta 0, rows 0..31 fresh), then
    registry hits with probability 0.75 (lengths uniform in [32,512], delta
    uniform in [-65536, 65536]) and fresh chunks.  Every hit is a distinct pool
    chunk, so each KV row is read from HBM once."""
    rng = np.random.default_rng(seed)
    lay = _Layout()
    prefix_end = int(round(ctx / 3))
    for _ in range(batch):
        lay.add_sequence(_decode_sequence(rng, ctx, prefix_end, 0.75, _uniform_len, 65536))
    chunks, seq_first, n_rows = lay.finish(rng)
    pool = randn_bf16(rng, (n_rows, ROW))
    q_lat, q_rope = _queries(rng, batch, heads)
    return Workload(f"batched_decode_b{batch}_n{ctx}_h{heads}", pool, chunks, seq_first,
                    n_heads=heads, q_lat=q_lat, q_rope=q_rope, n_splits=n_splits, kind="decode")


def long_decode(seed: int = 1004, batch: int = 32, ctx: int = 32768, heads: int = 128,
                n_splits: int = 16) -> Workload:
    """Rows 0..31 fresh, then registry hits with probability 0.9 (CDC-like
    lengths, mean ~128, delta uniform in [-131072, 131072]) and fresh chunks."""
    rng = np.random.default_rng(seed)
    lay = _Layout()
    for _ in range(batch):
        lay.add_sequence(_decode_sequence(rng, ctx, 0, 0.9, _cdc_like_len, 131072))
    chunks, seq_first, n_rows = lay.finish(rng)
    pool = randn_bf16(rng, (n_rows, ROW))
    q_lat, q_rope = _queries(rng, batch, heads)
    return Workload(f"long_decode_b{batch}_n{ctx}_h{heads}", pool, chunks, seq_first,
                    n_heads=heads, q_lat=q_lat, q_rope=q_rope, n_splits=n_splits, kind="decode")


def tail_prefill(seed: int = 1005, n_q: int = 4096, prefix_end: int = 16384,
                 hits_end: int = 57344, total: int = 65536, heads: int = 16,
                 delta_abs: int = 65536) -> Workload:
    """One sequence: rows 0..31 fresh, an exact prefix up to ``prefix_end``,
    registry hits (lengths uniform in [32,512], delta uniform in
    [-delta_abs, delta_abs]) up to ``hits_end``, then fresh rows: the previous
    tail chunk and the current tail's own ``n_q`` rows.  Queries sit at the
    last ``n_q`` positions."""
    rng = np.random.default_rng(seed)
    lay = _Layout()
    ents = [("fresh", CARVE_OUT, 0, 0)]
    if prefix_end > CARVE_OUT:
        ents.append(("prefix", prefix_end - CARVE_OUT, CARVE_OUT, CARVE_OUT))
    pos = max(prefix_end, CARVE_OUT)
    while pos < hits_end:
        ln = min(_uniform_len(rng), hits_end - pos)
        delta = int(rng.integers(-delta_abs, delta_abs + 1))
        ents.append(("hit", ln, pos - delta, pos))
        pos += ln
    q_pos0 = total - n_q
    if q_pos0 > pos:
        ents.append(("fresh", q_pos0 - pos, pos, pos))
    ents.append(("fresh", n_q, q_pos0, q_pos0))
    lay.add_sequence(ents)
    chunks, seq_first, n_rows = lay.finish(rng)
    pool = randn_bf16(rng, (n_rows, ROW))
    q_lat, q_rope = _queries(rng, n_q, heads)
    return Workload(f"tail_prefill_q{n_q}_kv{total}_h{heads}", pool, chunks, seq_first,
                    n_heads=heads, q_lat=q_lat, q_rope=q_rope, q_pos0=q_pos0, kind="prefill")


def random_table(seed: int, seq_lens: List[int], heads: int = 16, p_hit: float = 0.6,
                 prefix_frac: float = 0.0, delta_abs: int = 131072,
                 len_fn: Callable = _uniform_len, n_q: int = 0,
                 kind: str = "decode") -> Workload:
    """Small ragged workload for parity tests: one sequence per entry of
    ``seq_lens`` (each >= 1), mixing fresh, exact-prefix and hit entries.  For
    ``kind == 'prefill'`` only one sequence is allowed and the last ``n_q``
    positions carry queries."""
    rng = np.random.default_rng(seed)
    lay = _Layout()
    for L in seq_lens:
        pe = int(L * prefix_frac)
        lay.add_sequence(_decode_sequence(rng, L, pe, p_hit, len_fn, delta_abs))
    chunks, seq_first, n_rows = lay.finish(rng)
    pool = randn_bf16(rng, (n_rows, ROW))
    if kind == "prefill":
        assert len(seq_lens) == 1 and 1 <= n_q <= seq_lens[0]
        q_lat, q_rope = _queries(rng, n_q, heads)
        return Workload(f"random_prefill_{seed}", pool, chunks, seq_first, n_heads=heads,
                        q_lat=q_lat, q_rope=q_rope, q_pos0=seq_lens[0] - n_q, kind="prefill")
    q_lat, q_rope = _queries(rng, len(seq_lens), heads)
    return Workload(f"random_{kind}_{seed}", pool, chunks, seq_first, n_heads=heads,
                    q_lat=q_lat, q_rope=q_rope, kind=kind)


def token_requests(seed: int = 1006, n_req: int = 64, req_len: int = 32768, n_docs: int = 256,
                   doc_len: Tuple[int, int] = (1024, 8192), p_doc: float = 0.8,
                   fresh_len: Tuple[int, int] = (64, 2048), vocab: int = 128000,
                   library_seed: int = 2006) -> List[np.ndarray]:
    """Token streams for the chunk-table producer: each request concatenates
    segments until ``req_len`` tokens, a whole shared document (drawn from a
    library of ``n_docs`` documents with lengths uniform in ``doc_len``) with
    probability ``p_doc``, else fresh tokens (lengths uniform in
    ``fresh_len``); the last segment is truncated.  Token ids are uniform in
    [0, vocab).  The library depends only on ``library_seed``, so batches with
    different ``seed`` share documents at shifted offsets (the agentic reuse
    pattern the pages describe)."""
    lib_rng = np.random.default_rng(library_seed)
    docs = [lib_rng.integers(0, vocab, size=int(lib_rng.integers(doc_len[0], doc_len[1] + 1)), dtype=np.int32)
            for _ in range(n_docs)]
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n_req):
        parts, n = [], 0
        while n < req_len:
            if rng.random() < p_doc:
                seg = docs[int(rng.integers(0, n_docs))]
            else:
                seg = rng.integers(0, vocab, size=int(rng.integers(fresh_len[0], fresh_len[1] + 1)), dtype=np.int32)
            seg = seg[:req_len - n]
            parts.append(seg)
            n += seg.size
        out.append(np.concatenate(parts).astype(np.int32))
    return out


WORKLOADS = {
    "tiny_decode": tiny_decode,
    "rotate_gather": rotate_gather_batch,
    "rotate_gather_cdc": rotate_gather_cdc_batch,
    "batched_decode": batched_decode,
    "long_decode": long_decode,
    "tail_prefill": tail_prefill,
}


def make_workload(name: str, **kw) -> Workload:
    return WORKLOADS[name](**kw)
