"""Python binding of libirm (MLA position-independent KV path on MI355X).

Thin ctypes marshalling over the C ABI in include/irm.h: every step of the
path runs in the HIP kernels of libirm.so.  torch is used only for device
memory and streams.  Importing this package does not load the library;
the first call does, and raises if libirm.so has not been built.
"""
from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libirm.so")

D_LATENT = 512
D_ROPE = 64
ROW = 576
CARVE_OUT = 32
FRESH = 1
DEFAULT_SCALE = 1.0 / math.sqrt(192.0)

STATUS = {0: "OK", 1: "EINVAL", 2: "ERANGE", 3: "ELAYOUT", 4: "ECARVEOUT",
          5: "EWORKSPACE", 6: "EUNSUPPORTED", 7: "EHIP"}

CHUNK_DTYPE = np.dtype(
    [("pool_row", "<u4"), ("len", "<u4"), ("p_src", "<i4"), ("p_tgt", "<i4"), ("flags", "<u4")]
)

EXPORTS = (
    "irm_last_error", "irm_rope_inv_freq", "irm_rope_inv_freq_dim", "irm_table_create", "irm_table_destroy",
    "irm_table_info", "irm_table_gather_stats", "irm_table_seq_base", "irm_table_expand_host", "irm_table_upload",
    "irm_table_set_rope", "irm_table_prepare",
    "irm_table_gather_index", "irm_rotate_gather", "irm_mla_decode_workspace",
    "irm_mla_decode", "irm_mla_decode_noalloc", "irm_mla_prefill_tail", "irm_mla_prefill_assembled", "irm_gqa_workspace",
    "irm_gqa_rotate_gather", "irm_mla_kv_upproj", "irm_mla_prefill_nonabsorbed",
    "irm_cdc_params_default", "irm_cdc_split", "irm_xxh64", "irm_registry_create",
    "irm_registry_destroy", "irm_registry_info", "irm_registry_assemble",
)


class CdcParams(ctypes.Structure):
    """irm_cdc_params: Gear seed, mask bits, chunk length bounds."""
    _fields_ = [("seed", ctypes.c_uint64), ("mask_bits", ctypes.c_uint32), ("min_len", ctypes.c_uint32),
                ("max_len", ctypes.c_uint32), ("fallback_window", ctypes.c_uint32)]


class IrmError(RuntimeError):
    def __init__(self, status: int, fn: str, msg: str):
        self.status = status
        self.code = STATUS.get(status, str(status))
        super().__init__(f"{fn}: {self.code}: {msg}")


_lib = None


def lib() -> ctypes.CDLL:
    """Load libirm.so (built in-tree by _build.build()); raise if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                           "python mla_position_independent_amd/_build.py")
    L = ctypes.CDLL(LIB_PATH)
    vp, u32, u64, i32, sz = ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_int32, ctypes.c_size_t
    P = ctypes.POINTER
    sig = {
        "irm_last_error": (ctypes.c_char_p, []),
        "irm_rope_inv_freq": (ctypes.c_int, [ctypes.c_double, vp]),
        "irm_rope_inv_freq_dim": (ctypes.c_int, [ctypes.c_double, u32, vp]),
        "irm_table_create": (ctypes.c_int, [vp, u32, vp, u32, u64, P(vp)]),
        "irm_table_destroy": (ctypes.c_int, [vp]),
        "irm_table_info": (ctypes.c_int, [vp, P(u32), P(u32), P(u64), P(u32), P(sz)]),
        "irm_table_gather_stats": (ctypes.c_int, [vp, P(u32), P(u64), P(u64), P(sz)]),
        "irm_table_seq_base": (ctypes.c_int, [vp, vp]),
        "irm_table_expand_host": (ctypes.c_int, [vp, vp, vp, vp]),
        "irm_table_upload": (ctypes.c_int, [vp, vp, vp, sz, vp]),
        "irm_table_set_rope": (ctypes.c_int, [vp, vp, vp]),
        "irm_table_prepare": (ctypes.c_int, [vp, vp, vp]),
        "irm_table_gather_index": (ctypes.c_int, [vp, vp, vp, vp]),
        "irm_rotate_gather": (ctypes.c_int, [vp, vp, u64, vp, vp, vp]),
        "irm_mla_decode_workspace": (ctypes.c_int, [vp, u32, u32, P(sz)]),
        "irm_mla_decode": (ctypes.c_int, [vp, vp, vp, vp, u64, u32, u32, ctypes.c_float, vp, vp, vp, sz, vp]),
        "irm_mla_decode_noalloc": (ctypes.c_int, [vp, vp, vp, vp, u64, u32, u32, ctypes.c_float, vp, vp, vp]),
        "irm_mla_prefill_tail": (ctypes.c_int, [vp, vp, i32, u32, vp, vp, u64, u32, ctypes.c_float, vp, vp, vp]),
        "irm_mla_prefill_assembled": (ctypes.c_int, [vp, vp, i32, u32, vp, u64, u32, ctypes.c_float, vp, vp, vp]),
        "irm_gqa_workspace": (ctypes.c_int, [vp, u32, P(sz)]),
        "irm_mla_kv_upproj": (ctypes.c_int, [vp, u64, vp, vp, u32, vp, vp]),
        "irm_mla_prefill_nonabsorbed": (ctypes.c_int, [vp, vp, i32, u32, vp, vp, u64, u32, ctypes.c_float, vp, vp,
                                                       vp]),
        "irm_gqa_rotate_gather": (ctypes.c_int, [vp, vp, u64, u32, u32, vp, vp, sz, vp, vp]),
        "irm_cdc_params_default": (ctypes.c_int, [P(CdcParams)]),
        "irm_cdc_split": (ctypes.c_int, [P(CdcParams), vp, u64, vp, u64, P(u64)]),
        "irm_xxh64": (ctypes.c_int, [vp, u64, u64, P(u64)]),
        "irm_registry_create": (ctypes.c_int, [u64, P(vp)]),
        "irm_registry_destroy": (ctypes.c_int, [vp]),
        "irm_registry_info": (ctypes.c_int, [vp, P(u64), P(u64)]),
        "irm_registry_assemble": (ctypes.c_int, [vp, P(CdcParams), vp, vp, u32, vp, vp, u32, vp, vp, u32, vp,
                                                 P(u32)]),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def _check(st: int, fn: str):
    if st != 0:
        raise IrmError(st, fn, lib().irm_last_error().decode())


def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _on_stream(stream):
    """Context in which the binding allocates its temporaries: the stream the
    kernels run on, so the caching allocator hands a freed block (say, the
    decode workspace) only to work ordered after those kernels."""
    import contextlib
    import torch
    if stream is None:
        return contextlib.nullcontext()
    if isinstance(stream, int):
        stream = torch.cuda.ExternalStream(stream)
    return torch.cuda.stream(stream)


def check_out(out, shape, device, name: str = "out", dtype=None):
    """Refuse a caller-supplied output the kernels could overrun: the C ABI
    takes no size for outputs and writes exactly ``shape`` elements, so the
    tensor must have that shape, the dtype (bfloat16 unless given), be
    contiguous and live on ``device``."""
    import torch
    dtype = torch.bfloat16 if dtype is None else dtype
    if not isinstance(out, torch.Tensor):
        raise TypeError(f"{name} must be a torch tensor")
    if tuple(out.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(out.shape)}")
    if out.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {out.dtype}")
    if not out.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if out.device != torch.device(device):
        raise ValueError(f"{name} must be on {device}, got {out.device}")


def rope_inv_freq(theta: float = 10000.0) -> np.ndarray:
    """theta^(-2i/64), i = 0..31, computed by the library."""
    out = np.zeros(32, dtype=np.float64)
    _check(lib().irm_rope_inv_freq(float(theta), out.ctypes.data), "irm_rope_inv_freq")
    return out


class Table:
    """A validated chunk table (host image) and, after upload(), its device copy."""

    def __init__(self, chunks: np.ndarray, seq_first: np.ndarray, pool_rows: int):
        chunks = np.ascontiguousarray(chunks, dtype=CHUNK_DTYPE)
        seq_first = np.ascontiguousarray(seq_first, dtype=np.uint32)
        self._h = ctypes.c_void_p()
        L = lib()
        _check(L.irm_table_create(chunks.ctypes.data if chunks.size else None, chunks.shape[0],
                                  seq_first.ctypes.data, seq_first.shape[0] - 1, int(pool_rows),
                                  ctypes.byref(self._h)), "irm_table_create")
        n_seq, n_chunks, mx = ctypes.c_uint32(), ctypes.c_uint32(), ctypes.c_uint32()
        total, dbytes = ctypes.c_uint64(), ctypes.c_size_t()
        _check(L.irm_table_info(self._h, ctypes.byref(n_seq), ctypes.byref(n_chunks), ctypes.byref(total),
                                ctypes.byref(mx), ctypes.byref(dbytes)), "irm_table_info")
        self.n_seq, self.n_chunks = n_seq.value, n_chunks.value
        self.total_rows, self.max_seq_len, self.device_bytes = total.value, mx.value, dbytes.value
        self.pool_rows = int(pool_rows)
        self._dev = None

    def gather_stats(self) -> dict:
        """How the rotate-gather works through this table: work records and
        items, the pool rows one call reads (each shared run once) and the
        bytes an upload copies from the host."""
        g, it, rr, hb = ctypes.c_uint32(), ctypes.c_uint64(), ctypes.c_uint64(), ctypes.c_size_t()
        _check(lib().irm_table_gather_stats(self._h, ctypes.byref(g), ctypes.byref(it), ctypes.byref(rr),
                                            ctypes.byref(hb)), "irm_table_gather_stats")
        return {"n_groups": g.value, "n_items": it.value, "read_rows": rr.value, "host_bytes": hb.value}

    def close(self):
        if getattr(self, "_h", None) is not None and self._h.value:
            lib().irm_table_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    @property
    def handle(self) -> ctypes.c_void_p:
        return self._h

    def seq_base(self) -> np.ndarray:
        out = np.zeros(self.n_seq + 1, dtype=np.uint64)
        _check(lib().irm_table_seq_base(self._h, out.ctypes.data), "irm_table_seq_base")
        return out

    def expand_host(self) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
        n = self.total_rows
        pr = np.zeros(n, np.int64)
        de = np.zeros(n, np.int32)
        fr = np.zeros(n, np.uint8)
        _check(lib().irm_table_expand_host(self._h, pr.ctypes.data, de.ctypes.data, fr.ctypes.data),
               "irm_table_expand_host")
        return pr, de, fr

    def upload(self, inv_freq: Optional[np.ndarray] = None, dev_buf=None, stream=None) -> "Table":
        """Copy the device image to dev_buf (a torch uint8 CUDA tensor; allocated
        here if None) and compute the per-entry trig on the GPU."""
        import torch
        if inv_freq is None:
            inv_freq = rope_inv_freq(10000.0)
        inv = np.ascontiguousarray(inv_freq, dtype=np.float64)
        assert inv.shape == (32,)
        if dev_buf is None:
            with _on_stream(stream):
                dev_buf = torch.empty(max(self.device_bytes, 256), dtype=torch.uint8, device="cuda")
        elif dev_buf.dtype != torch.uint8 or not dev_buf.is_cuda or not dev_buf.is_contiguous():
            raise ValueError("dev_buf must be a contiguous uint8 CUDA tensor")
        _check(lib().irm_table_upload(self._h, inv.ctypes.data, _ptr(dev_buf), dev_buf.numel(),
                                      _stream(stream)), "irm_table_upload")
        self._dev = dev_buf
        self._inv = inv
        return self

    def prepare(self, inv_freq: Optional[np.ndarray] = None, stream=None) -> "Table":
        """Rebuild the row map and the per-entry cos/sin of the uploaded image
        on the GPU (the device passes of upload(), without its copy)."""
        inv = self._inv if inv_freq is None else np.ascontiguousarray(inv_freq, dtype=np.float64)
        assert inv.shape == (32,)
        _check(lib().irm_table_prepare(self._h, inv.ctypes.data, _stream(stream)), "irm_table_prepare")
        self._inv = inv
        return self

    def set_rope(self, inv_freq: np.ndarray, stream=None) -> "Table":
        """Recompute the per-entry cos/sin on the GPU (no host-to-device copy)."""
        inv = np.ascontiguousarray(inv_freq, dtype=np.float64)
        assert inv.shape == (32,)
        _check(lib().irm_table_set_rope(self._h, inv.ctypes.data, _stream(stream)), "irm_table_set_rope")
        self._inv = inv
        return self

    def gather_index(self, stream=None):
        import torch
        with _on_stream(stream):
            pr = torch.empty(self.total_rows, dtype=torch.int64, device="cuda")
            de = torch.empty(self.total_rows, dtype=torch.int32, device="cuda")
        _check(lib().irm_table_gather_index(self._h, _ptr(pr), _ptr(de), _stream(stream)),
               "irm_table_gather_index")
        return pr, de


def _bf16_2d(t, cols: int, name: str):
    import torch
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{name} must hold bf16 bits (bfloat16/int16/uint16), got {t.dtype}")
    if not t.is_cuda or not t.is_contiguous() or t.shape[-1] != cols:
        raise ValueError(f"{name} must be a contiguous CUDA tensor with last dim {cols}")


def rotate_gather(table: Table, pool, out=None, kr_f32: bool = False, stream=None):
    """Assemble every sequence of ``table`` from ``pool`` (bf16 [rows][576]).
    Returns out (bf16 [total_rows][576]) and, if kr_f32, the float rotated k_r."""
    import torch
    _bf16_2d(pool, ROW, "pool")
    with _on_stream(stream):
        if out is None:
            out = torch.empty((table.total_rows, ROW), dtype=torch.bfloat16, device=pool.device)
        kr = torch.empty((table.total_rows, D_ROPE), dtype=torch.float32, device=pool.device) if kr_f32 else None
    check_out(out, (table.total_rows, ROW), pool.device)
    _check(lib().irm_rotate_gather(table.handle, _ptr(pool), pool.shape[0], _ptr(out), _ptr(kr),
                                   _stream(stream)), "irm_rotate_gather")
    return (out, kr) if kr_f32 else out


def decode_workspace_bytes(table: Table, n_heads: int, n_splits: int = 0) -> int:
    b = ctypes.c_size_t()
    _check(lib().irm_mla_decode_workspace(table.handle, n_heads, n_splits, ctypes.byref(b)),
           "irm_mla_decode_workspace")
    return b.value


def mla_decode(q_lat, q_rope, table: Table, pool, n_splits: int = 0, scale: float = DEFAULT_SCALE,
               out=None, want_lse: bool = False, workspace=None, stream=None):
    """Absorbed MLA decode with k_r rotated on load.  q_lat bf16 [B][H][512],
    q_rope bf16 [B][H][64].  Returns out bf16 [B][H][512] (and lse [B][H])."""
    import torch
    _bf16_2d(pool, ROW, "pool")
    _bf16_2d(q_lat, D_LATENT, "q_lat")
    _bf16_2d(q_rope, D_ROPE, "q_rope")
    B, H = q_lat.shape[0], q_lat.shape[1]
    if B != table.n_seq or tuple(q_rope.shape) != (B, H, D_ROPE):
        raise ValueError("q_lat/q_rope must be [n_seq][H][512] / [n_seq][H][64]")
    need = decode_workspace_bytes(table, H, n_splits)
    with _on_stream(stream):
        if out is None:
            out = torch.empty((B, H, D_LATENT), dtype=torch.bfloat16, device=pool.device)
        lse = torch.empty((B, H), dtype=torch.float32, device=pool.device) if want_lse else None
        if workspace is None or workspace.numel() < need:
            workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=pool.device)
    check_out(out, (B, H, D_LATENT), pool.device)
    check_out(workspace, (workspace.numel(),), pool.device, "workspace", torch.uint8)
    _check(lib().irm_mla_decode(_ptr(q_lat), _ptr(q_rope), table.handle, _ptr(pool), pool.shape[0], H,
                                n_splits, float(scale), _ptr(out), _ptr(lse), _ptr(workspace),
                                workspace.numel(), _stream(stream)), "irm_mla_decode")
    return (out, lse) if want_lse else out


def mla_decode_noalloc(q_lat, q_rope, table: Table, pool, out, lse=None, n_splits: int = 0,
                       scale: float = DEFAULT_SCALE, stream=None):
    """mla_decode without any device allocation: the caller passes out (bf16
    [B][H][512]) and optionally lse (float [B][H]); the library keeps the
    split partials in its own per-GPU scratch array (calls that overlap on
    one GPU race; order them on one stream)."""
    import torch
    _bf16_2d(pool, ROW, "pool")
    _bf16_2d(q_lat, D_LATENT, "q_lat")
    _bf16_2d(q_rope, D_ROPE, "q_rope")
    B, H = q_lat.shape[0], q_lat.shape[1]
    if B != table.n_seq or tuple(q_rope.shape) != (B, H, D_ROPE):
        raise ValueError("q_lat/q_rope must be [n_seq][H][512] / [n_seq][H][64]")
    check_out(out, (B, H, D_LATENT), pool.device)
    if lse is not None:
        check_out(lse, (B, H), pool.device, "lse", torch.float32)
    _check(lib().irm_mla_decode_noalloc(_ptr(q_lat), _ptr(q_rope), table.handle, _ptr(pool), pool.shape[0], H,
                                        n_splits, float(scale), _ptr(out), _ptr(lse), _stream(stream)),
           "irm_mla_decode_noalloc")
    return (out, lse) if lse is not None else out


def mla_prefill_tail(q_lat, q_rope, q_pos0: int, table: Table, pool, scale: float = DEFAULT_SCALE,
                     out=None, want_lse: bool = False, stream=None):
    """Causal tail-prefill of n_q queries at q_pos0.. over the one sequence of
    ``table``.  q_lat bf16 [n_q][H][512], q_rope [n_q][H][64]."""
    import torch
    _bf16_2d(pool, ROW, "pool")
    _bf16_2d(q_lat, D_LATENT, "q_lat")
    _bf16_2d(q_rope, D_ROPE, "q_rope")
    nq, H = q_lat.shape[0], q_lat.shape[1]
    if tuple(q_rope.shape) != (nq, H, D_ROPE):
        raise ValueError("q_rope must be [n_q][H][64]")
    with _on_stream(stream):
        if out is None:
            out = torch.empty((nq, H, D_LATENT), dtype=torch.bfloat16, device=pool.device)
        lse = torch.empty((nq, H), dtype=torch.float32, device=pool.device) if want_lse else None
    check_out(out, (nq, H, D_LATENT), pool.device)
    _check(lib().irm_mla_prefill_tail(_ptr(q_lat), _ptr(q_rope), int(q_pos0), nq, table.handle, _ptr(pool),
                                      pool.shape[0], H, float(scale), _ptr(out), _ptr(lse),
                                      _stream(stream)), "irm_mla_prefill_tail")
    return (out, lse) if want_lse else out


def mla_prefill_assembled(q_lat, q_rope, q_pos0: int, kv, scale: float = DEFAULT_SCALE, out=None,
                          want_lse: bool = False, stream=None):
    """Causal tail-prefill over an assembled cache kv (bf16 [rows][576], row r
    at position r, e.g. the output of rotate_gather for one sequence)."""
    import torch
    _bf16_2d(kv, ROW, "kv")
    _bf16_2d(q_lat, D_LATENT, "q_lat")
    _bf16_2d(q_rope, D_ROPE, "q_rope")
    nq, H = q_lat.shape[0], q_lat.shape[1]
    if tuple(q_rope.shape) != (nq, H, D_ROPE):
        raise ValueError("q_rope must be [n_q][H][64]")
    with _on_stream(stream):
        if out is None:
            out = torch.empty((nq, H, D_LATENT), dtype=torch.bfloat16, device=kv.device)
        lse = torch.empty((nq, H), dtype=torch.float32, device=kv.device) if want_lse else None
    check_out(out, (nq, H, D_LATENT), kv.device)
    _check(lib().irm_mla_prefill_assembled(_ptr(q_lat), _ptr(q_rope), int(q_pos0), nq, _ptr(kv), kv.shape[0], H,
                                           float(scale), _ptr(out), _ptr(lse), _stream(stream)),
           "irm_mla_prefill_assembled")
    return (out, lse) if want_lse else out


D_NOPE = 128   # per-head nope key width of the non-absorbed form
D_V = 128      # per-head value width of the non-absorbed form


def mla_kv_upproj(kv, w_uk, w_uv, out=None, stream=None):
    """Per-head up-projection of an assembled cache: kv bf16 [rows][576],
    w_uk / w_uv bf16 [H][128][512] -> bf16 [H][rows][256] = [W_UK c_KV | W_UV c_KV]."""
    import torch
    _bf16_2d(kv, ROW, "kv")
    _bf16_2d(w_uk, D_LATENT, "w_uk")
    _bf16_2d(w_uv, D_LATENT, "w_uv")
    H = w_uk.shape[0]
    if tuple(w_uk.shape) != (H, D_NOPE, D_LATENT) or tuple(w_uv.shape) != (H, D_V, D_LATENT):
        raise ValueError("w_uk and w_uv must be [H][128][512]")
    rows = kv.shape[0]
    if out is None:
        with _on_stream(stream):
            out = torch.empty((H, rows, D_NOPE + D_V), dtype=torch.bfloat16, device=kv.device)
    check_out(out, (H, rows, D_NOPE + D_V), kv.device)
    _check(lib().irm_mla_kv_upproj(_ptr(kv), rows, _ptr(w_uk), _ptr(w_uv), H, _ptr(out), _stream(stream)),
           "irm_mla_kv_upproj")
    return out


def mla_prefill_nonabsorbed(q_nope, q_rope, q_pos0: int, kv, kvh, scale: float = DEFAULT_SCALE, out=None,
                            want_lse: bool = False, stream=None):
    """Causal prefill with per-head keys [k_nope | k_r] and values from
    mla_kv_upproj (kvh bf16 [H][rows][256]); k_r from the assembled kv."""
    import torch
    _bf16_2d(kv, ROW, "kv")
    _bf16_2d(kvh, D_NOPE + D_V, "kvh")
    _bf16_2d(q_nope, D_NOPE, "q_nope")
    _bf16_2d(q_rope, D_ROPE, "q_rope")
    nq, H = q_nope.shape[0], q_nope.shape[1]
    if tuple(q_rope.shape) != (nq, H, D_ROPE):
        raise ValueError("q_rope must be [n_q][H][64]")
    if tuple(kvh.shape) != (H, kv.shape[0], D_NOPE + D_V):
        raise ValueError("kvh must be [H][rows][256] for the rows of kv")
    with _on_stream(stream):
        if out is None:
            out = torch.empty((nq, H, D_V), dtype=torch.bfloat16, device=kv.device)
        lse = torch.empty((nq, H), dtype=torch.float32, device=kv.device) if want_lse else None
    check_out(out, (nq, H, D_V), kv.device)
    _check(lib().irm_mla_prefill_nonabsorbed(_ptr(q_nope), _ptr(q_rope), int(q_pos0), nq, _ptr(kv), _ptr(kvh),
                                             kv.shape[0], H, float(scale), _ptr(out), _ptr(lse), _stream(stream)),
           "irm_mla_prefill_nonabsorbed")
    return (out, lse) if want_lse else out


def gqa_inv_freq(theta: float, head_dim: int) -> np.ndarray:
    """theta^(-2i/head_dim), i < head_dim/2 (plain RoPE frequencies of a GQA
    head), computed by the library."""
    out = np.zeros(max(1, head_dim // 2), dtype=np.float64)
    _check(lib().irm_rope_inv_freq_dim(float(theta), int(head_dim), out.ctypes.data), "irm_rope_inv_freq_dim")
    return out


def gqa_rotate_gather(table: Table, pool, n_kv_heads: int, head_dim: int, inv_freq, out=None, stream=None):
    """Assemble GQA rows (bf16 [K heads | V heads]) with the whole key of each
    KV head rotated by the entry's delta (the GQA/MHA comparison path)."""
    import torch
    width = 2 * n_kv_heads * head_dim
    _bf16_2d(pool, width, "pool")
    inv = np.ascontiguousarray(inv_freq, dtype=np.float64)
    if inv.size != head_dim // 2:
        raise ValueError("inv_freq must hold head_dim / 2 values")
    nb = ctypes.c_size_t()
    _check(lib().irm_gqa_workspace(table.handle, head_dim, ctypes.byref(nb)), "irm_gqa_workspace")
    with _on_stream(stream):
        if out is None:
            out = torch.empty((table.total_rows, width), dtype=torch.bfloat16, device=pool.device)
        ws = torch.empty(max(16, nb.value), dtype=torch.uint8, device=pool.device)
    check_out(out, (table.total_rows, width), pool.device)
    _check(lib().irm_gqa_rotate_gather(table.handle, _ptr(pool), pool.shape[0], n_kv_heads, head_dim,
                                       inv.ctypes.data, _ptr(ws), ws.numel(), _ptr(out), _stream(stream)),
           "irm_gqa_rotate_gather")
    return out


def to_device_bf16(bits: np.ndarray):
    """uint16 bf16 bit patterns (host) -> torch.bfloat16 CUDA tensor."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda").view(torch.bfloat16)


def from_device_bf16(t) -> np.ndarray:
    """torch bf16 CUDA tensor -> uint16 bit patterns (host)."""
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


# ---------------------------------------------------------------- chunk-table producer (host)
def cdc_params(seed: int = 0, mask_bits: Optional[int] = None, min_len: Optional[int] = None,
               max_len: Optional[int] = None, fallback_window: int = 0) -> CdcParams:
    """CDC parameters: the library defaults (mask 7 bits, [32, 512], no S1
    fallback) unless given; fallback_window=128 is the pages' S1 fallback."""
    p = CdcParams()
    _check(lib().irm_cdc_params_default(ctypes.byref(p)), "irm_cdc_params_default")
    p.seed = int(seed) & (2**64 - 1)
    if mask_bits is not None:
        p.mask_bits = mask_bits
    if min_len is not None:
        p.min_len = min_len
    if max_len is not None:
        p.max_len = max_len
    p.fallback_window = int(fallback_window)
    return p


def cdc_split(tokens, params: Optional[CdcParams] = None) -> np.ndarray:
    """Chunk lengths (uint32) of a token stream."""
    toks = np.ascontiguousarray(tokens, dtype=np.int32)
    p = cdc_params() if params is None else params
    n = ctypes.c_uint64()
    cap = max(1, toks.size // max(1, p.min_len) + 1)
    lens = np.zeros(cap, dtype=np.uint32)
    _check(lib().irm_cdc_split(ctypes.byref(p), toks.ctypes.data, toks.size, lens.ctypes.data, cap,
                               ctypes.byref(n)), "irm_cdc_split")
    return lens[:n.value].copy()


def xxh64(data: bytes, seed: int = 0) -> int:
    out = ctypes.c_uint64()
    buf = ctypes.create_string_buffer(bytes(data), max(1, len(data)))
    _check(lib().irm_xxh64(buf, len(data), int(seed) & (2**64 - 1), ctypes.byref(out)), "irm_xxh64")
    return out.value


class Registry:
    """Content registry (fingerprint -> pool_row, len, p_src) with its
    fresh-row allocation counter, owned by the library."""

    def __init__(self, first_free_row: int = 0):
        h = ctypes.c_void_p()
        _check(lib().irm_registry_create(int(first_free_row), ctypes.byref(h)), "irm_registry_create")
        self._h = h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.irm_registry_destroy(h)
            self._h = None

    def info(self) -> Tuple[int, int]:
        n, nxt = ctypes.c_uint64(), ctypes.c_uint64()
        _check(lib().irm_registry_info(self._h, ctypes.byref(n), ctypes.byref(nxt)), "irm_registry_info")
        return n.value, nxt.value

    def assemble(self, requests, prefix_len=None, prefix_row=None, params: Optional[CdcParams] = None,
                 n_threads: int = 0):
        """requests: sequence of int32 token arrays.  Returns (chunks
        [CHUNK_DTYPE], seq_first [uint32, n_req + 1], fingerprints [uint64])."""
        reqs = [np.ascontiguousarray(r, dtype=np.int32) for r in requests]
        n_req = len(reqs)
        tok_first = np.zeros(n_req + 1, dtype=np.uint64)
        tok_first[1:] = np.cumsum([r.size for r in reqs]) if n_req else []
        toks = np.concatenate(reqs) if n_req and tok_first[-1] else np.zeros(1, dtype=np.int32)
        pl = None if prefix_len is None else np.ascontiguousarray(prefix_len, dtype=np.uint32)
        pr = None if prefix_row is None else np.ascontiguousarray(prefix_row, dtype=np.uint32)
        p = cdc_params() if params is None else params
        seq_first = np.zeros(n_req + 1, dtype=np.uint32)
        n = ctypes.c_uint32()
        cap = 16
        while True:
            chunks = np.zeros(cap, dtype=CHUNK_DTYPE)
            prints = np.zeros(cap, dtype=np.uint64)
            st = lib().irm_registry_assemble(
                self._h, ctypes.byref(p), toks.ctypes.data, tok_first.ctypes.data, n_req,
                None if pl is None else pl.ctypes.data, None if pr is None else pr.ctypes.data, int(n_threads),
                chunks.ctypes.data, prints.ctypes.data, cap, seq_first.ctypes.data, ctypes.byref(n))
            if st == 2 and n.value > cap:      # ERANGE: grow to the count the library reports
                cap = n.value
                continue
            _check(st, "irm_registry_assemble")
            return chunks[:n.value].copy(), seq_first, prints[:n.value].copy()

