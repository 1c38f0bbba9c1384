"""ctypes binding of libtq.so (argument marshalling only).

Every function here has the name of the C entry point it calls.  torch is
used for device memory and streams; all arithmetic of the method runs in the
library's HIP kernels.  If libtq.so is missing, importing the functions
raises: there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# TQ_LIBRARY names another build of the same library (the sanitizer build of
# the host sources); by default the in-tree libtq.so is loaded
LIB_PATH = os.environ.get("TQ_LIBRARY") or os.path.join(_HERE, "libtq.so")

TQ_OK, TQ_ERR_INVALID, TQ_ERR_UNSUPPORTED, TQ_ERR_HIP, TQ_ERR_ALLOC, TQ_ERR_NUMERIC = range(6)
TQ_F32, TQ_BF16, TQ_F16 = 0, 1, 2
TQ_LAYOUT_ROW, TQ_LAYOUT_TILE32 = 0, 1

# every symbol include/tq.h declares
EXPORTS = (
    "tq_codebook_build", "tq_codebook_destroy", "tq_codebook_export", "tq_codebook_values",
    "tq_code_row_bytes", "tq_quantize_kv", "tq_attn_decode_workspace", "tq_attn_decode",
    "tq_ip_topk_workspace", "tq_ip_topk", "tq_dequantize", "tq_quantize_kv_paged",
    "tq_attn_decode_paged_workspace", "tq_attn_decode_paged", "tq_profile_enable", "tq_profile_read",
    "tq_codebook_solver_limits", "tq_profile_durations", "tq_stream_read", "tq_stream_write", "tq_attn_decode_noalloc",
    "tq_attn_decode_append",
    "tq_polar_codebook_build", "tq_polar_codebook_values", "tq_ip_topk_exact_scan", "tq_ip_topk_scan_count",
    "tq_last_error",
)
TQ_KERNEL_QUANTIZE, TQ_KERNEL_DECODE_SPLIT, TQ_KERNEL_TOPK, TQ_KERNEL_DEQUANTIZE = 0, 1, 2, 3


class TQError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"tq status {status}: {msg}")
        self.status = status


class tq_params(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("bits", ctypes.c_int32), ("qjl_m", ctypes.c_int32),
                ("norm_correction", ctypes.c_int32), ("rot_seed", ctypes.c_uint64),
                ("qjl_seed", ctypes.c_uint64)]


class tq_codes(ctypes.Structure):
    _fields_ = [("idx", ctypes.c_void_p), ("sign", ctypes.c_void_p), ("scale", ctypes.c_void_p),
                ("rnorm", ctypes.c_void_p), ("idx_row_bytes", ctypes.c_int64),
                ("sign_row_bytes", ctypes.c_int64), ("seq_stride", ctypes.c_int64),
                ("layout", ctypes.c_int32), ("reserved", ctypes.c_int32)]


_LIB = None


def lib() -> ctypes.CDLL:
    """Load libtq.so (once).  Raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          "`python -m kv_cache_vector_quantize_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, dp = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.POINTER(ctypes.c_double)
    L.tq_last_error.restype = ctypes.c_char_p
    L.tq_last_error.argtypes = []
    L.tq_codebook_build.argtypes = [ctypes.POINTER(tq_params), ctypes.POINTER(vp)]
    L.tq_codebook_destroy.argtypes = [vp]
    L.tq_codebook_export.argtypes = [vp, dp, dp, dp, dp]
    L.tq_codebook_values.argtypes = [ctypes.POINTER(tq_params), dp, dp, dp, dp]
    L.tq_codebook_solver_limits.argtypes = [i32, i32]
    L.tq_ip_topk_exact_scan.argtypes = [i32]
    L.tq_ip_topk_scan_count.argtypes = [vp, vp, i64, i64, i32, vp, ctypes.POINTER(i64)]
    L.tq_polar_codebook_build.argtypes = [ctypes.POINTER(tq_polar_params), ctypes.POINTER(vp)]
    L.tq_polar_codebook_values.argtypes = [ctypes.POINTER(tq_polar_params), dp, dp, dp, dp]
    L.tq_code_row_bytes.argtypes = [vp, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    L.tq_quantize_kv.argtypes = [vp, vp, vp, vp, i32, i64, i64, i64,
                                 ctypes.POINTER(tq_codes), ctypes.POINTER(tq_codes), vp]
    L.tq_attn_decode_workspace.argtypes = [i64, i64, i64, i64, i32, ctypes.POINTER(ctypes.c_size_t)]
    L.tq_attn_decode.argtypes = [vp, vp, vp, i32, i64, i64, i64, ctypes.POINTER(tq_codes),
                                 ctypes.POINTER(tq_codes), vp, i64, ctypes.c_float, vp, vp, vp,
                                 ctypes.c_size_t, vp]
    L.tq_attn_decode_append.argtypes = [vp, vp, vp, vp, i32, i64, i64, vp, i32, i64, i64, i64,
                                         ctypes.POINTER(tq_codes), ctypes.POINTER(tq_codes), vp, i64,
                                         ctypes.c_float, vp, vp, vp, ctypes.c_size_t, vp]
    L.tq_attn_decode_noalloc.argtypes = [vp, vp, vp, i32, i64, i64, i64, ctypes.POINTER(tq_codes),
                                         ctypes.POINTER(tq_codes), vp, i64, ctypes.c_float, vp, vp, vp]
    L.tq_ip_topk_workspace.argtypes = [i64, i64, i32, i32, ctypes.POINTER(ctypes.c_size_t)]
    L.tq_ip_topk.argtypes = [vp, vp, i64, ctypes.POINTER(tq_codes), i64, i32, vp, vp, vp,
                             ctypes.c_size_t, vp]
    L.tq_dequantize.argtypes = [vp, ctypes.POINTER(tq_codes), i64, i64, i64, vp, i32, vp]
    L.tq_quantize_kv_paged.argtypes = [vp, vp, vp, vp, i32, i64, i64, i64, i64, vp, i64, i32,
                                       ctypes.POINTER(tq_codes), ctypes.POINTER(tq_codes), vp]
    L.tq_attn_decode_paged_workspace.argtypes = [i64, i64, i64, i64, i32, i32, ctypes.POINTER(ctypes.c_size_t)]
    L.tq_attn_decode_paged.argtypes = [vp, vp, vp, i32, i64, i64, i64, ctypes.POINTER(tq_codes),
                                       ctypes.POINTER(tq_codes), vp, i64, i32, vp, i64, ctypes.c_float,
                                       vp, vp, vp, ctypes.c_size_t, vp]
    L.tq_profile_enable.argtypes = [i32]
    L.tq_profile_read.argtypes = [i32, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(i64)]
    L.tq_profile_durations.argtypes = [i32, dp, i64, ctypes.POINTER(i64)]
    L.tq_stream_read.argtypes = [vp, i64, vp, vp]
    L.tq_stream_write.argtypes = [vp, i64, ctypes.c_uint32, vp]
    for name in EXPORTS:
        if name != "tq_last_error":
            getattr(L, name).restype = ctypes.c_int
    _LIB = L
    return L


def _check(status: int):
    if status != TQ_OK:
        raise TQError(status, lib().tq_last_error().decode())


def _dptr(a: np.ndarray | None):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _dtype_code(t) -> int:
    import torch
    return {torch.float32: TQ_F32, torch.bfloat16: TQ_BF16, torch.float16: TQ_F16}[t.dtype]


def _stream_handle(stream):
    import torch
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


# ------------------------------------------------------------------ codebook


def _params(d, bits, qjl_m, norm_correction, rot_seed, qjl_seed) -> tq_params:
    return tq_params(int(d), int(bits), int(qjl_m), int(bool(norm_correction)),
                     int(rot_seed), int(qjl_seed))


def tq_codebook_values(d, bits, qjl_m=0, norm_correction=False, rot_seed=1, qjl_seed=2):
    """Host-only float64 codebook values: dict(centroids, boundaries, rot, qjl)."""
    L = 1 << int(bits)
    c, t = np.zeros(L), np.zeros(L - 1)
    r = np.zeros((d, d))
    q = np.zeros((qjl_m, d)) if qjl_m > 0 else None
    p = _params(d, bits, qjl_m, norm_correction, rot_seed, qjl_seed)
    _check(lib().tq_codebook_values(ctypes.byref(p), _dptr(c), _dptr(t), _dptr(r), _dptr(q)))
    return dict(centroids=c, boundaries=t, rot=r, qjl=q)


def tq_codebook_solver_limits(lloyd_iters=0, newton_iters=0):
    """Iteration limits of the codebook solve on this thread (0: defaults)."""
    _check(lib().tq_codebook_solver_limits(int(lloyd_iters), int(newton_iters)))


def tq_ip_topk_scan_count(cb, workspace, nq, n_db, k, stream=None) -> int:
    """Queries of the last tq_ip_topk call with this workspace that the exact
    scan answered (waits for the call)."""
    out = ctypes.c_int64(0)
    _check(lib().tq_ip_topk_scan_count(cb.handle, ctypes.c_void_p(workspace.data_ptr()), int(nq), int(n_db),
                                       int(k), _stream_handle(stream), ctypes.byref(out)))
    return int(out.value)


def tq_ip_topk_exact_scan(always: bool):
    """Diagnostic switch: True sends every top-k query to the exact float64
    scan of the database; False (the default) scans only the queries the
    candidates do not settle."""
    _check(lib().tq_ip_topk_exact_scan(1 if always else 0))


class Codebook:
    """Owns a tq_codebook (built on the current HIP device)."""

    def __init__(self, d, bits, qjl_m=0, norm_correction=False, rot_seed=1, qjl_seed=2):
        self.d, self.bits, self.m = int(d), int(bits), int(qjl_m)
        self.nc = bool(norm_correction)
        self.rot_seed, self.qjl_seed = int(rot_seed), int(qjl_seed)
        self._h = ctypes.c_void_p()
        p = _params(d, bits, qjl_m, norm_correction, rot_seed, qjl_seed)
        _check(lib().tq_codebook_build(ctypes.byref(p), ctypes.byref(self._h)))

    @property
    def handle(self):
        return self._h

    def export(self):
        L = 1 << self.bits
        c, t = np.zeros(L), np.zeros(L - 1)
        r = np.zeros((self.d, self.d))
        q = np.zeros((self.m, self.d)) if self.m > 0 else None
        _check(lib().tq_codebook_export(self._h, _dptr(c), _dptr(t), _dptr(r), _dptr(q)))
        return dict(centroids=c, boundaries=t, rot=r, qjl=q)

    def row_bytes(self):
        a, b = ctypes.c_int64(), ctypes.c_int64()
        _check(lib().tq_code_row_bytes(self._h, ctypes.byref(a), ctypes.byref(b)))
        return a.value, b.value

    def close(self):
        if self._h:
            lib().tq_codebook_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class tq_polar_params(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("bits_first", ctypes.c_int32), ("bits_rest", ctypes.c_int32),
                ("qjl_m", ctypes.c_int32), ("rot_seed", ctypes.c_uint64), ("qjl_seed", ctypes.c_uint64)]


def _polar_sizes(d, b1, br):
    levels = int(d).bit_length() - 1
    nc = (1 << b1) + (levels - 1) * (1 << br)
    return levels, nc, nc - levels


def tq_polar_codebook_values(d, bits_first=4, bits_rest=2, qjl_m=0, rot_seed=1, qjl_seed=2):
    """Host-only float64 values of a polar codebook: dict(centroids,
    boundaries) concatenated per level (level 1 first), rot, qjl."""
    _, nc, nb = _polar_sizes(d, bits_first, bits_rest)
    c, t = np.zeros(max(1, nc)), np.zeros(max(1, nb))
    r = np.zeros((d, d))
    q = np.zeros((qjl_m, d)) if qjl_m > 0 else None
    p = tq_polar_params(int(d), int(bits_first), int(bits_rest), int(qjl_m), int(rot_seed), int(qjl_seed))
    _check(lib().tq_polar_codebook_values(ctypes.byref(p), _dptr(c), _dptr(t), _dptr(r), _dptr(q)))
    return dict(centroids=c[:nc], boundaries=t[:nb], rot=r, qjl=q)


class PolarCodebook(Codebook):
    """Owns a PolarQuant tq_codebook: b1 bits per level-1 angle, br bits per
    angle of every higher level."""

    def __init__(self, d, bits_first=4, bits_rest=2, qjl_m=0, rot_seed=1, qjl_seed=2):
        self.d, self.b1, self.br, self.m = int(d), int(bits_first), int(bits_rest), int(qjl_m)
        self.bits, self.nc, self.polar = self.b1, False, True
        self.rot_seed, self.qjl_seed = int(rot_seed), int(qjl_seed)
        self._h = ctypes.c_void_p()
        p = tq_polar_params(self.d, self.b1, self.br, self.m, self.rot_seed, self.qjl_seed)
        _check(lib().tq_polar_codebook_build(ctypes.byref(p), ctypes.byref(self._h)))

    def export(self):
        _, nc, nb = _polar_sizes(self.d, self.b1, self.br)
        c, t = np.zeros(max(1, nc)), np.zeros(max(1, nb))
        r = np.zeros((self.d, self.d))
        q = np.zeros((self.m, self.d)) if self.m > 0 else None
        _check(lib().tq_codebook_export(self._h, _dptr(c), _dptr(t), _dptr(r), _dptr(q)))
        return dict(centroids=c[:nc], boundaries=t[:nb], rot=r, qjl=q)


class Codes:
    """Device code planes of one tensor (torch tensors) plus their layout."""

    def __init__(self, cb: Codebook, n_seq: int, seq_stride: int, layout: int = TQ_LAYOUT_ROW,
                 device="cuda"):
        import torch
        self.cb, self.n_seq, self.seq_stride, self.layout = cb, int(n_seq), int(seq_stride), int(layout)
        n = self.n_seq * self.seq_stride
        if layout == TQ_LAYOUT_ROW:
            self.idx_row_bytes, self.sign_row_bytes = cb.row_bytes()
            self.idx = torch.zeros(max(1, n * self.idx_row_bytes), dtype=torch.uint8, device=device)
        else:
            if seq_stride % 32:
                raise ValueError("tile32 codes need seq_stride % 32 == 0")
            self.idx_row_bytes, self.sign_row_bytes = 0, 0
            block = 64 * ((cb.d + 15) // 16) * cb.bits
            self.idx = torch.zeros(max(1, self.n_seq * (self.seq_stride // 32) * block),
                                   dtype=torch.uint8, device=device)
        self.scale = torch.zeros(max(1, n), dtype=torch.float32, device=device)
        if cb.m > 0:
            if layout == TQ_LAYOUT_ROW:
                self.sign = torch.zeros(max(1, n * self.sign_row_bytes), dtype=torch.uint8, device=device)
            else:
                self.sign = None
            self.rnorm = torch.zeros(max(1, n), dtype=torch.float32, device=device)
        else:
            self.sign, self.rnorm = None, None

    def descriptor(self) -> tq_codes:
        return tq_codes(self.idx.data_ptr(),
                        self.sign.data_ptr() if self.sign is not None else None,
                        self.scale.data_ptr(),
                        self.rnorm.data_ptr() if self.rnorm is not None else None,
                        self.idx_row_bytes, self.sign_row_bytes, self.seq_stride, self.layout, 0)

    def nbytes_per_vector(self) -> float:
        b = self.idx_row_bytes + 4 if getattr(self.cb, "polar", False) else self.cb.d * self.cb.bits / 8 + 4
        if self.cb.m > 0:
            b += self.cb.m / 8 + 4
        return b


# ------------------------------------------------------------------ calls


def tq_quantize_kv(kcb, vcb, k, v, k_out: Codes | None, v_out: Codes | None,
                   tok_offset: int = 0, stream=None):
    """k, v: torch tensors [n_seq, n_tok, d] (contiguous, same dtype), or None."""
    ref = k if k is not None else v
    n_seq, n_tok = ref.shape[0], ref.shape[1]
    for t in (k, v):
        if t is not None and not t.is_contiguous():
            raise ValueError("inputs must be contiguous")
    kd = k_out.descriptor() if k_out is not None else None
    vd = v_out.descriptor() if v_out is not None else None
    _check(lib().tq_quantize_kv(
        kcb.handle if kcb is not None else None, vcb.handle if vcb is not None else None,
        k.data_ptr() if k is not None else None, v.data_ptr() if v is not None else None,
        _dtype_code(ref), n_seq, n_tok, int(tok_offset),
        ctypes.byref(kd) if kd is not None else None, ctypes.byref(vd) if vd is not None else None,
        _stream_handle(stream)))


def tq_dequantize(cb, codes: Codes, n_seq: int, n_tok: int, tok_offset: int = 0, out=None,
                  dtype=None, stream=None):
    """Vectors of positions [tok_offset, tok_offset + n_tok) of sequences
    0..n_seq-1 back from their codes.  Returns out ([n_seq, n_tok, d], fp32
    unless dtype / out say otherwise)."""
    import torch
    if out is None:
        out = torch.empty((n_seq, n_tok, cb.d), dtype=dtype or torch.float32, device=codes.scale.device)
    if not out.is_contiguous():
        raise ValueError("out must be contiguous")
    cd = codes.descriptor()
    _check(lib().tq_dequantize(cb.handle, ctypes.byref(cd), int(n_seq), int(n_tok), int(tok_offset),
                               out.data_ptr(), _dtype_code(out), _stream_handle(stream)))
    return out


def tq_attn_decode_workspace(B, Hq, Hkv, n_ctx, d) -> int:
    out = ctypes.c_size_t()
    _check(lib().tq_attn_decode_workspace(int(B), int(Hq), int(Hkv), int(n_ctx), int(d),
                                          ctypes.byref(out)))
    return out.value


def tq_attn_decode(kcb, vcb, q, k_codes: Codes, v_codes: Codes, n_ctx: int, sm_scale: float,
                   seq_lens=None, out=None, logits=None, workspace=None, stream=None):
    """q: [B, Hq, d] torch tensor.  Returns out (fp32 [B, Hq, d])."""
    import torch
    B, Hq, d = q.shape
    Hkv = k_codes.n_seq // B
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if workspace is None:
        ws = tq_attn_decode_workspace(B, Hq, Hkv, n_ctx, d)
        workspace = torch.empty(max(ws, 256), dtype=torch.uint8, device=q.device)
    kd, vd = k_codes.descriptor(), v_codes.descriptor()
    _check(lib().tq_attn_decode(
        kcb.handle, vcb.handle, q.data_ptr(), _dtype_code(q), B, Hq, Hkv, ctypes.byref(kd),
        ctypes.byref(vd), seq_lens.data_ptr() if seq_lens is not None else None, int(n_ctx),
        float(sm_scale), out.data_ptr(), logits.data_ptr() if logits is not None else None,
        workspace.data_ptr(), workspace.numel(), _stream_handle(stream)))
    return out


def tq_attn_decode_append(kcb, vcb, k_new, v_new, tok_offset: int, q, k_codes: Codes, v_codes: Codes,
                          n_ctx: int, sm_scale: float, seq_lens=None, out=None, logits=None, workspace=None,
                          stream=None):
    """One decode step: k_new, v_new ([B*Hkv, n_new, d] torch tensors, same
    dtype) go to positions [tok_offset, tok_offset + n_new) of their
    sequences, then q ([B, Hq, d]) attends.  Returns out (fp32 [B, Hq, d])."""
    import torch
    B, Hq, d = q.shape
    Hkv = k_codes.n_seq // B
    for t in (k_new, v_new):
        if not t.is_contiguous():
            raise ValueError("inputs must be contiguous")
    n_new = k_new.shape[1]
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if workspace is None:
        ws = tq_attn_decode_workspace(B, Hq, Hkv, n_ctx, d)
        workspace = torch.empty(max(ws, 256), dtype=torch.uint8, device=q.device)
    kd, vd = k_codes.descriptor(), v_codes.descriptor()
    _check(lib().tq_attn_decode_append(
        kcb.handle, vcb.handle, k_new.data_ptr(), v_new.data_ptr(), _dtype_code(k_new), int(n_new),
        int(tok_offset), q.data_ptr(), _dtype_code(q), B, Hq, Hkv, ctypes.byref(kd), ctypes.byref(vd),
        seq_lens.data_ptr() if seq_lens is not None else None, int(n_ctx), float(sm_scale), out.data_ptr(),
        logits.data_ptr() if logits is not None else None, workspace.data_ptr(), workspace.numel(),
        _stream_handle(stream)))
    return out


def tq_attn_decode_noalloc(kcb, vcb, q, k_codes: Codes, v_codes: Codes, n_ctx: int, sm_scale: float,
                           seq_lens=None, out=None, logits=None, stream=None):
    """tq_attn_decode without a workspace (the library's fixed per-device
    scratch).  ``out`` must be given by callers that cannot allocate."""
    import torch
    B, Hq, d = q.shape
    Hkv = k_codes.n_seq // B
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    kd, vd = k_codes.descriptor(), v_codes.descriptor()
    _check(lib().tq_attn_decode_noalloc(
        kcb.handle, vcb.handle, q.data_ptr(), _dtype_code(q), B, Hq, Hkv, ctypes.byref(kd),
        ctypes.byref(vd), seq_lens.data_ptr() if seq_lens is not None else None, int(n_ctx),
        float(sm_scale), out.data_ptr(), logits.data_ptr() if logits is not None else None,
        _stream_handle(stream)))
    return out


def _table(block_table):
    import torch
    if block_table.dtype != torch.int32 or block_table.dim() != 2 or not block_table.is_contiguous():
        raise ValueError("block_table must be a contiguous int32 [B, max_pages] tensor")
    return block_table


def tq_quantize_kv_paged(kcb, vcb, k, v, k_pool: Codes | None, v_pool: Codes | None, block_table,
                         page_tokens: int, tok_offset: int = 0, stream=None):
    """k, v: [B*Hkv, n_tok, d] (sequence b*Hkv + h) or None; the pools hold
    Hkv planes (n_seq = Hkv); block_table: int32 [B, max_pages]."""
    ref = k if k is not None else v
    pool = k_pool if k is not None else v_pool
    bt = _table(block_table)
    B, Hkv = bt.shape[0], pool.n_seq
    if ref.shape[0] != B * Hkv:
        raise ValueError("inputs must have B * Hkv rows (B from block_table, Hkv from the pool)")
    for t in (k, v):
        if t is not None and not t.is_contiguous():
            raise ValueError("inputs must be contiguous")
    kd = k_pool.descriptor() if k_pool is not None else None
    vd = v_pool.descriptor() if v_pool is not None else None
    _check(lib().tq_quantize_kv_paged(
        kcb.handle if kcb is not None else None, vcb.handle if vcb is not None else None,
        k.data_ptr() if k is not None else None, v.data_ptr() if v is not None else None,
        _dtype_code(ref), int(B), int(Hkv), int(ref.shape[1]), int(tok_offset), bt.data_ptr(),
        int(bt.shape[1]), int(page_tokens),
        ctypes.byref(kd) if kd is not None else None, ctypes.byref(vd) if vd is not None else None,
        _stream_handle(stream)))


def tq_attn_decode_paged_workspace(B, Hq, Hkv, n_ctx, d, page_tokens) -> int:
    out = ctypes.c_size_t()
    _check(lib().tq_attn_decode_paged_workspace(int(B), int(Hq), int(Hkv), int(n_ctx), int(d),
                                                int(page_tokens), ctypes.byref(out)))
    return out.value


def tq_attn_decode_paged(kcb, vcb, q, k_pool: Codes, v_pool: Codes, block_table, page_tokens: int,
                         n_ctx: int, sm_scale: float, seq_lens=None, out=None, logits=None,
                         workspace=None, stream=None):
    """q: [B, Hq, d]; the pools hold Hkv planes; block_table int32 [B, max_pages].
    Returns out (fp32 [B, Hq, d])."""
    import torch
    B, Hq, d = q.shape
    Hkv = k_pool.n_seq
    bt = _table(block_table)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=q.device)
    if workspace is None:
        ws = tq_attn_decode_paged_workspace(B, Hq, Hkv, n_ctx, d, page_tokens)
        workspace = torch.empty(max(ws, 256), dtype=torch.uint8, device=q.device)
    kd, vd = k_pool.descriptor(), v_pool.descriptor()
    _check(lib().tq_attn_decode_paged(
        kcb.handle, vcb.handle, q.data_ptr(), _dtype_code(q), B, Hq, Hkv, ctypes.byref(kd),
        ctypes.byref(vd), bt.data_ptr(), int(bt.shape[1]), int(page_tokens),
        seq_lens.data_ptr() if seq_lens is not None else None, int(n_ctx), float(sm_scale),
        out.data_ptr(), logits.data_ptr() if logits is not None else None,
        workspace.data_ptr(), workspace.numel(), _stream_handle(stream)))
    return out


def tq_ip_topk_workspace(nq, n_db, k, d) -> int:
    out = ctypes.c_size_t()
    _check(lib().tq_ip_topk_workspace(int(nq), int(n_db), int(k), int(d), ctypes.byref(out)))
    return out.value


def tq_ip_topk(cb, queries, db: Codes, n_db: int, k: int, out_idx=None, out_score=None,
               workspace=None, stream=None):
    """queries: fp32 [nq, d] torch tensor; db: codes of sequence 0.
    Returns (idx int64 [nq, k], score fp32 [nq, k])."""
    import torch
    nq, d = queries.shape
    if out_idx is None:
        out_idx = torch.empty((nq, k), dtype=torch.int64, device=queries.device)
    if out_score is None:
        out_score = torch.empty((nq, k), dtype=torch.float32, device=queries.device)
    if workspace is None:
        ws = tq_ip_topk_workspace(nq, n_db, k, d)
        workspace = torch.empty(max(ws, 256), dtype=torch.uint8, device=queries.device)
    dd = db.descriptor()
    _check(lib().tq_ip_topk(cb.handle, queries.data_ptr(), int(nq), ctypes.byref(dd), int(n_db),
                            int(k), out_idx.data_ptr(), out_score.data_ptr(), workspace.data_ptr(),
                            workspace.numel(), _stream_handle(stream)))
    return out_idx, out_score


def tq_profile_enable(on: bool = True):
    _check(lib().tq_profile_enable(1 if on else 0))


def tq_profile_read(kernel: int):
    """(total milliseconds, launches) recorded for one kernel id."""
    ms, n = ctypes.c_double(), ctypes.c_int64()
    _check(lib().tq_profile_read(int(kernel), ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def tq_profile_durations(kernel: int):
    """Milliseconds of every recorded launch of one kernel id (numpy array)."""
    n = ctypes.c_int64()
    _check(lib().tq_profile_durations(int(kernel), None, 0, ctypes.byref(n)))
    ms = np.zeros(max(1, n.value))
    _check(lib().tq_profile_durations(int(kernel), _dptr(ms), n.value, ctypes.byref(n)))
    return ms[:n.value]


def tq_stream_write(buf, value=0, stream=None):
    """Enqueue a write-only pass over the device tensor ``buf`` (its byte size
    a multiple of 16): every 32-bit word becomes ``value``."""
    nbytes = buf.numel() * buf.element_size()
    _check(lib().tq_stream_write(ctypes.c_void_p(buf.data_ptr()), nbytes, ctypes.c_uint32(value & 0xFFFFFFFF),
                                 _stream_handle(stream)))


def tq_stream_read(buf, sink, stream=None):
    """Enqueue a read-only pass over the device tensor ``buf`` (its byte size
    a multiple of 16); ``sink`` is a device tensor of >= 4 bytes."""
    nbytes = buf.numel() * buf.element_size()
    _check(lib().tq_stream_read(ctypes.c_void_p(buf.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()),
                                _stream_handle(stream)))
