"""Host-side checks of libtq.so that need no GPU: exports, the library's own
codebook construction against the oracle's independent one, and argument
validation that fails before any device call."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle as O
import kv_cache_vector_quantize_amd as tq
from kv_cache_vector_quantize_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    txt = open(os.path.join(ROOT, "include", "tq.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(tq_[a-z_]+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    L = tq.lib()
    decl = _declared()
    assert set(decl) == set(tq.EXPORTS)
    for name in decl:
        assert hasattr(L, name), name


@pytest.mark.parametrize("d,bits,m", [(3, 2, 0), (8, 3, 8), (64, 4, 16), (128, 1, 0), (128, 2, 0),
                                      (128, 3, 128), (128, 4, 0), (200, 4, 200), (128, 8, 0)])
def test_host_codebook_matches_oracle(d, bits, m):
    lib_v = tq.tq_codebook_values(d, bits, m, rot_seed=1, qjl_seed=2)
    ref = O.Codebook(d, bits, qjl_m=m, rot_seed=1, qjl_seed=2)
    # the 256-level fixed point amplifies fp64 residuals ~1e4x, so two
    # independent solvers agree to ~1e-11 there; fp32 storage needs ~1e-8
    assert np.max(np.abs(lib_v["centroids"] - ref.centroids)) < 1e-10
    assert np.max(np.abs(lib_v["boundaries"] - ref.boundaries)) < 1e-10
    # Householder (library) vs Gram-Schmidt (oracle): same Q by uniqueness
    assert np.max(np.abs(lib_v["rot"] - ref.rot)) < 1e-12
    if m:
        assert np.max(np.abs(lib_v["qjl"] - ref.qjl)) < 1e-13


def test_host_codebook_seeds_and_nc():
    a = tq.tq_codebook_values(16, 3, 8, norm_correction=True, rot_seed=7, qjl_seed=9)
    ref = O.Codebook(16, 3, qjl_m=8, nc=True, rot_seed=7, qjl_seed=9)
    assert np.max(np.abs(a["rot"] - ref.rot)) < 1e-12
    assert np.max(np.abs(a["qjl"] - ref.qjl)) < 1e-13


@pytest.mark.parametrize("kw", [dict(d=2, bits=3), dict(d=300, bits=3), dict(d=16, bits=0),
                                dict(d=16, bits=9), dict(d=16, bits=3, qjl_m=-1),
                                dict(d=16, bits=3, qjl_m=257)])
def test_invalid_params_rejected(kw):
    with pytest.raises(tq.TQError) as e:
        tq.tq_codebook_values(**kw)
    assert e.value.status == _lib.TQ_ERR_INVALID


def test_norm_correction_flag_validated():
    p = _lib.tq_params(16, 3, 0, 2, 1, 2)
    st = tq.lib().tq_codebook_values(ctypes.byref(p), None, None, None, None)
    assert st == _lib.TQ_ERR_INVALID
    assert b"norm_correction" in tq.lib().tq_last_error()


def test_decode_workspace_validation():
    assert tq.tq_attn_decode_workspace(8, 64, 8, 131072, 128) > 0
    assert tq.tq_attn_decode_workspace(1, 8, 1, 0, 128) > 0
    with pytest.raises(tq.TQError):
        tq.tq_attn_decode_workspace(1, 7, 2, 100, 128)       # Hq not a multiple of Hkv
    # every head dimension of a codebook (3..256) has a decode path; the
    # workspace grows with the padded dimension
    for d in (3, 64, 100, 200, 256):
        assert tq.tq_attn_decode_workspace(2, 16, 2, 1000, d) > 0
    assert tq.tq_attn_decode_workspace(2, 16, 2, 100000, 256) > tq.tq_attn_decode_workspace(2, 16, 2, 100000, 64)
    for d in (2, 257):
        with pytest.raises(tq.TQError) as e:
            tq.tq_attn_decode_workspace(1, 8, 1, 100, d)
        assert e.value.status == _lib.TQ_ERR_INVALID


def test_quantize_rejects_null_inputs_before_device():
    L = tq.lib()
    st = L.tq_quantize_kv(None, None, None, None, 0, 1, 1, 0, None, None, None)
    assert st == _lib.TQ_ERR_INVALID
    st = L.tq_quantize_kv(None, None, None, None, 7, 1, 1, 0, None, None, None)
    assert st == _lib.TQ_ERR_INVALID and b"dtype" in L.tq_last_error()


def test_decode_rejects_null_codebooks():
    L = tq.lib()
    st = L.tq_attn_decode(None, None, None, 0, 1, 8, 1, None, None, None, 16, 0.1, None, None,
                          None, 0, None)
    assert st == _lib.TQ_ERR_INVALID


def test_paged_workspace_and_page_size_validation():
    # paged plans take whole pages per wave (at most 64); the workspace query
    # is host-only and rejects page sizes that are not powers of two >= 32
    for pt in (32, 64, 128, 4096):
        assert tq.tq_attn_decode_paged_workspace(8, 64, 8, 131072, 128, pt) > 0
    assert tq.tq_attn_decode_paged_workspace(2, 16, 2, 0, 128, 64) > 0
    for pt in (0, 16, 48, 100, 1 << 17):
        with pytest.raises(tq.TQError) as e:
            tq.tq_attn_decode_paged_workspace(2, 16, 2, 300, 128, pt)
        assert e.value.status == _lib.TQ_ERR_INVALID
    assert tq.tq_attn_decode_paged_workspace(2, 16, 2, 300, 64, 64) > 0
    with pytest.raises(tq.TQError) as e:
        tq.tq_attn_decode_paged_workspace(2, 16, 2, 300, 300, 64)
    assert e.value.status == _lib.TQ_ERR_INVALID


def test_paged_calls_reject_bad_pages_before_device():
    L = tq.lib()
    bf16 = 1
    # page size, missing table and too few table entries fail before any device call
    st = L.tq_quantize_kv_paged(None, None, ctypes.c_void_p(16), None, bf16, 1, 1, 10, 0, ctypes.c_void_p(16), 1,
                                48, None, None, None)
    assert st == _lib.TQ_ERR_INVALID and b"page_tokens" in L.tq_last_error()
    st = L.tq_quantize_kv_paged(None, None, ctypes.c_void_p(16), None, bf16, 1, 1, 10, 0, None, 1, 64,
                                None, None, None)
    assert st == _lib.TQ_ERR_INVALID and b"block_table" in L.tq_last_error()
    st = L.tq_quantize_kv_paged(None, None, ctypes.c_void_p(16), None, bf16, 1, 1, 100, 0, ctypes.c_void_p(16), 1,
                                64, None, None, None)
    assert st == _lib.TQ_ERR_INVALID and b"max_pages" in L.tq_last_error()
    st = L.tq_attn_decode_paged(None, None, None, 0, 1, 8, 1, None, None, ctypes.c_void_p(16), 1, 64, None, 100,
                                0.1, None, None, None, 0, None)
    assert st == _lib.TQ_ERR_INVALID and b"max_pages" in L.tq_last_error()


def test_solver_limit_forces_numeric_error():
    # too few iterations leave the midpoint residual above 1e-12: the
    # construction fails with TQ_ERR_NUMERIC instead of returning a codebook
    try:
        tq.tq_codebook_solver_limits(5, 1)
        with pytest.raises(tq.TQError) as e:
            tq.tq_codebook_values(128, 4)
        assert e.value.status == _lib.TQ_ERR_NUMERIC
        assert "converge" in str(e.value)
    finally:
        tq.tq_codebook_solver_limits(0, 0)
    v = tq.tq_codebook_values(128, 4)
    ref = O.Codebook(128, 4)
    assert np.max(np.abs(v["centroids"] - ref.centroids)) < 1e-10


def test_exact_scan_switch_validated():
    L = tq.lib()
    assert L.tq_ip_topk_exact_scan(2) == _lib.TQ_ERR_INVALID
    assert b"always" in L.tq_last_error()
    assert L.tq_ip_topk_exact_scan(0) == _lib.TQ_OK


def test_scan_count_validates_arguments():
    L = tq.lib()
    c = ctypes.c_int64(5)
    assert L.tq_ip_topk_scan_count(None, None, 1, 10, 1, None, ctypes.byref(c)) == _lib.TQ_ERR_INVALID


def test_argument_trace_on_stderr():
    """TQ_LOG=1 makes each hot-path entry point print its arguments, and each
    failure its status and message, on stderr (host-only calls here)."""
    import subprocess
    import sys
    code = (
        "import ctypes, kv_cache_vector_quantize_amd as tq\n"
        "L = tq.lib()\n"
        "L.tq_quantize_kv(None, None, None, None, 1, 2, 3, 4, None, None, None)\n"
        "L.tq_ip_topk(None, None, 5, None, 6, 7, None, None, None, 0, None)\n"
    )
    env = dict(os.environ, TQ_LOG="1")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120,
                       cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert r.returncode == 0, r.stderr
    assert "[tq] tq_quantize_kv" in r.stderr and "n_seq=2 n_tok=3 tok_offset=4" in r.stderr
    assert "[tq] tq_ip_topk" in r.stderr and "nq=5 n_db=6 k=7" in r.stderr
    assert "[tq] -> status 1: codebook is NULL" in r.stderr
    env["TQ_LOG"] = "0"
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=120,
                       cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert "[tq]" not in r.stderr
