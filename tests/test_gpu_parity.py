"""GPU parity: libtq.so (HIP kernels via the C ABI) against the CPU oracle.

Tolerances are those in tq_testutil.  Inputs come from ``synth`` (seeded);
the oracle reads the very tensors the GPU quantized.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import synth
import kv_cache_vector_quantize_amd as tq
from kv_cache_vector_quantize_amd import TQ_LAYOUT_ROW, TQ_LAYOUT_TILE32

import tq_testutil as U

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tq.lib()
    return "cuda"


# ----------------------------------------------------------------- codebook


def test_device_codebook_export_matches_oracle(dev):
    _say("codebook export d=128 b=3 m=128")
    cb = tq.Codebook(128, 3, qjl_m=128)
    ex = cb.export()
    ref = O.Codebook(128, 3, qjl_m=128)
    assert np.max(np.abs(ex["centroids"] - ref.centroids)) < 1e-10
    assert np.max(np.abs(ex["rot"] - ref.rot)) < 1e-12
    assert cb.row_bytes() == (48, 16)


# ----------------------------------------------------------------- quantize


def _quant_case(dev, d, bits, m, nc, dtype, n_seq, n_tok, tok_offset=0, layout=TQ_LAYOUT_ROW,
                seed=0, stride=None, factor=20.0):
    cb = tq.Codebook(d, bits, qjl_m=m, norm_correction=nc, rot_seed=3, qjl_seed=4)
    S = stride or ((tok_offset + n_tok + 31) // 32 * 32)
    codes = tq.Codes(cb, n_seq, S, layout)
    x = synth.kv_gaussian(1, n_seq, n_tok, d, seed, dtype=dtype, device="cpu",
                          channels=[i for i in (3, 77, 101) if i < d], factor=factor)[0]
    xg = x.to(dev).contiguous()
    tq.tq_quantize_kv(cb, None, xg, None, codes, None, tok_offset=tok_offset)
    torch.cuda.synchronize()
    return cb, codes, x


@pytest.mark.parametrize("d,bits,m,nc,dtype", [
    (128, 3, 128, False, "f32"),   # keys of the tiny configuration
    (128, 4, 0, False, "f32"),     # values of the tiny configuration
    (128, 4, 0, False, "bf16"),
    (128, 2, 0, True, "bf16"),
    (128, 8, 0, False, "bf16"),
    (128, 3, 0, True, "f16"),      # d = 128 without a sketch: bf16-split MFMA kernel, odd widths
    (128, 5, 0, False, "bf16"),
    (128, 6, 0, False, "f16"),
    (128, 7, 0, True, "f32"),
    (128, 1, 0, False, "bf16"),
    (128, 1, 64, False, "f16"),
    (128, 3, 128, True, "bf16"),   # keys with a sketch: split-bf16 rotation and sketch
    (128, 4, 100, False, "bf16"),
    (128, 5, 128, True, "f32"),
    (128, 2, 32, False, "f16"),
    (96, 3, 96, True, "bf16"),
    (64, 4, 32, False, "f32"),
    (40, 5, 40, False, "f32"),
    (5, 2, 3, False, "f32"),
    (200, 4, 200, False, "f32"),   # vector-search shape (wide kernel)
    (256, 3, 256, True, "bf16"),
    (160, 8, 0, False, "bf16"),
    (128, 3, 200, False, "f32"),   # sketch wider than 128 rows (wide kernel)
    (128, 6, 128, False, "bf16"),  # wide codes with a sketch: |r| < 0.03, rnorm's |x| floor applies
    (128, 8, 128, True, "f32"),
    (128, 8, 64, False, "f16"),
    (64, 7, 64, False, "f32"),     # generic kernel, wide codes with a sketch
    (200, 8, 200, True, "bf16"),
])
def test_quantize_rows_parity(dev, d, bits, m, nc, dtype):
    n_seq, n_tok = 3, 333
    _say("quantize rows", d, bits, m, nc, dtype)
    cb, codes, x = _quant_case(dev, d, bits, m, nc, dtype, n_seq, n_tok, seed=d + bits)
    got = U.read_codes(codes, n_tok)
    ocb = U.oracle_codebook(cb)
    x64 = x.float().numpy().astype(np.float64).reshape(-1, d)
    flat = dict(idx=got["idx"].reshape(-1, d), scale=got["scale"].reshape(-1),
                sign=None if got["sign"] is None else got["sign"].reshape(-1, m),
                rnorm=None if got["rnorm"] is None else got["rnorm"].reshape(-1))
    st, ref = U.compare_quant(ocb, x64, flat, name=f"d{d}b{bits}m{m}")
    ok = st.pop("vec_ok").reshape(n_seq, n_tok)
    # packed format: rows of vectors without a (zone) mismatch equal the
    # oracle's packing of its own indices byte for byte (padding bits zero)
    ridx = ref["idx"].reshape(n_seq, n_tok, d)
    for s in range(n_seq):
        ib, sb = U.seq_bytes(codes, s, n_tok)
        exp = O.pack_rows(ridx[s], bits, codes.idx_row_bytes)
        assert np.array_equal(ib[ok[s]], exp[ok[s]])
        if m:
            exs = O.pack_signs(ref["sign"].reshape(n_seq, n_tok, m)[s], codes.sign_row_bytes)
            # sign bytes may differ only where |S r| is inside the zone
            zone = (np.abs(ref["u"].reshape(n_seq, n_tok, m)[s]) < U.ZONE).any(axis=1)
            keep = ok[s] & ~zone
            assert np.array_equal(sb[keep], exs[keep])
    print(st)


@pytest.mark.parametrize("bits,layout", [(4, TQ_LAYOUT_ROW), (4, TQ_LAYOUT_TILE32), (3, TQ_LAYOUT_ROW),
                                         (5, TQ_LAYOUT_ROW), (8, TQ_LAYOUT_TILE32)])
def test_quantize_zone_rate_large(dev, bits, layout):
    """16384 bf16 vectors (2.1 M coordinates) with outlier channels: every
    index outside the 1e-5 boundary zone matches the oracle and the zone
    mismatches stay within 1e-4 of the coordinates.  This is the check that
    bounds the rotation's split-bf16 error (two parts of Pi up to 4 bits,
    three beyond)."""
    _say("quantize zone rate", bits, layout)
    n_seq, n_tok, d = 8, 2048, 128
    cb, codes, x = _quant_case(dev, d, bits, 0, False, "bf16", n_seq, n_tok, layout=layout, seed=100 + bits)
    got = U.read_codes(codes, n_tok)
    ocb = U.oracle_codebook(cb)
    x64 = x.float().numpy().astype(np.float64).reshape(-1, d)
    flat = dict(idx=got["idx"].reshape(-1, d), scale=got["scale"].reshape(-1), sign=None, rnorm=None)
    st, _ = U.compare_quant(ocb, x64, flat, name=f"zone b{bits}")
    st.pop("vec_ok")
    print(st, "mismatch rate", st["idx_mismatch"] / (n_seq * n_tok * d))


@pytest.mark.parametrize("bits,m,nc,dtype", [(3, 128, False, "bf16"), (4, 128, True, "bf16"),
                                          (2, 96, False, "f32"), (6, 128, False, "bf16"),
                                          (8, 128, True, "bf16")])
def test_quantize_sketch_large(dev, bits, m, nc, dtype):
    """16384 vectors with outlier channels through the d = 128 key kernel
    (three-part split-bf16 rotation, two-part split-bf16 sketch): indices
    outside the 1e-5 boundary zone, sign bits outside |S r| < 1e-5, scales
    (2e-6) and residual norms (1e-5) meet the oracle on 2.1 M coordinates and
    up to 2.1 M sign bits."""
    _say("quantize sketch large", bits, m, nc, dtype)
    n_seq, n_tok, d = 8, 2048, 128
    cb, codes, x = _quant_case(dev, d, bits, m, nc, dtype, n_seq, n_tok, seed=200 + bits + m)
    got = U.read_codes(codes, n_tok)
    ocb = U.oracle_codebook(cb)
    x64 = x.float().numpy().astype(np.float64).reshape(-1, d)
    flat = dict(idx=got["idx"].reshape(-1, d), scale=got["scale"].reshape(-1),
                sign=got["sign"].reshape(-1, m), rnorm=got["rnorm"].reshape(-1))
    st, _ = U.compare_quant(ocb, x64, flat, name=f"sketch b{bits} m{m}")
    st.pop("vec_ok")
    print(st)


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 5, 6, 7, 8])
def test_quantize_tile32_parity_and_append(dev, bits):
    """Values in the tile32 layout, written in three appends at unaligned
    offsets (read-modify-write of shared blocks)."""
    d, n_seq, total = 128, 2, 230
    _say("quantize tile32 append", bits)
    cb = tq.Codebook(d, bits, rot_seed=5)
    codes = tq.Codes(cb, n_seq, 256, TQ_LAYOUT_TILE32)
    x = synth.kv_gaussian(1, n_seq, total, d, 11, dtype="bf16", device="cpu", channels=[3], factor=20.0)[0]
    for a, b in [(0, 45), (45, 46), (46, 230)]:
        tq.tq_quantize_kv(None, cb, None, x[:, a:b].contiguous().to(dev), None, codes, tok_offset=a)
    torch.cuda.synchronize()
    got = U.read_codes(codes, total)
    ocb = U.oracle_codebook(cb)
    x64 = x.float().numpy().astype(np.float64).reshape(-1, d)
    flat = dict(idx=got["idx"].reshape(-1, d), scale=got["scale"].reshape(-1), sign=None, rnorm=None)
    st, ref = U.compare_quant(ocb, x64, flat, name=f"tile32 b{bits}")
    ok = st.pop("vec_ok").reshape(n_seq, total)
    # positions >= total keep zero bits and zero scale
    raw = U.seq_bytes(codes, 0, total)[0]
    assert np.all(U.read_tile32(raw, d, bits, 256)[total:] == 0)
    assert np.all(codes.scale.cpu().numpy()[total:256] == 0)
    # byte-exact against the oracle's packing of its own indices (blocks
    # holding a zone-exempt vector are skipped)
    ridx = ref["idx"].reshape(n_seq, total, d)
    for s in range(n_seq):
        ib = U.seq_bytes(codes, s, total)[0]
        exp = O.pack_tile32(ridx[s], bits, 8)
        for blk in range(8):
            toks = ok[s][blk * 32:min(total, blk * 32 + 32)]
            if toks.all():
                assert np.array_equal(ib[blk], exp[blk])


@pytest.mark.parametrize("d,bits,m,nc,layout,n_tok", [
    (128, 3, 128, False, TQ_LAYOUT_ROW, 1),
    (128, 4, 0, False, TQ_LAYOUT_TILE32, 1),
    (128, 3, 0, True, TQ_LAYOUT_TILE32, 3),
    (128, 8, 0, False, TQ_LAYOUT_TILE32, 8),
    (96, 2, 40, True, TQ_LAYOUT_ROW, 5),
    (64, 4, 64, False, TQ_LAYOUT_ROW, 2),
    (40, 5, 0, False, TQ_LAYOUT_TILE32, 1),
    (200, 4, 200, False, TQ_LAYOUT_ROW, 2),     # 256-coordinate append kernel
    (256, 3, 0, True, TQ_LAYOUT_TILE32, 3),
])
def test_quantize_append_path(dev, d, bits, m, nc, layout, n_tok):
    """Appends of a few tokens per sequence at unaligned offsets (the
    decode-time path), on top of a cache written by the bulk path."""
    _say("quantize append", d, bits, m, nc, layout, n_tok)
    n_seq, base = 3, 70
    cb = tq.Codebook(d, bits, qjl_m=m, norm_correction=nc, rot_seed=7, qjl_seed=8)
    codes = tq.Codes(cb, n_seq, 96, layout)
    x = synth.kv_gaussian(1, n_seq, base + 2 * n_tok, d, 21, dtype="bf16", device="cpu",
                          channels=[i for i in (3, 77) if i < d], factor=20.0)[0]
    tq.tq_quantize_kv(cb, None, x[:, :base].contiguous().to(dev), None, codes, None, tok_offset=0)
    tq.tq_quantize_kv(cb, None, x[:, base:base + n_tok].contiguous().to(dev), None, codes, None, tok_offset=base)
    # re-append over already written positions (must replace, not OR)
    tq.tq_quantize_kv(cb, None, x[:, base + n_tok:base + 2 * n_tok].contiguous().to(dev), None, codes, None,
                      tok_offset=base)
    torch.cuda.synchronize()
    total = base + n_tok
    expect = torch.cat([x[:, :base], x[:, base + n_tok:base + 2 * n_tok]], dim=1)
    got = U.read_codes(codes, total)
    flat = dict(idx=got["idx"].reshape(-1, d), scale=got["scale"].reshape(-1),
                sign=None if got["sign"] is None else got["sign"].reshape(-1, m),
                rnorm=None if got["rnorm"] is None else got["rnorm"].reshape(-1))
    st, _ = U.compare_quant(U.oracle_codebook(cb), expect.float().numpy().astype(np.float64).reshape(-1, d),
                            flat, name="append")
    if layout == TQ_LAYOUT_TILE32:
        assert np.all(U.read_tile32(U.seq_bytes(codes, 1, 96)[0], d, bits, 96)[total:] == 0)
    st.pop("vec_ok")
    print(st)


def test_quantize_rows_offset_and_untouched(dev):
    d, bits = 128, 4
    _say("quantize rows with offset")
    cb = tq.Codebook(d, bits)
    codes = tq.Codes(cb, 2, 128, TQ_LAYOUT_ROW)
    codes.scale.fill_(-7.0)
    x = synth.kv_gaussian(1, 2, 50, d, 3, dtype="f32", device="cpu")[0]
    tq.tq_quantize_kv(cb, None, x.to(dev), None, codes, None, tok_offset=37)
    torch.cuda.synchronize()
    sc = codes.scale.cpu().numpy().reshape(2, 128)
    assert np.all(sc[:, :37] == -7.0) and np.all(sc[:, 87:] == -7.0)
    got = U.read_codes(codes, 87)
    ocb = U.oracle_codebook(cb)
    flat = dict(idx=got["idx"][:, 37:].reshape(-1, d), scale=got["scale"][:, 37:].reshape(-1),
                sign=None, rnorm=None)
    st, _ = U.compare_quant(ocb, x.numpy().astype(np.float64).reshape(-1, d), flat)
    assert st["n"] == 100


def test_quantize_zero_vectors_and_empty(dev):
    _say("quantize zero vectors / empty")
    cb = tq.Codebook(128, 3, qjl_m=128)
    codes = tq.Codes(cb, 1, 32)
    x = torch.zeros((1, 32, 128), dtype=torch.float32, device=dev)
    tq.tq_quantize_kv(cb, None, x, None, codes, None)
    tq.tq_quantize_kv(cb, None, x[:, :0], None, codes, None)
    torch.cuda.synchronize()
    got = U.read_codes(codes, 32)
    assert np.all(got["idx"] == 4) and np.all(got["scale"] == 0) and np.all(got["rnorm"] == 0)
    ref = O.quantize(U.oracle_codebook(cb), np.zeros((32, 128)))
    assert np.array_equal(got["sign"][0], ref["sign"])


def test_quantize_argument_errors(dev):
    cb = tq.Codebook(128, 3, qjl_m=128)
    codes = tq.Codes(cb, 1, 32)
    x = torch.zeros((1, 40, 128), dtype=torch.float32, device=dev)
    with pytest.raises(tq.TQError):          # beyond seq_stride
        tq.tq_quantize_kv(cb, None, x, None, codes, None)
    tc = tq.Codes(cb, 1, 32, TQ_LAYOUT_TILE32)      # QJL signs have no tile32 layout
    tc.sign = torch.zeros(32 * 16, dtype=torch.uint8, device=dev)
    with pytest.raises(tq.TQError) as e:
        tq.tq_quantize_kv(cb, None, torch.zeros((1, 4, 128), device=dev), None, tc, None)
    assert e.value.status == 2


# ----------------------------------------------------------------- decode
#
# Decode parity: the oracle quantizes the seeded inputs and packs its own
# codes; those codes are uploaded and the GPU decodes them.  Both sides thus
# start from the same codes and the logit/output bars apply directly.  The
# GPU's own quantize -> decode chain is compared end to end as well.


def _decode_setup(dev, B, Hkv, Hq, N, kb, km, knc, vb, vnc, qdtype="bf16", kvdtype="bf16",
                  seed=0, channels=(3, 77, 101), factor=20.0):
    kcb = tq.Codebook(128, kb, qjl_m=km, norm_correction=knc, rot_seed=1, qjl_seed=2)
    vcb = tq.Codebook(128, vb, norm_correction=vnc, rot_seed=3)
    S = (N + 31) // 32 * 32
    k = synth.kv_gaussian(B, Hkv, N, 128, seed, dtype=kvdtype, device=dev, channels=list(channels), factor=factor)
    v = synth.kv_gaussian(B, Hkv, N, 128, seed + 1, dtype=kvdtype, device=dev, channels=list(channels), factor=factor)
    q = synth.queries_gaussian(B, Hq, 128, seed + 2, dtype=qdtype, device=dev)
    return kcb, vcb, S, k, v, q


def _oracle_codes_on_gpu(kcb, vcb, S, k, v, B, Hkv, N):
    okc, ovc = U.oracle_codebook(kcb), U.oracle_codebook(vcb)
    kc = tq.Codes(kcb, B * Hkv, S, TQ_LAYOUT_ROW)
    vc = tq.Codes(vcb, B * Hkv, S, TQ_LAYOUT_TILE32)
    k64 = U.to_f64(k).reshape(B * Hkv, N, 128)
    v64 = U.to_f64(v).reshape(B * Hkv, N, 128)
    rk = [O.quantize(okc, k64[s]) for s in range(B * Hkv)]
    rv = [O.quantize(ovc, v64[s]) for s in range(B * Hkv)]
    for s in range(B * Hkv):
        U.upload_oracle_codes(kc, s, rk[s], N)
        U.upload_oracle_codes(vc, s, rv[s], N)
    kd = U.oracle_cache(rk, B, Hkv, N, kcb.m > 0)
    vd = U.oracle_cache(rv, B, Hkv, N, False)
    return okc, ovc, kc, vc, kd, vd


def _run_decode(dev, kcb, vcb, q, kc, vc, N, seq_lens=None):
    B, Hq, _ = q.shape
    logits = torch.full((B, Hq, N), 123.0, dtype=torch.float32, device=dev)
    sl = torch.tensor(seq_lens, dtype=torch.int32, device=dev) if seq_lens is not None else None
    tau = 1.0 / math.sqrt(128)
    out = tq.tq_attn_decode(kcb, vcb, q, kc, vc, N, tau, seq_lens=sl, logits=logits)
    torch.cuda.synchronize()
    return logits.cpu().numpy(), out.cpu().numpy(), tau


def test_decode_tiny_configuration(dev):
    """1 KV head, 8 queries, d = 128, N = 4096, fp32 inputs with outlier
    channels 3/77/101 x20; keys 3-bit + QJL m=128, values 4-bit."""
    _say("decode tiny configuration")
    k, v, q = synth.tiny_case(0)
    N = 4096
    kcb = tq.Codebook(128, 3, qjl_m=128)
    vcb = tq.Codebook(128, 4, rot_seed=3)
    kg = torch.from_numpy(k)[None, None].to(dev)
    vg = torch.from_numpy(v)[None, None].to(dev)
    qg = torch.from_numpy(q)[None].to(dev)
    okc, ovc, kc, vc, kd, vd = _oracle_codes_on_gpu(kcb, vcb, N, kg, vg, 1, 1, N)
    lg, out, tau = _run_decode(dev, kcb, vcb, qg, kc, vc, N)
    st = U.check_decode(okc, ovc, q[None].astype(np.float64), kd, vd, tau, lg, out, name="tiny")
    # end to end: GPU quantize + GPU decode vs oracle quantize + oracle decode
    kc2 = tq.Codes(kcb, 1, N, TQ_LAYOUT_ROW)
    vc2 = tq.Codes(vcb, 1, N, TQ_LAYOUT_TILE32)
    tq.tq_quantize_kv(kcb, vcb, kg[0], vg[0], kc2, vc2)
    lg2, out2, _ = _run_decode(dev, kcb, vcb, qg, kc2, vc2, N)
    st_k, _ = U.compare_quant(okc, k.astype(np.float64), {n: a[0] if a is not None else None for n, a in U.read_codes(kc2, N).items()}, "K")
    st_v, _ = U.compare_quant(ovc, v.astype(np.float64), {n: a[0] if a is not None else None for n, a in U.read_codes(vc2, N).items()}, "V")
    lg_ref, out_ref = O.attn_decode(okc, ovc, q[None].astype(np.float64), kd, vd, tau)
    e2e = U.check_end_to_end(okc, ovc, q[None].astype(np.float64), kc2, vc2, N, 1, 1, tau, lg2, out2, out_ref,
                             [st_k, st_v])
    print(st, "end to end", e2e, "K zone mismatches", st_k["idx_mismatch"], "V", st_v["idx_mismatch"])


@pytest.mark.parametrize("B,Hkv,Hq,N,lens", [
    (2, 2, 16, 1000, None),          # ragged tail, two KV heads
    (3, 1, 8, 700, [700, 333, 0]),   # per-sequence lengths incl. empty
    (1, 2, 4, 96, None),             # g = 2 (<8 queries per KV head)
    (1, 2, 24, 160, [150]),          # g = 12: two query groups
    (1, 1, 8, 1, None),              # one token
])
def test_decode_shapes(dev, B, Hkv, Hq, N, lens):
    _say("decode shapes", B, Hkv, Hq, N, lens)
    kcb, vcb, S, k, v, q = _decode_setup(dev, B, Hkv, Hq, N, 3, 128, False, 4, False, seed=N)
    okc, ovc, kc, vc, kd, vd = _oracle_codes_on_gpu(kcb, vcb, S, k, v, B, Hkv, N)
    lg, out, tau = _run_decode(dev, kcb, vcb, q, kc, vc, N, seq_lens=lens)
    st = U.check_decode(okc, ovc, U.to_f64(q), kd, vd, tau, lg, out, n_valid=lens, name="shapes")
    if lens is not None and 0 in lens:
        assert np.all(out[lens.index(0)] == 0)
    print(st)


@pytest.mark.parametrize("kb,vb,nc", [(8, 4, False), (4, 4, True), (3, 4, True), (3, 3, True),
                                      (2, 2, True), (2, 2, False), (4, 8, False), (2, 3, False)])
def test_decode_bit_variants(dev, kb, vb, nc):
    _say("decode variant", kb, vb, nc)
    B, Hkv, Hq, N = 2, 2, 16, 512
    kcb, vcb, S, k, v, q = _decode_setup(dev, B, Hkv, Hq, N, kb, 0, nc, vb, nc, seed=kb * 10 + vb)
    okc, ovc, kc, vc, kd, vd = _oracle_codes_on_gpu(kcb, vcb, S, k, v, B, Hkv, N)
    lg, out, tau = _run_decode(dev, kcb, vcb, q, kc, vc, N)
    print(U.check_decode(okc, ovc, U.to_f64(q), kd, vd, tau, lg, out, name=f"k{kb}v{vb}"))


def test_decode_qjl_smaller_m_f32_query(dev):
    _say("decode QJL m=64, fp32 query")
    B, Hkv, Hq, N = 1, 1, 8, 256
    kcb, vcb, S, k, v, q = _decode_setup(dev, B, Hkv, Hq, N, 3, 64, False, 4, False, qdtype="f32")
    okc, ovc, kc, vc, kd, vd = _oracle_codes_on_gpu(kcb, vcb, S, k, v, B, Hkv, N)
    lg, out, tau = _run_decode(dev, kcb, vcb, q, kc, vc, N)
    U.check_decode(okc, ovc, U.to_f64(q), kd, vd, tau, lg, out, name="m64")


def test_decode_full_size_128k(dev):
    """The 128K decode layer at full size and in the launch configuration the
    benchmark times: B=8, Hq=64, Hkv=8, d=128, N=131072, bf16 K/V N(0,1) with
    channels 3/77/101 x20, bf16 queries, keys 3-bit + QJL m=128, values 4-bit.
    The GPU quantizes the whole cache; the oracle's codes then replace three
    sampled sequences (first, middle, last), and those sequences' outputs
    (call without logits, as timed) and logits (second call) must meet the
    bars against the oracle's decode of the same codes."""
    B, Hq, Hkv, N = 8, 64, 8, 131072
    _say("decode full size 128K")
    kcb, vcb, S, k, v, q = _decode_setup(dev, B, Hkv, Hq, N, 3, 128, False, 4, False, seed=0)
    kc = tq.Codes(kcb, B * Hkv, S, TQ_LAYOUT_ROW)
    vc = tq.Codes(vcb, B * Hkv, S, TQ_LAYOUT_TILE32)
    tq.tq_quantize_kv(kcb, vcb, k.view(B * Hkv, N, 128), v.view(B * Hkv, N, 128), kc, vc)
    okc, ovc = U.oracle_codebook(kcb), U.oracle_codebook(vcb)
    sampled = [(0, 0), (3, 5), (7, 7)]
    refs = {}
    for b, h in sampled:
        s = b * Hkv + h
        rk = O.quantize(okc, U.to_f64(k[b, h]))
        rv = O.quantize(ovc, U.to_f64(v[b, h]))
        U.upload_oracle_codes(kc, s, rk, N)
        U.upload_oracle_codes(vc, s, rv, N)
        refs[(b, h)] = (rk, rv)
    torch.cuda.synchronize()
    tau = 1.0 / math.sqrt(128)
    ws = torch.empty(tq.tq_attn_decode_workspace(B, Hq, Hkv, N, 128), dtype=torch.uint8, device=dev)
    out = torch.empty((B, Hq, 128), dtype=torch.float32, device=dev)
    tq.tq_attn_decode(kcb, vcb, q, kc, vc, N, tau, out=out, workspace=ws)
    torch.cuda.synchronize()
    out_np = out.cpu().numpy()
    assert np.all(np.isfinite(out_np))
    lg_t = torch.full((B, Hq, N), 123.0, dtype=torch.float32, device=dev)
    out2 = tq.tq_attn_decode(kcb, vcb, q, kc, vc, N, tau, logits=lg_t, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(out2, out), "outputs differ between the calls with and without logits"
    q64 = U.to_f64(q)
    g = Hq // Hkv
    worst = {}
    for (b, h), (rk, rv) in refs.items():
        heads = slice(h * g, (h + 1) * g)
        kd = U.oracle_cache([rk], 1, 1, N, True)
        vd = U.oracle_cache([rv], 1, 1, N, False)
        lg_gpu = lg_t[b, heads].cpu().numpy()[None]
        st = U.check_decode(okc, ovc, q64[b:b + 1, heads], kd, vd, tau, lg_gpu,
                            out_np[b:b + 1, heads], name=f"128K ({b},{h})")
        worst[(b, h)] = st
    print(worst)


@pytest.mark.parametrize("kb,vb,nc", [(8, 4, True), (4, 4, True), (3, 4, True), (3, 3, True),
                                      (2, 2, True), (2, 2, False)])
def test_decode_bit_sweep_full_shape(dev, kb, vb, nc):
    """Every variant of the bit-width sweep at the shape and in the launch
    configuration the benchmark times it (B=32, Hq=32, Hkv=4, d=128,
    N=32768: 16 waves per row, 2048 tokens = 64 tiles per wave, so both
    register buffers of the tile pipeline and the multi-tile online softmax
    run).  The GPU quantizes the whole cache; the oracle's codes replace two
    sampled sequences, whose keys carry planted tokens aligned with a query
    (logits ~25, ~40, ~60 at tiles 21, 40 and 59 of one wave's chunk, each
    more than 2^8 above the running maximum in base 2), so the lazy maximum
    moves mid-chunk, on both buffers.  Logits and outputs of the sampled rows
    meet the bars against the oracle's decode of the same codes."""
    B, Hq, Hkv, N, d = 32, 32, 4, 32768, 128
    g = Hq // Hkv
    _say("decode bit sweep full shape", kb, vb, nc)
    kcb, vcb, S, k, v, q = _decode_setup(dev, B, Hkv, Hq, N, kb, 0, nc, vb, nc, seed=20)
    kc = tq.Codes(kcb, B * Hkv, S, TQ_LAYOUT_ROW)
    vc = tq.Codes(vcb, B * Hkv, S, TQ_LAYOUT_TILE32)
    tq.tq_quantize_kv(kcb, vcb, k.view(B * Hkv, N, d), v.view(B * Hkv, N, d), kc, vc)
    okc, ovc = U.oracle_codebook(kcb), U.oracle_codebook(vcb)
    tau = 1.0 / math.sqrt(d)
    q64 = U.to_f64(q)
    chunk0 = 3 * 2048                           # the chunk of wave 3 of each row
    refs = {}
    for b, h in [(0, 0), (B - 1, Hkv - 1)]:
        k64 = U.to_f64(k[b, h])
        qa = q64[b, h * g]                        # first query head of the group
        for off, target in ((700, 25.0), (1300, 40.0), (1900, 60.0)):
            kk = qa * (target / (tau * (qa @ qa)))
            k64[chunk0 + off] = torch.tensor(kk, dtype=torch.float32).to(torch.bfloat16).double().numpy()
        rk = O.quantize(okc, k64)
        rv = O.quantize(ovc, U.to_f64(v[b, h]))
        U.upload_oracle_codes(kc, b * Hkv + h, rk, N)
        U.upload_oracle_codes(vc, b * Hkv + h, rv, N)
        refs[(b, h)] = (rk, rv)
    torch.cuda.synchronize()
    ws = torch.empty(tq.tq_attn_decode_workspace(B, Hq, Hkv, N, d), dtype=torch.uint8, device=dev)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    lg_t = torch.full((B, Hq, N), 123.0, dtype=torch.float32, device=dev)
    tq.tq_attn_decode(kcb, vcb, q, kc, vc, N, tau, out=out, logits=lg_t, workspace=ws)
    torch.cuda.synchronize()
    out_np = out.cpu().numpy()
    assert np.all(np.isfinite(out_np))
    worst = {}
    for (b, h), (rk, rv) in refs.items():
        heads = slice(h * g, (h + 1) * g)
        lg_gpu = lg_t[b, heads].cpu().numpy()[None]
        assert lg_gpu[0, 0, chunk0 + 1900] > 50.0, "planted logit missing"
        st = U.check_decode(okc, ovc, q64[b:b + 1, heads], U.oracle_cache([rk], 1, 1, N, False),
                            U.oracle_cache([rv], 1, 1, N, False), tau, lg_gpu, out_np[b:b + 1, heads],
                            name=f"k{kb}v{vb} ({b},{h})")
        worst[(b, h)] = st
    print(worst)


def test_quantize_and_dequantize_full_size(dev):
    """The quantize layer at full size and in the launch configuration the
    benchmark times: B=16, Hkv=8, 32768 tokens, d=128, bf16 K and V with 4
    outlier channels per head x15, 4-bit codes, K in the row layout and V in
    tile32, quantized in one call.  Three sampled sequences of each tensor
    meet the quantize rules against the oracle's quantization of the same
    inputs.  The oracle's codes of those sequences then replace the GPU's, the
    whole layer is dequantized to bf16 as the benchmark times it, and the
    sampled sequences match the oracle's reconstruction of its own codes
    (1e-4 of each vector's max |x_hat| plus one bf16 rounding)."""
    B, H, N, d = 16, 8, 32768, 128
    _say("quantize + dequantize full size")
    chk = synth.outlier_channels(10, H, d, 4)
    chv = synth.outlier_channels(11, H, d, 4)
    k = synth.kv_gaussian(B, H, N, d, 10, dtype="bf16", device=dev, per_head_channels=chk, factor=15.0)
    v = synth.kv_gaussian(B, H, N, d, 11, dtype="bf16", device=dev, per_head_channels=chv, factor=15.0)
    kcb, vcb = tq.Codebook(d, 4, rot_seed=1), tq.Codebook(d, 4, rot_seed=3)
    kc = tq.Codes(kcb, B * H, N, TQ_LAYOUT_ROW)
    vc = tq.Codes(vcb, B * H, N, TQ_LAYOUT_TILE32)
    tq.tq_quantize_kv(kcb, vcb, k.view(B * H, N, d), v.view(B * H, N, d), kc, vc)
    torch.cuda.synchronize()
    sampled = [0, 77, B * H - 1]
    refs = {}
    stats = {}
    for cb, codes, x, name in ((kcb, kc, k, "K"), (vcb, vc, v, "V")):
        ocb = U.oracle_codebook(cb)
        got = U.read_codes(codes, N, seqs=sampled)
        for i, sq in enumerate(sampled):
            x64 = U.to_f64(x.view(B * H, N, d)[sq])
            flat = dict(idx=got["idx"][i], scale=got["scale"][i], sign=None, rnorm=None)
            st, ref = U.compare_quant(ocb, x64, flat, name=f"{name} seq {sq}")
            st.pop("vec_ok")
            stats[(name, sq)] = st
            U.upload_oracle_codes(codes, sq, ref, N)
            refs[(name, sq)] = (ocb, ref)
    ko = torch.empty((B * H, N, d), dtype=torch.bfloat16, device=dev)
    vo = torch.empty_like(ko)
    tq.tq_dequantize(kcb, kc, B * H, N, out=ko)
    tq.tq_dequantize(vcb, vc, B * H, N, out=vo)
    torch.cuda.synchronize()
    for (name, sq), (ocb, ref) in refs.items():
        out = (ko if name == "K" else vo)[sq].float().cpu().numpy().astype(np.float64)
        xh = O.dequantize(ocb, ref["idx"], ref["scale"].astype(np.float32).astype(np.float64))
        amax = np.max(np.abs(xh), axis=1, keepdims=True)
        err = np.abs(out - xh)
        assert np.all(err <= 1e-4 * amax + 2.0 ** -8 * np.abs(xh)), f"{name} seq {sq}: dequantize"
    print(stats)


def test_decode_deterministic(dev):
    _say("decode determinism")
    B, Hkv, Hq, N = 2, 2, 16, 2048
    kcb, vcb, S, k, v, q = _decode_setup(dev, B, Hkv, Hq, N, 3, 128, False, 4, False, seed=5)
    kc = tq.Codes(kcb, B * Hkv, S, TQ_LAYOUT_ROW)
    vc = tq.Codes(vcb, B * Hkv, S, TQ_LAYOUT_TILE32)
    tq.tq_quantize_kv(kcb, vcb, k.reshape(B * Hkv, N, 128), v.reshape(B * Hkv, N, 128), kc, vc)
    idx1 = kc.idx.clone()
    lg1, out1, _ = _run_decode(dev, kcb, vcb, q, kc, vc, N)
    tq.tq_quantize_kv(kcb, vcb, k.reshape(B * Hkv, N, 128), v.reshape(B * Hkv, N, 128), kc, vc)
    lg2, out2, _ = _run_decode(dev, kcb, vcb, q, kc, vc, N)
    assert torch.equal(idx1, kc.idx)
    assert np.array_equal(lg1, lg2) and np.array_equal(out1, out2)


def test_stream_measurement_kernels(dev):
    """The streaming read and write kernels the ceilings are measured with:
    the write sets every word (and nothing past the range), the read leaves
    the sink alone unless the XOR of the buffer equals its fixed value."""
    _say("stream read / write helpers")
    buf = torch.zeros(4096 + 64, dtype=torch.int32, device=dev)
    tq.tq_stream_write(buf[:4096], 0x12345678)
    torch.cuda.synchronize()
    assert bool((buf[:4096] == 0x12345678).all()) and bool((buf[4096:] == 0).all())
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    tq.tq_stream_read(buf[:4096], sink)
    torch.cuda.synchronize()
    assert bool((sink == 0).all())
    with pytest.raises(tq.TQError):
        tq.tq_stream_write(buf[:3], 0)
