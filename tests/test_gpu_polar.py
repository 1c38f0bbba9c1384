"""GPU parity of the PolarQuant encoding (libtq.so through the C ABI)
against the polar oracle.

Page "什么是TurboQuant？…" (a2a-mcp.org blog), "第一阶段：随机旋转 +
PolarQuant 压缩" item 2; "第二阶段：QJL 残差校正"; "如何实现 TurboQuant" item 1
(attention straight from the stored codes).

Tolerances: an angle's code is bit-exact unless the oracle's pair point lies
within 1e-5 (in the rotated unit-scale domain: radius times |sin(angle - t)|)
of a decision ray of its level, the polar form of the scalar path's
boundary zone; such mismatches must stay <= 1e-4 of the angles.  Scale,
signs and rnorm as for the scalar codes; logits 1e-4 of the row's max, outputs
2e-3 max-abs.
"""
import math

import numpy as np
import pytest
import torch

import oracle as O
import synth
import kv_cache_vector_quantize_amd as tq
from kv_cache_vector_quantize_amd import TQ_LAYOUT_ROW, TQ_LAYOUT_TILE32, _lib

import tq_testutil as U

P = O.polar
pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tq.lib()
    return "cuda"


def _opcb(cb):
    return P.PolarCodebook(cb.d, cb.b1, cb.br, qjl_m=cb.m, rot_seed=cb.rot_seed, qjl_seed=cb.qjl_seed)


def _read_polar(raw, d, b1, br):
    """uint8 [n, row_bytes] -> per-level indices (plain bit arithmetic)."""
    bits = U._bits_le(raw).astype(np.int64)
    out, pos = [], 0
    for lv in range(1, d.bit_length()):
        b = b1 if lv == 1 else br
        nf = d >> lv
        p = pos + np.arange(nf)[:, None] * b + np.arange(b)[None, :]
        out.append((bits[:, p] << np.arange(b)).sum(-1))
        pos += nf * b
    return out


def _compare(ocb, x64, got_idx, got_scale, got_sign, got_rnorm, name):
    """Asserts the tolerances; returns (stats, oracle result, per-vector ok)."""
    ref = P.quantize(ocb, x64)
    zone = P.boundary_distance(ocb, ref)
    n = x64.shape[0]
    mism_vec = np.zeros(n, dtype=bool)
    total, mism_count = 0, 0
    for lv in range(ocb.levels):
        mis = got_idx[lv] != ref["idx"][lv]
        bad = mis & ~(zone[lv] < U.ZONE)
        assert not bad.any(), f"{name}: level {lv + 1}: {bad.sum()} mismatches outside the zone"
        mism_vec |= mis.any(axis=1)
        total += mis.size
        mism_count += int(mis.sum())
    assert mism_count <= max(1, U.IDX_BUDGET * total), f"{name}: {mism_count} zone mismatches"
    ok = ~mism_vec
    rel = np.abs(got_scale - ref["scale"]) / np.maximum(ref["scale"], 1e-30)
    assert np.all(rel <= 2e-6), f"{name}: scale rel err {rel.max()}"
    st = dict(n=n, mismatches=mism_count, scale_rel=float(rel.max()))
    if ocb.m > 0:
        smis = (got_sign != ref["sign"]) & ok[:, None] & (np.abs(ref["u"]) >= U.ZONE)
        assert not smis.any(), f"{name}: {smis.sum()} sign mismatches"
        nx = np.sqrt(np.sum(x64 * x64, axis=1))
        rerr = np.abs(got_rnorm - ref["rnorm"])
        okr = rerr <= np.maximum(1e-5 * ref["rnorm"], U.RNORM_XFLOOR * nx)
        assert np.all(okr[ok]), f"{name}: rnorm err {rerr[ok & ~okr].max()}"
        st["rnorm_rel"] = float((rerr / np.maximum(ref["rnorm"], 1e-30))[ok].max())
    return st, ref, ok


def _read_all(codes, cb, n_tok, s=0):
    ib, sb = U.seq_bytes(codes, s, n_tok)
    S = codes.seq_stride
    idx = _read_polar(ib, cb.d, cb.b1, cb.br)
    sc = codes.scale.cpu().numpy()[s * S:s * S + n_tok].astype(np.float64)
    sg = rn = None
    if cb.m > 0:
        sg = U._bits_le(sb)[:, :cb.m]
        rn = codes.rnorm.cpu().numpy()[s * S:s * S + n_tok].astype(np.float64)
    return idx, sc, sg, rn, ib


@pytest.mark.parametrize("d,b1,br,m,dtype", [
    (128, 4, 2, 0, "bf16"),
    (128, 4, 2, 128, "bf16"),     # the 3-bit-total keys with a sketch
    (128, 4, 2, 64, "f32"),
    (128, 8, 6, 128, "f32"),      # wide codes
    (128, 1, 1, 0, "f16"),
    (64, 5, 3, 64, "f16"),
    (32, 3, 2, 32, "f32"),
    (16, 4, 2, 0, "bf16"),
    (8, 2, 1, 8, "f32"),
    (4, 3, 2, 0, "f32"),
])
def test_polar_quantize_parity(dev, d, b1, br, m, dtype):
    _say("polar quantize", d, b1, br, m, dtype)
    n_seq, n_tok = 2, 300
    cb = tq.PolarCodebook(d, b1, br, qjl_m=m, rot_seed=3, qjl_seed=4)
    ocb = _opcb(cb)
    codes = tq.Codes(cb, n_seq, 320, TQ_LAYOUT_ROW)
    x = synth.kv_gaussian(1, n_seq, n_tok, d, d + b1, dtype=dtype, device="cpu",
                          channels=[i for i in (3, 77, 101) if i < d], factor=20.0)[0]
    # written in three calls: a bulk prefix, one appended token, the rest
    for a, b in [(0, 200), (200, 201), (201, n_tok)]:
        tq.tq_quantize_kv(cb, None, x[:, a:b].contiguous().to(dev), None, codes, None, tok_offset=a)
    torch.cuda.synchronize()
    for s in range(n_seq):
        x64 = x[s].float().numpy().astype(np.float64)
        idx, sc, sg, rn, ib = _read_all(codes, cb, n_tok, s)
        st, ref, ok = _compare(ocb, x64, idx, sc, sg, rn, f"d{d} ({b1},{br}) m{m} seq {s}")
        exp = P.pack_rows(ref["idx"], d, b1, br, codes.idx_row_bytes)
        assert np.array_equal(ib[ok], exp[ok]), "packed rows differ"
        print(st)
    # positions past the written range keep zero codes
    assert np.all(U.seq_bytes(codes, 0, 320)[0][n_tok:] == 0)


def test_polar_quantize_zero_vector_and_large(dev):
    _say("polar quantize 16384 vectors incl. zeros")
    d, n = 128, 16384
    cb = tq.PolarCodebook(d, 4, 2, qjl_m=128, rot_seed=1, qjl_seed=2)
    ocb = _opcb(cb)
    x = synth.kv_gaussian(1, 1, n, d, 77, dtype="bf16", device="cpu", channels=[3, 77, 101], factor=20.0)[0]
    x[0, 5] = 0
    codes = tq.Codes(cb, 1, n, TQ_LAYOUT_ROW)
    tq.tq_quantize_kv(cb, None, x.to(dev), None, codes, None)
    torch.cuda.synchronize()
    idx, sc, sg, rn, _ = _read_all(codes, cb, n)
    st, ref, _ = _compare(ocb, x[0].float().numpy().astype(np.float64), idx, sc, sg, rn, "large")
    assert sc[5] == 0 and rn[5] == 0
    print(st, "mismatch rate", st["mismatches"] / (n * (d - 1)))


@pytest.mark.parametrize("d,b1,br,m,out", [(128, 4, 2, 128, "f32"), (128, 4, 2, 0, "bf16"), (64, 5, 3, 64, "f32"),
                                          (16, 3, 2, 16, "f16")])
def test_polar_dequantize_parity(dev, d, b1, br, m, out):
    _say("polar dequantize", d, b1, br, m, out)
    n_seq, n_tok, off = 2, 150, 7
    cb = tq.PolarCodebook(d, b1, br, qjl_m=m, rot_seed=5, qjl_seed=6)
    ocb = _opcb(cb)
    codes = tq.Codes(cb, n_seq, 192, TQ_LAYOUT_ROW)
    x = np.random.default_rng(d).standard_normal((n_seq, 192, d)) * 3
    refs = [P.quantize(ocb, x[s]) for s in range(n_seq)]
    for s in range(n_seq):
        _upload(codes, s, refs[s], 192)
    dt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[out]
    o = torch.empty((n_seq, n_tok, d), dtype=dt, device=dev)
    tq.tq_dequantize(cb, codes, n_seq, n_tok, tok_offset=off, out=o)
    torch.cuda.synchronize()
    got = o.float().cpu().numpy().astype(np.float64)
    for s in range(n_seq):
        r = refs[s]
        sl = slice(off, off + n_tok)
        xh = P.dequantize(ocb, [a[sl] for a in r["idx"]], r["scale"][sl].astype(np.float32).astype(np.float64),
                          None if m == 0 else r["sign"][sl],
                          None if m == 0 else r["rnorm"][sl].astype(np.float32).astype(np.float64))
        amax = np.max(np.abs(xh), axis=1, keepdims=True)
        tol = 1e-5 * amax + {"f32": 0.0, "bf16": 2.0 ** -8, "f16": 2.0 ** -11}[out] * np.abs(xh)
        assert np.all(np.abs(got[s] - xh) <= tol), float(np.max(np.abs(got[s] - xh) / amax))


def _upload(codes, s, ref, n_tok):
    cb = codes.cb
    S = codes.seq_stride
    rows = P.pack_rows(ref["idx"], cb.d, cb.b1, cb.br, codes.idx_row_bytes)
    a = s * S * codes.idx_row_bytes
    codes.idx[a:a + rows.size] = torch.from_numpy(rows.reshape(-1)).to(codes.idx.device)
    codes.scale[s * S:s * S + n_tok] = torch.from_numpy(ref["scale"][:n_tok].astype(np.float32)).to(codes.scale.device)
    if cb.m > 0:
        sg = O.pack_signs(ref["sign"], codes.sign_row_bytes)
        a = s * S * codes.sign_row_bytes
        codes.sign[a:a + sg.size] = torch.from_numpy(sg.reshape(-1)).to(codes.sign.device)
        codes.rnorm[s * S:s * S + n_tok] = torch.from_numpy(ref["rnorm"][:n_tok].astype(np.float32)).to(codes.rnorm.device)


def _polar_cache(refs, B, Hkv, N, with_sign):
    kc = dict(idx=[np.stack([r["idx"][lv] for r in refs]).reshape(B, Hkv, N, -1) for lv in range(len(refs[0]["idx"]))],
              scale=np.stack([r["scale"].astype(np.float32) for r in refs]).astype(np.float64).reshape(B, Hkv, N))
    if with_sign:
        kc["sign"] = np.stack([r["sign"] for r in refs]).reshape(B, Hkv, N, -1)
        kc["rnorm"] = np.stack([r["rnorm"].astype(np.float32) for r in refs]).astype(np.float64).reshape(B, Hkv, N)
    return kc


def _check(okc, ovc, q64, kc, vc, tau, lg, out, lens=None, name=""):
    lg_ref, out_ref = P.attn_decode(okc, ovc, q64, kc, vc, tau, n_valid=lens)
    B, Hq, N = lg_ref.shape
    worst_l = 0.0
    for b in range(B):
        nb = N if lens is None else lens[b]
        for h in range(Hq):
            if nb < N:
                assert np.all(np.isneginf(lg[b, h, nb:]))
            if nb:
                err = np.max(np.abs(lg[b, h, :nb] - lg_ref[b, h, :nb]))
                sc = np.max(np.abs(lg_ref[b, h, :nb]))
                worst_l = max(worst_l, err / sc)
                assert err <= U.LOGIT_RTOL * sc, f"{name}: logits ({b},{h}) {err} vs {sc}"
    oerr = float(np.max(np.abs(out - out_ref)))
    assert oerr <= U.OUT_ATOL, f"{name}: outputs {oerr}"
    return dict(logit_rel=worst_l, out_abs=oerr)


@pytest.mark.parametrize("B,Hkv,Hq,N,m,lens", [
    (1, 1, 8, 4096, 128, None),     # the tiny configuration's shape, polar keys + sketch
    (2, 2, 16, 1000, 0, None),      # ragged tail, no sketch
    (3, 1, 8, 700, 128, [700, 333, 0]),
    (1, 2, 24, 160, 64, [150]),     # two query groups, m = 64
])
def test_polar_decode_parity(dev, B, Hkv, Hq, N, m, lens):
    _say("polar decode", B, Hkv, Hq, N, m, lens)
    d = 128
    kcb = tq.PolarCodebook(d, 4, 2, qjl_m=m, rot_seed=1, qjl_seed=2)
    vcb = tq.Codebook(d, 4, rot_seed=3)
    okc, ovc = _opcb(kcb), U.oracle_codebook(vcb)
    S = (N + 31) // 32 * 32
    k = synth.kv_gaussian(B, Hkv, N, d, N + m, dtype="bf16", device=dev, channels=[3, 77, 101], factor=20.0)
    v = synth.kv_gaussian(B, Hkv, N, d, N + m + 1, dtype="bf16", device=dev, channels=[3, 77, 101], factor=20.0)
    q = synth.queries_gaussian(B, Hq, d, N + m + 2, dtype="bf16", device=dev)
    kc = tq.Codes(kcb, B * Hkv, S, TQ_LAYOUT_ROW)
    vc = tq.Codes(vcb, B * Hkv, S, TQ_LAYOUT_TILE32)
    k64 = U.to_f64(k).reshape(B * Hkv, N, d)
    v64 = U.to_f64(v).reshape(B * Hkv, N, d)
    rk = [P.quantize(okc, k64[s]) for s in range(B * Hkv)]
    rv = [O.quantize(ovc, v64[s]) for s in range(B * Hkv)]
    for s in range(B * Hkv):
        _upload(kc, s, rk[s], N)
        U.upload_oracle_codes(vc, s, rv[s], N)
    tau = 1 / math.sqrt(d)
    sl = torch.tensor(lens, dtype=torch.int32, device=dev) if lens is not None else None
    lg = torch.full((B, Hq, N), 123.0, dtype=torch.float32, device=dev)
    out = tq.tq_attn_decode(kcb, vcb, q, kc, vc, N, tau, seq_lens=sl, logits=lg)
    torch.cuda.synchronize()
    st = _check(okc, ovc, U.to_f64(q), _polar_cache(rk, B, Hkv, N, m > 0), U.oracle_cache(rv, B, Hkv, N, False),
                tau, lg.cpu().numpy(), out.cpu().numpy(), lens, name="polar decode")
    print(st)


def test_polar_decode_full_size_128k(dev):
    """The 128K decode layer with polar keys (4, 2) + QJL m=128 and 4-bit
    values, in the launch configuration the benchmark times: the GPU
    quantizes the whole cache, the oracle's codes replace two sampled
    sequences, whose logits and outputs meet the bars."""
    B, Hq, Hkv, N, d = 8, 64, 8, 131072, 128
    g = Hq // Hkv
    _say("polar decode full size 128K")
    kcb = tq.PolarCodebook(d, 4, 2, qjl_m=128, rot_seed=1, qjl_seed=2)
    vcb = tq.Codebook(d, 4, rot_seed=3)
    okc, ovc = _opcb(kcb), U.oracle_codebook(vcb)
    k = synth.kv_gaussian(B, Hkv, N, d, 0, dtype="bf16", device=dev, channels=[3, 77, 101], factor=20.0)
    v = synth.kv_gaussian(B, Hkv, N, d, 1, dtype="bf16", device=dev, channels=[3, 77, 101], factor=20.0)
    q = synth.queries_gaussian(B, Hq, d, 2, dtype="bf16", device=dev)
    kc = tq.Codes(kcb, B * Hkv, N, TQ_LAYOUT_ROW)
    vc = tq.Codes(vcb, B * Hkv, N, TQ_LAYOUT_TILE32)
    tq.tq_quantize_kv(kcb, vcb, k.view(B * Hkv, N, d), v.view(B * Hkv, N, d), kc, vc)
    refs = {}
    for b, h in [(0, 0), (7, 7)]:
        rk = P.quantize(okc, U.to_f64(k[b, h]))
        rv = O.quantize(ovc, U.to_f64(v[b, h]))
        _upload(kc, b * Hkv + h, rk, N)
        U.upload_oracle_codes(vc, b * Hkv + h, rv, N)
        refs[(b, h)] = (rk, rv)
    tau = 1 / math.sqrt(d)
    lg = torch.full((B, Hq, N), 123.0, dtype=torch.float32, device=dev)
    out = tq.tq_attn_decode(kcb, vcb, q, kc, vc, N, tau, logits=lg)
    torch.cuda.synchronize()
    out_np = out.cpu().numpy()
    assert np.all(np.isfinite(out_np))
    q64 = U.to_f64(q)
    for (b, h), (rk, rv) in refs.items():
        hs = slice(h * g, (h + 1) * g)
        st = _check(okc, ovc, q64[b:b + 1, hs], _polar_cache([rk], 1, 1, N, True), U.oracle_cache([rv], 1, 1, N, False),
                    tau, lg[b, hs].cpu().numpy()[None], out_np[b:b + 1, hs], name=f"128K ({b},{h})")
        print((b, h), st)


def test_polar_end_to_end(dev):
    # GPU quantize + GPU decode against the oracle's quantize + decode
    _say("polar end to end")
    d, N = 128, 2048
    k, v, qn = synth.tiny_case(3, n=N)
    kcb = tq.PolarCodebook(d, 4, 2, qjl_m=128)
    vcb = tq.Codebook(d, 4, rot_seed=3)
    okc, ovc = _opcb(kcb), U.oracle_codebook(vcb)
    kc = tq.Codes(kcb, 1, N, TQ_LAYOUT_ROW)
    vc = tq.Codes(vcb, 1, N, TQ_LAYOUT_TILE32)
    tq.tq_quantize_kv(kcb, vcb, torch.from_numpy(k)[None].to(dev), torch.from_numpy(v)[None].to(dev), kc, vc)
    tau = 1 / math.sqrt(d)
    out = tq.tq_attn_decode(kcb, vcb, torch.from_numpy(qn)[None].to(dev), kc, vc, N, tau)
    torch.cuda.synchronize()
    rk, rv = P.quantize(okc, k.astype(np.float64)), O.quantize(ovc, v.astype(np.float64))
    _, ref = P.attn_decode(okc, ovc, qn[None].astype(np.float64), _polar_cache([rk], 1, 1, N, True),
                           U.oracle_cache([rv], 1, 1, N, False), tau)
    err = float(np.max(np.abs(out.cpu().numpy() - ref)))
    print("end-to-end max-abs", err)
    assert err <= U.OUT_ATOL


def test_polar_unsupported_combinations(dev):
    _say("polar unsupported combinations")
    cb = tq.PolarCodebook(128, 4, 2)
    t32 = tq.Codes(cb, 1, 64, TQ_LAYOUT_TILE32)
    with pytest.raises(tq.TQError) as e:
        tq.tq_quantize_kv(cb, None, torch.zeros((1, 4, 128), device=dev), None, t32, None)
    assert e.value.status == _lib.TQ_ERR_UNSUPPORTED
    kc = tq.Codes(cb, 1, 64, TQ_LAYOUT_ROW)
    with pytest.raises(tq.TQError) as e:
        tq.tq_ip_topk(cb, torch.zeros((1, 128), device=dev), kc, 64, 4)
    assert e.value.status == _lib.TQ_ERR_UNSUPPORTED
    k53 = tq.PolarCodebook(128, 5, 3)
    vcb = tq.Codebook(128, 4)
    with pytest.raises(tq.TQError) as e:
        tq.tq_attn_decode(k53, vcb, torch.zeros((1, 8, 128), device=dev), tq.Codes(k53, 1, 64, TQ_LAYOUT_ROW),
                          tq.Codes(vcb, 1, 64, TQ_LAYOUT_TILE32), 64, 0.1)
    assert e.value.status == _lib.TQ_ERR_UNSUPPORTED
