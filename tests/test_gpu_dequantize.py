"""GPU parity of tq_dequantize against the oracle's dequantize.

The oracle quantizes seeded synthetic vectors and its packed codes are
uploaded; the GPU reconstructs positions [tok_offset, tok_offset + n_tok) and
is compared element by element with the oracle's
x_hat = Pi^T (scale c[idx] + sqrt(pi/2)/m rnorm S^T (2 sign - 1)) of the same
codes (stored scalars rounded to fp32 as uploaded).

Bars (per vector, relative to max |x_hat_oracle| of that vector):
* d = 128, qjl_m <= 128 (bf16 MFMA on two-part splits of Pi, the centroids
  and the sketch operand; each product keeps ~2^-16 of its relative
  precision): 1e-4;
* other shapes (fp32 FMAs): 1e-5;
* 16-bit outputs add one rounding of the result: 2^-8 (bf16) or 2^-11
  (fp16) of |x_hat| element-wise on top of the fp32 bar.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
import kv_cache_vector_quantize_amd as tq
from kv_cache_vector_quantize_amd import TQ_LAYOUT_ROW, TQ_LAYOUT_TILE32

import tq_testutil as U

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    return "cuda"


def _say(*a):
    print("[case]", *a, flush=True)


def _case(dev, d, bits, m, nc, layout, n_seq, n_tok, tok_offset, odt, seed):
    cb = tq.Codebook(d, bits, qjl_m=m, norm_correction=nc, rot_seed=1, qjl_seed=2)
    ocb = U.oracle_codebook(cb)
    n_all = tok_offset + n_tok
    S = (n_all + 31) // 32 * 32 + (32 if layout == TQ_LAYOUT_TILE32 else 0)
    x = synth.kv_gaussian(1, n_seq, n_all, d, seed, dtype="f32", device="cpu",
                          channels=[c for c in (3, 77, 101) if c < d], factor=20.0)
    x64 = U.to_f64(x).reshape(n_seq, n_all, d)
    codes = tq.Codes(cb, n_seq, S, layout, device=dev)
    refs = []
    for s in range(n_seq):
        r = O.quantize(ocb, x64[s])
        U.upload_oracle_codes(codes, s, r, n_all)
        refs.append(r)
    out = tq.tq_dequantize(cb, codes, n_seq, n_tok, tok_offset, dtype=odt)
    torch.cuda.synchronize()
    got = out.float().cpu().numpy().astype(np.float64)
    fast = d == 128 and m <= 128
    tol = 1e-4 if fast else 1e-5
    worst = 0.0
    for s in range(n_seq):
        r = refs[s]
        sl = slice(tok_offset, tok_offset + n_tok)
        sc = r["scale"].astype(np.float32).astype(np.float64)[sl]
        sg = r["sign"][sl] if m > 0 else None
        rn = r["rnorm"].astype(np.float32).astype(np.float64)[sl] if m > 0 else None
        ref = O.dequantize(ocb, r["idx"][sl], sc, sg, rn)
        amax = np.max(np.abs(ref), axis=1, keepdims=True)
        err = np.abs(got[s] - ref)
        bar = tol * amax
        if odt == torch.bfloat16:
            bar = bar + 2.0 ** -8 * np.abs(ref)
        elif odt == torch.float16:
            bar = bar + 2.0 ** -11 * np.abs(ref)
        assert np.all(err <= bar), f"seq {s}: max err {np.max(err / np.maximum(amax, 1e-30))} of max |x_hat|"
        worst = max(worst, float(np.max(err / np.maximum(amax, 1e-30))))
    return worst


@pytest.mark.parametrize("bits,m,nc,layout", [
    (1, 0, False, TQ_LAYOUT_ROW), (2, 0, True, TQ_LAYOUT_ROW), (3, 0, False, TQ_LAYOUT_ROW),
    (4, 0, False, TQ_LAYOUT_ROW), (5, 0, False, TQ_LAYOUT_ROW), (6, 0, True, TQ_LAYOUT_ROW),
    (7, 0, False, TQ_LAYOUT_ROW), (8, 0, False, TQ_LAYOUT_ROW),
    (1, 0, False, TQ_LAYOUT_TILE32), (2, 0, False, TQ_LAYOUT_TILE32), (3, 0, True, TQ_LAYOUT_TILE32),
    (4, 0, False, TQ_LAYOUT_TILE32), (5, 0, False, TQ_LAYOUT_TILE32), (8, 0, True, TQ_LAYOUT_TILE32),
    (3, 128, False, TQ_LAYOUT_ROW), (4, 128, True, TQ_LAYOUT_ROW), (2, 64, False, TQ_LAYOUT_ROW),
    (8, 100, False, TQ_LAYOUT_ROW),
])
def test_dequantize_d128(dev, bits, m, nc, layout):
    _say("dequantize d=128", bits, m, nc, layout)
    w = _case(dev, 128, bits, m, nc, layout, n_seq=2, n_tok=77, tok_offset=5, odt=torch.float32,
              seed=100 + bits + m)
    print("worst rel", w)


@pytest.mark.parametrize("odt", [torch.bfloat16, torch.float16])
def test_dequantize_16bit_outputs(dev, odt):
    _say("dequantize 16-bit out", odt)
    _case(dev, 128, 3, 128, False, TQ_LAYOUT_ROW, n_seq=1, n_tok=64, tok_offset=0, odt=odt, seed=7)
    _case(dev, 128, 4, 0, False, TQ_LAYOUT_TILE32, n_seq=1, n_tok=40, tok_offset=3, odt=odt, seed=8)


@pytest.mark.parametrize("d,bits,m,layout", [
    (200, 4, 200, TQ_LAYOUT_ROW), (64, 3, 0, TQ_LAYOUT_TILE32), (128, 3, 200, TQ_LAYOUT_ROW),
    (96, 2, 32, TQ_LAYOUT_ROW),
])
def test_dequantize_generic_shapes(dev, d, bits, m, layout):
    _say("dequantize generic", d, bits, m, layout)
    w = _case(dev, d, bits, m, False, layout, n_seq=2, n_tok=45, tok_offset=2, odt=torch.float32,
              seed=d + bits)
    print("worst rel", w)


def test_dequantize_single_and_many_tiles(dev):
    _say("dequantize one token / many tiles")
    _case(dev, 128, 4, 128, False, TQ_LAYOUT_ROW, n_seq=3, n_tok=1, tok_offset=31, odt=torch.float32, seed=3)
    _case(dev, 128, 4, 0, False, TQ_LAYOUT_TILE32, n_seq=2, n_tok=700, tok_offset=0, odt=torch.float32, seed=4)


def test_dequantize_inner_products_match_decode_estimate(dev):
    """<q, x_hat> from the GPU reconstruction equals the oracle's score of the
    same codes (the estimate decode and top-k use) to the dequantize bar."""
    _say("dequantize vs code scores")
    d, n = 128, 256
    cb = tq.Codebook(d, 3, qjl_m=128, rot_seed=1, qjl_seed=2)
    ocb = U.oracle_codebook(cb)
    x = synth.kv_gaussian(1, 1, n, d, 21, dtype="f32", device="cpu", channels=[3, 77, 101], factor=20.0)
    x64 = U.to_f64(x).reshape(n, d)
    r = O.quantize(ocb, x64)
    codes = tq.Codes(cb, 1, n, TQ_LAYOUT_ROW, device=dev)
    U.upload_oracle_codes(codes, 0, r, n)
    xh = tq.tq_dequantize(cb, codes, 1, n).cpu().numpy().astype(np.float64)[0]
    q = np.random.default_rng(5).standard_normal((4, d))
    s_ref = np.stack([O.code_scores(ocb, q[i], r["idx"], r["scale"].astype(np.float32).astype(np.float64),
                                    r["sign"], r["rnorm"].astype(np.float32).astype(np.float64))
                      for i in range(q.shape[0])])
    s_gpu = q @ xh.T
    bar = 1e-4 * np.max(np.abs(xh), axis=1)[None, :] * np.sum(np.abs(q), axis=1)[:, None]
    assert np.all(np.abs(s_gpu - s_ref) <= bar)


def test_dequantize_argument_errors(dev):
    _say("dequantize argument errors")
    cb = tq.Codebook(128, 4)
    codes = tq.Codes(cb, 1, 64, TQ_LAYOUT_ROW, device=dev)
    with pytest.raises(tq.TQError):
        tq.tq_dequantize(cb, codes, 1, 60, 10)            # past seq_stride
    out = torch.empty((1, 8, 128), dtype=torch.float32, device=dev)
    with pytest.raises(tq.TQError):
        tq.tq_dequantize(cb, codes, 1, 8, -1, out=out)
    # empty ranges are no-ops
    tq.tq_dequantize(cb, codes, 0, 8, 0, out=out)
    tq.tq_dequantize(cb, codes, 1, 0, 0, out=out[:, :0])


def test_dequantize_then_attend_equals_decode_from_codes(dev):
    """Dense attention over the GPU's reconstructions of K and V (fp32,
    evaluated here in float64) equals the oracle's decode attention from the
    same codes, to the decode bars (logits 1e-4 of the row's max |logit|,
    outputs 2e-3 max-abs): reconstructing first and attending from the codes
    compute the same estimate."""
    _say("dequantize-then-attend vs decode from codes")
    B, Hq, Hkv, d, N = 1, 4, 2, 128, 200
    g = Hq // Hkv
    tau = 1.0 / np.sqrt(d)
    kcb = tq.Codebook(d, 3, qjl_m=128, rot_seed=1, qjl_seed=2)
    vcb = tq.Codebook(d, 4, rot_seed=3)
    okc, ovc = U.oracle_codebook(kcb), U.oracle_codebook(vcb)
    k = U.to_f64(synth.kv_gaussian(B, Hkv, N, d, 31, dtype="f32", device="cpu", channels=[3, 77, 101], factor=20.0))
    v = U.to_f64(synth.kv_gaussian(B, Hkv, N, d, 32, dtype="f32", device="cpu", channels=[3, 77, 101], factor=20.0))
    q = np.random.default_rng(33).standard_normal((B, Hq, d))
    S = (N + 31) // 32 * 32
    kc = tq.Codes(kcb, B * Hkv, S, TQ_LAYOUT_ROW, device=dev)
    vc = tq.Codes(vcb, B * Hkv, S, TQ_LAYOUT_TILE32, device=dev)
    kr = [O.quantize(okc, k.reshape(B * Hkv, N, d)[s]) for s in range(B * Hkv)]
    vr = [O.quantize(ovc, v.reshape(B * Hkv, N, d)[s]) for s in range(B * Hkv)]
    for s in range(B * Hkv):
        U.upload_oracle_codes(kc, s, kr[s], N)
        U.upload_oracle_codes(vc, s, vr[s], N)
    kh = tq.tq_dequantize(kcb, kc, B * Hkv, N).cpu().numpy().astype(np.float64).reshape(B, Hkv, N, d)
    vh = tq.tq_dequantize(vcb, vc, B * Hkv, N).cpu().numpy().astype(np.float64).reshape(B, Hkv, N, d)
    f32 = lambda a: a.astype(np.float32).astype(np.float64)
    stack = lambda rs, key: np.stack([r[key] for r in rs]).reshape(B, Hkv, N, *rs[0][key].shape[1:])
    okcodes = dict(idx=stack(kr, "idx"), scale=f32(stack(kr, "scale")), sign=stack(kr, "sign"),
                   rnorm=f32(stack(kr, "rnorm")))
    ovcodes = dict(idx=stack(vr, "idx"), scale=f32(stack(vr, "scale")))
    ref_lg, ref_out = O.attn_decode(okc, ovc, q, okcodes, ovcodes, tau)
    for b in range(B):
        for hq in range(Hq):
            h = hq // g
            lg = tau * (kh[b, h] @ q[b, hq])
            p = np.exp(lg - lg.max())
            out = (p / p.sum()) @ vh[b, h]
            assert np.max(np.abs(lg - ref_lg[b, hq])) <= 1e-4 * np.max(np.abs(ref_lg[b, hq]))
            assert np.max(np.abs(out - ref_out[b, hq])) <= 2e-3
