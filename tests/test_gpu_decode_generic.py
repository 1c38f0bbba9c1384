"""GPU parity of decode attention at the shapes the d = 128 MFMA kernels do not
take: head dimensions 3..256 other than 128, and at d = 128 the code widths
(1, 5, 6, 7 bits) and sketch sizes (m > 128) those kernels lack.  These run on
the any-shape kernels of decode_gen.hip (bf16 hi/lo MFMA operands, like the
d = 128 kernels).

The oracle quantizes the seeded inputs and packs its own codes; the GPU decodes
those codes and both sides are held to the decode bars (logits within 1e-4 of
the row's max |logit|, outputs within 2e-3 max-abs).  The GPU's own quantize ->
decode chain is compared end to end as well.
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


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    return "cuda"


def _say(*a):
    print("[case]", *a, flush=True)


def _setup(dev, d, B, Hkv, Hq, N, kb, km, vb, nc=False, seed=0, qdtype="bf16"):
    kcb = tq.Codebook(d, kb, qjl_m=km, norm_correction=nc, rot_seed=1, qjl_seed=2)
    vcb = tq.Codebook(d, vb, norm_correction=nc, rot_seed=3)
    ch = [c for c in (3, 77, 101) if c < d]
    k = synth.kv_gaussian(B, Hkv, N, d, seed, dtype="bf16", device=dev, channels=ch, factor=20.0)
    v = synth.kv_gaussian(B, Hkv, N, d, seed + 1, dtype="bf16", device=dev, channels=ch, factor=20.0)
    q = synth.queries_gaussian(B, Hq, d, seed + 2, dtype=qdtype, device=dev)
    return kcb, vcb, k, v, q


def _oracle_codes(kcb, vcb, k, v, B, Hkv, N):
    d = kcb.d
    S = (N + 31) // 32 * 32
    okc, ovc = U.oracle_codebook(kcb), U.oracle_codebook(vcb)
    kc = tq.Codes(kcb, B * Hkv, S, TQ_LAYOUT_ROW)
    vc = tq.Codes(vcb, B * Hkv, S, TQ_LAYOUT_TILE32)
    k64 = U.to_f64(k).reshape(B * Hkv, N, d)
    v64 = U.to_f64(v).reshape(B * Hkv, N, d)
    rk = [O.quantize(okc, k64[s]) for s in range(B * Hkv)]
    rv = [O.quantize(ovc, v64[s]) for s in range(B * Hkv)]
    for s in range(B * Hkv):
        U.upload_oracle_codes(kc, s, rk[s], N)
        U.upload_oracle_codes(vc, s, rv[s], N)
    kd = U.oracle_cache(rk, B, Hkv, N, kcb.m > 0)
    vd = U.oracle_cache(rv, B, Hkv, N, False)
    return okc, ovc, kc, vc, kd, vd


def _decode(dev, kcb, vcb, q, kc, vc, N, lens=None):
    B, Hq, d = q.shape
    logits = torch.full((B, Hq, N), 123.0, dtype=torch.float32, device=dev)
    sl = torch.tensor(lens, dtype=torch.int32, device=dev) if lens is not None else None
    tau = 1.0 / math.sqrt(d)
    out = tq.tq_attn_decode(kcb, vcb, q, kc, vc, N, tau, seq_lens=sl, logits=logits)
    torch.cuda.synchronize()
    return logits.cpu().numpy(), out.cpu().numpy(), tau


@pytest.mark.parametrize("d,kb,km,vb,nc", [
    (64, 3, 64, 4, False),     # a common small head dimension, with a sketch
    (96, 4, 0, 4, True),       # 3 groups of 32 coordinates, norm correction
    (200, 4, 200, 3, False),   # the vector-search dimension; 13 tile32 groups
    (256, 2, 256, 8, False),   # the largest d and m; 8-bit values
    (3, 1, 32, 1, False),      # the smallest d, 1-bit codes
    (48, 5, 100, 6, True),     # field widths that straddle words
    (160, 7, 0, 2, False),
    (128, 5, 0, 6, False),     # d = 128 widths the MFMA kernels lack
    (128, 3, 200, 4, False),   # d = 128 with a sketch of more than 128 rows
    (128, 1, 128, 7, True),
])
def test_generic_decode_matches_oracle(dev, d, kb, km, vb, nc):
    _say("generic decode", d, kb, km, vb, nc)
    B, Hkv, Hq, N = 2, 2, 16, 777
    kcb, vcb, k, v, q = _setup(dev, d, B, Hkv, Hq, N, kb, km, vb, nc, seed=d * 10 + kb)
    okc, ovc, kc, vc, kd, vd = _oracle_codes(kcb, vcb, k, v, B, Hkv, N)
    lg, out, tau = _decode(dev, kcb, vcb, q, kc, vc, N)
    print(U.check_decode(okc, ovc, U.to_f64(q), kd, vd, tau, lg, out, name=f"d{d}k{kb}m{km}v{vb}"))


@pytest.mark.parametrize("B,Hkv,Hq,N,lens", [
    (3, 1, 8, 700, [700, 333, 0]),   # per-sequence lengths incl. empty
    (1, 2, 4, 96, None),             # g = 2
    (1, 2, 24, 161, [150]),          # g = 12: two query groups, ragged tile
    (1, 1, 8, 1, None),              # one token
    (2, 1, 8, 65, [64, 65]),         # one full 64-token tile, then one token more
])
def test_generic_decode_shapes(dev, B, Hkv, Hq, N, lens):
    _say("generic decode shapes", B, Hkv, Hq, N, lens)
    d = 80
    kcb, vcb, k, v, q = _setup(dev, d, B, Hkv, Hq, N, 3, 96, 4, seed=N)
    okc, ovc, kc, vc, kd, vd = _oracle_codes(kcb, vcb, k, v, B, Hkv, N)
    lg, out, tau = _decode(dev, kcb, vcb, q, kc, vc, N, lens)
    st = U.check_decode(okc, ovc, U.to_f64(q), kd, vd, tau, lg, out, n_valid=lens, name="shapes")
    if lens is not None and 0 in lens:
        assert np.all(out[lens.index(0)] == 0)
    print(st)


def test_generic_decode_f32_and_f16_queries(dev):
    _say("generic decode fp32 / fp16 queries")
    d, B, Hkv, Hq, N = 112, 1, 2, 8, 300
    for qdt in ("f32", "f16"):
        kcb, vcb, k, v, q = _setup(dev, d, B, Hkv, Hq, N, 4, 64, 4, seed=5, qdtype=qdt)
        okc, ovc, kc, vc, kd, vd = _oracle_codes(kcb, vcb, k, v, B, Hkv, N)
        lg, out, tau = _decode(dev, kcb, vcb, q, kc, vc, N)
        print(qdt, U.check_decode(okc, ovc, U.to_f64(q), kd, vd, tau, lg, out, name=qdt))


def test_generic_decode_end_to_end(dev):
    """GPU quantize + GPU decode against oracle quantize + oracle decode, d = 200."""
    _say("generic decode end to end")
    d, B, Hkv, Hq, N = 200, 1, 2, 16, 1000
    kcb, vcb, k, v, q = _setup(dev, d, B, Hkv, Hq, N, 4, 200, 4, seed=9)
    okc, ovc, _, _, kd, vd = _oracle_codes(kcb, vcb, k, v, B, Hkv, N)
    S = (N + 31) // 32 * 32
    kc2 = tq.Codes(kcb, B * Hkv, S, TQ_LAYOUT_ROW)
    vc2 = tq.Codes(vcb, B * Hkv, S, TQ_LAYOUT_TILE32)
    tq.tq_quantize_kv(kcb, vcb, k.view(B * Hkv, N, d), v.view(B * Hkv, N, d), kc2, vc2)
    lg2, out2, tau = _decode(dev, kcb, vcb, q, kc2, vc2, N)
    flat = lambda c: {n: (a.reshape(-1, *a.shape[2:]) if a is not None else None)
                      for n, a in U.read_codes(c, N).items()}
    st_k, _ = U.compare_quant(okc, U.to_f64(k).reshape(-1, d), flat(kc2), "K")
    st_v, _ = U.compare_quant(ovc, U.to_f64(v).reshape(-1, d), flat(vc2), "V")
    _, out_ref = O.attn_decode(okc, ovc, U.to_f64(q), kd, vd, tau)
    print(U.check_end_to_end(okc, ovc, U.to_f64(q), kc2, vc2, N, B, Hkv, tau, lg2, out2, out_ref, [st_k, st_v]))


def test_generic_decode_long_context_sampled(dev):
    """d = 256, 64K context, 8 query heads per KV head, several workgroups per
    row: the GPU quantizes the cache, the oracle's codes replace two sequences,
    whose outputs are checked."""
    _say("generic decode long context")
    d, B, Hkv, Hq, N = 256, 2, 2, 16, 65536
    kcb, vcb, k, v, q = _setup(dev, d, B, Hkv, Hq, N, 3, 128, 4, seed=17)
    kc = tq.Codes(kcb, B * Hkv, N, TQ_LAYOUT_ROW)
    vc = tq.Codes(vcb, B * Hkv, N, TQ_LAYOUT_TILE32)
    tq.tq_quantize_kv(kcb, vcb, k.view(B * Hkv, N, d), v.view(B * Hkv, N, d), kc, vc)
    okc, ovc = U.oracle_codebook(kcb), U.oracle_codebook(vcb)
    seqs = [0, B * Hkv - 1]
    refs = {}
    for s in seqs:
        rk = O.quantize(okc, U.to_f64(k.view(B * Hkv, N, d)[s]))
        rv = O.quantize(ovc, U.to_f64(v.view(B * Hkv, N, d)[s]))
        U.upload_oracle_codes(kc, s, rk, N)
        U.upload_oracle_codes(vc, s, rv, N)
        refs[s] = (rk, rv)
    lg, out, tau = _decode(dev, kcb, vcb, q, kc, vc, N)
    g = Hq // Hkv
    q64 = U.to_f64(q)
    for s in seqs:
        b, h = divmod(s, Hkv)
        rk, rv = refs[s]
        kd = U.oracle_cache([rk], 1, 1, N, True)
        vd = U.oracle_cache([rv], 1, 1, N, False)
        qs = q64[b:b + 1, h * g:(h + 1) * g]
        st = U.check_decode(okc, ovc, qs, kd, vd, tau, lg[b:b + 1, h * g:(h + 1) * g],
                            out[b:b + 1, h * g:(h + 1) * g], name=f"seq{s}")
        print(s, st)


def test_generic_noalloc_matches_workspace_call(dev):
    _say("generic decode, allocation-free entry point")
    d, B, Hkv, Hq, N = 64, 2, 2, 16, 500
    kcb, vcb, k, v, q = _setup(dev, d, B, Hkv, Hq, N, 4, 64, 4, seed=3)
    S = (N + 31) // 32 * 32
    kc = tq.Codes(kcb, B * Hkv, S, TQ_LAYOUT_ROW)
    vc = tq.Codes(vcb, B * Hkv, S, TQ_LAYOUT_TILE32)
    tq.tq_quantize_kv(kcb, vcb, k.view(B * Hkv, N, d), v.view(B * Hkv, N, d), kc, vc)
    tau = 1.0 / math.sqrt(d)
    out_ws = tq.tq_attn_decode(kcb, vcb, q, kc, vc, N, tau)
    out_na = torch.full((B, Hq, d), 5.0, dtype=torch.float32, device=dev)
    tq.tq_attn_decode_noalloc(kcb, vcb, q, kc, vc, N, tau, out=out_na)
    torch.cuda.synchronize()
    assert torch.equal(out_ws, out_na)
