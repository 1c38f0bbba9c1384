"""Pins of the oracle's decode attention and top-k search from codes.

Sources: page "什么是TurboQuant？…" (a2a-mcp.org blog): "如何实现 TurboQuant"
item 1 (rotate the query once, dot products straight from the indices),
"基准测试与实际性能表现" (top-k inner-product search from codes).
"""
import math

import numpy as np
import pytest

import oracle as O


def _brute_decode(kcb, vcb, qv, kx, vx, tau):
    """Python-loop decode for one query against one head (tiny sizes)."""
    d = len(qv)
    kq = O.quantize(kcb, kx)
    vq = O.quantize(vcb, vx)
    qt = [sum(kcb.rot[i][j] * qv[j] for j in range(d)) for i in range(d)]
    tq = None
    if kcb.m:
        tq = [sum(kcb.qjl[r][i] * qt[i] for i in range(d)) for r in range(kcb.m)]
    logits = []
    for n in range(len(kx)):
        s = sum(qt[i] * kcb.centroids[kq["idx"][n][i]] for i in range(d)) * kq["scale"][n]
        if kcb.m:
            s += math.sqrt(math.pi / 2) / kcb.m * kq["rnorm"][n] * sum(
                tq[r] * (1.0 if kq["sign"][n][r] else -1.0) for r in range(kcb.m))
        logits.append(tau * s)
    mx = max(logits)
    w = [math.exp(v - mx) for v in logits]
    tot = sum(w)
    out = [0.0] * d
    for n in range(len(vx)):
        # value n dequantized explicitly: scale * Pi_V^T c[idx]
        yv = [vcb.centroids[vq["idx"][n][i]] for i in range(d)]
        vh = [vq["scale"][n] * sum(vcb.rot[i][j] * yv[i] for i in range(d)) for j in range(d)]
        for j in range(d):
            out[j] += w[n] / tot * vh[j]
    return np.array(logits), np.array(out)


def _as_cache(qd, B=1, H=1):
    N = qd["idx"].shape[0]
    c = dict(idx=qd["idx"].reshape(B, H, N // (B * H), -1) if B * H > 1 else qd["idx"][None, None],
             scale=qd["scale"][None, None])
    if qd["sign"] is not None:
        c["sign"] = qd["sign"][None, None]
        c["rnorm"] = qd["rnorm"][None, None]
    return c


@pytest.mark.parametrize("d,N,m", [(3, 1, 0), (4, 2, 4), (4, 7, 3), (8, 64, 8)])
def test_decode_bruteforce_tiny(d, N, m):
    rng = np.random.default_rng(d * 100 + N)
    kcb = O.Codebook(d, 3, qjl_m=m, rot_seed=3, qjl_seed=4)
    vcb = O.Codebook(d, 2, rot_seed=5)
    kx, vx = rng.standard_normal((N, d)), rng.standard_normal((N, d))
    qv = rng.standard_normal(d)
    tau = 1 / math.sqrt(d)
    lg_ref, out_ref = _brute_decode(kcb, vcb, qv, kx, vx, tau)
    lg, out = O.attn_decode(kcb, vcb, qv[None, None, :], _as_cache(O.quantize(kcb, kx)),
                            _as_cache(O.quantize(vcb, vx)), tau)
    assert np.allclose(lg[0, 0], lg_ref, atol=1e-12)
    assert np.allclose(out[0, 0], out_ref, atol=1e-12)


def test_decode_single_token_returns_its_value():
    d = 16
    rng = np.random.default_rng(1)
    kcb, vcb = O.Codebook(d, 3, qjl_m=16), O.Codebook(d, 4, rot_seed=9)
    kx, vx = rng.standard_normal((1, d)), rng.standard_normal((1, d))
    vq = O.quantize(vcb, vx)
    _, out = O.attn_decode(kcb, vcb, rng.standard_normal((1, 1, d)),
                           _as_cache(O.quantize(kcb, kx)), _as_cache(vq), 0.25)
    assert np.allclose(out[0, 0], O.dequantize(vcb, vq["idx"], vq["scale"])[0], atol=1e-13)


def test_decode_equal_logits_average_values():
    # identical keys -> identical codes -> equal logits -> mean of values
    d, N = 16, 9
    rng = np.random.default_rng(2)
    kcb, vcb = O.Codebook(d, 3, qjl_m=16), O.Codebook(d, 4, rot_seed=9)
    kx = np.repeat(rng.standard_normal((1, d)), N, axis=0)
    vx = rng.standard_normal((N, d))
    vq = O.quantize(vcb, vx)
    lg, out = O.attn_decode(kcb, vcb, rng.standard_normal((1, 1, d)),
                            _as_cache(O.quantize(kcb, kx)), _as_cache(vq), 0.3)
    assert np.allclose(lg[0, 0], lg[0, 0, 0])
    assert np.allclose(out[0, 0], O.dequantize(vcb, vq["idx"], vq["scale"]).mean(0), atol=1e-13)


def test_decode_gqa_head_mapping_and_lengths():
    # query head hq reads kv head hq // (Hq/Hkv); n_valid cuts the context
    d, N, B, Hkv, g = 8, 20, 2, 2, 3
    rng = np.random.default_rng(3)
    kcb, vcb = O.Codebook(d, 2, qjl_m=8), O.Codebook(d, 3, rot_seed=7)
    kx = rng.standard_normal((B, Hkv, N, d))
    vx = rng.standard_normal((B, Hkv, N, d))
    q = rng.standard_normal((B, Hkv * g, d))
    kq = O.quantize(kcb, kx.reshape(-1, d))
    vq = O.quantize(vcb, vx.reshape(-1, d))
    kc = dict(idx=kq["idx"].reshape(B, Hkv, N, d), scale=kq["scale"].reshape(B, Hkv, N),
              sign=kq["sign"].reshape(B, Hkv, N, 8), rnorm=kq["rnorm"].reshape(B, Hkv, N))
    vc = dict(idx=vq["idx"].reshape(B, Hkv, N, d), scale=vq["scale"].reshape(B, Hkv, N))
    nval = [N, 13]
    lg, out = O.attn_decode(kcb, vcb, q, kc, vc, 0.35, n_valid=nval)
    for b in range(B):
        for hq in range(Hkv * g):
            h = hq // g
            nb = nval[b]
            lr, orf = _brute_decode(kcb, vcb, q[b, hq], kx[b, h, :nb], vx[b, h, :nb], 0.35)
            assert np.allclose(lg[b, hq, :nb], lr, atol=1e-12)
            assert np.all(np.isneginf(lg[b, hq, nb:]))
            assert np.allclose(out[b, hq], orf, atol=1e-12)


def test_decode_logits_equal_dequantized_key_path():
    # rotated-query logits == tau * <q, x_hat> with explicitly dequantized keys
    d, N, m = 32, 50, 32
    rng = np.random.default_rng(4)
    kcb, vcb = O.Codebook(d, 3, qjl_m=m), O.Codebook(d, 4)
    kx, vx = rng.standard_normal((N, d)) * 2, rng.standard_normal((N, d))
    qv = rng.standard_normal(d)
    kq = O.quantize(kcb, kx)
    lg, _ = O.attn_decode(kcb, vcb, qv[None, None], _as_cache(kq), _as_cache(O.quantize(vcb, vx)), 0.2)
    xh = O.dequantize(kcb, kq["idx"], kq["scale"], kq["sign"], kq["rnorm"])
    assert np.allclose(lg[0, 0], 0.2 * (xh @ qv), atol=1e-12)


def test_decode_converges_to_exact_attention_with_bits():
    # error against exact attention falls as bits grow (no QJL)
    d, N = 64, 300
    rng = np.random.default_rng(5)
    kx, vx = rng.standard_normal((N, d)), rng.standard_normal((N, d))
    qv = rng.standard_normal((1, 1, d)) * 2
    tau = 1 / math.sqrt(d)
    ex = O.exact_attention(qv, kx[None, None], vx[None, None], tau)
    errs = []
    for b in (2, 3, 4, 8):
        kcb, vcb = O.Codebook(d, b), O.Codebook(d, b, rot_seed=11)
        _, out = O.attn_decode(kcb, vcb, qv, _as_cache(O.quantize(kcb, kx)),
                               _as_cache(O.quantize(vcb, vx)), tau)
        errs.append(np.linalg.norm(out - ex) / np.linalg.norm(ex))
    assert all(errs[i + 1] < errs[i] for i in range(3)), errs
    # error scales like sqrt(D_b): D_2 / D_8 is about 2900
    assert errs[-1] < errs[0] / 20


def test_exact_attention_bruteforce():
    rng = np.random.default_rng(6)
    q, k, v = rng.standard_normal((1, 2, 3)), rng.standard_normal((1, 1, 4, 3)), rng.standard_normal((1, 1, 4, 3))
    out = O.exact_attention(q, k, v, 0.7)
    for hq in range(2):
        lg = [0.7 * sum(q[0, hq, i] * k[0, 0, n, i] for i in range(3)) for n in range(4)]
        w = [math.exp(x - max(lg)) for x in lg]
        ref = [sum(w[n] * v[0, 0, n, j] for n in range(4)) / sum(w) for j in range(3)]
        assert np.allclose(out[0, hq], ref, atol=1e-14)


# ----------------------------------------------------------------- top-k


def test_topk_bruteforce_and_ties():
    d, n = 12, 60
    rng = np.random.default_rng(7)
    cb = O.Codebook(d, 4, qjl_m=12)
    db = rng.standard_normal((n, d))
    db[40] = db[3]          # duplicate vectors -> equal scores
    db[41] = db[3]
    qs = rng.standard_normal((5, d))
    qs[0] = db[3] * 3       # makes the duplicates the top results
    qd = O.quantize(cb, db)
    codes = dict(idx=qd["idx"], scale=qd["scale"], sign=qd["sign"], rnorm=qd["rnorm"])
    ti, ts = O.ip_topk(cb, qs, codes, 7)
    for i in range(5):
        s = O.code_scores(cb, qs[i], qd["idx"], qd["scale"], qd["sign"], qd["rnorm"])
        ref = sorted(range(n), key=lambda j: (-s[j], j))[:7]
        assert list(ti[i]) == ref
        assert np.allclose(ts[i], s[ref])
    assert list(ti[0][:3]) == [3, 40, 41]


def test_topk_recall_high_at_8_bits():
    d, n = 32, 2000
    rng = np.random.default_rng(8)
    db = rng.standard_normal((n, d))
    qs = rng.standard_normal((20, d))
    cb = O.Codebook(d, 8, qjl_m=32)
    qd = O.quantize(cb, db)
    codes = dict(idx=qd["idx"], scale=qd["scale"], sign=qd["sign"], rnorm=qd["rnorm"])
    ti, _ = O.ip_topk(cb, qs, codes, 10)
    te, _ = O.exact_topk(qs, db, 10)
    recall = np.mean([len(set(a) & set(b)) / 10 for a, b in zip(ti, te)])
    assert recall > 0.9


def test_exact_topk_bruteforce_with_ties():
    # pure-Python inner products and ordering (descending, ties to the lower
    # index) on a small database with duplicated rows
    rng = np.random.default_rng(9)
    d, n, k = 5, 40, 6
    db = rng.integers(-3, 4, size=(n, d)).astype(np.float64)
    db[17] = db[2]
    db[30] = db[2]
    qs = rng.integers(-2, 3, size=(4, d)).astype(np.float64)
    qs[0] = db[2]
    ti, ts = O.exact_topk(qs, db, k)
    for i in range(len(qs)):
        s = [sum(qs[i, c] * db[j, c] for c in range(d)) for j in range(n)]
        ref = sorted(range(n), key=lambda j: (-s[j], j))[:k]
        assert list(ti[i]) == ref
        assert list(ts[i]) == [s[j] for j in ref]
    assert list(ti[0][:3]) == [2, 17, 30]
