"""Pins of the oracle's quantizer, packing and QJL sketch.

Sources: page "什么是TurboQuant？…" (a2a-mcp.org blog), "第一阶段" item 2
(normalise, Lloyd-Max index per coordinate), "第二阶段：QJL 残差校正" (1-bit
sign sketch of the residual that removes inner-product bias).
"""
import math

import numpy as np
import pytest

import oracle as O


# ----------------------------------------------------------------- index rule


def test_index_is_nearest_centroid_with_upper_ties():
    cb = O.Codebook(16, 3)
    rng = np.random.default_rng(0)
    x = rng.standard_normal((400, 16))
    q = O.quantize(cb, x)
    # brute force: argmin |y - c_k|, ties to the larger k
    dist = np.abs(q["y"][:, :, None] - cb.centroids[None, None, :])
    best = np.array([[max(np.flatnonzero(r == r.min())) for r in row] for row in dist])
    assert np.array_equal(q["idx"], best)


def test_index_exact_boundary_goes_up():
    c, t = O.lloyd_max(8, 2)
    # a coordinate exactly on boundary k lands in cell k (the upper one)
    assert list(O.coord_index(t, t)) == [1, 2, 3]
    assert list(O.coord_index(np.nextafter(t, -1), t)) == [0, 1, 2]
    assert list(O.coord_index([-1.0, 1.0], t)) == [0, 3]


def test_zero_vector():
    cb = O.Codebook(32, 3, qjl_m=32)
    q = O.quantize(cb, np.zeros((2, 32)))
    assert np.all(q["y"] == 0) and np.all(q["scale"] == 0) and np.all(q["rnorm"] == 0)
    assert np.all(q["idx"] == 4)
    xh = O.dequantize(cb, q["idx"], q["scale"], q["sign"], q["rnorm"])
    assert np.all(xh == 0)


# ----------------------------------------------------------------- distortion


@pytest.mark.parametrize("b", [2, 3, 4])
def test_empirical_mse_matches_closed_form(b):
    # original-domain relative error |x - x_hat|^2 / |x|^2 on isotropic data
    d, n = 128, 6000
    cb = O.Codebook(d, b)
    x = np.random.default_rng(b).standard_normal((n, d)) * 3.0
    q = O.quantize(cb, x)
    xh = O.dequantize(cb, q["idx"], q["scale"])
    err = np.sum((x - xh) ** 2, axis=1) / np.sum(x * x, axis=1)
    D = O.mse_closed_form(d, cb.centroids, cb.boundaries)
    assert abs(err.mean() - D) < 4 * err.std() / math.sqrt(n)


def test_mean_cosine_3bit_page_value():
    d, n = 128, 4000
    cb = O.Codebook(d, 3)
    x = np.random.default_rng(3).standard_normal((n, d))
    q = O.quantize(cb, x)
    xh = O.dequantize(cb, q["idx"], q["scale"])
    cos = np.sum(x * xh, axis=1) / (np.linalg.norm(x, axis=1) * np.linalg.norm(xh, axis=1))
    assert abs(cos.mean() - 0.983) < 1e-3


def test_rotation_is_not_transposed():
    # a wrong orientation of Pi (x Pi instead of Pi x) would leave the
    # reconstruction error at ~2, not at D_b
    d = 64
    cb = O.Codebook(d, 4)
    x = np.random.default_rng(9).standard_normal((500, d))
    q = O.quantize(cb, x)
    assert np.allclose(q["y"] * np.linalg.norm(x, axis=1)[:, None], x @ cb.rot.T)
    xh = O.dequantize(cb, q["idx"], q["scale"])
    assert np.mean(np.sum((x - xh) ** 2, 1) / np.sum(x * x, 1)) < 0.02


def test_norm_correction_preserves_norm():
    d = 128
    cb = O.Codebook(d, 2, nc=True)
    x = np.random.default_rng(4).standard_normal((300, d)) * 2
    q = O.quantize(cb, x)
    xh = O.dequantize(cb, q["idx"], q["scale"])
    assert np.allclose(np.linalg.norm(xh, axis=1), np.linalg.norm(x, axis=1), rtol=1e-12)
    # same indices as without norm correction
    q0 = O.quantize(O.Codebook(d, 2, nc=False), x)
    assert np.array_equal(q["idx"], q0["idx"])


# ----------------------------------------------------------------- QJL


def test_qjl_sign_identity_m1():
    # E[(g.a) sign(g.b)] = sqrt(2/pi) a.b/|b| for g ~ N(0, I)
    rng = np.random.default_rng(1)
    a, b = rng.standard_normal(5), rng.standard_normal(5)
    g = rng.standard_normal((400000, 5))
    est = np.mean((g @ a) * np.sign(g @ b))
    ref = math.sqrt(2 / math.pi) * a @ b / np.linalg.norm(b)
    sd = math.sqrt(a @ a - (2 / math.pi) * (a @ b / np.linalg.norm(b)) ** 2) / math.sqrt(len(g))
    assert abs(est - ref) < 4 * sd


def test_qjl_estimator_unbiased_over_seeds():
    # fixed q, x; average the code inner product over many QJL seeds
    d, m, b = 32, 32, 2
    rng = np.random.default_rng(5)
    x = rng.standard_normal(d)
    qv = rng.standard_normal(d)
    cb0 = O.Codebook(d, b, qjl_m=m, qjl_seed=100)
    q0 = O.quantize(cb0, x[None, :])
    n = np.linalg.norm(x)
    qt = cb0.rot @ qv
    r = q0["y"][0] - cb0.centroids[q0["idx"][0]]
    target = n * (qt @ (cb0.centroids[q0["idx"][0]] + r))          # = <q, x>
    assert abs(target - qv @ x) < 1e-10
    rho = np.linalg.norm(r)
    var = (n * rho) ** 2 / m * (math.pi / 2 * qt @ qt - (qt @ r / rho) ** 2)
    ests = []
    for s in range(3000):
        cb = O.Codebook(d, b, qjl_m=m, qjl_seed=1000 + s)
        qq = O.quantize(cb, x[None, :])
        ests.append(O.code_scores(cb, qv, qq["idx"], qq["scale"], qq["sign"], qq["rnorm"])[0])
    ests = np.array(ests)
    z = (ests.mean() - target) / math.sqrt(var / len(ests))
    assert abs(z) < 4, z
    # the sample variance matches the closed form
    assert abs(ests.var() / var - 1) < 0.15
    # without the sketch the MSE-stage estimate is biased away from <q, x>
    mse_only = n * (qt @ cb0.centroids[q0["idx"][0]])
    assert abs(mse_only - target) > 0


def _sketch_estimates(d, m, b, nc, x, qv, seeds, wrong_residual=False):
    """Code inner products <q, x> over independent sketch matrices (the
    rotation stays fixed: only S is redrawn per seed).  With
    ``wrong_residual`` the sketch is taken of y - c[idx] instead of the
    residual of the direction actually used (a planted mistake)."""
    cb = O.Codebook(d, b, qjl_m=m, nc=nc)
    ests = []
    for s in seeds:
        cb.qjl = O.qjl_matrix(m, d, s)
        q = O.quantize(cb, x[None, :])
        sign, rnorm = q["sign"], q["rnorm"]
        if wrong_residual:
            r = q["y"] - cb.centroids[q["idx"]]
            sign = (r @ cb.qjl.T >= 0).astype(np.uint8)
            rnorm = np.linalg.norm(x) * np.linalg.norm(r, axis=1)
        ests.append(O.code_scores(cb, qv, q["idx"], q["scale"], sign, rnorm)[0])
    return cb, np.array(ests)


def test_qjl_estimator_unbiased_with_norm_correction():
    # nc on: scale = n/|c[idx]| and the sketched residual is y - c[idx]/|c[idx]|,
    # so scale <q~, c[idx]> + n <q~, r> = n <q~, y> = <q, x> exactly and the
    # sketch term keeps the estimate unbiased.  q is correlated with x so that
    # a residual taken against c[idx] (not c[idx]/|c[idx]|) shows its bias,
    # n <q~, c[idx]> (1/|c[idx]| - 1), far outside the 4-sigma band.
    d, m, b = 32, 32, 2
    rng = np.random.default_rng(12)
    x = rng.standard_normal(d)
    qv = x + 0.5 * rng.standard_normal(d)
    seeds = range(5000, 8000)
    cb, ests = _sketch_estimates(d, m, b, True, x, qv, seeds)
    q0 = O.quantize(cb, x[None, :])
    n = np.linalg.norm(x)
    qt = cb.rot @ qv
    c = cb.centroids[q0["idx"][0]]
    used = c / np.linalg.norm(c)
    r = q0["y"][0] - used
    rho = np.linalg.norm(r)
    assert abs(q0["scale"][0] * (qt @ c) + n * (qt @ r) - qv @ x) < 1e-10
    var = (n * rho) ** 2 / m * (math.pi / 2 * qt @ qt - (qt @ r / rho) ** 2)
    z = (ests.mean() - qv @ x) / math.sqrt(var / len(ests))
    assert abs(z) < 4, z
    assert abs(ests.var() / var - 1) < 0.15
    # the planted mistake fails the same test
    _, bad = _sketch_estimates(d, m, b, True, x, qv, seeds, wrong_residual=True)
    zb = (bad.mean() - qv @ x) / math.sqrt(var / len(bad))
    assert abs(zb) > 10, zb


def test_dequantized_keys_match_code_scores_nc():
    # the two-path identity with norm correction on
    d, m = 40, 24
    cb = O.Codebook(d, 2, qjl_m=m, nc=True)
    rng = np.random.default_rng(13)
    x = rng.standard_normal((60, d)) * 3
    qv = rng.standard_normal(d)
    q = O.quantize(cb, x)
    xh = O.dequantize(cb, q["idx"], q["scale"], q["sign"], q["rnorm"])
    s = O.code_scores(cb, qv, q["idx"], q["scale"], q["sign"], q["rnorm"])
    assert np.max(np.abs(xh @ qv - s)) < 1e-11 * np.max(np.abs(s))
    # and the residual norm is that of y - c/|c|, not of y - c
    c = cb.centroids[q["idx"]]
    r = q["y"] - c / np.linalg.norm(c, axis=1, keepdims=True)
    assert np.allclose(q["rnorm"], np.linalg.norm(x, axis=1) * np.linalg.norm(r, axis=1), rtol=1e-12)
    assert not np.allclose(q["rnorm"], np.linalg.norm(x, axis=1) * np.linalg.norm(q["y"] - c, axis=1),
                           rtol=1e-3)


def test_dequantized_keys_match_code_scores():
    # two paths: <q, x_hat> with explicit dequantization (incl. QJL term)
    # equals the rotated-query score taken from the codes
    d, m = 48, 40
    cb = O.Codebook(d, 3, qjl_m=m)
    rng = np.random.default_rng(6)
    x = rng.standard_normal((50, d))
    qv = rng.standard_normal(d)
    q = O.quantize(cb, x)
    xh = O.dequantize(cb, q["idx"], q["scale"], q["sign"], q["rnorm"])
    s = O.code_scores(cb, qv, q["idx"], q["scale"], q["sign"], q["rnorm"])
    assert np.max(np.abs(xh @ qv - s)) < 1e-12 * np.max(np.abs(s)) * 10


# ----------------------------------------------------------------- packing


def test_pack_rows_hand_example():
    # b = 3, indices [5, 3]: bits 1,0,1 then 1,1,0 -> byte 0 = 0b00011101 = 29
    rows = O.pack_rows(np.array([[5, 3]]), 3)
    assert rows.shape == (1, 12)  # 4*b*ceil(2/32)
    assert rows[0, 0] == 29 and np.all(rows[0, 1:] == 0)
    # b = 4, [0xA, 0x5, 0xF] -> bytes 0x5A, 0x0F
    rows = O.pack_rows(np.array([[10, 5, 15]]), 4)
    assert rows[0, 0] == 0x5A and rows[0, 1] == 0x0F


def test_pack_rows_straddling_fields_bruteforce():
    rng = np.random.default_rng(7)
    for b in range(1, 9):
        idx = rng.integers(0, 1 << b, size=(5, 40))
        rows = O.pack_rows(idx, b)
        assert rows.shape[1] == 4 * b * 2
        # brute-force bit check with python integers
        for r in range(5):
            word = int.from_bytes(bytes(rows[r]), "little")
            for i in range(40):
                assert (word >> (i * b)) & ((1 << b) - 1) == idx[r, i]
            assert word >> (40 * b) == 0
        assert np.array_equal(O.unpack_rows(rows, 40, b), idx)


def test_pack_signs():
    s = np.zeros((1, 40), dtype=np.uint8)
    s[0, [0, 9, 39]] = 1
    rows = O.pack_signs(s)
    assert rows.shape == (1, 8)
    assert rows[0, 0] == 1 and rows[0, 1] == 2 and rows[0, 4] == 0x80
    assert np.array_equal(O.unpack_signs(rows, 40), s)


def test_tile32_layout_and_roundtrip():
    # hand example: d = 16, b = 4 -> one coordinate group, record r = 16 G + C
    # holds coordinate C for tokens 4G..4G+3 (slots 0-3) and 16+4G.. (4-7)
    assert O.tile32_position(0, 0, 4, 16) == 0
    assert O.tile32_position(0, 1, 4, 16) == 4
    assert O.tile32_position(0, 16, 4, 16) == 16          # slot 4 of record 0
    assert O.tile32_position(1, 0, 4, 16) == 32           # record 1 = coordinate 1
    assert O.tile32_position(0, 4, 4, 16) == 16 * 32      # record 16 = group G=1
    # d = 128: coordinate i = 16 j + C sits in group j of record 16 G + C
    assert O.tile32_position(17, 5, 4, 128) == ((16 * 1 + 1) * 8 + 1) * 8 * 4 + 1 * 4
    rng = np.random.default_rng(8)
    for d, b in ((128, 4), (128, 3), (40, 2), (16, 8), (5, 3)):
        idx = rng.integers(0, 1 << b, size=(70, d))
        blocks = O.pack_tile32(idx, b, 3)
        assert blocks.shape == (3, O.tile32_block_bytes(d, b))
        assert np.array_equal(O.unpack_tile32(blocks, d, b, 70), idx)
        # brute force on block 1 with python integers
        word = int.from_bytes(bytes(blocks[1]), "little")
        for t in range(32):
            for i in range(d):
                p = O.tile32_position(i, t, b, d)
                assert (word >> p) & ((1 << b) - 1) == idx[32 + t, i]
        # tokens beyond 70 leave zero bits
        w2 = int.from_bytes(bytes(blocks[2]), "little")
        for t in range(6, 32):
            for i in range(d):
                assert (w2 >> O.tile32_position(i, t, b, d)) & ((1 << b) - 1) == 0


def test_dequantize_sketch_term_is_unbiased_over_sketches():
    # Averaged over independent Gaussian sketches S, the residual term of the
    # reconstruction returns the residual itself (E[g sign(g.r)] = sqrt(2/pi)
    # r/|r| per row), so the mean of x_hat over sketch seeds converges to x at
    # rate ~ sqrt(d (pi/2) D / (m n)); without the term it stays at the MSE
    # error sqrt(D).  A flipped sign leaves ~2 sqrt(D), the constant
    # sqrt(2/pi) in place of sqrt(pi/2) ~0.36 sqrt(D), S in place of S^T
    # fails on the shapes (m != d).
    d, m, bits, n = 32, 48, 2, 400
    x = np.random.default_rng(11).standard_normal((4, d)) * 2.0
    acc = np.zeros_like(x)
    for s in range(n):
        cb = O.Codebook(d, bits, qjl_m=m, qjl_seed=1000 + s)
        q = O.quantize(cb, x)
        acc += O.dequantize(cb, q["idx"], q["scale"], q["sign"], q["rnorm"])
    rel = np.linalg.norm(acc / n - x, axis=1) / np.linalg.norm(x, axis=1)
    xh0 = O.dequantize(cb, q["idx"], q["scale"])
    rel0 = np.linalg.norm(xh0 - x, axis=1) / np.linalg.norm(x, axis=1)
    D = O.mse_closed_form(d, cb.centroids, cb.boundaries)
    expect = math.sqrt(d * (math.pi / 2) * D / (m * n))
    assert np.all(rel < 4 * expect), (rel, expect)
    assert np.all(rel0 > 0.5 * math.sqrt(D)), (rel0, D)


@pytest.mark.parametrize("m,nc", [(0, False), (40, False), (24, True)])
def test_code_scores_many_match_dequantized_keys(m, nc):
    # the batched scores equal <q_i, x_hat_j> with explicit dequantization,
    # for every query and row (a transposed operand or a dropped sketch term
    # fails this)
    d = 48
    cb = O.Codebook(d, 3, qjl_m=m, nc=nc)
    rng = np.random.default_rng(21)
    x = rng.standard_normal((70, d))
    qs = rng.standard_normal((9, d))
    q = O.quantize(cb, x)
    xh = O.dequantize(cb, q["idx"], q["scale"], q.get("sign"), q.get("rnorm"))
    s = O.code_scores_many(cb, qs, q["idx"], q["scale"], q.get("sign"), q.get("rnorm"))
    assert s.shape == (70, 9)
    ref = xh @ qs.T
    assert np.max(np.abs(s - ref)) < 1e-11 * np.max(np.abs(ref))
