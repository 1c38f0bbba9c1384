"""Pins of the PolarQuant oracle against facts fixed by the page and by
mathematics (closed forms, brute force, library routines, invariants).

Page "什么是TurboQuant？…" (a2a-mcp.org blog), "第一阶段：随机旋转 +
PolarQuant 压缩" item 2 (recursive pairing into radius and angles, Lloyd-Max
codebooks for the angles' known law), "第二阶段：QJL 残差校正".
"""
import math

import numpy as np
import pytest
from scipy import stats
from scipy.integrate import quad
from scipy.special import betainc, betaln

import oracle as O

P = O.polar


def _unit(n, d, seed):
    g = np.random.default_rng(seed).standard_normal((n, d))
    return g / np.linalg.norm(g, axis=1, keepdims=True)


# ----------------------------------------------------------------- transform


def test_transform_inverse_roundtrip_and_radius():
    y = _unit(200, 64, 1)
    ang, rad = P.polar_transform(y)
    assert len(ang) == 6 and ang[0].shape == (200, 32) and ang[5].shape == (200, 1)
    assert np.allclose(rad[-1][:, 0], 1.0, atol=1e-14)          # the last radius is |y|
    assert np.max(np.abs(P.polar_inverse(ang) - y)) < 1e-14
    assert np.all(ang[0] >= -math.pi) and np.all(ang[0] <= math.pi)
    for a in ang[1:]:
        assert np.all(a >= 0) and np.all(a <= math.pi / 2)


def test_d4_explicit_formula():
    # d = 4: y = (cos p cos f1, cos p sin f1, sin p cos f2, sin p sin f2)
    rng = np.random.default_rng(2)
    f1, f2 = rng.uniform(-math.pi, math.pi, 5), rng.uniform(-math.pi, math.pi, 5)
    p = rng.uniform(0, math.pi / 2, 5)
    y = np.stack([np.cos(p) * np.cos(f1), np.cos(p) * np.sin(f1), np.sin(p) * np.cos(f2),
                  np.sin(p) * np.sin(f2)], axis=1)
    got = P.polar_inverse([np.stack([f1, f2], 1), p[:, None]])
    assert np.max(np.abs(got - y)) < 1e-15
    ang, _ = P.polar_transform(y)
    assert np.allclose(ang[0], np.stack([f1, f2], 1), atol=1e-12)
    assert np.allclose(ang[1][:, 0], p, atol=1e-12)


# ----------------------------------------------------------------- angle laws


def test_level1_angles_uniform():
    # first-level angles of isotropic pairs are uniform on [-pi, pi]
    x = np.random.default_rng(3).standard_normal((4000, 32))
    cb = P.PolarCodebook(32, 4, 2)
    ang = P.quantize(cb, x)["angles"][0].ravel()
    assert stats.kstest(ang, lambda v: (v + math.pi) / (2 * math.pi)).pvalue > 1e-3


@pytest.mark.parametrize("level", [2, 3, 4, 5, 6, 7])
def test_higher_level_angle_laws(level):
    # sin^2 of a level-l angle ~ Beta(k/2, k/2), k = 2^(l-1): KS against the
    # library CDF, on Haar-rotated Gaussian vectors
    x = np.random.default_rng(10 + level).standard_normal((3000, 128))
    cb = P.PolarCodebook(128, 4, 2)
    ang = P.quantize(cb, x)["angles"][level - 1][:, :8].ravel()
    k = 2 ** (level - 1)
    assert stats.kstest(np.sin(ang) ** 2, lambda u: betainc(k / 2, k / 2, u)).pvalue > 1e-3
    # the oracle's CDF is that law
    grid = np.linspace(0.01, 1.55, 7)
    assert np.allclose(P.angle_cdf(grid, level), betainc(k / 2, k / 2, np.sin(grid) ** 2), atol=1e-15)


@pytest.mark.parametrize("level", [1, 2, 3, 5, 7])
def test_angle_density_normalised(level):
    lo, hi = (-math.pi, math.pi) if level == 1 else (0.0, math.pi / 2)
    tot = quad(lambda p: float(P.angle_density(p, level)), lo, hi, limit=200)[0]
    assert abs(tot - 1) < 1e-10
    for p in np.linspace(lo + 0.1, hi - 0.1, 5):
        h = 1e-6
        num = (P.angle_cdf(p + h, level) - P.angle_cdf(p - h, level)) / (2 * h)
        assert abs(num - P.angle_density(p, level)) < 1e-6


# ----------------------------------------------------------------- codebooks


@pytest.mark.parametrize("bits", [1, 2, 3, 4, 6])
def test_level1_codebook_is_uniform_quantizer(bits):
    c, t = P.angle_codebook(1, bits)
    L = 1 << bits
    w = 2 * math.pi / L
    assert np.allclose(c, -math.pi + w * (np.arange(L) + 0.5), atol=1e-15)
    assert np.allclose(t, -math.pi + w * np.arange(1, L), atol=1e-15)
    assert t[L // 2 - 1] == 0.0


@pytest.mark.parametrize("bits", [1, 2, 3, 4])
def test_level2_codebook_closed_form(bits):
    # level 2: density sin(2 psi), mass F = sin^2, first moment
    # -psi cos(2 psi)/2 + sin(2 psi)/4: the centroid condition in closed form
    c, t = P.angle_codebook(2, bits)
    L = 1 << bits
    e = np.concatenate([[0.0], t, [math.pi / 2]])
    mass = np.sin(e[1:]) ** 2 - np.sin(e[:-1]) ** 2
    F1 = lambda p: -p * np.cos(2 * p) / 2 + np.sin(2 * p) / 4
    mom = F1(e[1:]) - F1(e[:-1])
    assert np.max(np.abs(mom / mass - c)) < 1e-12
    assert np.max(np.abs(t - 0.5 * (c[:-1] + c[1:]))) < 1e-15
    assert abs(t[L // 2 - 1] - math.pi / 4) == 0.0 if L > 1 else True
    assert np.allclose(c, math.pi / 2 - c[::-1], atol=1e-15)


@pytest.mark.parametrize("level,bits", [(3, 2), (4, 2), (5, 3), (7, 2), (8, 2)])
def test_higher_codebook_centroid_condition_in_u(level, bits):
    # centroid condition checked in the variable u = sin^2(psi) (a different
    # integrand from the oracle's): E[psi | cell] = int arcsin(sqrt u)
    # Beta(u; k/2, k/2) du over the cell's u-range / its Beta mass
    c, t = P.angle_codebook(level, bits)
    k = 2 ** (level - 1)
    a = k / 2
    ue = np.sin(np.concatenate([[0.0], t, [math.pi / 2]])) ** 2
    lb = betaln(a, a)
    for j in range(len(c)):
        m = betainc(a, a, ue[j + 1]) - betainc(a, a, ue[j])
        g = lambda u: math.asin(math.sqrt(u)) * math.exp((a - 1) * (math.log(u) + math.log1p(-u)) - lb)
        mom = quad(g, ue[j], ue[j + 1], epsabs=0, epsrel=1e-12, limit=400)[0]
        assert abs(mom / m - c[j]) < 1e-10, (j, mom / m, c[j])


# ----------------------------------------------------------------- distortion


@pytest.mark.parametrize("L", [4, 8, 16, 64])
def test_d2_mse_closed_form(L):
    # d = 2, one level: uniform angle, cells of width 2 pi / L with centred
    # centroids: E|y - y_hat|^2 = 2 - 2 sin(pi/L) / (pi/L)
    b = L.bit_length() - 1
    cb = P.PolarCodebook(2, b, 1)
    x = np.random.default_rng(4).standard_normal((200000, 2))
    r = P.quantize(cb, x)
    err = np.sum((r["y"] - r["y_hat"]) ** 2, axis=1)
    D = 2 - 2 * math.sin(math.pi / L) / (math.pi / L)
    assert abs(err.mean() - D) < 4 * err.std() / math.sqrt(len(err))


def test_reconstruction_unit_norm_and_zero_vector():
    cb = P.PolarCodebook(64, 4, 2, qjl_m=16)
    x = np.random.default_rng(5).standard_normal((50, 64)) * 3
    x[7] = 0
    r = P.quantize(cb, x)
    assert np.max(np.abs(np.linalg.norm(r["y_hat"], axis=1) - 1)) < 1e-14
    assert r["scale"][7] == 0 and r["rnorm"][7] == 0
    xh = P.dequantize(cb, r["idx"], r["scale"], r["sign"], r["rnorm"])
    assert np.all(xh[7] == 0)


def test_mse_falls_with_bits_and_round_trip_converges():
    d = 64
    x = np.random.default_rng(6).standard_normal((1500, d))
    errs = []
    for b1, br in ((2, 1), (3, 1), (4, 2), (5, 3), (6, 4), (8, 6)):
        cb = P.PolarCodebook(d, b1, br)
        r = P.quantize(cb, x)
        xh = P.dequantize(cb, r["idx"], r["scale"])
        errs.append(np.mean(np.sum((x - xh) ** 2, 1) / np.sum(x * x, 1)))
    assert all(errs[i + 1] < errs[i] for i in range(len(errs) - 1)), errs
    assert errs[-1] < 1e-3


def test_mse_comparable_to_scalar_at_three_bits():
    # the page's "3 bits in total" main stage: (4, 2) spends 3d - 2 bits;
    # its distortion is within 10 % of the scalar 3-bit Lloyd-Max (0.033966)
    d = 128
    x = np.random.default_rng(7).standard_normal((3000, d))
    cb = P.PolarCodebook(d, 4, 2)
    assert cb.field_bits() == 3 * d - 2
    r = P.quantize(cb, x)
    xh = P.dequantize(cb, r["idx"], r["scale"])
    e = np.mean(np.sum((x - xh) ** 2, 1) / np.sum(x * x, 1))
    D3 = O.mse_closed_form(d, *O.lloyd_max(d, 3))
    assert 0.9 * D3 < e < 1.1 * D3, (e, D3)


# ----------------------------------------------------------------- QJL


def test_polar_qjl_unbiased_and_two_paths():
    d, m = 16, 16
    rng = np.random.default_rng(8)
    x = rng.standard_normal(d)
    qv = x + 0.5 * rng.standard_normal(d)
    cb = P.PolarCodebook(d, 3, 1, qjl_m=m)
    q0 = P.quantize(cb, x[None])
    n = np.linalg.norm(x)
    qt = cb.rot @ qv
    r = q0["y"][0] - q0["y_hat"][0]
    rho = np.linalg.norm(r)
    assert abs(n * (qt @ q0["y_hat"][0]) + n * (qt @ r) - qv @ x) < 1e-10
    var = (n * rho) ** 2 / m * (math.pi / 2 * qt @ qt - (qt @ r / rho) ** 2)
    ests = []
    for s in range(3000):
        cb.qjl = O.qjl_matrix(m, d, 9000 + s)
        qq = P.quantize(cb, x[None])
        ests.append(P.code_scores(cb, qv, qq["idx"], qq["scale"], qq["sign"], qq["rnorm"])[0])
    ests = np.array(ests)
    z = (ests.mean() - qv @ x) / math.sqrt(var / len(ests))
    assert abs(z) < 4, z
    assert abs(ests.var() / var - 1) < 0.15
    # two paths: explicit reconstruction vs scores from the codes
    X = rng.standard_normal((40, d))
    qq = P.quantize(cb, X)
    xh = P.dequantize(cb, qq["idx"], qq["scale"], qq["sign"], qq["rnorm"])
    s = P.code_scores(cb, qv, qq["idx"], qq["scale"], qq["sign"], qq["rnorm"])
    assert np.max(np.abs(xh @ qv - s)) < 1e-11 * np.max(np.abs(s))


# ----------------------------------------------------------------- packing


def test_pack_hand_example_and_roundtrip():
    # d = 4, b1 = 3, br = 2: level-1 fields [5, 3] then level-2 field [2]:
    # bits 1,0,1 | 1,1,0 | 0,1 (bit 0 first) -> byte 0 = 0b10011101 = 157
    rows = P.pack_rows([np.array([[5, 3]]), np.array([[2]])], 4, 3, 2)
    assert rows.shape == (1, 4)
    assert rows[0, 0] == 157 and np.all(rows[0, 1:] == 0)
    rng = np.random.default_rng(9)
    for d, b1, br in ((128, 4, 2), (64, 5, 3), (8, 3, 1), (32, 8, 7)):
        idx = [rng.integers(0, 1 << P.level_bits(lv, b1, br), size=(6, d >> lv))
               for lv in range(1, P.n_levels(d) + 1)]
        rows = P.pack_rows(idx, d, b1, br)
        assert rows.shape[1] == P.row_bytes(d, b1, br)
        back = P.unpack_rows(rows, d, b1, br)
        assert all(np.array_equal(a, b) for a, b in zip(idx, back))
        word = int.from_bytes(bytes(rows[2]), "little")
        pos = 0
        for lv in range(1, P.n_levels(d) + 1):
            b = P.level_bits(lv, b1, br)
            for i in range(d >> lv):
                assert (word >> pos) & ((1 << b) - 1) == idx[lv - 1][2, i]
                pos += b
        assert word >> pos == 0


# ----------------------------------------------------------------- decode


def test_polar_attention_bruteforce_tiny():
    # d = 4, N = 3: logits from explicitly rebuilt keys (trigonometric
    # formula), softmax and the scalar value reconstruction
    d, N = 4, 3
    rng = np.random.default_rng(10)
    kx, vx, q = rng.standard_normal((N, d)), rng.standard_normal((N, d)), rng.standard_normal((1, 2, d))
    kcb, vcb = P.PolarCodebook(d, 3, 2), O.Codebook(d, 3, rot_seed=5)
    rk, rv = P.quantize(kcb, kx), O.quantize(vcb, vx)
    kc = dict(idx=[a[None, None] for a in rk["idx"]], scale=rk["scale"][None, None])
    vc = dict(idx=rv["idx"][None, None], scale=rv["scale"][None, None])
    lg, out = P.attn_decode(kcb, vcb, q, kc, vc, 0.5)
    c1, c2 = kcb.books[1][0], kcb.books[2][0]
    vh = O.dequantize(vcb, rv["idx"], rv["scale"])
    for hq in range(2):
        ref_l = []
        for j in range(N):
            f1, f2 = c1[rk["idx"][0][j]]
            p = c2[rk["idx"][1][j, 0]]
            yh = [math.cos(p) * math.cos(f1), math.cos(p) * math.sin(f1), math.sin(p) * math.cos(f2),
                  math.sin(p) * math.sin(f2)]
            xh = [sum(kcb.rot[i, c] * yh[i] for i in range(d)) * rk["scale"][j] for c in range(d)]
            ref_l.append(0.5 * sum(q[0, hq, c] * xh[c] for c in range(d)))
        w = [math.exp(v - max(ref_l)) for v in ref_l]
        ref_o = [sum(w[j] * vh[j, c] for j in range(N)) / sum(w) for c in range(d)]
        assert np.allclose(lg[0, hq], ref_l, atol=1e-13)
        assert np.allclose(out[0, hq], ref_o, atol=1e-13)


def test_boundary_distance_zero_on_a_ray():
    cb = P.PolarCodebook(4, 2, 1)
    cb.rot = np.eye(4)                         # test the rotated domain directly
    t1 = cb.books[1][1][0]                     # a level-1 decision ray
    y = np.array([[math.cos(t1) * 0.6, math.sin(t1) * 0.6, 0.8, 0.0]])
    r = P.quantize(cb, y)
    dist = P.boundary_distance(cb, r)
    assert dist[0][0, 0] < 1e-15
    assert dist[0][0, 1] < 1e-15                # (0.8, 0): on the ray at angle 0
    assert r["idx"][0][0, 0] == 1               # a tie goes to the upper cell
    # level 2 pairs the radii (0.6, 0.8): distance = 1 * |sin(psi - t)|
    psi = math.atan2(0.8, 0.6)
    t2 = cb.books[2][1]
    assert dist[1].shape == (1, 1)
    assert abs(dist[1][0, 0] - np.min(np.abs(np.sin(psi - t2)))) < 1e-15
    # shapes: one distance per angle at every level (d = 16)
    cb16 = P.PolarCodebook(16, 3, 2)
    r16 = P.quantize(cb16, np.random.default_rng(1).standard_normal((3, 16)))
    assert [x.shape for x in P.boundary_distance(cb16, r16)] == [a.shape for a in r16["angles"]]
    assert all(np.allclose(pr, np.hypot(*([r16["y"][:, 0::2], r16["y"][:, 1::2]] if lv == 0 else
                                            [r16["pair_radius"][lv - 1][:, 0::2], r16["pair_radius"][lv - 1][:, 1::2]])))
               for lv, pr in enumerate(r16["pair_radius"]))
