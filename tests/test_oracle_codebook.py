"""Pins of the oracle's codebook pieces against facts fixed by the pages and
by mathematics (not against the oracle itself).

Density, Lloyd-Max and the generator follow the page "什么是TurboQuant？…"
(a2a-mcp.org blog), section "第一阶段" items 1-2.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy import stats
from scipy.integrate import quad
from scipy.special import betainc, betaln, gammaln

import oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------- density


def test_density_d3_is_uniform():
    # d = 3: coordinates of a uniform point on the 2-sphere are Uniform[-1,1]
    y = np.linspace(-0.999, 0.999, 101)
    assert np.allclose(O.coord_density(y, 3), 0.5, atol=1e-15)
    assert np.allclose(O.coord_cdf(y, 3), (1 + y) / 2, atol=1e-15)


@pytest.mark.parametrize("d", [3, 8, 128, 200])
def test_density_normalised_and_second_moment(d):
    # integrates to 1 and E[Y^2] = 1/d (a unit vector's coordinates)
    tot = quad(lambda y: O.coord_density(y, d), -1, 1, limit=200, epsabs=1e-14)[0]
    m2 = quad(lambda y: y * y * O.coord_density(y, d), -1, 1, limit=200, epsabs=1e-14)[0]
    assert abs(tot - 1) < 1e-10
    assert abs(m2 - 1.0 / d) < 1e-10


@pytest.mark.parametrize("d", [4, 16, 128])
def test_density_matches_sphere_coordinates(d):
    # Monte Carlo: first coordinate of uniform unit vectors (numpy normals,
    # normalised) follows the law; KS test against the oracle CDF.
    rng = np.random.default_rng(11 + d)
    g = rng.standard_normal((20000, d))
    y = g[:, 0] / np.linalg.norm(g, axis=1)
    p = stats.kstest(y, lambda v: O.coord_cdf(v, d)).pvalue
    assert p > 1e-3


def test_cdf_against_quadrature():
    d = 128
    for y in [-0.3, -0.1, -0.01, 0.0, 0.05, 0.2]:
        ref = quad(lambda t: O.coord_density(t, d), -1, y, limit=200, epsabs=1e-15)[0]
        assert abs(O.coord_cdf(y, d) - ref) < 1e-12


# ----------------------------------------------------------------- Lloyd-Max


@pytest.mark.parametrize("d,b", [(3, 1), (3, 2), (3, 3), (3, 5), (8, 3), (128, 1), (128, 2),
                                 (128, 3), (128, 4), (200, 4), (128, 8)])
def test_lloyd_max_conditions(d, b):
    c, t = O.lloyd_max(d, b)
    L = 1 << b
    assert c.shape == (L,) and t.shape == (L - 1,)
    assert np.all(np.diff(c) > 0)
    # symmetry and exact centre boundary
    assert np.allclose(c, -c[::-1], atol=0, rtol=0)
    assert t[L // 2 - 1] == 0.0
    # midpoint condition
    assert np.max(np.abs(t - 0.5 * (c[:-1] + c[1:]))) < 1e-15
    # centroid condition from closed forms (the oracle solves with quadrature):
    # P = I_{(1+v)/2}(a, a) - I_{(1+u)/2}(a, a) and
    # int_u^v y f_d = ((1-u^2)^a - (1-v^2)^a) / (2 a B(1/2, a)); the lower
    # half's cells (no cancellation in P), the upper half by symmetry above
    a = (d - 1) / 2
    edges = np.concatenate([[-1.0], t, [1.0]])
    for k in range(L // 2):
        lo, hi = edges[k], edges[k + 1]
        P = betainc(a, a, (1 + hi) / 2) - betainc(a, a, (1 + lo) / 2)
        M = ((1 - lo * lo) ** a - (1 - hi * hi) ** a) / (2 * a * math.exp(betaln(0.5, a)))
        assert abs(M / P - c[k]) < 1e-10, (k, M / P, c[k])


def test_lloyd_max_d3_uniform_closed_form():
    # uniform law on [-1,1]: optimal levels are cell midpoints of L equal cells
    for b in range(1, 6):
        L = 1 << b
        c, t = O.lloyd_max(3, b)
        assert np.allclose(c, (2 * np.arange(L) + 1) / L - 1, atol=1e-12)
        # per-vector MSE: 3 coordinates * (2/L)^2 / 12
        assert abs(O.mse_closed_form(3, c, t) - 3 * (2 / L) ** 2 / 12) < 1e-12


@pytest.mark.parametrize("d", [3, 16, 128, 200])
def test_lloyd_max_one_bit_is_mean_abs(d):
    # b = 1: c = +-E|Y| = +-Gamma(d/2) / (sqrt(pi) Gamma((d+1)/2))
    c, _ = O.lloyd_max(d, 1)
    eab = math.exp(gammaln(d / 2) - gammaln((d + 1) / 2)) / math.sqrt(math.pi)
    assert abs(c[1] - eab) < 1e-13
    if d == 128:
        assert abs(c[1] - 0.0706616) < 1e-7


def test_lloyd_max_gaussian_limit_max1960():
    tab = json.load(open(os.path.join(GOLD, "max1960_gaussian.json")))["levels"]
    d = 65536
    for L_s, levels in tab.items():
        L = int(L_s)
        c, _ = O.lloyd_max(d, L.bit_length() - 1)
        got = math.sqrt(d) * c[L // 2:]
        # table printed to 4 significant digits
        assert np.allclose(got, levels, rtol=6e-4, atol=0), (L, got, levels)
    # at d = 128 the O(1/d) gap is still within 1 %
    c, _ = O.lloyd_max(128, 3)
    assert np.allclose(math.sqrt(128) * c[4:], tab["8"], rtol=1e-2)


def test_mse_closed_form_values():
    # distortion per unit vector, decreasing about 4x per extra bit
    D = [O.mse_closed_form(128, *O.lloyd_max(128, b)) for b in (1, 2, 3, 4)]
    assert all(D[i + 1] < D[i] / 3 for i in range(3))
    assert abs(D[2] - 0.033966) < 2e-6


def test_page_cosine_value_3bit():
    # the page's ">= 0.983 at 3 bits": sqrt(1 - D_3) at d = 128
    page = json.load(open(os.path.join(GOLD, "page_values.json")))
    c, t = O.lloyd_max(128, 3)
    D3 = O.mse_closed_form(128, c, t)
    # the page prints the figure to 3 decimals
    assert abs(math.sqrt(1 - D3) - page["cosine_3bit_at_least"]["value"]) < 5e-4
    assert abs(math.sqrt(1 - D3) - 0.98287) < 1e-5


# ----------------------------------------------------------------- generator


def test_splitmix64_published_vector():
    # reference outputs of splitmix64 seeded with 1234567
    ref = [6457827717110365317, 3203168211198807973, 9817491932198370423,
           4593380528125082431, 16408922859458223821]
    assert [int(v) for v in O.splitmix64(1234567, 5)] == ref


def test_gaussians_are_standard_normal():
    z = O.gaussians(5, 200000)
    assert abs(z.mean()) < 5 * 1 / math.sqrt(len(z))
    assert abs(z.var() - 1) < 5 * math.sqrt(2 / len(z))
    assert stats.kstest(z[:50000], "norm").pvalue > 1e-3


# ----------------------------------------------------------------- rotation


@pytest.mark.parametrize("d", [3, 16, 128, 200])
def test_rotation_orthogonal_and_unique(d):
    P = O.rotation_matrix(d, 1)
    assert np.max(np.abs(P @ P.T - np.eye(d))) < 1e-12
    # uniqueness of QR with positive diag(R): LAPACK Householder agrees
    G = O.gaussians(1, d * d).reshape(d, d)
    Q, R = np.linalg.qr(G)
    Q = Q * np.sign(np.diag(R))[None, :]
    assert np.max(np.abs(Q - P)) < 1e-12
    # G = Pi R with R upper triangular, positive diagonal
    R2 = P.T @ G
    assert np.max(np.abs(np.tril(R2, -1))) < 1e-10
    assert np.all(np.diag(R2) > 0)


def test_rotation_haar_coordinate_law():
    # coordinates of Pi e_d (the last, fully orthogonalised column) over
    # many seeds follow the Beta law (d = 6)
    d = 6
    ys = np.array([O.rotation_matrix(d, s)[:, d - 1] for s in range(1, 1501)]).ravel()
    assert stats.kstest(ys, lambda v: O.coord_cdf(v, d)).pvalue > 1e-3


def test_rotation_seed_changes_matrix():
    assert not np.allclose(O.rotation_matrix(16, 1), O.rotation_matrix(16, 2))
