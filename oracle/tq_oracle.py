"""Float64 CPU oracle of TurboQuant-style online KV-vector quantization.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg; never by the GPU product path.

Sources (web pages; cited by title and section):

* [WIT] "什么是TurboQuant？谷歌突破性AI压缩技术实现6倍KV缓存缩减和8倍推理加速"
  (a2a-mcp.org blog, "What is TurboQuant?").  Sections used:
  - "TurboQuant 工作原理" > "第一阶段" item 1: every KV vector is multiplied by
    one data-independent random orthogonal matrix obtained from the QR
    decomposition of a Gaussian matrix; afterwards each coordinate on [-1, 1]
    follows Beta((d-1)/2, (d-1)/2), so optimal centroids can be computed
    analytically in advance.
  - "第一阶段" item 2: vectors are normalised; a Lloyd-Max quantizer that is
    MSE-optimal for that Beta law maps each coordinate to a few bits.
  - "第二阶段：QJL 残差校正": the remaining residual gets a 1-bit (+1/-1)
    quantized Johnson-Lindenstrauss sketch that removes inner-product bias.
  - "如何实现 TurboQuant" item 1: the Lloyd-Max codebook is precomputed per
    head dimension and bit width; the query is rotated once and attention dot
    products are taken straight from the stored indices.
  - "基准测试与实际性能表现": top-k inner-product search on d=200 vectors.
* [AGENT] "6倍KV缓存压缩零精度损失：谷歌TurboQuant技术如何提升智能体运行效率",
  section "三、工程实现" item 1: the method comes as a compress / decompress
  pair (no formula given for the decompress side).
* [VLLM] "A First Comprehensive Study of TurboQuant: Accuracy and Performance"
  (papercache.org summary), section A3: variant names k8v4, 4bit_nc,
  k3v4_nc, 3bit_nc ("nc" = norm correction; not defined further).

Readings where the pages are silent (each is listed in the design notes):

* R1 density: (1+y)/2 ~ Beta(a, a) with a = (d-1)/2, i.e.
  f_d(y) = (1-y^2)^(a-1) / B(1/2, a) on [-1, 1]; needs d >= 3.
* R2 Lloyd-Max: the unique quantizer meeting the centroid and midpoint
  conditions for f_d (unique because f_d is log-concave).  Computed by
  damped Newton steps on the midpoint residual from the quantile start, with
  every cell mass and moment taken by adaptive Gauss-Kronrod quadrature of
  f_d; centroids symmetric, c[L-1-k] = -c[k], so the middle boundary is 0.
* R3 generator: splitmix64 (Steele, Lea, Flood 2014) seeded with the seed;
  uniform u = (x >> 11) * 2^-53; one normal per two uniforms by Box-Muller,
  z = sqrt(-2 ln(1 - u1)) * cos(2 pi u2); matrices filled row-major.
* R4 rotation: G = QR with diag(R) > 0 and Pi = Q (unique per G, Haar);
  y = Pi x / |x|, and y = 0 when x = 0.
* R5 index: idx_i = #{k : y_i >= t_k} (a tie goes to the upper cell).
* R6 norm correction (nc): the stored scale is |x| / |c[idx]| so the unit
  direction is rebuilt as c[idx]/|c[idx]|; without nc the scale is |x|.
* R7 QJL: m sketch rows S ~ N(0,1)^{m x d} (own seed); residual
  r = y - (scale/|x|) c[idx] in the rotated unit-scale domain; one sign bit
  per row, sigma_j = [ (S r)_j >= 0 ]; stored rnorm = |x| |r|; estimator
  <q, x> ~ scale <Pi q, c[idx]> + sqrt(pi/2)/m * rnorm * <S Pi q, 2 sigma - 1>,
  unbiased because E[(g.a) sign(g.b)] = sqrt(2/pi) a.b/|b| for g ~ N(0, I).
* R8 decode: logit_j = tau * (that estimate); softmax over all cached tokens
  (no mask); output = sum_j p_j * scale^V_j * Pi_V^T c_V[idx^V_j].
* R9 top-k: the same estimate without tau; descending score, ties to the
  lower database index.
* R10 packed formats (pages silent; "bit-packed indices"):
  - row layout: index i of a vector at bits [i*b, i*b+b) of a little-endian
    bit stream (bit p in byte p>>3, position p&7), row padded with zero bits
    to 4*b*ceil(d/32) bytes; sign j at bit j of a 4*ceil(m/32)-byte row.
  - tile32 layout (value codes): per sequence, blocks of 32 tokens; inside a
    block, the bit of (coordinate i, token t) is given by tile32_position:
    64 records of 8 tokens x ceil(d/16) coordinates, so that one GPU lane
    reads the codes of its 8 tokens for 8 coordinates as one contiguous run.
* R13 dequantize: both stages inverted in the original domain,
  x_hat = Pi^T (scale c[idx]) + rnorm sqrt(pi/2)/m Pi^T S^T (2 sigma - 1), so
  that <q, x_hat> is the R7 estimate for every q.
"""
from __future__ import annotations

import math

import numpy as np
from scipy.integrate import quad
from scipy.special import betainc, betaincinv, betaln

SQRT_HALF_PI = math.sqrt(math.pi / 2.0)

# ---------------------------------------------------------------------------
# R1: coordinate law after a Haar rotation ([WIT] 第一阶段 item 1)
# ---------------------------------------------------------------------------


def beta_alpha(d: int) -> float:
    if d < 3:
        raise ValueError("the Beta coordinate law needs d >= 3")
    return (d - 1) / 2.0


def coord_density(y, d: int):
    """f_d(y) = (1 - y^2)^((d-3)/2) / B(1/2, (d-1)/2) on [-1, 1]."""
    a = beta_alpha(d)
    y = np.asarray(y, dtype=np.float64)
    inside = np.abs(y) <= 1.0
    w = np.where(inside, 1.0 - y * y, 0.0)
    return np.where(inside, np.power(w, a - 1.0) * math.exp(-betaln(0.5, a)), 0.0)


def coord_cdf(y, d: int):
    """P(Y <= y) = I_{(1+y)/2}(a, a)."""
    a = beta_alpha(d)
    y = np.clip(np.asarray(y, dtype=np.float64), -1.0, 1.0)
    return betainc(a, a, (1.0 + y) / 2.0)


def _density_scalar(d: int):
    """f_d as a plain float function of one point (the quadrature integrand)."""
    a = beta_alpha(d)
    log_norm = betaln(0.5, a)

    def f(y: float) -> float:
        w = 1.0 - y * y
        if w <= 0.0:
            return math.exp(-log_norm) if a == 1.0 else 0.0
        return math.exp((a - 1.0) * math.log(w) - log_norm)

    return f


def _cell_integrals(edges, f):
    """Mass P_k = int f and first moment M_k = int y f over each cell
    [edges[k], edges[k+1]] of a density f (a float function of one point),
    by adaptive Gauss-Kronrod quadrature (QUADPACK through
    scipy.integrate.quad) of the density itself: no antiderivative, no
    incomplete-beta function."""
    n = len(edges) - 1
    P, M = np.empty(n), np.empty(n)
    for k in range(n):
        u, v = float(edges[k]), float(edges[k + 1])
        P[k] = quad(f, u, v, epsabs=0.0, epsrel=1e-13, limit=400)[0]
        M[k] = quad(lambda y: y * f(y), u, v, epsabs=0.0, epsrel=1e-13, limit=400)[0]
    return P, M


def symmetric_lloyd_max(f, lo: float, mid: float, start, *, max_newton: int = 100, what: str = ""):
    """Lloyd-Max quantizer with L = 2 len(start) levels of a density f on
    [lo, 2 mid - lo] that is symmetric about mid.

    The quantizer is the one whose boundaries are the midpoints of adjacent
    centroids and whose centroids are the conditional means of their cells
    (unique for a log-concave f).  By symmetry only the cells inside
    [lo, mid] are solved, with inner boundaries t_1..t_{h-1} (h = L/2) and
    t_h = mid; the upper half is the mirror image.  The boundaries are found
    by damped Newton steps on the midpoint residual
        R_k(t) = t_k - (c_{k-1}(t) + c_k(t)) / 2,   c_k(t) = M_k / P_k,
    started from the midpoints of ``start`` (lower-half centroid guesses,
    increasing); cell masses and moments come from adaptive quadrature, and
    dc_k/dt of a cell edge from the density there.  Returns
    (centroids[L], boundaries[L-1]) in float64, increasing, with the middle
    boundary exactly mid.
    """
    start = np.asarray(start, dtype=np.float64)
    h = len(start)
    L = 2 * h

    def centroids_of(t):
        edges = np.concatenate([[lo], t, [mid]])
        P, M = _cell_integrals(edges, f)
        return edges, P, M / P

    if h == 1:
        _, _, c = centroids_of(np.empty(0))
    else:
        t = 0.5 * (start[:-1] + start[1:])
        edges, P, c = centroids_of(t)
        R = t - 0.5 * (c[:-1] + c[1:])
        r = np.max(np.abs(R))
        for _ in range(max_newton):
            if r == 0.0:
                break
            fe = np.array([f(x) for x in edges])
            dl = fe[:-1] * (c - edges[:-1]) / P      # dc_k / d(lower edge of cell k)
            dr = fe[1:] * (edges[1:] - c) / P        # dc_k / d(upper edge of cell k)
            J = np.zeros((h - 1, h - 1))
            for k in range(1, h):                    # row of R_k, column of t_j
                J[k - 1, k - 1] = 1.0 - 0.5 * (dr[k - 1] + dl[k])
                if k >= 2:
                    J[k - 1, k - 2] = -0.5 * dl[k - 1]
                if k <= h - 2:
                    J[k - 1, k] = -0.5 * dr[k]
            step = np.linalg.solve(J, R)
            lam, accepted = 1.0, False
            while lam >= 2.0 ** -20:
                tn = t - lam * step
                if np.all(np.diff(np.concatenate([[lo], tn, [mid]])) > 0):
                    en, Pn, cn = centroids_of(tn)
                    Rn = tn - 0.5 * (cn[:-1] + cn[1:])
                    rn = np.max(np.abs(Rn))
                    if rn < r:
                        accepted = True
                        break
                lam *= 0.5
            if not accepted:
                break
            t, edges, P, c, R, r = tn, en, Pn, cn, Rn, rn
        if r > 1e-13 * max(1.0, abs(mid - lo)):
            raise ArithmeticError(f"Lloyd-Max did not converge ({what}, residual {r:.3g})")
    cent = np.concatenate([c, 2.0 * mid - c[::-1]])
    bnd = 0.5 * (cent[:-1] + cent[1:])
    bnd[h - 1] = mid
    return cent, bnd


# ---------------------------------------------------------------------------
# R2: Lloyd-Max for f_d ([WIT] 第一阶段 item 2; 如何实现 item 1)
# ---------------------------------------------------------------------------


_LM_CACHE: dict = {}


def lloyd_max(d: int, bits: int):
    """Cached :func:`lloyd_max_solve` (a pure function of d and bits)."""
    key = (int(d), int(bits))
    if key not in _LM_CACHE:
        _LM_CACHE[key] = lloyd_max_solve(*key)
    c, t = _LM_CACHE[key]
    return c.copy(), t.copy()


def lloyd_max_solve(d: int, bits: int):
    """Lloyd-Max quantizer of f_d with L = 2^bits levels (symmetric about 0
    on [-1, 1]), started from the cell-centre quantiles (k + 1/2)/L of the
    law.  Returns (centroids[L], boundaries[L-1]) in float64, increasing,
    with the middle boundary exactly 0."""
    if not 1 <= bits <= 8:
        raise ValueError("bits must be in 1..8")
    L = 1 << bits
    a = beta_alpha(d)
    start = 2.0 * betaincinv(a, a, (np.arange(L // 2) + 0.5) / L) - 1.0
    return symmetric_lloyd_max(_density_scalar(d), -1.0, 0.0, start, what=f"d={d}, bits={bits}")


def mse_closed_form(d: int, centroids, boundaries) -> float:
    """Per-vector distortion E|y - c[idx(y)]|^2 for unit y (centroid form):
    1 - d * sum_k c_k^2 P_k."""
    t = np.concatenate([[-1.0], boundaries, [1.0]])
    P = coord_cdf(t[1:], d) - coord_cdf(t[:-1], d)
    return 1.0 - d * float(np.sum(np.asarray(centroids) ** 2 * P))


# ---------------------------------------------------------------------------
# R3: seeded Gaussian matrices (splitmix64 + Box-Muller)
# ---------------------------------------------------------------------------

_GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)


def splitmix64(seed: int, count: int) -> np.ndarray:
    """First ``count`` outputs of splitmix64 started from state ``seed``."""
    with np.errstate(over="ignore"):
        k = np.arange(1, count + 1, dtype=np.uint64)
        z = np.uint64(seed & 0xFFFFFFFFFFFFFFFF) + k * _GAMMA
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
        z = z ^ (z >> np.uint64(31))
    return z


def gaussians(seed: int, count: int) -> np.ndarray:
    x = splitmix64(seed, 2 * count)
    u = (x >> np.uint64(11)).astype(np.float64) * (2.0 ** -53)
    u1, u2 = u[0::2], u[1::2]
    return np.sqrt(-2.0 * np.log1p(-u1)) * np.cos(2.0 * math.pi * u2)


def rotation_matrix(d: int, seed: int) -> np.ndarray:
    """Pi = Q of G = QR, diag(R) > 0, G ~ N(0,1)^{d x d} row-major from seed
    ([WIT] 第一阶段 item 1).  Modified Gram-Schmidt on G's columns with one
    re-orthogonalisation pass."""
    G = gaussians(seed, d * d).reshape(d, d)
    Q = np.zeros((d, d))
    for j in range(d):
        v = G[:, j].copy()
        for _ in range(2):
            for i in range(j):
                v -= np.dot(Q[:, i], v) * Q[:, i]
        Q[:, j] = v / np.linalg.norm(v)
    return Q


def qjl_matrix(m: int, d: int, seed: int) -> np.ndarray:
    """S ~ N(0,1)^{m x d}, row-major from seed ([WIT] 第二阶段)."""
    return gaussians(seed, m * d).reshape(m, d)


class Codebook:
    """Everything a (d, bits, m, nc, seeds) choice fixes, in float64."""

    def __init__(self, d, bits, qjl_m=0, nc=False, rot_seed=1, qjl_seed=2):
        self.d, self.bits, self.m, self.nc = int(d), int(bits), int(qjl_m), bool(nc)
        self.rot_seed, self.qjl_seed = int(rot_seed), int(qjl_seed)
        self.centroids, self.boundaries = lloyd_max(self.d, self.bits)
        self.rot = rotation_matrix(self.d, self.rot_seed)
        self.qjl = qjl_matrix(self.m, self.d, self.qjl_seed) if self.m > 0 else None

    @property
    def levels(self):
        return 1 << self.bits


# ---------------------------------------------------------------------------
# Quantizer: rotation, norm, index, scale, QJL sign sketch
# ---------------------------------------------------------------------------


def coord_index(y, boundaries):
    """R5: idx = #{k : y >= t_k}; a coordinate on a boundary goes up."""
    y = np.asarray(y, dtype=np.float64)
    idx = np.zeros(y.shape, dtype=np.int16)
    for t in boundaries:
        idx += (y >= t)
    return idx


def quantize(cb: Codebook, x):
    """Quantize vectors x [n, d] (any float dtype; taken exactly into fp64).

    Returns a dict: idx int16 [n,d], scale [n], sign uint8 [n,m] or None,
    rnorm [n] or None, plus y [n,d] and u [n,m] (S r) for boundary-zone
    accounting.
    """
    x = np.asarray(x, dtype=np.float64)
    n = np.sqrt(np.sum(x * x, axis=1))
    z = x @ cb.rot.T                                   # Pi x
    safe = np.where(n > 0, n, 1.0)
    y = np.where(n[:, None] > 0, z / safe[:, None], 0.0)
    idx = coord_index(y, cb.boundaries)
    yh = cb.centroids[idx]
    if cb.nc:
        nh = np.sqrt(np.sum(yh * yh, axis=1))
        scale = n / nh
        used = yh / nh[:, None]
    else:
        scale = n.copy()
        used = yh
    out = dict(idx=idx, scale=scale, sign=None, rnorm=None, y=y, u=None)
    if cb.m > 0:
        r = y - used
        rho = np.sqrt(np.sum(r * r, axis=1))
        u = r @ cb.qjl.T
        out["sign"] = (u >= 0).astype(np.uint8)
        out["rnorm"] = n * rho
        out["u"] = u
    return out


def dequantize(cb: Codebook, idx, scale, sign=None, rnorm=None):
    """x_hat in the original domain (R13; [AGENT] 三、工程实现 item 1, [WIT]
    第一阶段 and 第二阶段): scale * Pi^T c[idx], plus (when signs are given)
    the QJL term rnorm * sqrt(pi/2)/m * Pi^T S^T (2 sigma - 1)."""
    yh = cb.centroids[np.asarray(idx)] * np.asarray(scale, dtype=np.float64)[:, None]
    if sign is not None and cb.m > 0:
        pm = 2.0 * np.asarray(sign, dtype=np.float64) - 1.0
        yh = yh + (SQRT_HALF_PI / cb.m) * np.asarray(rnorm)[:, None] * (pm @ cb.qjl)
    return yh @ cb.rot


# ---------------------------------------------------------------------------
# R10: packed formats
# ---------------------------------------------------------------------------


def idx_row_bytes(d: int, bits: int) -> int:
    return 4 * bits * ((d + 31) // 32)


def sign_row_bytes(m: int) -> int:
    return 4 * ((m + 31) // 32)


def pack_rows(idx, bits: int, row_bytes: int | None = None) -> np.ndarray:
    """idx [n, d] -> uint8 [n, row_bytes]: LSB-first bit stream per row."""
    idx = np.asarray(idx, dtype=np.int64)
    n, d = idx.shape
    rb = idx_row_bytes(d, bits) if row_bytes is None else row_bytes
    bitarr = np.zeros((n, rb * 8), dtype=np.uint8)
    for bb in range(bits):
        bitarr[:, np.arange(d) * bits + bb] = (idx >> bb) & 1
    return np.packbits(bitarr, axis=1, bitorder="little")


def unpack_rows(rows, d: int, bits: int) -> np.ndarray:
    rows = np.asarray(rows, dtype=np.uint8)
    bitarr = np.unpackbits(rows, axis=1, bitorder="little").astype(np.int64)
    out = np.zeros((rows.shape[0], d), dtype=np.int64)
    for bb in range(bits):
        out |= bitarr[:, np.arange(d) * bits + bb] << bb
    return out


def pack_signs(sign, row_bytes: int | None = None) -> np.ndarray:
    sign = np.asarray(sign, dtype=np.uint8)
    n, m = sign.shape
    rb = sign_row_bytes(m) if row_bytes is None else row_bytes
    bitarr = np.zeros((n, rb * 8), dtype=np.uint8)
    bitarr[:, :m] = sign
    return np.packbits(bitarr, axis=1, bitorder="little")


def unpack_signs(rows, m: int) -> np.ndarray:
    return np.unpackbits(np.asarray(rows, dtype=np.uint8), axis=1,
                         bitorder="little")[:, :m]


def tile32_position(i: int, t: int, bits: int, d: int) -> int:
    """Bit position of (coordinate i, token t in 0..31) inside a tile32 block.

    The block is 64 records; record r = 16*G + C holds coordinates
    i = 16*j + C (j = 0..ceil(d/16)-1, one b-byte group each) for the eight
    token slots e = 0..7 of slot group G, where slot e holds token
    4*G + (e % 4) + 16*(e // 4).  Inside the group, slot e is at bits
    [e*b, e*b + b)."""
    ndb = (d + 15) // 16
    C, j = i % 16, i // 16
    G = (t % 16) // 4
    e = (t % 4) + 4 * (t // 16)
    r = 16 * G + C
    return ((r * ndb + j) * 8 + e) * bits


def tile32_block_bytes(d: int, bits: int) -> int:
    return 64 * ((d + 15) // 16) * bits


def _tile32_positions(d: int, bits: int) -> np.ndarray:
    """[32, d] bit positions of (token, coordinate) inside a block."""
    return np.array([[tile32_position(i, t, bits, d) for i in range(d)] for t in range(32)],
                    dtype=np.int64)


def pack_tile32(idx, bits: int, n_blocks: int) -> np.ndarray:
    """idx [n_tok, d] of one sequence -> uint8 [n_blocks, block_bytes].
    Tokens >= n_tok and padding coordinates leave zero bits."""
    idx = np.asarray(idx, dtype=np.int64)
    n_tok, d = idx.shape
    pos = _tile32_positions(d, bits)
    full = np.zeros((n_blocks * 32, d), dtype=np.int64)
    full[:n_tok] = idx
    full = full.reshape(n_blocks, 32, d)
    out = np.zeros((n_blocks, tile32_block_bytes(d, bits) * 8), dtype=np.uint8)   # one byte per bit
    for bb in range(bits):
        out[:, (pos + bb).reshape(-1)] = ((full >> bb) & 1).reshape(n_blocks, -1)
    return np.packbits(out, axis=1, bitorder="little")


def unpack_tile32(blocks, d: int, bits: int, n_tok: int) -> np.ndarray:
    blocks = np.asarray(blocks, dtype=np.uint8)
    nb = blocks.shape[0]
    bitarr = np.unpackbits(blocks, axis=1, bitorder="little").astype(np.int64)
    pos = _tile32_positions(d, bits).reshape(-1)
    out = np.zeros((nb, 32 * d), dtype=np.int64)
    for bb in range(bits):
        out |= bitarr[:, pos + bb] << bb
    return out.reshape(nb * 32, d)[:n_tok]


# ---------------------------------------------------------------------------
# R8: decode attention from codes ([WIT] 如何实现 item 1; 工作原理 end)
# ---------------------------------------------------------------------------


def code_scores(kcb: Codebook, q, idx, scale, sign=None, rnorm=None):
    """Inner-product estimates of one query q [d] against coded vectors:
    scale_j <Pi q, c[idx_j]> + sqrt(pi/2)/m rnorm_j <S Pi q, 2 sigma_j - 1>."""
    qt = kcb.rot @ np.asarray(q, dtype=np.float64)
    s = np.asarray(scale, dtype=np.float64) * (kcb.centroids[np.asarray(idx)] @ qt)
    if sign is not None and kcb.m > 0:
        tq = kcb.qjl @ qt
        pm = 2.0 * np.asarray(sign, dtype=np.float64) - 1.0
        s = s + (SQRT_HALF_PI / kcb.m) * np.asarray(rnorm, dtype=np.float64) * (pm @ tq)
    return s


def code_scores_many(kcb: Codebook, queries, idx, scale, sign=None, rnorm=None):
    """code_scores of several queries [nq, d] at once, as a matrix [n, nq]:
    the same two terms, each one matrix product over all queries."""
    qt = np.asarray(queries, dtype=np.float64) @ kcb.rot.T            # row i: Pi q_i
    s = np.asarray(scale, dtype=np.float64)[:, None] * (kcb.centroids[np.asarray(idx)] @ qt.T)
    if sign is not None and kcb.m > 0:
        tq = qt @ kcb.qjl.T                                             # row i: S Pi q_i
        pm = 2.0 * np.asarray(sign, dtype=np.float64) - 1.0
        s = s + (SQRT_HALF_PI / kcb.m) * np.asarray(rnorm, dtype=np.float64)[:, None] * (pm @ tq.T)
    return s


def attn_decode(kcb: Codebook, vcb: Codebook, q, kc: dict, vc: dict, sm_scale: float,
                n_valid=None):
    """q [B, Hq, d]; kc/vc hold unpacked codes with leading dims [B, Hkv, N]:
    kc: idx [B,Hkv,N,d], scale [B,Hkv,N], sign [B,Hkv,N,m] | None, rnorm | None;
    vc: idx, scale.  ``n_valid`` [B] optional per-sequence lengths.
    Returns (logits [B,Hq,N] with -inf beyond n_valid, out [B,Hq,d])."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv, N = kc["idx"].shape[1], kc["idx"].shape[2]
    g = Hq // Hkv
    logits = np.full((B, Hq, N), -np.inf)
    out = np.zeros((B, Hq, d))
    for b in range(B):
        nb = N if n_valid is None else int(n_valid[b])
        for h in range(Hkv):
            if nb == 0:
                continue
            sg = None if kc.get("sign") is None else kc["sign"][b, h, :nb]
            rn = None if kc.get("rnorm") is None else kc["rnorm"][b, h, :nb]
            vhat = dequantize(vcb, vc["idx"][b, h, :nb], vc["scale"][b, h, :nb])
            for j in range(g):
                hq = h * g + j
                lg = sm_scale * code_scores(kcb, q[b, hq], kc["idx"][b, h, :nb],
                                            kc["scale"][b, h, :nb], sg, rn)
                p = np.exp(lg - np.max(lg))
                p /= np.sum(p)
                logits[b, hq, :nb] = lg
                out[b, hq] = p @ vhat
    return logits, out


def exact_attention(q, k, v, sm_scale: float):
    """softmax(tau q K^T) V on unquantized inputs, float64.
    q [B,Hq,d], k/v [B,Hkv,N,d]."""
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv = k.shape[1]
    g = Hq // Hkv
    out = np.zeros((B, Hq, d))
    for b in range(B):
        for hq in range(Hq):
            h = hq // g
            kk = np.asarray(k[b, h], dtype=np.float64)
            lg = sm_scale * (kk @ q[b, hq])
            p = np.exp(lg - lg.max())
            out[b, hq] = (p / p.sum()) @ np.asarray(v[b, h], dtype=np.float64)
    return out


# ---------------------------------------------------------------------------
# R9: inner-product top-k from codes ([WIT] 基准测试与实际性能表现)
# ---------------------------------------------------------------------------


def ip_topk(cb: Codebook, queries, codes: dict, k: int):
    """queries [nq, d]; codes: idx [n,d], scale [n], sign/rnorm or None.
    Returns (idx int64 [nq,k], score [nq,k]) by descending score, ties to the
    lower index."""
    queries = np.asarray(queries, dtype=np.float64)
    nq = queries.shape[0]
    oi = np.zeros((nq, k), dtype=np.int64)
    os_ = np.zeros((nq, k))
    for i in range(nq):
        s = code_scores(cb, queries[i], codes["idx"], codes["scale"],
                        codes.get("sign"), codes.get("rnorm"))
        order = np.argsort(-s, kind="stable")[:k]
        oi[i], os_[i] = order, s[order]
    return oi, os_


def exact_topk(queries, db, k: int):
    """Brute-force exact inner-product top-k on raw vectors (float64)."""
    s = np.asarray(queries, dtype=np.float64) @ np.asarray(db, dtype=np.float64).T
    order = np.argsort(-s, axis=1, kind="stable")[:, :k]
    return order, np.take_along_axis(s, order, axis=1)
