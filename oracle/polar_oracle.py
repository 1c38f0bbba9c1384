"""Float64 CPU oracle of the PolarQuant stage-1 encoding.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the
benchmark's CPU-baseline leg; never by the GPU product path.

Source: page "什么是TurboQuant？谷歌突破性AI压缩技术实现6倍KV缓存缩减和8倍推理加速"
(a2a-mcp.org blog), section "TurboQuant 工作原理" > "第一阶段：随机旋转 +
PolarQuant 压缩", item 2: after the random rotation the vector is
normalised and carried from Cartesian to polar coordinates by pairing
dimensions recursively; the radius holds the magnitude and the angles the
direction; the angles' law is concentrated and known in advance, so no
per-block normalisation constant is stored; a Lloyd-Max quantizer that is
MSE-optimal for that law maps each value to a few bits (the page's example:
3 bits in total for the main stage).  "第二阶段：QJL 残差校正" then sketches what
PolarQuant leaves over, as for the scalar encoding.

Readings where the page is silent (listed in the design notes as R-P1..8):

* R-P1 transform: y = Pi x / |x| as in the scalar path (the same rotation),
  d a power of two.  Level 1 pairs coordinates: (y[2i], y[2i+1]) ->
  radius rho1[i] = hypot and angle phi[i] = atan2(y[2i+1], y[2i]) in
  [-pi, pi].  Level l >= 2 pairs the radii of level l-1:
  (rho[2i], rho[2i+1]) -> radius and angle atan2(rho[2i+1], rho[2i]) in
  [0, pi/2].  After log2(d) levels one radius is left, |y| = 1; the stored
  scale is |x| (the magnitude), so x = 0 gives y = 0 and scale 0.
* R-P2 angle laws for a Haar-rotated (uniform) direction: level-1 angles
  are uniform on [-pi, pi]; at level l >= 2 each radius pools k = 2^(l-1)
  coordinates, so sin^2(psi) ~ Beta(k/2, k/2), i.e. psi has density
  2 sin^(k-1)(psi) cos^(k-1)(psi) / B(k/2, k/2) on [0, pi/2].
* R-P3 codebooks: one Lloyd-Max quantizer per level for that level's law.
  Level 1: the uniform law's quantizer, 2^b1 equal cells of [-pi, pi] with
  centroids at their centres.  Levels >= 2: the unique (log-concave law)
  Lloyd-Max quantizer with 2^br levels, symmetric about pi/4.
* R-P4 bits: b1 bits for each level-1 angle and br bits for each angle of
  every higher level: (d/2) b1 + (d/2 - 1) br bits per vector.  The default
  (b1, br) = (4, 2) gives 3d - 2 bits, the page's "3 bits in total".
* R-P5 index: idx = #{k : angle >= t_k}, a tie goes to the upper cell.
* R-P6 reconstruction: the quantized angles rebuild y_hat top-down from
  radius 1, so |y_hat| = 1 exactly; x_hat = scale Pi^T y_hat.
* R-P7 QJL: as for the scalar path, on r = y - y_hat: sign bits of S r,
  stored rnorm = |x| |r|, estimator scale <Pi q, y_hat> +
  sqrt(pi/2)/m rnorm <S Pi q, 2 sigma - 1>.
* R-P8 packing: one little-endian bit stream per vector, level-major: the
  d/2 level-1 fields of b1 bits (field i at bits [i b1, i b1 + b1)), then
  the d/4 level-2 fields of br bits, and so on up to the single top field;
  zero bits pad the row to 4 ceil(T/32) bytes (T the field bits).
"""
from __future__ import annotations

import math

import numpy as np
from scipy.special import betainc, betaincinv, betaln

from .tq_oracle import SQRT_HALF_PI, coord_index, qjl_matrix, rotation_matrix, symmetric_lloyd_max


def n_levels(d: int) -> int:
    if d < 2 or d & (d - 1):
        raise ValueError("PolarQuant needs d to be a power of two >= 2")
    return d.bit_length() - 1


def level_bits(level: int, b1: int, br: int) -> int:
    return b1 if level == 1 else br


# ---------------------------------------------------------------------------
# R-P2: angle laws
# ---------------------------------------------------------------------------


def angle_density(psi, level: int):
    """Density of a level's angle for a uniform direction (R-P2)."""
    psi = np.asarray(psi, dtype=np.float64)
    if level == 1:
        return np.where(np.abs(psi) <= math.pi, 1.0 / (2.0 * math.pi), 0.0)
    k = 2 ** (level - 1)
    inside = (psi >= 0.0) & (psi <= math.pi / 2)
    s, c = np.sin(psi), np.cos(psi)
    val = 2.0 * np.power(np.abs(s), k - 1) * np.power(np.abs(c), k - 1) * math.exp(-betaln(k / 2, k / 2))
    return np.where(inside, val, 0.0)


def angle_cdf(psi, level: int):
    psi = np.asarray(psi, dtype=np.float64)
    if level == 1:
        return np.clip((psi + math.pi) / (2.0 * math.pi), 0.0, 1.0)
    k = 2 ** (level - 1)
    p = np.clip(psi, 0.0, math.pi / 2)
    return betainc(k / 2, k / 2, np.sin(p) ** 2)


# ---------------------------------------------------------------------------
# R-P3: per-level Lloyd-Max codebooks
# ---------------------------------------------------------------------------

_ANGLE_CACHE: dict = {}


def angle_codebook(level: int, bits: int):
    """(centroids[L], boundaries[L-1]) of one level's angle quantizer."""
    key = (int(level), int(bits))
    if key not in _ANGLE_CACHE:
        _ANGLE_CACHE[key] = _angle_codebook_solve(*key)
    c, t = _ANGLE_CACHE[key]
    return c.copy(), t.copy()


def _angle_codebook_solve(level: int, bits: int):
    if not 1 <= bits <= 8:
        raise ValueError("bits must be in 1..8")
    L = 1 << bits
    if level == 1:
        # the uniform law's Lloyd-Max quantizer: equal cells, centres
        w = 2.0 * math.pi / L
        cent = -math.pi + w * (np.arange(L) + 0.5)
        bnd = -math.pi + w * np.arange(1, L)
        bnd[L // 2 - 1] = 0.0
        return cent, bnd
    k = 2 ** (level - 1)
    log_norm = betaln(k / 2, k / 2)

    def f(p: float) -> float:
        s, c = math.sin(p), math.cos(p)
        if s <= 0.0 or c <= 0.0:
            return math.exp(math.log(2.0) - log_norm) if k == 1 else 0.0
        return math.exp(math.log(2.0) + (k - 1) * (math.log(s) + math.log(c)) - log_norm)

    start = np.arcsin(np.sqrt(betaincinv(k / 2, k / 2, (np.arange(L // 2) + 0.5) / L)))
    return symmetric_lloyd_max(f, 0.0, math.pi / 4, start, what=f"angle level {level}, bits={bits}")


class PolarCodebook:
    """Everything a (d, b1, br, m, seeds) choice fixes, in float64."""

    def __init__(self, d, bits_first=4, bits_rest=2, qjl_m=0, rot_seed=1, qjl_seed=2):
        self.d, self.b1, self.br, self.m = int(d), int(bits_first), int(bits_rest), int(qjl_m)
        self.levels = n_levels(self.d)
        self.rot_seed, self.qjl_seed = int(rot_seed), int(qjl_seed)
        self.books = {lv: angle_codebook(lv, level_bits(lv, self.b1, self.br))
                      for lv in range(1, self.levels + 1)}
        self.rot = rotation_matrix(self.d, self.rot_seed)
        self.qjl = qjl_matrix(self.m, self.d, self.qjl_seed) if self.m > 0 else None

    def field_bits(self) -> int:
        return (self.d // 2) * self.b1 + (self.d // 2 - 1) * self.br


# ---------------------------------------------------------------------------
# R-P1, R-P6: the recursive polar transform and its inverse
# ---------------------------------------------------------------------------


def polar_transform(y):
    """y [n, d] -> (angles, radii): angles[l-1] [n, d/2^l] is level l's
    angle array; radii[l-1] [n, d/2^l] the radii level l produces."""
    y = np.asarray(y, dtype=np.float64)
    d = y.shape[1]
    angles, radii = [], []
    a, b = y[:, 0::2], y[:, 1::2]
    for _ in range(n_levels(d)):
        angles.append(np.arctan2(b, a))
        rho = np.hypot(a, b)
        radii.append(rho)
        a, b = rho[:, 0::2], rho[:, 1::2]
    return angles, radii


def polar_inverse(angles):
    """Angles per level (as from polar_transform) -> unit vectors [n, d]
    rebuilt top-down from radius 1."""
    n = angles[0].shape[0]
    rho = np.ones((n, 1))
    for lv in range(len(angles), 0, -1):
        ang = angles[lv - 1]
        nxt = np.empty((n, 2 * rho.shape[1]))
        nxt[:, 0::2] = rho * np.cos(ang)
        nxt[:, 1::2] = rho * np.sin(ang)
        rho = nxt
    return rho


# ---------------------------------------------------------------------------
# Quantizer
# ---------------------------------------------------------------------------


def quantize(pcb: PolarCodebook, x):
    """Quantize vectors x [n, d].  Returns a dict: idx (list of int16 arrays
    per level), scale [n], sign uint8 [n, m] or None, rnorm [n] or None,
    plus y, y_hat, the exact angles and the radius of the pair each angle
    is taken from (zone accounting), and u = S r."""
    x = np.asarray(x, dtype=np.float64)
    n = np.sqrt(np.sum(x * x, axis=1))
    z = x @ pcb.rot.T
    safe = np.where(n > 0, n, 1.0)
    y = np.where(n[:, None] > 0, z / safe[:, None], 0.0)
    angles, radii = polar_transform(y)
    idx, qang = [], []
    for lv in range(1, pcb.levels + 1):
        c, t = pcb.books[lv]
        ii = coord_index(angles[lv - 1], t)
        idx.append(ii)
        qang.append(c[ii])
    # the pair an angle of level l is taken from has the radius level l makes
    pair_r = list(radii)
    yh = polar_inverse(qang)
    out = dict(idx=idx, scale=n.copy(), sign=None, rnorm=None, y=y, y_hat=yh, angles=angles,
               pair_radius=pair_r, u=None)
    if pcb.m > 0:
        r = y - yh
        rho = np.sqrt(np.sum(r * r, axis=1))
        u = r @ pcb.qjl.T
        out["sign"] = (u >= 0).astype(np.uint8)
        out["rnorm"] = n * rho
        out["u"] = u
    return out


def reconstruct_unit(pcb: PolarCodebook, idx):
    """Unit vectors [n, d] from per-level indices."""
    return polar_inverse([pcb.books[lv][0][np.asarray(idx[lv - 1])] for lv in range(1, pcb.levels + 1)])


def dequantize(pcb: PolarCodebook, idx, scale, sign=None, rnorm=None):
    """x_hat = Pi^T (scale y_hat + rnorm sqrt(pi/2)/m S^T (2 sigma - 1))."""
    yh = reconstruct_unit(pcb, idx) * np.asarray(scale, dtype=np.float64)[:, None]
    if sign is not None and pcb.m > 0:
        pm = 2.0 * np.asarray(sign, dtype=np.float64) - 1.0
        yh = yh + (SQRT_HALF_PI / pcb.m) * np.asarray(rnorm, dtype=np.float64)[:, None] * (pm @ pcb.qjl)
    return yh @ pcb.rot


def code_scores(pcb: PolarCodebook, q, idx, scale, sign=None, rnorm=None):
    """<q, x> estimates of one query q [d] against coded vectors."""
    qt = pcb.rot @ np.asarray(q, dtype=np.float64)
    s = np.asarray(scale, dtype=np.float64) * (reconstruct_unit(pcb, idx) @ qt)
    if sign is not None and pcb.m > 0:
        tq = pcb.qjl @ qt
        pm = 2.0 * np.asarray(sign, dtype=np.float64) - 1.0
        s = s + (SQRT_HALF_PI / pcb.m) * np.asarray(rnorm, dtype=np.float64) * (pm @ tq)
    return s


def boundary_distance(pcb: PolarCodebook, ref):
    """Per level, the distance [n, fields] of each angle's pair point from
    the nearest decision ray of its level (radius times |sin(angle - t)|,
    and for level 1 also the rays at +-pi)."""
    out = []
    for lv in range(1, pcb.levels + 1):
        _, t = pcb.books[lv]
        if lv == 1:
            t = np.concatenate([[-math.pi], t, [math.pi]])
        ang = ref["angles"][lv - 1]
        dmin = np.min(np.abs(np.sin(ang[..., None] - t)), axis=-1)
        out.append(ref["pair_radius"][lv - 1] * dmin)
    return out


# ---------------------------------------------------------------------------
# R-P8: packing
# ---------------------------------------------------------------------------


def row_bytes(d: int, b1: int, br: int) -> int:
    bits = (d // 2) * b1 + (d // 2 - 1) * br
    return 4 * ((bits + 31) // 32)


def pack_rows(idx, d: int, b1: int, br: int, rb: int | None = None) -> np.ndarray:
    """Per-level indices -> uint8 [n, rb] level-major LSB-first bit streams."""
    n = np.asarray(idx[0]).shape[0]
    rb = row_bytes(d, b1, br) if rb is None else rb
    bitarr = np.zeros((n, rb * 8), dtype=np.uint8)
    pos = 0
    for lv in range(1, n_levels(d) + 1):
        b = level_bits(lv, b1, br)
        v = np.asarray(idx[lv - 1], dtype=np.int64)
        nf = v.shape[1]
        for bb in range(b):
            bitarr[:, pos + np.arange(nf) * b + bb] = (v >> bb) & 1
        pos += nf * b
    return np.packbits(bitarr, axis=1, bitorder="little")


def unpack_rows(rows, d: int, b1: int, br: int):
    rows = np.asarray(rows, dtype=np.uint8)
    bitarr = np.unpackbits(rows, axis=1, bitorder="little").astype(np.int64)
    out, pos = [], 0
    for lv in range(1, n_levels(d) + 1):
        b = level_bits(lv, b1, br)
        nf = d >> lv
        v = np.zeros((rows.shape[0], nf), dtype=np.int64)
        for bb in range(b):
            v |= bitarr[:, pos + np.arange(nf) * b + bb] << bb
        out.append(v)
        pos += nf * b
    return out


# ---------------------------------------------------------------------------
# Decode with polar-coded keys ([WIT] 如何实现 item 1: rotate the query once,
# take the attention products from the stored codes)
# ---------------------------------------------------------------------------


def attn_decode(kpcb: PolarCodebook, vcb, q, kc: dict, vc: dict, sm_scale: float, n_valid=None):
    """q [B, Hq, d]; kc: idx (list per level of [B, Hkv, N, fields]), scale
    [B, Hkv, N], sign/rnorm or None; vc: scalar value codes (idx [B,Hkv,N,d],
    scale) of the scalar path's codebook vcb.  Returns (logits with -inf
    beyond n_valid, out [B, Hq, d])."""
    from .tq_oracle import dequantize as scalar_dequantize
    q = np.asarray(q, dtype=np.float64)
    B, Hq, d = q.shape
    Hkv, N = kc["scale"].shape[1], kc["scale"].shape[2]
    g = Hq // Hkv
    logits = np.full((B, Hq, N), -np.inf)
    out = np.zeros((B, Hq, d))
    for b in range(B):
        nb = N if n_valid is None else int(n_valid[b])
        for h in range(Hkv):
            if nb == 0:
                continue
            kidx = [a[b, h, :nb] for a in kc["idx"]]
            sg = None if kc.get("sign") is None else kc["sign"][b, h, :nb]
            rn = None if kc.get("rnorm") is None else kc["rnorm"][b, h, :nb]
            vhat = scalar_dequantize(vcb, vc["idx"][b, h, :nb], vc["scale"][b, h, :nb])
            for j in range(g):
                hq = h * g + j
                lg = sm_scale * code_scores(kpcb, q[b, hq], kidx, kc["scale"][b, h, :nb], sg, rn)
                p = np.exp(lg - np.max(lg))
                p /= np.sum(p)
                logits[b, hq, :nb] = lg
                out[b, hq] = p @ vhat
    return logits, out
