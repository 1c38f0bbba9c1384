"""Shared helpers of the GPU parity tests: read GPU codes back to the host
(with the oracle's format readers) and compare them with the oracle under
the stated tolerances.

Tolerances (floating point decides an integer here, and the GPU rotates in
fp32 while the oracle works in fp64):
* indices: bit-exact, except where the oracle's rotated coordinate lies
  within 1e-5 of a decision boundary; such mismatches are counted and must
  stay <= 1e-4 of the elements;
* QJL sign bits: bit-exact except where |(S r)_j| < 1e-5 or the vector had
  an index mismatch;
* scale within 2e-6 relative, rnorm within 1e-5 relative (vectors without
  index mismatches);
* logits: per (query, head) row, max |l_gpu - l_ref| <= 1e-4 * max |l_ref|,
  with l_ref computed by the oracle from the GPU's own codes;
* outputs: max-abs <= 2e-3 against the oracle on the same codes.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle as O
from kv_cache_vector_quantize_amd import TQ_LAYOUT_ROW

ZONE = 1e-5
IDX_BUDGET = 1e-4
LOGIT_RTOL = 1e-4
OUT_ATOL = 2e-3


def oracle_codebook(cb):
    return O.Codebook(cb.d, cb.bits, qjl_m=cb.m, nc=cb.nc, rot_seed=cb.rot_seed,
                      qjl_seed=cb.qjl_seed)


def read_codes(codes, n_tok: int, seqs=None):
    """GPU codes -> dict of host arrays with leading dims [n_seq_sel, n_tok]."""
    cb = codes.cb
    seqs = list(range(codes.n_seq)) if seqs is None else list(seqs)
    S = codes.seq_stride
    out = {}
    idx_b = codes.idx.cpu().numpy()
    sc = codes.scale.cpu().numpy()
    idx_l, sc_l, sg_l, rn_l = [], [], [], []
    for s in seqs:
        if codes.layout == TQ_LAYOUT_ROW:
            rows = idx_b[s * S * codes.idx_row_bytes:(s * S + n_tok) * codes.idx_row_bytes]
            rows = rows.reshape(n_tok, codes.idx_row_bytes)
            idx_l.append(O.unpack_rows(rows, cb.d, cb.bits))
        else:
            nb = S // 32
            blk_bytes = cb.d * cb.bits * 4
            raw = idx_b[s * nb * blk_bytes:(s + 1) * nb * blk_bytes].reshape(nb, cb.d, cb.bits * 4)
            idx_l.append(O.unpack_tile32(raw, cb.d, cb.bits, n_tok))
        sc_l.append(sc[s * S:s * S + n_tok])
        if cb.m > 0:
            sg = codes.sign.cpu().numpy()
            rows = sg[s * S * codes.sign_row_bytes:(s * S + n_tok) * codes.sign_row_bytes]
            sg_l.append(O.unpack_signs(rows.reshape(n_tok, codes.sign_row_bytes), cb.m))
            rn_l.append(codes.rnorm.cpu().numpy()[s * S:s * S + n_tok])
    out["idx"] = np.stack(idx_l)
    out["scale"] = np.stack(sc_l).astype(np.float64)
    out["sign"] = np.stack(sg_l) if sg_l else None
    out["rnorm"] = np.stack(rn_l).astype(np.float64) if rn_l else None
    return out


def raw_rows(codes, s, n_tok):
    """Packed ROW-layout bytes of sequence s: [n_tok, idx_row_bytes]."""
    S = codes.seq_stride
    b = codes.idx.cpu().numpy()
    return b[s * S * codes.idx_row_bytes:(s * S + n_tok) * codes.idx_row_bytes].reshape(
        n_tok, codes.idx_row_bytes)


def boundary_distance(t: np.ndarray, y: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Distance of y to the nearest boundary; idx = #{k : y >= t_k}, so the
    neighbours are t[idx-1] (below) and t[idx] (above)."""
    tt = np.concatenate([[-np.inf], t, [np.inf]])
    i = idx.astype(np.int64)
    return np.minimum(np.abs(y - tt[i]), np.abs(tt[i + 1] - y))


def compare_quant(ocb, x64: np.ndarray, got: dict, name=""):
    """x64 [n, d] exact inputs; got: codes of the same n vectors (flattened).
    Returns a stats dict; asserts the tolerances."""
    ref = O.quantize(ocb, x64)
    gidx = got["idx"].reshape(ref["idx"].shape)
    mism = gidx != ref["idx"]
    # distance of each rotated coordinate to its nearest boundary
    in_zone = boundary_distance(ocb.boundaries, ref["y"], ref["idx"]) < ZONE
    bad = mism & ~in_zone
    assert not bad.any(), f"{name}: {bad.sum()} index mismatches outside the boundary zone"
    n_el = mism.size
    assert mism.sum() <= max(1, IDX_BUDGET * n_el), f"{name}: {mism.sum()} zone mismatches"
    vec_ok = ~mism.any(axis=1)
    gsc = got["scale"].reshape(-1)
    rel = np.abs(gsc - ref["scale"]) / np.maximum(np.abs(ref["scale"]), 1e-30)
    assert np.all(rel[vec_ok] <= 2e-6), f"{name}: scale rel err {rel[vec_ok].max()}"
    stats = dict(n=len(x64), idx_mismatch=int(mism.sum()), zone=int(in_zone.sum()),
                 scale_rel=float(rel[vec_ok].max() if vec_ok.any() else 0.0))
    if ocb.m > 0:
        gs = got["sign"].reshape(ref["sign"].shape)
        smis = (gs != ref["sign"]) & vec_ok[:, None] & (np.abs(ref["u"]) >= ZONE)
        assert not smis.any(), f"{name}: {smis.sum()} sign mismatches"
        grn = got["rnorm"].reshape(-1)
        rr = np.abs(grn - ref["rnorm"]) / np.maximum(np.abs(ref["rnorm"]), 1e-30)
        assert np.all(rr[vec_ok] <= 1e-5), f"{name}: rnorm rel err {rr[vec_ok].max()}"
        stats["sign_mismatch_total"] = int((gs != ref["sign"]).sum())
        stats["rnorm_rel"] = float(rr[vec_ok].max() if vec_ok.any() else 0.0)
    return stats


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_decode(ocb_k, ocb_v, q64, kc, vc, sm_scale, logits_gpu, out_gpu, n_valid=None,
                 name=""):
    """Oracle decode on the GPU's own codes; asserts logit and output bars."""
    lg_ref, out_ref = O.attn_decode(ocb_k, ocb_v, q64, kc, vc, sm_scale, n_valid=n_valid)
    worst_l, worst_o = 0.0, 0.0
    B, Hq, N = lg_ref.shape
    for b in range(B):
        nb = N if n_valid is None else int(n_valid[b])
        for h in range(Hq):
            if logits_gpu is not None:
                gl = logits_gpu[b, h]
                if nb < N:
                    assert np.all(np.isneginf(gl[nb:])), f"{name}: logits beyond length not -inf"
                if nb > 0:
                    err = np.max(np.abs(gl[:nb] - lg_ref[b, h, :nb]))
                    scale = np.max(np.abs(lg_ref[b, h, :nb]))
                    worst_l = max(worst_l, err / scale)
                    assert err <= LOGIT_RTOL * scale, f"{name}: logit row ({b},{h}) err {err} vs {scale}"
    worst_o = float(np.max(np.abs(out_gpu - out_ref))) if out_ref.size else 0.0
    assert worst_o <= OUT_ATOL, f"{name}: output max-abs err {worst_o}"
    return dict(logit_rel=worst_l, out_abs=worst_o)
