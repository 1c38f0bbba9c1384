"""Shared helpers of the GPU parity tests.

Direction of data: every expected value comes from the oracle run on the
seeded inputs (``synth``).  GPU outputs are only read back and compared.  For
decode parity the oracle's own packed codes are uploaded and the GPU decodes
them, so both sides start from identical codes.

Tolerances (floating point decides an integer here, and the GPU rotates in
fp32 while the oracle works in fp64):
* indices: bit-exact, except where the oracle's rotated coordinate lies
  within 1e-5 of a decision boundary; such mismatches are counted and must
  stay <= 1e-4 of the elements;
* QJL sign bits: bit-exact except where |(S r)_j| < 1e-5 or the vector had
  an index mismatch;
* scale within 2e-6 relative, rnorm within 1e-5 relative or 1e-6 |x|,
  whichever is larger (vectors without index mismatches);
* logits: per (query, head) row, max |l_gpu - l_ref| <= 1e-4 * max |l_ref|;
* outputs: max-abs <= 2e-3.
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
RNORM_XFLOOR = 1e-6


def oracle_codebook(cb):
    return O.Codebook(cb.d, cb.bits, qjl_m=cb.m, nc=cb.nc, rot_seed=cb.rot_seed,
                      qjl_seed=cb.qjl_seed)


# ------------------------------------------------------------- test-side readers
# (plain bit arithmetic, independent of the oracle's packers)


def _bits_le(b: np.ndarray) -> np.ndarray:
    """uint8 [..., nbytes] -> uint8 bits [..., nbytes*8], bit p = byte p>>3, pos p&7."""
    shifts = np.arange(8, dtype=np.uint8)
    return ((b[..., :, None] >> shifts) & 1).reshape(*b.shape[:-1], b.shape[-1] * 8)


def read_rows(raw: np.ndarray, d: int, bits: int) -> np.ndarray:
    bt = _bits_le(raw).astype(np.int64)
    pos = np.arange(d)[:, None] * bits + np.arange(bits)[None, :]
    return (bt[:, pos] << np.arange(bits)[None, None, :]).sum(-1)


def read_tile32(raw: np.ndarray, d: int, bits: int, n_tok: int) -> np.ndarray:
    """raw [n_blocks, block_bytes] -> idx [n_tok, d].  Record r = 16 G + C of
    a block holds coordinates 16 j + C (one b-byte group per j) for the tokens
    4G + e%4 + 16 (e//4) of slots e = 0..7."""
    ndb = (d + 15) // 16
    nb = raw.shape[0]
    bt = _bits_le(raw).astype(np.int64).reshape(nb, 64, ndb, 8, bits)   # [blk, r, j, e, bit]
    v = (bt << np.arange(bits)).sum(-1)                                  # [blk, r, j, e]
    out = np.zeros((nb, 32, ndb * 16), dtype=np.int64)
    for G in range(4):
        for e in range(8):
            t = 4 * G + e % 4 + 16 * (e // 4)
            rec = v[:, 16 * G:16 * G + 16, :, e]                         # [blk, C, j]
            out[:, t, :] = rec.transpose(0, 2, 1).reshape(nb, ndb * 16)   # coordinate 16 j + C
    return out.reshape(nb * 32, ndb * 16)[:n_tok, :d]


def seq_bytes(codes, s: int, n_tok: int):
    """Raw code bytes of sequence s: (idx bytes, sign bytes or None)."""
    S = codes.seq_stride
    b = codes.idx.cpu().numpy()
    if codes.layout == TQ_LAYOUT_ROW:
        ib = b[s * S * codes.idx_row_bytes:(s * S + n_tok) * codes.idx_row_bytes].reshape(
            n_tok, codes.idx_row_bytes)
    else:
        nb = S // 32
        blk = O.tile32_block_bytes(codes.cb.d, codes.cb.bits)
        ib = b[s * nb * blk:(s + 1) * nb * blk].reshape(nb, blk)
    sb = None
    if codes.sign is not None:
        sg = codes.sign.cpu().numpy()
        sb = sg[s * S * codes.sign_row_bytes:(s * S + n_tok) * codes.sign_row_bytes].reshape(
            n_tok, codes.sign_row_bytes)
    return ib, sb


def read_codes(codes, n_tok: int, seqs=None):
    """GPU codes -> dict(idx [ns, n_tok, d], scale, sign [ns, n_tok, m], rnorm)."""
    cb = codes.cb
    seqs = list(range(codes.n_seq)) if seqs is None else list(seqs)
    S = codes.seq_stride
    sc = codes.scale.cpu().numpy()
    rn = codes.rnorm.cpu().numpy() if codes.rnorm is not None else None
    idx_l, sc_l, sg_l, rn_l = [], [], [], []
    for s in seqs:
        ib, sb = seq_bytes(codes, s, n_tok)
        if codes.layout == TQ_LAYOUT_ROW:
            idx_l.append(read_rows(ib, cb.d, cb.bits))
        else:
            idx_l.append(read_tile32(ib, cb.d, cb.bits, n_tok))
        sc_l.append(sc[s * S:s * S + n_tok])
        if sb is not None:
            sg_l.append(_bits_le(sb)[:, :cb.m])
            rn_l.append(rn[s * S:s * S + n_tok])
    return dict(idx=np.stack(idx_l), scale=np.stack(sc_l).astype(np.float64),
                sign=np.stack(sg_l) if sg_l else None,
                rnorm=np.stack(rn_l).astype(np.float64) if rn_l else None)


# ------------------------------------------------------------- comparisons


def boundary_distance(t: np.ndarray, y: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Distance of y to the nearest boundary; idx = #{k : y >= t_k}, so the
    neighbours are t[idx-1] (below) and t[idx] (above)."""
    tt = np.concatenate([[-np.inf], t, [np.inf]])
    i = idx.astype(np.int64)
    return np.minimum(np.abs(y - tt[i]), np.abs(tt[i + 1] - y))


def compare_quant(ocb, x64: np.ndarray, got: dict, name="", ref=None):
    """x64 [n, d] exact inputs; got: GPU codes of the same n vectors
    (flattened).  Asserts the tolerances; returns (stats, oracle result)."""
    if ref is None:
        ref = O.quantize(ocb, x64)
    gidx = got["idx"].reshape(ref["idx"].shape)
    mism = gidx != ref["idx"]
    in_zone = boundary_distance(ocb.boundaries, ref["y"], ref["idx"]) < ZONE
    bad = mism & ~in_zone
    assert not bad.any(), f"{name}: {bad.sum()} index mismatches outside the boundary zone"
    assert mism.sum() <= max(1, IDX_BUDGET * mism.size), f"{name}: {mism.sum()} zone mismatches"
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
        nx = np.sqrt(np.sum(x64 * x64, axis=1))
        # 1e-5 relative, with a floor of 1e-6 |x|: an fp32 rotation leaves y
        # ~3e-7 (in norm) from the fp64 one, which moves |r| by as much; for
        # codes of >= 6 bits |r| < 0.03 and the relative bar alone is unmeetable
        rerr = np.abs(grn - ref["rnorm"])
        rr = rerr / np.maximum(np.abs(ref["rnorm"]), 1e-30)
        okr = rerr <= np.maximum(1e-5 * np.abs(ref["rnorm"]), RNORM_XFLOOR * nx)
        assert np.all(okr[vec_ok]), f"{name}: rnorm err {rerr[vec_ok & ~okr].max()}"
        stats["sign_mismatch_total"] = int((gs != ref["sign"]).sum())
        stats["rnorm_rel"] = float(rr[vec_ok].max() if vec_ok.any() else 0.0)
    stats["vec_ok"] = vec_ok
    return stats, ref


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


# ------------------------------------------------------------- oracle codes -> GPU


def upload_oracle_codes(codes, s: int, ref: dict, n_tok: int):
    """Write the oracle's quantization of sequence s (packed by the oracle's
    packers) into the GPU code buffers."""
    cb = codes.cb
    S = codes.seq_stride
    if codes.layout == TQ_LAYOUT_ROW:
        rows = O.pack_rows(ref["idx"], cb.bits, codes.idx_row_bytes)
        a = s * S * codes.idx_row_bytes
        codes.idx[a:a + rows.size] = torch.from_numpy(rows.reshape(-1)).to(codes.idx.device)
    else:
        nb = S // 32
        blk = O.tile32_block_bytes(cb.d, cb.bits)
        blocks = O.pack_tile32(ref["idx"], cb.bits, nb)
        a = s * nb * blk
        codes.idx[a:a + blocks.size] = torch.from_numpy(blocks.reshape(-1)).to(codes.idx.device)
    codes.scale[s * S:s * S + n_tok] = torch.from_numpy(ref["scale"].astype(np.float32)).to(codes.scale.device)
    if cb.m > 0:
        sg = O.pack_signs(ref["sign"], codes.sign_row_bytes)
        a = s * S * codes.sign_row_bytes
        codes.sign[a:a + sg.size] = torch.from_numpy(sg.reshape(-1)).to(codes.sign.device)
        codes.rnorm[s * S:s * S + n_tok] = torch.from_numpy(ref["rnorm"].astype(np.float32)).to(codes.rnorm.device)


def oracle_cache(refs, B, Hkv, N, with_sign):
    """Stack per-sequence oracle quantizations into decode-oracle inputs, with
    the stored scalars rounded to fp32 exactly as uploaded."""
    d = dict(idx=np.stack([r["idx"] for r in refs]).reshape(B, Hkv, N, -1),
             scale=np.stack([r["scale"].astype(np.float32) for r in refs]).astype(np.float64).reshape(B, Hkv, N))
    if with_sign:
        d["sign"] = np.stack([r["sign"] for r in refs]).reshape(B, Hkv, N, -1)
        d["rnorm"] = np.stack([r["rnorm"].astype(np.float32) for r in refs]).astype(np.float64).reshape(B, Hkv, N)
    return d


def check_decode(ocb_k, ocb_v, q64, kc, vc, sm_scale, logits_gpu, out_gpu, n_valid=None,
                 name="", rows=None):
    """Oracle decode of the same codes; asserts the logit and output bars.
    ``rows``: optional list of (b, hq) to check (default: all)."""
    lg_ref, out_ref = O.attn_decode(ocb_k, ocb_v, q64, kc, vc, sm_scale, n_valid=n_valid)
    worst_l = 0.0
    B, Hq, N = lg_ref.shape
    sel = rows if rows is not None else [(b, h) for b in range(B) for h in range(Hq)]
    for b, h in sel:
        nb = N if n_valid is None else int(n_valid[b])
        if logits_gpu is not None:
            gl = logits_gpu[b, h]
            if nb < N:
                assert np.all(np.isneginf(gl[nb:])), f"{name}: logits beyond length not -inf"
            if nb > 0:
                err = np.max(np.abs(gl[:nb] - lg_ref[b, h, :nb]))
                scale = np.max(np.abs(lg_ref[b, h, :nb]))
                worst_l = max(worst_l, err / scale)
                assert err <= LOGIT_RTOL * scale, f"{name}: logit row ({b},{h}) err {err} vs {scale}"
    diffs = [np.max(np.abs(out_gpu[b, h] - out_ref[b, h])) for b, h in sel]
    worst_o = float(max(diffs)) if diffs else 0.0
    assert worst_o <= OUT_ATOL, f"{name}: output max-abs err {worst_o}"
    return dict(logit_rel=worst_l, out_abs=worst_o)


def check_end_to_end(ocb_k, ocb_v, q64, k_codes, v_codes, n_tok, B, Hkv, sm_scale, lg_gpu, out_gpu,
                     out_ref, code_stats):
    """GPU quantize -> GPU decode.  The zone rule lets a GPU code differ from
    the oracle's where the oracle's y lies within 1e-5 of a boundary (or u of
    0), and such a token's logit moves with its code, by more than the decode
    bars allow.  So: with no differing code the chain must meet the output bar
    against the oracle's quantize -> decode (``out_ref``); in every case the
    GPU decode must equal the oracle's decode of the GPU's own codes (read
    back) to the decode bars.  ``code_stats``: compare_quant stats of the K
    and V codes."""
    gk, gv = read_codes(k_codes, n_tok), read_codes(v_codes, n_tok)
    shape = lambda a: a.reshape(B, Hkv, n_tok, *a.shape[2:])
    kd = dict(idx=shape(gk["idx"]), scale=shape(gk["scale"]))
    if gk["sign"] is not None:
        kd.update(sign=shape(gk["sign"]), rnorm=shape(gk["rnorm"]))
    vd = dict(idx=shape(gv["idx"]), scale=shape(gv["scale"]))
    st = check_decode(ocb_k, ocb_v, q64, kd, vd, sm_scale, lg_gpu, out_gpu, name="end-to-end codes")
    differ = sum(int(c["idx_mismatch"]) + int(c.get("sign_mismatch_total", 0)) for c in code_stats)
    e2e = float(np.max(np.abs(out_gpu - out_ref)))
    if differ == 0:
        assert e2e <= OUT_ATOL, f"end-to-end output max-abs {e2e} with identical codes"
    return dict(st, e2e_out=e2e, differing_codes=differ)
