"""GPU parity of the paged-pool calls (tq_quantize_kv_paged,
tq_attn_decode_paged).

* Decode: the oracle's codes are laid out in a pool through a shuffled
  block table (byte copies only) and the paged decode is compared with the
  oracle's decode of the same codes (decode bars: logits within 1e-4 of the
  row's max |logit|, outputs within 2e-3 max-abs), and with the contiguous
  decode of the same codes (the two differ only in the order of the split-K
  partial sums).
* Quantize: the same inputs quantized into a pool and into contiguous codes
  give byte-identical planes once the pool's pages are gathered back in
  logical order (bulk prefill and single-token appends, both layouts).
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


def _planes(c: "tq.Codes"):
    """Per-position views of a Codes' planes: dict name -> tensor [n_seq, S, bytes]
    (tile32 idx: [n_seq, S / 32, block bytes])."""
    n, S = c.n_seq, c.seq_stride
    out = {}
    if c.layout == TQ_LAYOUT_ROW:
        out["idx"] = c.idx[:n * S * c.idx_row_bytes].view(n, S, c.idx_row_bytes)
    else:
        blk = c.idx.numel() // (n * (S // 32))
        out["idx32"] = c.idx.view(n, S // 32, blk)
    out["scale"] = c.scale[:n * S].view(n, S, 1)
    if c.sign is not None:
        out["sign"] = c.sign[:n * S * c.sign_row_bytes].view(n, S, c.sign_row_bytes)
        out["rnorm"] = c.rnorm[:n * S].view(n, S, 1)
    return out


def _move_pages(src: "tq.Codes", dst: "tq.Codes", table, Hkv, pt, n_lp, to_pool: bool):
    """Copy logical page i of sequence (b, h) of contiguous codes to pool page
    table[b, i] of plane h (to_pool) or back (byte copies only)."""
    cont, pool = (src, dst) if to_pool else (dst, src)
    cp, pp = _planes(cont), _planes(pool)
    B = table.shape[0]
    for b in range(B):
        for h in range(Hkv):
            s = b * Hkv + h
            for i in range(n_lp):
                p = int(table[b, i])
                for name in cp:
                    u = pt // 32 if name == "idx32" else pt
                    c_sl = cp[name][s, i * u:(i + 1) * u]
                    p_sl = pp[name][h, p * u:(p + 1) * u]
                    if to_pool:
                        p_sl.copy_(c_sl)
                    else:
                        c_sl.copy_(p_sl)


def _table(B, n_lp, n_pages, seed):
    perm = np.random.default_rng(seed).permutation(n_pages)[:B * n_lp]
    return perm.reshape(B, n_lp).astype(np.int32)


@pytest.mark.parametrize("pt,N,lens,d,kb,km,vb", [
    (64, 300, None, 128, 3, 128, 4), (32, 200, [200, 77], 128, 3, 128, 4), (128, 513, [1, 513], 128, 3, 128, 4),
    # head dimensions of the any-shape kernels (decode_gen.hip)
    (32, 200, [200, 77], 96, 4, 64, 3), (64, 300, None, 200, 2, 200, 4)])
def test_paged_decode_matches_oracle(dev, pt, N, lens, d, kb, km, vb):
    _say("paged decode", pt, N, lens, d, kb, km, vb)
    B, Hq, Hkv = 2, 16, 2
    tau = 1.0 / np.sqrt(d)
    kcb = tq.Codebook(d, kb, qjl_m=km, rot_seed=1, qjl_seed=2)
    vcb = tq.Codebook(d, vb, rot_seed=3)
    okc, ovc = U.oracle_codebook(kcb), U.oracle_codebook(vcb)
    ch = [c for c in (3, 77, 101) if c < d]
    k = U.to_f64(synth.kv_gaussian(B, Hkv, N, d, 41, dtype="f32", device="cpu", channels=ch, factor=20.0))
    v = U.to_f64(synth.kv_gaussian(B, Hkv, N, d, 42, dtype="f32", device="cpu", channels=ch, factor=20.0))
    q = np.random.default_rng(43).standard_normal((B, Hq, d))
    n_lp = (N + pt - 1) // pt
    n_pages = B * n_lp + 3
    S = n_lp * pt
    kc = tq.Codes(kcb, B * Hkv, S, TQ_LAYOUT_ROW, device=dev)
    vc = tq.Codes(vcb, B * Hkv, S, TQ_LAYOUT_TILE32, device=dev)
    kr = [O.quantize(okc, k.reshape(B * Hkv, N, d)[s]) for s in range(B * Hkv)]
    vr = [O.quantize(ovc, v.reshape(B * Hkv, N, d)[s]) for s in range(B * Hkv)]
    for s in range(B * Hkv):
        U.upload_oracle_codes(kc, s, kr[s], N)
        U.upload_oracle_codes(vc, s, vr[s], N)
    table = _table(B, n_lp, n_pages, pt + N)
    kp = tq.Codes(kcb, Hkv, n_pages * pt, TQ_LAYOUT_ROW, device=dev)
    vp = tq.Codes(vcb, Hkv, n_pages * pt, TQ_LAYOUT_TILE32, device=dev)
    _move_pages(kc, kp, table, Hkv, pt, n_lp, True)
    _move_pages(vc, vp, table, Hkv, pt, n_lp, True)
    qt = torch.from_numpy(q).float().to(dev)
    bt = torch.from_numpy(table).to(dev)
    sl = torch.tensor(lens, dtype=torch.int32, device=dev) if lens else None
    lg_p = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    lg_c = torch.empty_like(lg_p)
    out_p = tq.tq_attn_decode_paged(kcb, vcb, qt, kp, vp, bt, pt, N, tau, seq_lens=sl, logits=lg_p)
    out_c = tq.tq_attn_decode(kcb, vcb, qt, kc, vc, N, tau, seq_lens=sl, logits=lg_c)
    torch.cuda.synchronize()
    f32 = lambda a: a.astype(np.float32).astype(np.float64)
    stack = lambda rs, key: np.stack([r[key] for r in rs]).reshape(B, Hkv, N, *rs[0][key].shape[1:])
    okcodes = dict(idx=stack(kr, "idx"), scale=f32(stack(kr, "scale")))
    if km:
        okcodes.update(sign=stack(kr, "sign"), rnorm=f32(stack(kr, "rnorm")))
    ovcodes = dict(idx=stack(vr, "idx"), scale=f32(stack(vr, "scale")))
    ref_lg, ref_out = O.attn_decode(okc, ovc, q, okcodes, ovcodes, tau, n_valid=lens)
    op, oc = out_p.cpu().numpy().astype(np.float64), out_c.cpu().numpy().astype(np.float64)
    lp, lc = lg_p.cpu().numpy().astype(np.float64), lg_c.cpu().numpy().astype(np.float64)
    assert np.max(np.abs(op - ref_out)) <= 2e-3
    assert np.max(np.abs(op - oc)) <= 1e-4 * max(1.0, np.max(np.abs(oc)))
    for b in range(B):
        nb = N if lens is None else lens[b]
        for hq in range(Hq):
            r = ref_lg[b, hq, :nb]
            assert np.max(np.abs(lp[b, hq, :nb] - r)) <= 1e-4 * np.max(np.abs(r))
            # same tiles and arithmetic; only the chunk's reference maximum
            # (added back to the stored logit) may differ
            assert np.max(np.abs(lp[b, hq, :nb] - lc[b, hq, :nb])) <= 1e-6 * np.max(np.abs(r))
            assert np.all(np.isneginf(lp[b, hq, nb:]))


@pytest.mark.parametrize("bits,m,layout,pt", [(3, 128, TQ_LAYOUT_ROW, 64), (4, 0, TQ_LAYOUT_ROW, 32),
                                              (4, 0, TQ_LAYOUT_TILE32, 64), (3, 0, TQ_LAYOUT_TILE32, 32),
                                              (2, 64, TQ_LAYOUT_ROW, 128)])
def test_paged_quantize_equals_contiguous(dev, bits, m, layout, pt):
    _say("paged quantize", bits, m, layout, pt)
    B, Hkv, d, N0, n_app = 2, 3, 128, 150, 3
    N = N0 + n_app
    cb = tq.Codebook(d, bits, qjl_m=m, rot_seed=5, qjl_seed=6)
    x = synth.kv_gaussian(B, Hkv, N, d, 51, dtype="bf16", device=dev, channels=[3, 77, 101],
                          factor=20.0).view(B * Hkv, N, d)
    n_lp = (N + pt - 1) // pt
    n_pages = B * n_lp + 5
    table = _table(B, n_lp, n_pages, 7 * pt + bits)
    bt = torch.from_numpy(table).to(dev)
    cont = tq.Codes(cb, B * Hkv, n_lp * pt, layout, device=dev)
    pool = tq.Codes(cb, Hkv, n_pages * pt, layout, device=dev)
    # prefill N0 positions (bulk kernels), then single-token appends
    tq.tq_quantize_kv(cb, None, x[:, :N0].contiguous(), None, cont, None)
    tq.tq_quantize_kv_paged(cb, None, x[:, :N0].contiguous(), None, pool, None, bt, pt)
    for t in range(N0, N):
        xt = x[:, t:t + 1].contiguous()
        tq.tq_quantize_kv(cb, None, xt, None, cont, None, tok_offset=t)
        tq.tq_quantize_kv_paged(cb, None, xt, None, pool, None, bt, pt, tok_offset=t)
    back = tq.Codes(cb, B * Hkv, n_lp * pt, layout, device=dev)
    _move_pages(pool, back, table, Hkv, pt, n_lp, False)
    torch.cuda.synchronize()
    for name, a in _planes(cont).items():
        assert torch.equal(a, _planes(back)[name]), name


def test_paged_argument_errors(dev):
    _say("paged argument errors")
    cb = tq.Codebook(128, 4)
    kcb = tq.Codebook(128, 3, qjl_m=128)
    pool = tq.Codes(cb, 2, 4 * 64, TQ_LAYOUT_TILE32, device=dev)
    kpool = tq.Codes(kcb, 2, 4 * 64, TQ_LAYOUT_ROW, device=dev)
    bt = torch.zeros((1, 2), dtype=torch.int32, device=dev)
    x = torch.zeros((2, 100, 128), dtype=torch.bfloat16, device=dev)
    with pytest.raises(tq.TQError):      # page size not a power of two
        tq.tq_quantize_kv_paged(cb, None, x, None, pool, None, bt, 48)
    with pytest.raises(tq.TQError):      # 2 pages of 32 do not cover 100 positions
        tq.tq_quantize_kv_paged(cb, None, x, None, pool, None, bt, 32)
    with pytest.raises(tq.TQError):      # pool stride 256 is not a multiple of 512
        tq.tq_quantize_kv_paged(cb, None, x, None, pool, None, bt, 512)
    q = torch.zeros((1, 8, 128), dtype=torch.float32, device=dev)
    with pytest.raises(tq.TQError):      # n_ctx beyond max_pages * page_tokens
        tq.tq_attn_decode_paged(kcb, cb, q, kpool, pool, bt, 64, 200, 0.1)
    with pytest.raises(ValueError):      # table dtype
        tq.tq_attn_decode_paged(kcb, cb, q, kpool, pool, bt.long(), 64, 100, 0.1)
