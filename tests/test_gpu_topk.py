"""GPU parity of tq_ip_topk (inner-product top-k from codes) against the oracle.

Both sides score the same codes: the oracle quantizes the seeded database and
its packed codes are uploaded, so the GPU never produces an oracle input.

Several answers are correct when scores tie or nearly tie (the GPU forms the
scores with bf16 hi/lo splits, about 2^-16 relative), so the checks are:
* indices are distinct and in range, scores are non-increasing, and equal
  scores come in ascending index order;
* each returned score equals the oracle's score of that index within
  SCORE_RTOL x max |oracle score| of the query;
* each returned index has an oracle score >= the oracle's k-th score - 2 tol,
  and every index whose oracle score exceeds the k-th score + 2 tol is returned.
"""
import numpy as np
import pytest
import torch

import oracle as O
import synth
import kv_cache_vector_quantize_amd as tq
from kv_cache_vector_quantize_amd import TQ_LAYOUT_ROW

import tq_testutil as U

pytestmark = pytest.mark.gpu

SCORE_RTOL = 1e-4


def _say(*a):
    print("[case]", *a, flush=True)


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    tq.lib()
    return "cuda"


def _db_codes(cb, ocb, db64, dev, chunk=250000):
    """Oracle codes of db64 [n, d] uploaded into GPU row-layout codes."""
    n = db64.shape[0]
    codes = tq.Codes(cb, 1, n, TQ_LAYOUT_ROW)
    parts = []
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        r = O.quantize(ocb, db64[s:e])
        rows = O.pack_rows(r["idx"], cb.bits, codes.idx_row_bytes)
        codes.idx[s * codes.idx_row_bytes:e * codes.idx_row_bytes] = torch.from_numpy(rows.reshape(-1)).to(dev)
        codes.scale[s:e] = torch.from_numpy(r["scale"].astype(np.float32)).to(dev)
        part = dict(idx=r["idx"].astype(np.int16), scale=r["scale"].astype(np.float32).astype(np.float64))
        if cb.m > 0:
            sg = O.pack_signs(r["sign"], codes.sign_row_bytes)
            codes.sign[s * codes.sign_row_bytes:e * codes.sign_row_bytes] = torch.from_numpy(sg.reshape(-1)).to(dev)
            codes.rnorm[s:e] = torch.from_numpy(r["rnorm"].astype(np.float32)).to(dev)
            part["sign"] = r["sign"]
            part["rnorm"] = r["rnorm"].astype(np.float32).astype(np.float64)
        parts.append(part)
    ref = {key: np.concatenate([p[key] for p in parts]) for key in parts[0]}
    return codes, ref


def _check_query(ocb, q64, ref, gi, gs, k, name):
    s = O.code_scores(ocb, q64, ref["idx"], ref["scale"], ref.get("sign"), ref.get("rnorm"))
    n = s.shape[0]
    tol = SCORE_RTOL * max(np.max(np.abs(s)), 1e-30)
    assert len(set(gi.tolist())) == k, f"{name}: repeated indices {gi}"
    assert np.all((gi >= 0) & (gi < n)), f"{name}: index out of range {gi}"
    assert np.all(np.diff(gs) <= 0), f"{name}: scores not sorted {gs}"
    eq = np.diff(gs) == 0
    assert np.all(np.diff(gi)[eq] > 0), f"{name}: equal scores not in index order"
    err = np.max(np.abs(gs - s[gi]))
    assert err <= tol, f"{name}: score error {err} > {tol}"
    kth = np.sort(s)[::-1][k - 1]
    assert np.all(s[gi] >= kth - 2 * tol), f"{name}: returned index below the k-th score"
    must = np.nonzero(s > kth + 2 * tol)[0]
    assert set(must.tolist()) <= set(gi.tolist()), f"{name}: missed a clear top-k member"
    return err / tol


@pytest.mark.parametrize("d,bits,m,nc,n_db,nq,k", [
    (200, 4, 200, False, 3001, 21, 10),    # vector-search shape, ragged tiles and query blocks
    (128, 3, 128, False, 2000, 8, 1),
    (256, 8, 0, True, 1500, 13, 32),
    (64, 2, 64, False, 999, 5, 7),
    (96, 5, 0, False, 777, 3, 4),
    (200, 1, 0, False, 500, 9, 10),
    (40, 4, 40, True, 33, 2, 33 - 1),
])
def test_topk_parity(dev, d, bits, m, nc, n_db, nq, k):
    _say("topk", d, bits, m, nc, n_db, nq, k)
    cb = tq.Codebook(d, bits, qjl_m=m, norm_correction=nc, rot_seed=5, qjl_seed=6)
    ocb = U.oracle_codebook(cb)
    db = synth.mixture_db(n_db, d, 16, seed=1 + d).numpy().astype(np.float64)
    qs = synth.mixture_db(nq, d, 16, seed=2 + d).numpy()
    codes, ref = _db_codes(cb, ocb, db, dev)
    gi, gs = tq.tq_ip_topk(cb, torch.from_numpy(qs).to(dev), codes, n_db, k)
    torch.cuda.synchronize()
    gi, gs = gi.cpu().numpy(), gs.cpu().numpy().astype(np.float64)
    worst = max(_check_query(ocb, qs[i].astype(np.float64), ref, gi[i], gs[i], k, f"q{i}")
                for i in range(nq))
    print("worst score error / tol", worst)


def test_topk_ties_go_to_lower_index(dev):
    """Duplicated database rows have identical codes and scores; the lower
    index must come first and win the last place."""
    _say("topk ties")
    d, n_half, k = 128, 700, 9
    cb = tq.Codebook(d, 4, qjl_m=128, rot_seed=9, qjl_seed=10)
    ocb = U.oracle_codebook(cb)
    half = synth.mixture_db(n_half, d, 8, seed=31).numpy().astype(np.float64)
    db = np.concatenate([half, half])
    codes, ref = _db_codes(cb, ocb, db, dev)
    qs = synth.mixture_db(6, d, 8, seed=32).numpy()
    gi, gs = tq.tq_ip_topk(cb, torch.from_numpy(qs).to(dev), codes, 2 * n_half, k)
    torch.cuda.synchronize()
    gi, gs = gi.cpu().numpy(), gs.cpu().numpy()
    for i in range(len(qs)):
        _check_query(ocb, qs[i].astype(np.float64), ref, gi[i], gs[i].astype(np.float64), k, f"q{i}")
        for j in range(k):
            a = gi[i, j] % n_half
            # a duplicate pair is taken in index order: the copy is only
            # present together with (and after) the original
            if gi[i, j] >= n_half:
                assert a in gi[i, :j].tolist(), f"q{i}: copy {gi[i, j]} taken before its original"


def test_topk_argument_errors(dev):
    _say("topk errors")
    cb = tq.Codebook(64, 4)
    codes = tq.Codes(cb, 1, 64, TQ_LAYOUT_ROW)
    q = torch.zeros((3, 64), dtype=torch.float32, device=dev)
    with pytest.raises(tq.TQError) as e:
        tq.tq_ip_topk(cb, q, codes, 64, 33)
    assert e.value.status == 2
    with pytest.raises(tq.TQError) as e:
        tq.tq_ip_topk(cb, q, codes, 10, 11)
    assert e.value.status == 1
    gi = torch.full((3, 0), 5, dtype=torch.int64, device=dev)
    gs = torch.full((3, 0), 5.0, dtype=torch.float32, device=dev)
    tq.tq_ip_topk(cb, q, codes, 64, 0, out_idx=gi, out_score=gs)      # k = 0: no-op
    tile = tq.Codes(cb, 1, 64, tq.TQ_LAYOUT_TILE32)
    with pytest.raises(tq.TQError):
        tq.tq_ip_topk(cb, q, tile, 64, 5)


@pytest.mark.timeout(600)
def test_topk_full_size_vector_search(dev):
    """1,000,000 database vectors at d = 200 (unit-norm 256-cluster mixture),
    4-bit + QJL m = 200, 1,000 queries, k = 10 in the launch configuration the
    benchmark times.  Every query's returned scores are checked against the
    oracle's scores of those indices; 16 sampled queries get the full check."""
    _say("topk full size 1e6 x 200")
    d, n_db, nq, k = 200, 1_000_000, 1000, 10
    cb = tq.Codebook(d, 4, qjl_m=200, rot_seed=1, qjl_seed=2)
    ocb = U.oracle_codebook(cb)
    db = synth.mixture_db(n_db, d, 256, seed=7).numpy()
    qs = synth.mixture_db(nq, d, 256, seed=8).numpy()
    codes, ref = _db_codes(cb, ocb, db.astype(np.float64), dev)
    del db
    gi, gs = tq.tq_ip_topk(cb, torch.from_numpy(qs).to(dev), codes, n_db, k)
    torch.cuda.synchronize()
    gi, gs = gi.cpu().numpy(), gs.cpu().numpy().astype(np.float64)
    assert np.all((gi >= 0) & (gi < n_db))
    assert np.all(np.diff(gs, axis=1) <= 0)
    qt = qs.astype(np.float64) @ ocb.rot.T
    tq_ = qt @ ocb.qjl.T
    for i in range(nq):
        rows = gi[i]
        s = ref["scale"][rows] * (ocb.centroids[ref["idx"][rows]] @ qt[i])
        pm = 2.0 * ref["sign"][rows].astype(np.float64) - 1.0
        s = s + (O.SQRT_HALF_PI / ocb.m) * ref["rnorm"][rows] * (pm @ tq_[i])
        tol = SCORE_RTOL * max(np.max(np.abs(s)), 1e-30)
        assert np.max(np.abs(gs[i] - s)) <= 2 * tol, f"q{i}: returned scores differ from the oracle"
    rng = np.random.default_rng(123)
    for i in rng.choice(nq, 16, replace=False):
        _check_query(ocb, qs[i].astype(np.float64), ref, gi[i], gs[i], k, f"q{i}")
