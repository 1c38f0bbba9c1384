"""GPU parity of tq_ip_topk (inner-product top-k from codes) against the oracle.

Both sides score the same codes: the oracle quantizes the seeded database and
its packed codes are uploaded, so the GPU never produces an oracle input.

tq_ip_topk returns the exact top-k of the float64 score from the codes, with
each score rounded to fp32.  The oracle's scores (its own float64 rotation
and sketch, built independently of the library's) agree with the library's
float64 scores to about 1e-12 relative, so with EPS = 1e-9 x the largest
|score| of the query's top rows the checks on every query are:
* indices are distinct and in range, scores are non-increasing;
* each returned score is the oracle score of its index rounded to fp32
  (within 2^-23 relative + EPS);
* the returned set is the oracle's top-k: every row whose score exceeds the
  k-th by more than EPS is returned and no returned row falls below the k-th
  by more than EPS;
* without near-ties (gaps <= EPS) among the first k + 1 oracle scores, the
  returned list equals the oracle's list, position by position.
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

EPS_REL = 1e-9
F32_REL = 2.0 ** -23


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


def _oracle_top(ocb, qs, ref, keep, block=50000):
    """Per query, the `keep` best rows by oracle score (score desc, index
    asc) and their scores, from blockwise oracle scores of the whole
    database."""
    nq = qs.shape[0]
    n = ref["idx"].shape[0]
    best_i = np.zeros((nq, 0), dtype=np.int64)
    best_s = np.zeros((nq, 0))
    for s0 in range(0, n, block):
        e0 = min(n, s0 + block)
        sc = O.code_scores_many(ocb, qs, ref["idx"][s0:e0], ref["scale"][s0:e0],
                                None if "sign" not in ref else ref["sign"][s0:e0],
                                None if "rnorm" not in ref else ref["rnorm"][s0:e0]).T   # [nq, rows]
        kk = min(keep, e0 - s0)
        part = np.argpartition(-sc, kk - 1, axis=1)[:, :kk]
        cand_i = np.concatenate([best_i, part + s0], axis=1)
        cand_s = np.concatenate([best_s, np.take_along_axis(sc, part, axis=1)], axis=1)
        order = np.lexsort((cand_i, -cand_s), axis=1)[:, :keep]
        best_i = np.take_along_axis(cand_i, order, axis=1)
        best_s = np.take_along_axis(cand_s, order, axis=1)
    return best_i, best_s


def _row_scores(ocb, q64, ref, rows):
    return O.code_scores(ocb, q64, ref["idx"][rows], ref["scale"][rows],
                         None if "sign" not in ref else ref["sign"][rows],
                         None if "rnorm" not in ref else ref["rnorm"][rows])


def _check_query(ocb, q64, ref, top_i, top_s, gi, gs, k, name):
    """top_i/top_s: the oracle's best k + 1 (or more) rows of this query.
    Returns True when the list had to match position by position."""
    n = ref["idx"].shape[0]
    eps = EPS_REL * max(np.max(np.abs(top_s[:k + 1])), 1e-30)
    assert len(set(gi.tolist())) == k, f"{name}: repeated indices {gi}"
    assert np.all((gi >= 0) & (gi < n)), f"{name}: index out of range {gi}"
    assert np.all(np.diff(gs) <= 0), f"{name}: scores not sorted {gs}"
    s_g = _row_scores(ocb, q64, ref, gi)
    err = np.abs(gs - s_g)
    assert np.all(err <= F32_REL * np.abs(s_g) + eps), f"{name}: score error {err.max()}"
    kth = top_s[k - 1]
    assert np.all(s_g >= kth - eps), f"{name}: returned row below the k-th score"
    must = top_i[:k][top_s[:k] > kth + eps]
    assert set(must.tolist()) <= set(gi.tolist()), f"{name}: missed a top-k row"
    head = top_s[:k + 1] if len(top_s) > k else top_s[:k]
    strict = bool(np.all(-np.diff(head) > eps))
    if strict:
        assert np.array_equal(gi, top_i[:k]), f"{name}: {gi} != oracle {top_i[:k]}"
    return strict


def _run(cb, qs, codes, n_db, k, dev):
    gi, gs = tq.tq_ip_topk(cb, torch.from_numpy(qs).to(dev), codes, n_db, k)
    torch.cuda.synchronize()
    return gi.cpu().numpy(), gs.cpu().numpy().astype(np.float64)


def _check_all(ocb, qs, ref, gi, gs, k, tag):
    top_i, top_s = _oracle_top(ocb, qs.astype(np.float64), ref, k + 1)
    n_strict = sum(_check_query(ocb, qs[i].astype(np.float64), ref, top_i[i], top_s[i], gi[i], gs[i], k,
                                f"{tag} q{i}") for i in range(qs.shape[0]))
    print(tag, "queries matched position by position:", n_strict, "of", qs.shape[0])
    return n_strict


@pytest.mark.parametrize("d,bits,m,nc,n_db,nq,k", [
    (200, 4, 200, False, 3001, 21, 10),    # vector-search shape, ragged tiles and query blocks
    (128, 3, 128, False, 2000, 8, 1),
    (256, 8, 0, True, 1500, 13, 32),       # 64 candidates
    (64, 2, 64, False, 999, 5, 7),
    (96, 5, 0, False, 777, 3, 4),
    (200, 1, 0, False, 500, 9, 10),
    (40, 4, 40, True, 33, 2, 33 - 1),      # every row is a candidate
    (128, 3, 128, False, 5000, 40, 16),    # 32 candidates
    (200, 4, 200, False, 3001, 21, 20),    # 40 candidates
])
def test_topk_parity(dev, d, bits, m, nc, n_db, nq, k):
    _say("topk", d, bits, m, nc, n_db, nq, k)
    cb = tq.Codebook(d, bits, qjl_m=m, norm_correction=nc, rot_seed=5, qjl_seed=6)
    ocb = U.oracle_codebook(cb)
    db = synth.mixture_db(n_db, d, 16, seed=1 + d).numpy().astype(np.float64)
    qs = synth.mixture_db(nq, d, 16, seed=2 + d).numpy()
    codes, ref = _db_codes(cb, ocb, db, dev)
    gi, gs = _run(cb, qs, codes, n_db, k, dev)
    _check_all(ocb, qs, ref, gi, gs, k, "default")
    # the exact scan alone gives the same answer
    ws = torch.empty(tq.tq_ip_topk_workspace(nq, n_db, k, d), dtype=torch.uint8, device=dev)
    try:
        tq.tq_ip_topk_exact_scan(True)
        si, ss = tq.tq_ip_topk(cb, torch.from_numpy(qs).to(dev), codes, n_db, k, workspace=ws)
        n_scan = tq.tq_ip_topk_scan_count(cb, ws, nq, n_db, k)
    finally:
        tq.tq_ip_topk_exact_scan(False)
    si, ss = si.cpu().numpy(), ss.cpu().numpy().astype(np.float64)
    assert np.array_equal(si, gi)
    assert np.array_equal(ss, gs)
    # every query was scanned unless all rows are candidates
    assert n_scan == (nq if n_db > (16 if k <= 10 else min(2 * k, 64)) else 0)


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
    gi, gs = _run(cb, qs, codes, 2 * n_half, k, dev)
    _check_all(ocb, qs, ref, gi, gs, k, "ties")
    for i in range(len(qs)):
        for j in range(k):
            a = gi[i, j] % n_half
            # a duplicate pair is taken in index order: the copy is only
            # present together with (and after) the original
            if gi[i, j] >= n_half:
                assert a in gi[i, :j].tolist(), f"q{i}: copy {gi[i, j]} taken before its original"


def test_topk_many_copies_take_the_scan(dev):
    """40 copies of each of 50 vectors: the candidates of a query are copies
    of its best vector, the k-th exact score equals the kc-th approximate one,
    so the test cannot settle the query and the exact scan answers it."""
    _say("topk many copies")
    d, n_u, copies, k = 64, 50, 40, 10
    cb = tq.Codebook(d, 3, qjl_m=64, rot_seed=3, qjl_seed=4)
    ocb = U.oracle_codebook(cb)
    base = synth.mixture_db(n_u, d, 4, seed=41).numpy().astype(np.float64)
    perm = np.random.default_rng(42).permutation(n_u * copies)
    db = np.tile(base, (copies, 1))[perm]
    codes, ref = _db_codes(cb, ocb, db, dev)
    qs = synth.mixture_db(7, d, 4, seed=43).numpy()
    ws = torch.empty(tq.tq_ip_topk_workspace(len(qs), n_u * copies, k, d), dtype=torch.uint8, device=dev)
    gi, gs = tq.tq_ip_topk(cb, torch.from_numpy(qs).to(dev), codes, n_u * copies, k, workspace=ws)
    assert tq.tq_ip_topk_scan_count(cb, ws, len(qs), n_u * copies, k) == len(qs)
    gi, gs = gi.cpu().numpy(), gs.cpu().numpy().astype(np.float64)
    _check_all(ocb, qs, ref, gi, gs, k, "copies")
    for i in range(len(qs)):
        # the k returned rows are the k lowest indices holding the best vector
        s = _row_scores(ocb, qs[i].astype(np.float64), ref, np.arange(n_u * copies))
        src = perm[gi[i]] % n_u
        best = src[0]
        holders = np.sort(np.nonzero(perm % n_u == best)[0])
        assert np.all(src == best), f"q{i}: mixed vectors {src}"
        assert np.array_equal(gi[i], holders[:k]), f"q{i}: {gi[i]} != {holders[:k]}"
        assert np.all(gs[i] == gs[i][0])
        assert abs(gs[i][0] - s[holders[0]]) <= F32_REL * abs(s[holders[0]]) + EPS_REL * abs(s[holders[0]])


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
def test_topk_mid_size_sample_pass(dev):
    """300,000 vectors at d = 128 (3-bit + QJL m = 128): past the size where
    the sample pass sets each query's floor; all 300 queries get the full
    check, and the exact scan alone returns the same lists."""
    _say("topk 3e5 x 128")
    d, n_db, nq, k = 128, 300_000, 300, 10
    cb = tq.Codebook(d, 3, qjl_m=128, rot_seed=11, qjl_seed=12)
    ocb = U.oracle_codebook(cb)
    db = synth.mixture_db(n_db, d, 128, seed=51).numpy().astype(np.float64)
    qs = synth.mixture_db(nq, d, 128, seed=52).numpy()
    codes, ref = _db_codes(cb, ocb, db, dev)
    del db
    gi, gs = _run(cb, qs, codes, n_db, k, dev)
    n_strict = _check_all(ocb, qs, ref, gi, gs, k, "3e5")
    assert n_strict >= nq - 3
    try:
        tq.tq_ip_topk_exact_scan(True)
        si, ss = _run(cb, qs, codes, n_db, k, dev)
    finally:
        tq.tq_ip_topk_exact_scan(False)
    assert np.array_equal(si, gi)
    assert np.array_equal(ss, gs)


@pytest.mark.timeout(900)
def test_topk_full_size_vector_search(dev):
    """1,000,000 database vectors at d = 200 (unit-norm 256-cluster mixture),
    4-bit + QJL m = 200, 1,000 queries, k = 10 in the launch configuration the
    benchmark times.  Every query gets the full check against the oracle's
    scores of the whole database."""
    _say("topk full size 1e6 x 200")
    d, n_db, nq, k = 200, 1_000_000, 1000, 10
    cb = tq.Codebook(d, 4, qjl_m=200, rot_seed=1, qjl_seed=2)
    ocb = U.oracle_codebook(cb)
    db = synth.mixture_db(n_db, d, 256, seed=7).numpy()
    qs = synth.mixture_db(nq, d, 256, seed=8).numpy()
    codes, ref = _db_codes(cb, ocb, db.astype(np.float64), dev)
    del db
    ws = torch.empty(tq.tq_ip_topk_workspace(nq, n_db, k, d), dtype=torch.uint8, device=dev)
    gi, gs = tq.tq_ip_topk(cb, torch.from_numpy(qs).to(dev), codes, n_db, k, workspace=ws)
    print("queries answered by the exact scan:", tq.tq_ip_topk_scan_count(cb, ws, nq, n_db, k))
    gi, gs = gi.cpu().numpy(), gs.cpu().numpy().astype(np.float64)
    n_strict = _check_all(ocb, qs, ref, gi, gs, k, "1e6")
    assert n_strict >= nq - 5
