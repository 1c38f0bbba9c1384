"""The allocation-free decode entry point (tq_attn_decode_noalloc) against
tq_attn_decode with its own workspace, through the C ABI: two calls in a row
on the library's fixed scratch, the second on a smaller input, each meeting
the decode bars (logits 1e-4 of the row max, outputs 2e-3 max-abs) against the
workspace call on the same codes; and a shape whose scratch exceeds the fixed
array is refused before anything runs."""
import math

import numpy as np
import pytest
import torch

import synth
import kv_cache_vector_quantize_amd as tq
from kv_cache_vector_quantize_amd import TQ_LAYOUT_ROW, TQ_LAYOUT_TILE32, _lib

import tq_testutil as U

pytestmark = pytest.mark.gpu


def _say(*a):
    print("[case]", *a, flush=True)


def _case(dev, B, Hkv, Hq, N, seed, lens=None):
    kcb = tq.Codebook(128, 3, qjl_m=128, rot_seed=1, qjl_seed=2)
    vcb = tq.Codebook(128, 4, rot_seed=3)
    S = (N + 31) // 32 * 32
    k = synth.kv_gaussian(B, Hkv, N, 128, seed, dtype="bf16", device=dev, channels=[3, 77, 101], factor=20.0)
    v = synth.kv_gaussian(B, Hkv, N, 128, seed + 1, dtype="bf16", device=dev, channels=[3, 77, 101], factor=20.0)
    q = synth.queries_gaussian(B, Hq, 128, seed + 2, dtype="bf16", device=dev)
    kc = tq.Codes(kcb, B * Hkv, S, TQ_LAYOUT_ROW)
    vc = tq.Codes(vcb, B * Hkv, S, TQ_LAYOUT_TILE32)
    tq.tq_quantize_kv(kcb, vcb, k.view(B * Hkv, N, 128), v.view(B * Hkv, N, 128), kc, vc)
    sl = torch.tensor(lens, dtype=torch.int32, device=dev) if lens is not None else None
    tau = 1.0 / math.sqrt(128)
    lg_ws = torch.full((B, Hq, N), 7.0, dtype=torch.float32, device=dev)
    out_ws = tq.tq_attn_decode(kcb, vcb, q, kc, vc, N, tau, seq_lens=sl, logits=lg_ws)
    lg_na = torch.full((B, Hq, N), 9.0, dtype=torch.float32, device=dev)
    out_na = torch.full((B, Hq, 128), 5.0, dtype=torch.float32, device=dev)
    tq.tq_attn_decode_noalloc(kcb, vcb, q, kc, vc, N, tau, seq_lens=sl, out=out_na, logits=lg_na)
    torch.cuda.synchronize()
    return (lg_ws.cpu().numpy(), out_ws.cpu().numpy()), (lg_na.cpu().numpy(), out_na.cpu().numpy()), lens


def _check(ref, got, lens):
    (lr, orf), (lg, og) = ref, got
    B, Hq, N = lr.shape
    for b in range(B):
        nb = N if lens is None else lens[b]
        assert np.all(np.isneginf(lg[b, :, nb:]))
        for h in range(Hq):
            if nb:
                scale = np.max(np.abs(lr[b, h, :nb]))
                assert np.max(np.abs(lg[b, h, :nb] - lr[b, h, :nb])) <= U.LOGIT_RTOL * scale
    assert np.max(np.abs(og - orf)) <= U.OUT_ATOL
    return bool(np.array_equal(lg, lr) and np.array_equal(og, orf))


def test_noalloc_decode_matches_workspace_call():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    dev = "cuda"
    _say("noalloc call 1: B=2 Hkv=2 Hq=16 N=5000")
    ref, got, lens = _case(dev, 2, 2, 16, 5000, seed=31)
    same1 = _check(ref, got, lens)
    _say("noalloc call 2 (smaller): B=1 Hkv=1 Hq=8 N=300, length 211")
    ref, got, lens = _case(dev, 1, 1, 8, 300, seed=41, lens=[211])
    same2 = _check(ref, got, lens)
    print("bit-identical to the workspace call:", same1, same2)


def test_noalloc_decode_rejects_oversized_shape():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    _say("noalloc oversized shape")
    kcb = tq.Codebook(128, 3, qjl_m=128, rot_seed=1, qjl_seed=2)
    vcb = tq.Codebook(128, 4, rot_seed=3)
    B, Hq, Hkv, N = 128, 64, 8, 131072          # 17 MB of scratch
    assert tq.tq_attn_decode_workspace(B, Hq, Hkv, N, 128) > (8 << 20)
    st = tq.lib().tq_attn_decode_noalloc(kcb.handle, vcb.handle, None, 1, B, Hq, Hkv, None, None, None, N,
                                         0.1, None, None, None)
    assert st == _lib.TQ_ERR_UNSUPPORTED
    assert b"scratch" in tq.lib().tq_last_error()
