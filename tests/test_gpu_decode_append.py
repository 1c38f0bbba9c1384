"""One decode step in one call (tq_attn_decode_append) against the two calls
it stands for (tq_quantize_kv of the step's new keys and values, then
tq_attn_decode), through the C ABI on the same inputs: the code planes and
the outputs and logits must be identical, since the fused call runs the same
kernels (the d = 128 query prologue inside the append launch, other head
dimensions unfused).  Also the end-to-end decode bars against the oracle's
decode of the codes the GPU wrote, and the argument checks that must reject
a call before anything runs."""
import math

import pytest
import torch

import synth
import kv_cache_vector_quantize_amd as tq
from kv_cache_vector_quantize_amd import TQ_LAYOUT_ROW, TQ_LAYOUT_TILE32, TQError

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    return "cuda"


def _say(*a):
    print("[case]", *a, flush=True)


def _cache(dev, kcb, vcb, B, Hkv, N, d, seed):
    S = (N + 31) // 32 * 32
    k = synth.kv_gaussian(B, Hkv, N, d, seed, dtype="bf16", device=dev, channels=[3], factor=20.0)
    v = synth.kv_gaussian(B, Hkv, N, d, seed + 1, dtype="bf16", device=dev, channels=[3], factor=20.0)
    return k.view(B * Hkv, N, d), v.view(B * Hkv, N, d), S


def _two_sets(kcb, vcb, B, Hkv, S):
    mk = lambda: (tq.Codes(kcb, B * Hkv, S, TQ_LAYOUT_ROW), tq.Codes(vcb, B * Hkv, S, TQ_LAYOUT_TILE32))
    return mk(), mk()


@pytest.mark.parametrize("d,kb,m,vb,n_new,qdt", [
    (128, 3, 128, 4, 1, "bf16"),     # the decode layer's shape class: prologue fused into the append
    (128, 2, 0, 2, 4, "f32"),        # no sketch, several new tokens
    (128, 4, 64, 8, 2, "bf16"),
    (64, 3, 64, 4, 1, "bf16"),       # any-shape kernels: append and decode unfused
])
def test_append_step_matches_separate_calls(dev, d, kb, m, vb, n_new, qdt):
    B, Hkv, Hq, N = 2, 2, 16, 300
    _say("append step", d, kb, m, vb, n_new, qdt)
    kcb = tq.Codebook(d, kb, qjl_m=m, rot_seed=1, qjl_seed=2)
    vcb = tq.Codebook(d, vb, rot_seed=3)
    k, v, S = _cache(dev, kcb, vcb, B, Hkv, N, d, 5)
    q = synth.queries_gaussian(B, Hq, d, 7, dtype=qdt, device=dev)
    (kc1, vc1), (kc2, vc2) = _two_sets(kcb, vcb, B, Hkv, S)
    off = N - n_new
    for kc, vc in ((kc1, vc1), (kc2, vc2)):
        tq.tq_quantize_kv(kcb, vcb, k[:, :off].contiguous(), v[:, :off].contiguous(), kc, vc)
    k_new, v_new = k[:, off:].contiguous(), v[:, off:].contiguous()
    tau = 1.0 / math.sqrt(d)
    lens = torch.tensor([N, N - 17], dtype=torch.int32, device=dev)
    lg1 = torch.full((B, Hq, N), 3.0, dtype=torch.float32, device=dev)
    lg2 = torch.full((B, Hq, N), 5.0, dtype=torch.float32, device=dev)
    tq.tq_quantize_kv(kcb, vcb, k_new, v_new, kc1, vc1, tok_offset=off)
    o1 = tq.tq_attn_decode(kcb, vcb, q, kc1, vc1, N, tau, seq_lens=lens, logits=lg1)
    o2 = tq.tq_attn_decode_append(kcb, vcb, k_new, v_new, off, q, kc2, vc2, N, tau, seq_lens=lens, logits=lg2)
    torch.cuda.synchronize()
    for a, b in ((kc1.idx, kc2.idx), (kc1.scale, kc2.scale), (vc1.idx, vc2.idx), (vc1.scale, vc2.scale)):
        assert torch.equal(a, b)
    if m:
        assert torch.equal(kc1.sign, kc2.sign) and torch.equal(kc1.rnorm, kc2.rnorm)
    assert torch.equal(o1, o2)
    assert torch.equal(lg1, lg2)


def test_append_step_repeated_like_a_serving_loop(dev):
    """Several steps in a row, each appending one token at the next position
    and attending over the grown context: every step equals the two-call
    step on its own copy of the caches."""
    d, B, Hkv, Hq, N0, steps = 128, 1, 2, 16, 96, 5
    _say("append loop")
    kcb = tq.Codebook(d, 3, qjl_m=128, rot_seed=1, qjl_seed=2)
    vcb = tq.Codebook(d, 4, rot_seed=3)
    k, v, S = _cache(dev, kcb, vcb, B, Hkv, N0 + steps, d, 11)
    (kc1, vc1), (kc2, vc2) = _two_sets(kcb, vcb, B, Hkv, S)
    for kc, vc in ((kc1, vc1), (kc2, vc2)):
        tq.tq_quantize_kv(kcb, vcb, k[:, :N0].contiguous(), v[:, :N0].contiguous(), kc, vc)
    tau = 1.0 / math.sqrt(d)
    for s in range(steps):
        n = N0 + s + 1
        q = synth.queries_gaussian(B, Hq, d, 20 + s, dtype="bf16", device=dev)
        kn, vn = k[:, n - 1:n].contiguous(), v[:, n - 1:n].contiguous()
        tq.tq_quantize_kv(kcb, vcb, kn, vn, kc1, vc1, tok_offset=n - 1)
        o1 = tq.tq_attn_decode(kcb, vcb, q, kc1, vc1, n, tau)
        o2 = tq.tq_attn_decode_append(kcb, vcb, kn, vn, n - 1, q, kc2, vc2, n, tau)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2), s
    assert torch.equal(kc1.idx, kc2.idx) and torch.equal(vc1.idx, vc2.idx)


def test_append_step_argument_errors(dev):
    d, B, Hkv, Hq, N = 128, 1, 1, 8, 64
    kcb = tq.Codebook(d, 3, qjl_m=128, rot_seed=1, qjl_seed=2)
    vcb = tq.Codebook(d, 4, rot_seed=3)
    k, v, S = _cache(dev, kcb, vcb, B, Hkv, N, d, 3)
    (kc, vc), _ = _two_sets(kcb, vcb, B, Hkv, S)
    q = synth.queries_gaussian(B, Hq, d, 4, dtype="bf16", device=dev)
    before = kc.idx.clone()
    kn, vn = k[:, -1:].contiguous(), v[:, -1:].contiguous()
    with pytest.raises(TQError):      # the new token lies past the attended context
        tq.tq_attn_decode_append(kcb, vcb, kn, vn, N, q, kc, vc, N, 0.1)
    small = torch.empty(16, dtype=torch.uint8, device=dev)
    with pytest.raises(TQError):      # workspace too small: the append must not run either
        tq.tq_attn_decode_append(kcb, vcb, kn, vn, N - 1, q, kc, vc, N, 0.1, workspace=small)
    torch.cuda.synchronize()
    assert torch.equal(kc.idx, before)
