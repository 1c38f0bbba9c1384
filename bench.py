#!/usr/bin/env python3
"""Benchmark of the hot path on one MI355X.

A step is one serving-style pass over the 128K-context decode layer
(B=8, 64 query heads, 8 KV heads, d=128, context 131072; keys 3-bit + 1-bit
QJL m=128, values 4-bit): quantize the step's new key/value vector of every
sequence into the compressed cache (position ctx-1), then decode attention
for all 512 query heads straight from the packed codes, in one
tq_attn_decode_append call (append + query prologue in one launch, then the
split and combine launches).  Inputs and the
compressed cache are resident in HBM before the timed region.

Printed: ONE JSON line with the contract fields plus
* roofline of the dominant kernel (the decode split kernel), from HIP events
  recorded on its stream around every launch in the timed region;
* quantize: tq_quantize_kv bandwidth on the quantize-only layer
  (B=16, 8 KV heads, d=128, 32768 tokens, bf16 K and V, 4-bit, no QJL);
* bit_sweep: decode KV tokens/s, HBM fraction and error against exact
  attention for k8v4, k4v4, k3v4, k3v3, k2v2 on the 32K GQA layer
  (B=32, 32 query / 4 KV heads);
* vector_search: tq_ip_topk queries/s, MFMA rate and recall on 1e6 coded
  vectors of d=200 with 1000 queries;
* copy_GBps: the box's device-to-device copy rate (1 GiB); read_GBps and
  write_GBps: the rates of a kernel that only reads and of one that only
  writes 1 GiB (the ceilings of read- and store-dominated kernels);
* cpu_baseline: the float64 CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_split_128k_traffic.txt")
SPLIT_SOURCE = os.path.join(ROOT, "kv_cache_vector_quantize_amd", "csrc", "decode.hip")


def split_traffic():
    """HBM bytes per split launch from the committed FETCH_SIZE / WRITE_SIZE
    summary, or None when the kernel source changed since it was taken."""
    import hashlib
    try:
        kv = {}
        with open(TRAFFIC_FILE) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    kv[k.strip()] = v.strip()
        with open(SPLIT_SOURCE, "rb") as f:
            sha = hashlib.sha256(f.read()).hexdigest()
        if kv.get("kernel_source_sha256") != sha:
            return None
        return int(kv["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


METRIC = "KV tokens/s in compressed decode attention & quantize GB/s, % of HBM peak"


def spread(ms):
    """median, p10 and p90 (milliseconds) of per-iteration times."""
    a = np.asarray(ms, dtype=np.float64)
    if a.size == 0:
        return None
    return dict(median=round(float(np.median(a)), 5), p10=round(float(np.percentile(a, 10)), 5),
                p90=round(float(np.percentile(a, 90)), 5), n=int(a.size))


def timed_iters(torch, fn, iters):
    """Run fn iters times between a synchronize on either side, with an event
    at every iteration boundary on the current stream.  Returns (mean ms over
    the whole region, per-iteration ms list)."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(iters + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(iters):
        fn()
        ev[i + 1].record()
    torch.cuda.synchronize()
    per = [ev[i].elapsed_time(ev[i + 1]) for i in range(iters)]
    return ev[0].elapsed_time(ev[iters]) / iters, per


def kernel_spread(tq, kernel):
    """(mean ms, spread) of every recorded launch of one library kernel."""
    d = tq.tq_profile_durations(kernel)
    return (float(d.mean()) if d.size else 0.0), spread(d)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-quantize", action="store_true")
    ap.add_argument("--no-sweep", action="store_true", help="skip the bit-width sweep leg")
    ap.add_argument("--no-search", action="store_true", help="skip the vector-search leg")
    ap.add_argument("--no-ab", action="store_true", help="skip the dequantize-then-attend leg")
    ap.add_argument("--no-paged", action="store_true", help="skip the paged-cache leg")
    ap.add_argument("--no-polar", action="store_true", help="skip the PolarQuant-keys leg")
    ap.add_argument("--no-dims", action="store_true", help="skip the other-head-dimension leg")
    ap.add_argument("--calib-copy", action="store_true",
                    help="accepted for profiling commands; the 1 GiB copy always runs")
    return ap.parse_args()


def decode_workload(torch, tq, synth, dev):
    B, Hq, Hkv, d, N = 8, 64, 8, 128, 131072
    kcb = tq.Codebook(d, 3, qjl_m=128, rot_seed=1, qjl_seed=2)
    vcb = tq.Codebook(d, 4, rot_seed=3)
    k = synth.kv_gaussian(B, Hkv, N, d, 0, dtype="bf16", device=dev, channels=[3, 77, 101], factor=20.0)
    v = synth.kv_gaussian(B, Hkv, N, d, 1, dtype="bf16", device=dev, channels=[3, 77, 101], factor=20.0)
    q = synth.queries_gaussian(B, Hq, d, 2, dtype="bf16", device=dev)
    kc = tq.Codes(kcb, B * Hkv, N, tq.TQ_LAYOUT_ROW)
    vc = tq.Codes(vcb, B * Hkv, N, tq.TQ_LAYOUT_TILE32)
    # cache build (untimed): all N positions
    tq.tq_quantize_kv(kcb, vcb, k.view(B * Hkv, N, d), v.view(B * Hkv, N, d), kc, vc)
    # the step's new token per sequence = the last position
    k_new = k[:, :, N - 1:N].reshape(B * Hkv, 1, d).contiguous()
    v_new = v[:, :, N - 1:N].reshape(B * Hkv, 1, d).contiguous()
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    ws = torch.empty(tq.tq_attn_decode_workspace(B, Hq, Hkv, N, d), dtype=torch.uint8, device=dev)
    tau = 1.0 / math.sqrt(d)

    def step():
        # one call: the new token of every sequence is quantized into the
        # caches at position N - 1 (the query prologue rides in that launch),
        # then the 8 query heads of each KV head attend over all N positions
        tq.tq_attn_decode_append(kcb, vcb, k_new, v_new, N - 1, q, kc, vc, N, tau, out=out, workspace=ws)

    per_token_head = (3 * d // 8) + 4 * ((128 + 31) // 32) + 4 + 4 + (4 * d // 8) + 4   # 140 B
    cfg = dict(workload="decode-128k GQA layer", B=B, Hq=Hq, Hkv=Hkv, d=d, context=N,
               keys="3-bit Lloyd-Max + 1-bit QJL m=128", values="4-bit Lloyd-Max",
               kv_input="bf16, N(0,1), channels 3/77/101 x20", query="bf16")
    return dict(step=step, B=B, Hq=Hq, Hkv=Hkv, d=d, N=N, kcb=kcb, vcb=vcb, k=k, v=v, q=q, kc=kc, vc=vc,
                out=out, ws=ws, tau=tau, bytes_per_token_head=per_token_head, cfg=cfg)


def quantize_leg(torch, tq, synth, dev, iters, warm):
    B, H, N, d = 16, 8, 32768, 128
    chk = synth.outlier_channels(10, H, d, 4)
    chv = synth.outlier_channels(11, H, d, 4)
    k = synth.kv_gaussian(B, H, N, d, 10, dtype="bf16", device=dev, per_head_channels=chk, factor=15.0)
    v = synth.kv_gaussian(B, H, N, d, 11, dtype="bf16", device=dev, per_head_channels=chv, factor=15.0)
    kcb = tq.Codebook(d, 4, rot_seed=1)
    vcb = tq.Codebook(d, 4, rot_seed=3)
    kc = tq.Codes(kcb, B * H, N, tq.TQ_LAYOUT_ROW)
    vc = tq.Codes(vcb, B * H, N, tq.TQ_LAYOUT_TILE32)
    kf, vf = k.view(B * H, N, d), v.view(B * H, N, d)
    for _ in range(warm):
        tq.tq_quantize_kv(kcb, vcb, kf, vf, kc, vc)
    torch.cuda.synchronize()
    tq.tq_profile_enable(True)
    ms, per = timed_iters(torch, lambda: tq.tq_quantize_kv(kcb, vcb, kf, vf, kc, vc), iters)
    tq.tq_profile_enable(False)
    kern_ms, kern_spread = kernel_spread(tq, tq.TQ_KERNEL_QUANTIZE)
    n_vec = 2 * B * H * N
    in_bytes = n_vec * d * 2
    out_bytes = n_vec * (d * 4 // 8 + 4)
    gbs = (in_bytes + out_bytes) / (ms * 1e-3) / 1e9
    per_launch_bytes = (in_bytes + out_bytes) / 2
    flops = 2.0 * d * d * n_vec
    # the rotation runs as bf16 MFMAs on a two-part split of Pi (bf16 input,
    # codes of up to 4 bits): two issued products per useful one
    mfma_flops = 2 * flops
    deq = dequantize_leg(torch, tq, kcb, vcb, kc, vc, B * H, N, iters, warm)
    del k, v, kc, vc
    return dict(workload="quantize-only layer: B=16, Hkv=8, d=128, 32768 tokens, bf16 K and V "
                         "(4 outlier channels/head x15), 4-bit, no QJL",
                GB_per_s=round(gbs, 1), frac_hbm=round(gbs / HBM_PEAK_GBS, 4), ms_per_call=round(ms, 4),
                call_ms_spread=spread(per), kernel_ms=round(kern_ms, 4), kernel_ms_spread=kern_spread,
                kernel_GB_per_s=round(per_launch_bytes / (kern_ms * 1e-3) / 1e9, 1),
                rotation_TFLOP_per_s=round(flops / (ms * 1e-3) / 1e12, 2),
                mfma_TFLOP_per_s=round(mfma_flops / (ms * 1e-3) / 1e12, 2),
                mfma_frac_bf16_peak=round(mfma_flops / (ms * 1e-3) / 2.5e15, 4),
                bytes_per_call=int(in_bytes + out_bytes), read_bytes_per_call=int(in_bytes),
                write_bytes_per_call=int(out_bytes), dequantize=deq)


def sketch_build_leg(torch, tq, W, iters, warm):
    """Keys with a sketch: the whole key cache of the 128K decode layer
    (8388608 bf16 vectors, 3-bit + QJL m=128) quantized again into its own
    code planes (the same codes are rewritten)."""
    B, Hkv, N, d = W["B"], W["Hkv"], W["N"], W["d"]
    kf = W["k"].view(B * Hkv, N, d)
    call = lambda: tq.tq_quantize_kv(W["kcb"], None, kf, None, W["kc"], None)
    for _ in range(warm):
        call()
    torch.cuda.synchronize()
    tq.tq_profile_enable(True)
    ms, per = timed_iters(torch, call, iters)
    tq.tq_profile_enable(False)
    kms, kspread = kernel_spread(tq, tq.TQ_KERNEL_QUANTIZE)
    n = B * Hkv * N
    bpv = 2 * d + 3 * d // 8 + 128 // 8 + 4 + 4      # bf16 in; idx, signs, scale, rnorm out
    return dict(workload="keys of the decode-128k layer with a sketch: 8388608 bf16 vectors, d=128, "
                         "3-bit + QJL m=128, row layout",
                ms_per_call=round(ms, 4), call_ms_spread=spread(per), kernel_ms=round(kms, 4),
                kernel_ms_spread=kspread, bytes_per_vector=bpv,
                kernel_GB_per_s=round(bpv * n / (kms * 1e-3) / 1e9, 1),
                frac_hbm=round(bpv * n / (kms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4))


def dequantize_leg(torch, tq, kcb, vcb, kc, vc, n_seq, n_tok, iters, warm):
    """tq_dequantize of the quantize layer's K (row) and V (tile32) codes back
    to bf16: reads 68 B of codes and writes 256 B per vector."""
    d = kcb.d
    ko = torch.empty((n_seq, n_tok, d), dtype=torch.bfloat16, device="cuda")
    vo = torch.empty_like(ko)

    def call():
        tq.tq_dequantize(kcb, kc, n_seq, n_tok, out=ko)
        tq.tq_dequantize(vcb, vc, n_seq, n_tok, out=vo)
    for _ in range(warm):
        call()
    torch.cuda.synchronize()
    tq.tq_profile_enable(True)
    ms, per = timed_iters(torch, call, iters)
    tq.tq_profile_enable(False)
    kern_ms, kern_spread = kernel_spread(tq, tq.TQ_KERNEL_DEQUANTIZE)
    n_vec = 2 * n_seq * n_tok
    rbytes = n_vec * (d * kcb.bits // 8 + 4)
    wbytes = n_vec * d * 2
    nbytes = rbytes + wbytes
    # Pi^T hi.hi + hi.lo + lo.hi on 32x32x16 bf16 MFMAs: three issued products
    # per useful one
    mfma_flops = 3 * 2.0 * d * d * n_vec
    del ko, vo
    return dict(workload=f"dequantize the quantize layer's K (row) and V (tile32) {kcb.bits}-bit codes "
                         f"to bf16: {n_vec} vectors, d={d}",
                GB_per_s=round(nbytes / (ms * 1e-3) / 1e9, 1), frac_hbm=round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                ms_per_call=round(ms, 4), call_ms_spread=spread(per), kernel_ms=round(kern_ms, 4),
                kernel_ms_spread=kern_spread,
                kernel_GB_per_s=round(nbytes / 2 / (kern_ms * 1e-3) / 1e9, 1),
                mfma_TFLOP_per_s=round(mfma_flops / (ms * 1e-3) / 1e12, 2),
                bytes_per_call=int(nbytes), read_bytes_per_call=int(rbytes), write_bytes_per_call=int(wbytes))


def dequant_attend_leg(torch, tq, W, iters, warm, copy_gbps):
    """The 128K layer's attention done dequantize-first, against decode from
    the codes.  A: tq_dequantize of K (3-bit + QJL, row) and V (4-bit, tile32)
    to bf16, then dense bf16 attention over them (torch batched products and
    softmax: S = K_hat q^T, P = softmax(tau S) in fp32, o = P^T V_hat; every
    right operand contiguous).  B: tq_attn_decode straight from the codes.
    Both compute the same estimate: <q, K_hat_j> is the codes' logit
    estimate.  dense_floor_ms is the time to read the bf16 K and V once at
    the box's copy rate, the least any dense kernel over them needs."""
    B, Hq, Hkv, d, N, tau = W["B"], W["Hq"], W["Hkv"], W["d"], W["N"], W["tau"]
    g = Hq // Hkv
    S_ = B * Hkv
    kd = torch.empty((S_, N, d), dtype=torch.bfloat16, device="cuda")
    vd = torch.empty_like(kd)
    qt = W["q"].view(B, Hkv, g, d).reshape(S_, g, d).transpose(1, 2).contiguous()   # [S, d, g]

    def dequant():
        tq.tq_dequantize(W["kcb"], W["kc"], S_, N, out=kd)
        tq.tq_dequantize(W["vcb"], W["vc"], S_, N, out=vd)

    # logits straight to fp32 where this torch offers it (bf16 logits of
    # magnitude ~30 lose ~0.1 to rounding, which moves the softmax by ~1%)
    try:
        torch.bmm(kd[:1, :64], qt[:1], out_dtype=torch.float32)
        lg_dtype = "fp32"
    except (RuntimeError, TypeError):
        lg_dtype = "bf16"

    def attend():
        if lg_dtype == "fp32":
            s = torch.bmm(kd, qt, out_dtype=torch.float32)             # [S, N, g]
        else:
            s = torch.bmm(kd, qt).float()
        p = torch.softmax(s * tau, dim=1)                              # over the context
        pt = p.to(torch.bfloat16).transpose(1, 2).contiguous()         # [S, g, N]
        return torch.bmm(pt, vd)                                       # [S, g, d]

    def direct():
        tq.tq_attn_decode(W["kcb"], W["vcb"], W["q"], W["kc"], W["vc"], N, tau, out=W["out"], workspace=W["ws"])

    def timed(fn):
        for _ in range(warm):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(iters):
            r = fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / iters, r

    deq_ms, _ = timed(dequant)
    att_ms, o_ab = timed(attend)
    dir_ms, _ = timed(direct)
    o_ab = o_ab.float().view(B, Hkv, g, d).reshape(B, Hq, d)
    err = float((o_ab - W["out"]).abs().max() / W["out"].abs().max())
    kv_bytes = 2 * S_ * N * d * 2
    floor_ms = kv_bytes / (copy_gbps * 1e9) * 1e3 if copy_gbps else None
    del kd, vd
    return dict(workload="decode-128k GQA layer, dequantize K and V to bf16 then dense bf16 attention, "
                         "against decode from the codes",
                dequantize_ms=round(deq_ms, 4), dense_attend_ms=round(att_ms, 4),
                dequant_then_attend_ms=round(deq_ms + att_ms, 4),
                dense_floor_ms=round(floor_ms, 4) if floor_ms else None,
                decode_from_codes_ms=round(dir_ms, 4),
                speedup_vs_dequant_first=round((deq_ms + att_ms) / dir_ms, 2),
                max_rel_diff_of_outputs=round(err, 5), dense_logits=lg_dtype,
                bf16_kv_bytes=int(kv_bytes))


def paged_leg(torch, tq, W, iters, warm, page_tokens=64):
    """The headline step on a paged cache: the 128K layer's K and V codes in
    pools of page_tokens-position pages placed by a shuffled block table
    (every sequence's pages scattered over the pool), the step's append
    through tq_quantize_kv_paged and the decode through tq_attn_decode_paged.
    Timed like the headline; the split kernel's time is compared with the
    contiguous one."""
    B, Hq, Hkv, d, N, tau = W["B"], W["Hq"], W["Hkv"], W["d"], W["N"], W["tau"]
    n_lp = (N + page_tokens - 1) // page_tokens
    n_pages = B * n_lp
    g = torch.Generator(device="cpu")
    g.manual_seed(12345)
    table = torch.randperm(n_pages, generator=g).to(torch.int32).view(B, n_lp).contiguous().to("cuda")
    kp = tq.Codes(W["kcb"], Hkv, n_pages * page_tokens, tq.TQ_LAYOUT_ROW)
    vp = tq.Codes(W["vcb"], Hkv, n_pages * page_tokens, tq.TQ_LAYOUT_TILE32)
    kf, vf = W["k"].view(B * Hkv, N, d), W["v"].view(B * Hkv, N, d)
    tq.tq_quantize_kv_paged(W["kcb"], W["vcb"], kf, vf, kp, vp, table, page_tokens)   # cache build, untimed
    k_new = W["k"][:, :, N - 1:N].reshape(B * Hkv, 1, d).contiguous()
    v_new = W["v"][:, :, N - 1:N].reshape(B * Hkv, 1, d).contiguous()
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")
    ws = torch.empty(tq.tq_attn_decode_paged_workspace(B, Hq, Hkv, N, d, page_tokens), dtype=torch.uint8,
                     device="cuda")

    def step():
        tq.tq_quantize_kv_paged(W["kcb"], W["vcb"], k_new, v_new, kp, vp, table, page_tokens, tok_offset=N - 1)
        tq.tq_attn_decode_paged(W["kcb"], W["vcb"], W["q"], kp, vp, table, page_tokens, N, tau, out=out,
                                workspace=ws)
    for _ in range(warm):
        step()
    torch.cuda.synchronize()
    tq.tq_profile_enable(True)
    ms, per = timed_iters(torch, step, iters)
    tq.tq_profile_enable(False)
    split_ms, split_spread = kernel_spread(tq, tq.TQ_KERNEL_DECODE_SPLIT)
    diff = float((out - W["out"]).abs().max() / W["out"].abs().max())
    del kp, vp, ws
    alg = W["bytes_per_token_head"] * B * Hkv * N
    return dict(workload=f"decode-128k GQA layer on a paged cache: {page_tokens}-position pages, "
                         f"{n_pages} pages per KV head placed by a shuffled block table",
                KV_tokens_per_s=round(B * N / (ms * 1e-3), 1), ms_per_step=round(ms, 5),
                step_ms_spread=spread(per), split_kernel_ms=round(split_ms, 5),
                split_kernel_ms_spread=split_spread, split_GBps=round(alg / (split_ms * 1e-3) / 1e9, 1),
                frac_hbm=round(alg / (split_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                max_rel_diff_vs_contiguous=round(diff, 7))


def polar_leg(torch, tq, W, iters, warm):
    """PolarQuant keys on the 128K decode layer: the same K inputs coded as
    (b1, br) = (4, 2) polar angles + QJL m=128 (48 + 16 + 8 B per key, as
    the 3-bit scalar keys) against the scalar path's keys, with the same
    4-bit values.  Reports the decode step's KV tokens/s and split-kernel
    rate beside the scalar path's, the polar quantize rate of the key cache,
    and the keys' reconstruction error |k - k_hat|^2 / |k|^2 (mean over one
    sequence of 131072 keys, GPU dequantize, without the sketch term) for
    both encodings."""
    B, Hq, Hkv, d, N, tau = W["B"], W["Hq"], W["Hkv"], W["d"], W["N"], W["tau"]
    pcb = tq.PolarCodebook(d, 4, 2, qjl_m=128, rot_seed=1, qjl_seed=2)
    kp = tq.Codes(pcb, B * Hkv, N, tq.TQ_LAYOUT_ROW)
    kf = W["k"].view(B * Hkv, N, d)
    tq.tq_quantize_kv(pcb, None, kf, None, kp, None)      # warm-up / cache build
    torch.cuda.synchronize()
    tq.tq_profile_enable(True)
    qms, _ = timed_iters(torch, lambda: tq.tq_quantize_kv(pcb, None, kf, None, kp, None), 3)
    tq.tq_profile_enable(False)
    n_vec = B * Hkv * N
    qbytes = n_vec * (d * 2 + kp.idx_row_bytes + kp.sign_row_bytes + 8)
    k_new = W["k"][:, :, N - 1:N].reshape(B * Hkv, 1, d).contiguous()
    v_new = W["v"][:, :, N - 1:N].reshape(B * Hkv, 1, d).contiguous()
    out = torch.empty((B, Hq, d), dtype=torch.float32, device="cuda")

    def step():
        tq.tq_quantize_kv(pcb, W["vcb"], k_new, v_new, kp, W["vc"], tok_offset=N - 1)
        tq.tq_attn_decode(pcb, W["vcb"], W["q"], kp, W["vc"], N, tau, out=out, workspace=W["ws"])
    for _ in range(warm):
        step()
    torch.cuda.synchronize()
    tq.tq_profile_enable(True)
    ms, per = timed_iters(torch, step, iters)
    tq.tq_profile_enable(False)
    split_ms, split_spread = kernel_spread(tq, tq.TQ_KERNEL_DECODE_SPLIT)
    bpt = kp.idx_row_bytes + kp.sign_row_bytes + 8 + d * 4 // 8 + 4
    alg = bpt * B * Hkv * N

    # reconstruction error of one sequence's keys, both encodings
    def rel_mse(cb, codes):
        xh = torch.empty((1, N, d), dtype=torch.float32, device="cuda")
        plain = tq.PolarCodebook(d, 4, 2, rot_seed=1) if cb is pcb else tq.Codebook(d, 3, rot_seed=1)
        c0 = tq.Codes(plain, 1, N, tq.TQ_LAYOUT_ROW)
        c0.idx.copy_(codes.idx[:N * codes.idx_row_bytes])
        c0.scale.copy_(codes.scale[:N])
        tq.tq_dequantize(plain, c0, 1, N, out=xh)
        x = kf[:1].float()
        return float((((x - xh) ** 2).sum(-1) / (x ** 2).sum(-1)).mean())
    mse_polar = rel_mse(pcb, kp)
    mse_scalar = rel_mse(W["kcb"], W["kc"])
    del kp
    return dict(workload="decode-128k GQA layer with PolarQuant keys: (b1, br) = (4, 2) angle codes "
                         "(382 bits, 48 B) + QJL m=128, 4-bit scalar values",
                KV_tokens_per_s=round(B * N / (ms * 1e-3), 1), ms_per_step=round(ms, 5), step_ms_spread=spread(per),
                split_kernel_ms=round(split_ms, 5), split_kernel_ms_spread=split_spread,
                bytes_per_token_head=bpt, split_GBps=round(alg / (split_ms * 1e-3) / 1e9, 1),
                frac_hbm=round(alg / (split_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                quantize_keys_ms=round(qms, 4), quantize_keys_GBps=round(qbytes / (qms * 1e-3) / 1e9, 1),
                key_rel_mse_polar=round(mse_polar, 6), key_rel_mse_scalar3=round(mse_scalar, 6))


def _exact_attention_np(q, k, v, tau):
    """float64 softmax(tau q k^T) v on the raw (bf16) inputs of one KV head;
    q [g, d], k/v [N, d] -> (logits [g, N], out [g, d])."""
    lg = tau * (q @ k.T)
    p = np.exp(lg - lg.max(axis=1, keepdims=True))
    return lg, (p / p.sum(axis=1, keepdims=True)) @ v


def bit_sweep_leg(torch, tq, synth, dev, iters, warm):
    """Bit-width sweep on the 32K GQA layer (B=32, 32 query / 4 KV heads,
    d=128, context 32768, bf16 K/V as the 128K layer, no QJL): per variant
    the decode KV tokens/s and HBM fraction of the split kernel, and the error
    of the outputs and logits against exact float64 attention on the raw
    inputs for two sampled (batch, KV head) rows."""
    B, Hq, Hkv, d, N = 32, 32, 4, 128, 32768
    g = Hq // Hkv
    tau = 1.0 / math.sqrt(d)
    k = synth.kv_gaussian(B, Hkv, N, d, 20, dtype="bf16", device=dev, channels=[3, 77, 101], factor=20.0)
    v = synth.kv_gaussian(B, Hkv, N, d, 21, dtype="bf16", device=dev, channels=[3, 77, 101], factor=20.0)
    q = synth.queries_gaussian(B, Hq, d, 22, dtype="bf16", device=dev)
    kf, vf = k.view(B * Hkv, N, d), v.view(B * Hkv, N, d)
    rows = [(0, 0), (B - 1, Hkv - 1)]
    ref = {}
    for (b, h) in rows:
        ref[(b, h)] = _exact_attention_np(q[b, h * g:(h + 1) * g].float().cpu().numpy().astype(np.float64),
                                          k[b, h].float().cpu().numpy().astype(np.float64),
                                          v[b, h].float().cpu().numpy().astype(np.float64), tau)
    out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
    logits = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    ws = torch.empty(tq.tq_attn_decode_workspace(B, Hq, Hkv, N, d), dtype=torch.uint8, device=dev)
    res = []
    for name, kb, vb, nc in [("k8v4", 8, 4, True), ("k4v4", 4, 4, True), ("k3v4", 3, 4, True),
                             ("k3v3", 3, 3, True), ("k2v2", 2, 2, True), ("k2v2 nc off", 2, 2, False)]:
        kcb = tq.Codebook(d, kb, norm_correction=nc, rot_seed=1)
        vcb = tq.Codebook(d, vb, norm_correction=nc, rot_seed=3)
        kc = tq.Codes(kcb, B * Hkv, N, tq.TQ_LAYOUT_ROW)
        vc = tq.Codes(vcb, B * Hkv, N, tq.TQ_LAYOUT_TILE32)
        tq.tq_quantize_kv(kcb, vcb, kf, vf, kc, vc)
        tq.tq_attn_decode(kcb, vcb, q, kc, vc, N, tau, out=out, logits=logits, workspace=ws)
        torch.cuda.synchronize()
        errs = dict(out_rel_l2=0.0, out_cos_min=1.0, logit_max_abs=0.0)
        for (b, h) in rows:
            lg_e, o_e = ref[(b, h)]
            o_g = out[b, h * g:(h + 1) * g].cpu().numpy().astype(np.float64)
            lg_g = logits[b, h * g:(h + 1) * g].cpu().numpy().astype(np.float64)
            errs["out_rel_l2"] = max(errs["out_rel_l2"], float(np.linalg.norm(o_g - o_e) / np.linalg.norm(o_e)))
            cos = np.sum(o_g * o_e, axis=1) / (np.linalg.norm(o_g, axis=1) * np.linalg.norm(o_e, axis=1))
            errs["out_cos_min"] = min(errs["out_cos_min"], float(cos.min()))
            errs["logit_max_abs"] = max(errs["logit_max_abs"], float(np.max(np.abs(lg_g - lg_e))))
        for _ in range(warm):
            tq.tq_attn_decode(kcb, vcb, q, kc, vc, N, tau, out=out, workspace=ws)
        torch.cuda.synchronize()
        tq.tq_profile_enable(True)
        ms, per = timed_iters(torch, lambda: tq.tq_attn_decode(kcb, vcb, q, kc, vc, N, tau, out=out,
                                                               workspace=ws), iters)
        tq.tq_profile_enable(False)
        split_ms, split_spread = kernel_spread(tq, tq.TQ_KERNEL_DECODE_SPLIT)
        bpt = kb * d // 8 + 4 + vb * d // 8 + 4
        gbs = bpt * B * Hkv * N / (split_ms * 1e-3) / 1e9
        res.append(dict(variant=name, KV_tokens_per_s=round(B * N / (ms * 1e-3), 1),
                        ms_per_decode=round(ms, 4), decode_ms_spread=spread(per),
                        split_kernel_ms=round(split_ms, 4), split_kernel_ms_spread=split_spread,
                        bytes_per_token_head=bpt, split_GBps=round(gbs, 1),
                        frac_hbm=round(gbs / HBM_PEAK_GBS, 4),
                        **{kk: round(vv, 6) for kk, vv in errs.items()}))
        del kc, vc, kcb, vcb
    del k, v
    return dict(workload="bit sweep: B=32, Hq=32, Hkv=4, d=128, context 32768, bf16 K/V N(0,1) "
                         "with channels 3/77/101 x20, no QJL; errors vs exact float64 attention "
                         "on the raw inputs of (b=0,h=0) and (b=31,h=3)",
                variants=res)


def head_dims_leg(torch, tq, synth, dev, iters, warm):
    """Decode at head dimensions other than 128 (the kernels of decode_gen.hip): the 32K
    GQA layer (B=32, 32 query / 4 KV heads, context 32768, bf16 K/V N(0,1)
    with outlier channels 3/77 x20) with 3-bit keys + QJL m=d and 4-bit
    values, for d = 64, 96 and 256, and at d = 128 with 5-bit keys (a width
    the MFMA kernels lack)."""
    B, Hq, Hkv, N = 32, 32, 4, 32768
    res = []
    for name, d, kb, km, vb in [("d64 k3+qjl v4", 64, 3, 64, 4), ("d96 k3+qjl v4", 96, 3, 96, 4),
                                ("d256 k3+qjl v4", 256, 3, 256, 4), ("d128 k5 v4", 128, 5, 0, 4)]:
        tau = 1.0 / math.sqrt(d)
        kcb = tq.Codebook(d, kb, qjl_m=km, rot_seed=1, qjl_seed=2)
        vcb = tq.Codebook(d, vb, rot_seed=3)
        kc = tq.Codes(kcb, B * Hkv, N, tq.TQ_LAYOUT_ROW)
        vc = tq.Codes(vcb, B * Hkv, N, tq.TQ_LAYOUT_TILE32)
        ch = [c for c in (3, 77) if c < d]
        k = synth.kv_gaussian(B, Hkv, N, d, 30, dtype="bf16", device=dev, channels=ch, factor=20.0)
        tq.tq_quantize_kv(kcb, None, k.view(B * Hkv, N, d), None, kc, None)
        del k
        v = synth.kv_gaussian(B, Hkv, N, d, 31, dtype="bf16", device=dev, channels=ch, factor=20.0)
        tq.tq_quantize_kv(None, vcb, None, v.view(B * Hkv, N, d), None, vc)
        del v
        q = synth.queries_gaussian(B, Hq, d, 32, dtype="bf16", device=dev)
        out = torch.empty((B, Hq, d), dtype=torch.float32, device=dev)
        ws = torch.empty(tq.tq_attn_decode_workspace(B, Hq, Hkv, N, d), dtype=torch.uint8, device=dev)
        call = lambda: tq.tq_attn_decode(kcb, vcb, q, kc, vc, N, tau, out=out, workspace=ws)
        for _ in range(warm):
            call()
        torch.cuda.synchronize()
        tq.tq_profile_enable(True)
        ms, per = timed_iters(torch, call, iters)
        tq.tq_profile_enable(False)
        split_ms, split_spread = kernel_spread(tq, tq.TQ_KERNEL_DECODE_SPLIT)
        bpt = (kb * d + km + vb * d) // 8 + 4 + (4 if km else 0) + 4
        gbs = bpt * B * Hkv * N / (split_ms * 1e-3) / 1e9
        res.append(dict(variant=name, KV_tokens_per_s=round(B * N / (ms * 1e-3), 1), ms_per_decode=round(ms, 4),
                        decode_ms_spread=spread(per), split_kernel_ms=round(split_ms, 4),
                        split_kernel_ms_spread=split_spread, bytes_per_token_head=bpt,
                        split_GBps=round(gbs, 1), frac_hbm=round(gbs / HBM_PEAK_GBS, 4)))
        del kc, vc, kcb, vcb, ws
    return dict(workload="decode at other head dimensions (any-shape MFMA kernels): B=32, Hq=32, Hkv=4, context 32768, "
                         "bf16 K/V N(0,1) with channels 3/77 (those below d) x20, bf16 queries",
                variants=res)


def vector_search_leg(torch, tq, synth, dev, iters, warm):
    """1,000,000 unit-norm vectors d=200 (256-cluster mixture), 4-bit + QJL
    m=200 codes, 1000 queries, k=10: queries/s of tq_ip_topk, MFMA
    utilisation of its score kernel and recall@10 against the exact top-10
    of the raw vectors."""
    d, n_db, nq, k, m = 200, 1_000_000, 1000, 10, 200
    db = synth.mixture_db(n_db, d, 256, seed=7, device=dev)
    qs = synth.mixture_db(nq, d, 256, seed=8, device=dev)
    cb = tq.Codebook(d, 4, qjl_m=m, rot_seed=1, qjl_seed=2)
    codes = tq.Codes(cb, 1, n_db, tq.TQ_LAYOUT_ROW)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record()
    tq.tq_quantize_kv(cb, None, db[None], None, codes, None)
    c1.record()
    torch.cuda.synchronize()
    quant_ms = c0.elapsed_time(c1)
    # the 133 MB of codes fit the 256 MB last-level cache: the timed calls
    # rotate over three copies, so each call reads its codes from HBM
    copies = [codes]
    for _ in range(2):
        c2 = tq.Codes(cb, 1, n_db, tq.TQ_LAYOUT_ROW)
        for name in ("idx", "sign", "scale", "rnorm"):
            getattr(c2, name).copy_(getattr(codes, name))
        copies.append(c2)
    ws = torch.empty(tq.tq_ip_topk_workspace(nq, n_db, k, d), dtype=torch.uint8, device=dev)
    gi = torch.empty((nq, k), dtype=torch.int64, device=dev)
    gs = torch.empty((nq, k), dtype=torch.float32, device=dev)
    ctr = [0]

    def call():
        c = copies[ctr[0] % len(copies)]
        ctr[0] += 1
        tq.tq_ip_topk(cb, qs, c, n_db, k, out_idx=gi, out_score=gs, workspace=ws)
    for _ in range(warm):
        call()
    torch.cuda.synchronize()
    tq.tq_profile_enable(True)
    ms, per = timed_iters(torch, call, iters)
    tq.tq_profile_enable(False)
    score_ms, score_spread = kernel_spread(tq, tq.TQ_KERNEL_TOPK)
    n_scan = tq.tq_ip_topk_scan_count(cb, ws, nq, n_db, k)
    # the last call's results are those of the first copy's codes (identical)
    # MFMA work the score kernel issues (fp16 16x16x32, 16384 flop each): per
    # 16-query block (queries padded to whole workgroups of 256) and 16-row
    # tile, dp/16 centroid MFMAs (hi and lo parts) and ceil(m/32) sign MFMAs,
    # over every tile and, in the sample pass, every 64th tile
    dp = (d + 31) // 32 * 32
    nqp = (nq + 255) // 256 * 256
    n_tiles = (n_db + 15) // 16
    tiles = n_tiles + (n_tiles // 64 if n_tiles >= 64 * 256 else 0)
    n_mfma = (nqp // 16) * tiles * (dp // 16 + (m + 31) // 32)
    mfma_tflops = n_mfma * 16384 / (score_ms * 1e-3) / 1e12
    useful = nq * n_db * (2 * d + 2 * m)
    # exact top-10 of the raw vectors (fp32 matmul, chunked) for recall
    ex_s = torch.full((nq, k), -float("inf"), device=dev)
    ex_i = torch.zeros((nq, k), dtype=torch.int64, device=dev)
    for s in range(0, n_db, 250000):
        sc = qs @ db[s:s + 250000].T
        cs, ci = torch.topk(sc, k, dim=1)
        allv = torch.cat([ex_s, cs], dim=1)
        alli = torch.cat([ex_i, ci + s], dim=1)
        ex_s, pos = torch.topk(allv, k, dim=1)
        ex_i = torch.gather(alli, 1, pos)
    hit = (gi[:, :, None] == ex_i[:, None, :]).any(dim=2).sum().item()
    hit1 = (gi == ex_i[:, :1]).any(dim=1).sum().item()
    del db, codes, copies
    return dict(workload="vector search: 1e6 unit-norm vectors d=200 (256-cluster mixture), "
                         "4-bit + QJL m=200, 1000 queries, top-10; timed calls rotate over 3 copies "
                         "of the codes (399 MB > the 256 MB last-level cache)",
                queries_per_s=round(nq / (ms * 1e-3), 1), ms_per_call=round(ms, 4),
                call_ms_spread=spread(per), score_kernel_ms=round(score_ms, 4),
                score_kernel_ms_spread=score_spread,
                mfma_TFLOPs=round(mfma_tflops, 1),
                mfma_frac_fp16_peak=round(mfma_tflops / 2500.0, 4),
                useful_TFLOPs=round(useful / (ms * 1e-3) / 1e12, 1),
                exact_scan_queries=n_scan,
                recall_10_at_10=round(hit / (nq * k), 4),
                recall_1_at_10=round(hit1 / nq, 4),
                quantize_db_ms=round(quant_ms, 3))


def host_info():
    """Host CPU model and logical core count (the oracle's machine)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count()
    return dict(host_nproc=os.cpu_count(), host_cpus_available=avail, cpu_model=model)


def cpu_baseline(torch, O, W, budget_s=10.0):
    """float64 oracle: per sampled (batch, KV head) pair, quantize the step's
    new vectors and decode its 8 query heads over the full context; pairs are
    taken in a fixed shuffled order until about budget_s of timed CPU work."""
    threads = _oracle_threads()
    B, Hkv, Hq, d, N = W["B"], W["Hkv"], W["Hq"], W["d"], W["N"]
    g = Hq // Hkv
    okc = O.Codebook(d, 3, qjl_m=128, rot_seed=1, qjl_seed=2)
    ovc = O.Codebook(d, 4, rot_seed=3)
    order = np.random.default_rng(123).permutation(B * Hkv)
    pairs = [(int(x) // Hkv, int(x) % Hkv) for x in order]
    q64 = W["q"].float().cpu().numpy().astype(np.float64)
    t_total = 0.0
    cpu_total = 0.0
    done = 0
    for (b, h) in pairs:
        if t_total >= budget_s:
            break
        done += 1
        k64 = W["k"][b, h].float().cpu().numpy().astype(np.float64)
        v64 = W["v"][b, h].float().cpu().numpy().astype(np.float64)
        rk = O.quantize(okc, k64[:N - 1])          # cache build (untimed)
        rv = O.quantize(ovc, v64[:N - 1])
        t0 = time.perf_counter()
        p0 = time.process_time()
        nk = O.quantize(okc, k64[N - 1:])
        nv = O.quantize(ovc, v64[N - 1:])
        kd = {n: np.concatenate([rk[n], nk[n]])[None, None] for n in ("idx", "scale", "sign", "rnorm")}
        vd = {n: np.concatenate([rv[n], nv[n]])[None, None] for n in ("idx", "scale")}
        O.attn_decode(okc, ovc, q64[b:b + 1, h * g:(h + 1) * g], kd, vd, W["tau"])
        t_total += time.perf_counter() - t0
        cpu_total += time.process_time() - p0
    kv_tokens = done * N / Hkv               # each pair is 1/Hkv of a batch row
    return dict(value=round(kv_tokens / t_total, 1), unit="KV tokens/s", cores=int(threads),
                kind="oracle", **host_info(),
                cores_busy=round(cpu_total / t_total, 2),
                cores_note="cores: the BLAS threads the oracle's numpy products may use; cores_busy: "
                           "process CPU time over wall time in the timed region",
                sample=f"{done} of {B * Hkv} (batch, KV head) pairs of the decode-128k layer at "
                       f"full context {N}, all {g} query heads each, float64; "
                       f"{t_total:.1f} s of CPU time, scaled to KV tokens/s")


def _oracle_threads():
    try:
        from threadpoolctl import threadpool_info
        return int(max([t.get("num_threads", 1) for t in threadpool_info()] or [1]))
    except Exception:
        return 1


def cpu_oracle_legs(O, synth, budget_s=2.0):
    """float64 oracle rates beside the secondary legs, each on a bounded
    sample of the leg's workload (repeated until ~budget_s of CPU time):
    quantize and dequantize of 32768 quantize-layer vectors (4-bit, d=128,
    outlier channels x15), and top-k (k=10) of 20 queries against a
    65536-vector sample of the d=200 search database (4-bit + QJL m=200),
    scaled to the 1e6-vector database."""
    threads = _oracle_threads()
    d = 128
    chk = synth.outlier_channels(10, 8, d, 4)
    x = synth.kv_gaussian(1, 8, 4096, d, 10, dtype="bf16", device="cpu", per_head_channels=chk, factor=15.0)
    x64 = x.float().numpy().astype(np.float64).reshape(-1, d)
    cb = O.Codebook(d, 4, rot_seed=1)

    def rate(fn):
        t, n = 0.0, 0
        while t < budget_s:
            t0 = time.perf_counter()
            fn()
            t += time.perf_counter() - t0
            n += 1
        return n, t
    r = O.quantize(cb, x64)
    nq_, tq_ = rate(lambda: O.quantize(cb, x64))
    nd_, td_ = rate(lambda: O.dequantize(cb, r["idx"], r["scale"]))
    vec_q = nq_ * len(x64) / tq_
    vec_d = nd_ * len(x64) / td_
    out = {}
    out["quantize"] = dict(value=round(vec_q * 324 / 1e9, 4), unit="GB/s", vectors_per_s=round(vec_q, 1),
                           cores=threads, kind="oracle",
                           sample=f"{len(x64)} quantize-layer vectors x {nq_} passes, float64, {tq_:.1f} s")
    out["dequantize"] = dict(value=round(vec_d * 324 / 1e9, 4), unit="GB/s", vectors_per_s=round(vec_d, 1),
                             cores=threads, kind="oracle",
                             sample=f"{len(x64)} quantize-layer vectors x {nd_} passes, float64, {td_:.1f} s")
    cb2 = O.Codebook(200, 4, qjl_m=200, rot_seed=1, qjl_seed=2)
    n_s, n_q = 65536, 20
    db = synth.mixture_db(n_s, 200, 256, seed=7).double().numpy()
    qs = synth.mixture_db(n_q, 200, 256, seed=8).double().numpy()
    codes = O.quantize(cb2, db)
    nt_, tt_ = rate(lambda: O.ip_topk(cb2, qs, codes, 10))
    qps = nt_ * n_q / tt_ * n_s / 1e6
    out["vector_search"] = dict(value=round(qps, 2), unit="queries/s", cores=threads, kind="oracle",
                                sample=f"{n_q} queries x {n_s} database vectors x {nt_} passes, float64, "
                                       f"{tt_:.1f} s, scaled to 1e6 vectors")
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the library has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    import torch
    import synth
    import kv_cache_vector_quantize_amd as tq
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    tq.lib()
    dev = "cuda"
    print("[bench] building decode-128k workload", file=sys.stderr, flush=True)
    W = decode_workload(torch, tq, synth, dev)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        W["step"]()
    torch.cuda.synchronize()
    print("[bench] timing", args.steps, "steps", file=sys.stderr, flush=True)
    tq.tq_profile_enable(True)
    ms_step, step_per = timed_iters(torch, W["step"], args.steps)
    tq.tq_profile_enable(False)
    split_avg, split_spread = kernel_spread(tq, tq.TQ_KERNEL_DECODE_SPLIT)
    B, Hkv, N = W["B"], W["Hkv"], W["N"]
    value = B * N / (ms_step * 1e-3)
    alg_bytes = W["bytes_per_token_head"] * B * Hkv * N
    achieved = alg_bytes / (split_avg * 1e-3) / 1e9
    res = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "KV tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "step_ms_spread": spread(step_per),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": W["cfg"],
        "roofline": {
            "bound": "hbm",
            "kernel": "decode split (k_split<3,4,qjl>)",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": split_traffic(),
            "kernel_ms": round(split_avg, 5),
            "kernel_ms_spread": split_spread,
            "algorithmic_bytes_per_launch": int(alg_bytes),
        },
    }
    if not args.no_paged:
        print("[bench] paged-cache leg", file=sys.stderr, flush=True)
        res["paged"] = paged_leg(torch, tq, W, iters=args.steps, warm=args.warmup)
    if not args.no_polar:
        print("[bench] polar-keys leg", file=sys.stderr, flush=True)
        res["polar"] = polar_leg(torch, tq, W, iters=args.steps, warm=args.warmup)
        res["polar"]["scalar_KV_tokens_per_s"] = res["value"]
        res["polar"]["scalar_split_kernel_ms"] = res["roofline"]["kernel_ms"]
    if not args.no_quantize:
        print("[bench] quantize leg", file=sys.stderr, flush=True)
        res["quantize"] = quantize_leg(torch, tq, synth, dev, iters=args.steps, warm=args.warmup)
        res["quantize"]["sketched_keys"] = sketch_build_leg(torch, tq, W, iters=max(5, args.steps // 5),
                                                            warm=2)
    if not args.no_sweep:
        print("[bench] bit-width sweep leg", file=sys.stderr, flush=True)
        res["bit_sweep"] = bit_sweep_leg(torch, tq, synth, dev, iters=args.steps, warm=args.warmup)
    if not args.no_dims:
        print("[bench] head-dimension leg", file=sys.stderr, flush=True)
        res["head_dims"] = head_dims_leg(torch, tq, synth, dev, iters=args.steps, warm=args.warmup)
    if not args.no_search:
        print("[bench] vector-search leg", file=sys.stderr, flush=True)
        res["vector_search"] = vector_search_leg(torch, tq, synth, dev, iters=max(10, args.steps // 2),
                                                 warm=max(2, args.warmup // 2))
    # codebook construction (host, float64 Lloyd-Max + QR + sketch, then the
    # device tables), once per (d, bits, m, seeds) in a serving process
    cbt = {}
    for name, (d_, b_, m_) in {"d128_b3_m128": (128, 3, 128), "d128_b4": (128, 4, 0),
                              "d200_b4_m200": (200, 4, 200)}.items():
        t0 = time.perf_counter()
        cb_ = tq.Codebook(d_, b_, qjl_m=m_, rot_seed=11, qjl_seed=12)
        torch.cuda.synchronize()
        cbt[name] = round((time.perf_counter() - t0) * 1e3, 2)
        del cb_
    res["codebook_build_ms"] = cbt
    # achievable device-to-device copy rate of this machine (1 GiB read + 1 GiB
    # written per copy); with --calib-copy it is also the counter calibration
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    n_copy = 3
    c0.record()
    for _ in range(n_copy):
        dst.copy_(src)
    c1.record()
    torch.cuda.synchronize()
    res["copy_GBps"] = round(2 * (1 << 30) * n_copy / (c0.elapsed_time(c1) * 1e-3) / 1e9, 1)
    del dst
    # streaming-read ceiling: a kernel that only reads 1 GiB (median of 20)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    for _ in range(3):
        tq.tq_stream_read(src, sink)
    _, rper = timed_iters(torch, lambda: tq.tq_stream_read(src, sink), 20)
    rmed = float(np.median(rper))
    res["read_GBps"] = round((1 << 30) / (rmed * 1e-3) / 1e9, 1)
    res["read_ms_spread"] = spread(rper)
    res["roofline"]["frac_of_read_ceiling"] = round(res["roofline"]["achieved"] / res["read_GBps"], 4)
    # streaming-write ceiling: a kernel that only writes 1 GiB (median of 20)
    for _ in range(3):
        tq.tq_stream_write(src, 0)
    _, wper = timed_iters(torch, lambda: tq.tq_stream_write(src, 0), 20)
    wmed = float(np.median(wper))
    res["write_GBps"] = round((1 << 30) / (wmed * 1e-3) / 1e9, 1)
    res["write_ms_spread"] = spread(wper)
    # the quantize and dequantize calls against the time their reads and
    # writes take at the streaming ceilings
    if "quantize" in res:
        for leg in (res["quantize"], res["quantize"]["dequantize"]):
            floor_ms = (leg["read_bytes_per_call"] / (res["read_GBps"] * 1e9)
                        + leg["write_bytes_per_call"] / (res["write_GBps"] * 1e9)) * 1e3
            leg["stream_floor_ms"] = round(floor_ms, 4)
            leg["frac_of_stream_ceiling"] = round(floor_ms / leg["ms_per_call"], 4)
    del src, sink
    if not args.no_ab:
        print("[bench] dequantize-then-attend leg", file=sys.stderr, flush=True)
        res["dequant_then_attend"] = dequant_attend_leg(torch, tq, W, iters=max(3, args.steps // 5),
                                                        warm=max(1, args.warmup // 5), copy_gbps=res["copy_GBps"])
    if not args.no_cpu_baseline:
        import oracle as O
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        res["cpu_baseline"] = cpu_baseline(torch, O, W)
        legs = cpu_oracle_legs(O, synth)
        if "quantize" in res:
            res["quantize"]["cpu_oracle"] = legs["quantize"]
            res["quantize"]["dequantize"]["cpu_oracle"] = legs["dequantize"]
        if "vector_search" in res:
            res["vector_search"]["cpu_oracle"] = legs["vector_search"]
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
