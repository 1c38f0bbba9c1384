"""Seeded synthetic workloads (random-number recipes only).

Every generator is a pure function of its seed and shape.  Two back ends
exist and they do NOT produce the same numbers:

* ``device="cpu"``: numpy ``default_rng`` streams, float64 normals, scaled,
  then rounded to the requested dtype (round-to-nearest-even).  Large tensors
  are drawn per (batch, head) slice from ``default_rng([seed, b, h])`` so any
  slice can be regenerated on its own.
* any other device: a ``torch.Generator`` on that device seeded with ``seed``
  draws float32 normals in place, slice by slice, which keeps multi-GB
  workloads off the host.

A test always compares the GPU library and the oracle on the *same* tensor
(the oracle reads device inputs back to the host), so the two back ends never
need to agree with each other.
"""
from __future__ import annotations

import numpy as np

_TORCH = None


def _torch():
    global _TORCH
    if _TORCH is None:
        import torch  # local import: the CPU oracle path does not need torch

        _TORCH = torch
    return _TORCH


def outlier_channels(seed: int, n_heads: int, d: int, count: int) -> np.ndarray:
    """``count`` distinct channel ids per head, int64 [n_heads, count]."""
    out = np.empty((n_heads, count), dtype=np.int64)
    for h in range(n_heads):
        rng = np.random.default_rng([seed, 7919, h])
        out[h] = np.sort(rng.choice(d, size=count, replace=False))
    return out


def tiny_case(seed: int = 0, n: int = 4096, d: int = 128, n_q: int = 8,
              channels=(3, 77, 101), factor: float = 20.0):
    """One head: K [n,d], V [n,d], Q [n_q,d] float32, drawn N(0,1) in the
    order K, V, Q from ``default_rng(seed)``; ``channels`` of K and V are
    multiplied by ``factor`` (outlier channels)."""
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((n, d))
    v = rng.standard_normal((n, d))
    q = rng.standard_normal((n_q, d))
    ch = list(channels)
    k[:, ch] *= factor
    v[:, ch] *= factor
    return k.astype(np.float32), v.astype(np.float32), q.astype(np.float32)


def _np_to_dtype(a64: np.ndarray, dtype: str):
    torch = _torch()
    t = torch.from_numpy(a64.astype(np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    elif dtype == "f16":
        t = t.to(torch.float16)
    elif dtype != "f32":
        raise ValueError(dtype)
    return t


def kv_gaussian(B: int, H: int, N: int, d: int, seed: int, *, dtype: str = "bf16",
                device: str = "cpu", channels=None, factor: float = 1.0,
                per_head_channels: np.ndarray | None = None):
    """Gaussian K or V tensor [B, H, N, d] with outlier channels.

    ``channels``: one fixed list of channel ids scaled by ``factor`` in every
    head; ``per_head_channels``: int array [H, c] of channel ids per head
    (e.g. from :func:`outlier_channels`).  Returns a torch tensor of ``dtype``
    on ``device``.
    """
    torch = _torch()
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dtype]
    # channel ids are checked here, on the host: a device index_put with an
    # id past d would access memory out of bounds
    ids = list(channels) if channels is not None else []
    if per_head_channels is not None:
        ids += [int(c) for c in np.asarray(per_head_channels).reshape(-1)]
    if any(c < 0 or c >= d for c in ids):
        raise ValueError(f"outlier channel ids must lie in [0, {d})")
    out = torch.empty((B, H, N, d), dtype=tdt, device=device)
    if device == "cpu":
        for b in range(B):
            for h in range(H):
                rng = np.random.default_rng([seed, b, h])
                x = rng.standard_normal((N, d))
                if channels is not None:
                    x[:, list(channels)] *= factor
                if per_head_channels is not None:
                    x[:, list(per_head_channels[h])] *= factor
                out[b, h] = _np_to_dtype(x, dtype)
        return out
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    scale = torch.ones((H, d), dtype=torch.float32, device=device)
    if channels is not None:
        scale[:, list(channels)] = factor
    if per_head_channels is not None:
        for h in range(H):
            scale[h, list(per_head_channels[h])] = factor
    tmp = torch.empty((N, d), dtype=torch.float32, device=device)
    for b in range(B):
        for h in range(H):
            tmp.normal_(generator=gen)
            tmp.mul_(scale[h])
            out[b, h].copy_(tmp)
    return out


def queries_gaussian(B: int, Hq: int, d: int, seed: int, *, dtype: str = "bf16",
                     device: str = "cpu"):
    """Decode queries [B, Hq, d] ~ N(0, 1)."""
    torch = _torch()
    if device == "cpu":
        rng = np.random.default_rng([seed, 31337])
        return _np_to_dtype(rng.standard_normal((B, Hq, d)), dtype)
    tdt = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dtype]
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed) + 31337)
    q = torch.empty((B, Hq, d), dtype=torch.float32, device=device)
    q.normal_(generator=gen)
    return q.to(tdt)


def mixture_db(n: int, d: int, n_clusters: int, seed: int, *, spread: float = 0.5,
               device: str = "cpu", centers_seed: int = 0):
    """Unit-normalised Gaussian-mixture vectors [n, d] float32.

    Centres mu_c = g/|g| with g ~ N(0, I_d) (from ``centers_seed``); each
    vector picks a centre uniformly, adds ``spread``*e/sqrt(d) with
    e ~ N(0, I_d), and is normalised to unit length.  Database and queries use
    the same centres and different ``seed``.
    """
    torch = _torch()
    crng = np.random.default_rng([centers_seed, 4242])
    cen = crng.standard_normal((n_clusters, d))
    cen /= np.linalg.norm(cen, axis=1, keepdims=True)
    if device == "cpu":
        rng = np.random.default_rng([seed, 4243])
        lab = rng.integers(0, n_clusters, size=n)
        x = cen[lab] + spread * rng.standard_normal((n, d)) / np.sqrt(d)
        x /= np.linalg.norm(x, axis=1, keepdims=True)
        return torch.from_numpy(x.astype(np.float32))
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed) + 4243)
    cen_t = torch.from_numpy(cen.astype(np.float32)).to(device)
    out = torch.empty((n, d), dtype=torch.float32, device=device)
    step = 1 << 18
    for s in range(0, n, step):
        e = min(n, s + step)
        lab = torch.randint(0, n_clusters, (e - s,), generator=gen, device=device)
        x = torch.empty((e - s, d), dtype=torch.float32, device=device).normal_(generator=gen)
        x = cen_t[lab] + (spread / np.sqrt(d)) * x
        out[s:e] = x / x.norm(dim=1, keepdim=True)
    return out
