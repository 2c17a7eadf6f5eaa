"""Seeded synthetic inputs for the MoE-layer workloads.

This module only draws random inputs; it holds none of the layer's
arithmetic, so both the HIP path and the CPU oracle can be fed from it
without sharing any of the method's code.

Recipe (every workload): one ``torch.Generator`` on the requested device,
seeded with the workload's seed, draws in this order
  x  [S,d]    ~ N(0,1)
  Wg [E,d]    ~ N(0, 1/d)                (fp32 router weight, stored [E,d])
  W1 [E,h,d]  ~ N(0, 1/d)    drawn expert by expert
  W2 [E,d,h]  ~ N(0, 1/h)    drawn expert by expert
as fp32 normals scaled by the standard deviation, then rounded to bf16
(round to nearest even) for bf16 workloads.  N(0,v) names the variance.
The skewed workload adds a router bias b_j = ln p_j with p_j proportional to
j^-1.2 over j = 1..E (a Zipf law), so expert 0 is the hottest.  The tiny fp32
workload passes explicit all-zero expert biases; the others pass none.

Values depend on (seed, device type): a CPU draw and a GPU draw differ, but
each side of a comparison always receives the same tensors.
"""
from __future__ import annotations

import dataclasses
import math

import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    S: int                  # tokens on this device
    d: int                  # model width
    h: int                  # expert hidden width
    E: int                  # experts
    k: int                  # experts per token
    capacity_factor: float
    dtype: str              # "f32" or "bf16": x, expert weights, buffers, y
    seed: int
    gate_bias: str | None = None    # None or "zipf1.2"
    ffn_bias: str | None = None     # None or "zeros"
    dropless: bool = False          # no capacity limit, compact expert segments
    reroute: bool = False           # dropped assignments offered to next-ranked experts

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("tiny_fp32", S=256, d=64, h=128, E=8, k=2, capacity_factor=1.25,
                 dtype="f32", seed=0, ffn_bias="zeros"),
        Workload("balanced_bf16", S=16384, d=1024, h=4096, E=128, k=2, capacity_factor=2.0,
                 dtype="bf16", seed=1),
        Workload("skewed_bf16", S=16384, d=1024, h=4096, E=128, k=2, capacity_factor=1.0,
                 dtype="bf16", seed=2, gate_bias="zipf1.2"),
        Workload("large_bf16", S=65536, d=2048, h=8192, E=64, k=2, capacity_factor=1.25,
                 dtype="bf16", seed=3),
        Workload("deepseek_bf16", S=8192, d=7168, h=2048, E=256, k=8, capacity_factor=1.5,
                 dtype="bf16", seed=4),
    ]
}
ORDER = list(WORKLOADS)


def get(name: str) -> Workload:
    return WORKLOADS[name]


def zipf_log_bias(E: int, alpha: float = 1.2) -> torch.Tensor:
    """b_j = ln p_j, p_j = (j+1)^-alpha / sum_i (i+1)^-alpha, j = 0..E-1 (fp32)."""
    ranks = torch.arange(1, E + 1, dtype=torch.float64)
    p = ranks.pow(-alpha)
    p = p / p.sum()
    return p.log().to(torch.float32)


def generate(w: Workload, device="cpu") -> dict:
    """Draw the workload's inputs on ``device``.  Returns a dict of tensors:
    x, wg, bg (or None), w1, b1 (or None), w2, b2 (or None)."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(w.seed)
    dt = w.torch_dtype

    def normal(shape, std):
        t = torch.randn(shape, generator=g, device=dev, dtype=torch.float32)
        if std != 1.0:
            t.mul_(std)
        return t.to(dt) if dt != torch.float32 else t

    x = normal((w.S, w.d), 1.0)
    wg = torch.randn((w.E, w.d), generator=g, device=dev, dtype=torch.float32).mul_(w.d ** -0.5)
    w1 = torch.empty((w.E, w.h, w.d), device=dev, dtype=dt)
    for e in range(w.E):
        w1[e] = normal((w.h, w.d), w.d ** -0.5)
    w2 = torch.empty((w.E, w.d, w.h), device=dev, dtype=dt)
    for e in range(w.E):
        w2[e] = normal((w.d, w.h), w.h ** -0.5)

    bg = None
    if w.gate_bias == "zipf1.2":
        bg = zipf_log_bias(w.E, 1.2).to(dev)
    elif w.gate_bias is not None:
        raise ValueError(w.gate_bias)
    b1 = b2 = None
    if w.ffn_bias == "zeros":
        b1 = torch.zeros((w.E, w.h), device=dev, dtype=dt)
        b2 = torch.zeros((w.E, w.d), device=dev, dtype=dt)
    elif w.ffn_bias is not None:
        raise ValueError(w.ffn_bias)
    return dict(x=x, wg=wg, bg=bg, w1=w1, b1=b1, w2=w2, b2=b2)


@dataclasses.dataclass(frozen=True)
class EPShare:
    """One GPU's share of an expert-parallel layer: `sources` GPUs of S tokens
    each route k of E_total experts; this GPU holds experts 0..E_local-1 and
    receives every row routed to them."""
    name: str
    sources: int
    S: int
    E_total: int
    k: int
    E_local: int
    d: int
    h: int
    seed: int


# DeepSeek-R1-shaped layout: 256 routed experts over 8 GPUs, 32 per GPU
EP_SHARES = {
    s.name: s
    for s in [EPShare("deepseek_ep8_share", sources=8, S=8192, E_total=256, k=8, E_local=32,
                      d=7168, h=2048, seed=5)]
}


def ep_share_counts(sh: EPShare):
    """Rows each local expert receives (int64 [E_local]).  Every token of every
    source picks k distinct experts uniformly at random (the balanced,
    uniform-router case); no capacity limit."""
    import numpy as np
    rng = np.random.default_rng(sh.seed)
    counts = np.zeros(sh.E_local, np.int64)
    for _ in range(sh.sources):
        u = rng.random((sh.S, sh.E_total), dtype=np.float32)
        top = np.argpartition(u, -sh.k, axis=1)[:, -sh.k:]
        counts += np.bincount(top.ravel(), minlength=sh.E_total)[:sh.E_local]
    return counts


def generate_ep_share(sh: EPShare, rows: int, device="cpu") -> dict:
    """Received rows xd [rows, d] ~ N(0,1) and the local experts' weights
    W1 [E_local,h,d] ~ N(0,1/d), W2 [E_local,d,h] ~ N(0,1/h), all bf16."""
    dev = torch.device(device)
    g = torch.Generator(device=dev)
    g.manual_seed(sh.seed)
    bf = torch.bfloat16
    xd = torch.randn((rows, sh.d), generator=g, device=dev).to(bf)
    w1 = torch.empty((sh.E_local, sh.h, sh.d), device=dev, dtype=bf)
    w2 = torch.empty((sh.E_local, sh.d, sh.h), device=dev, dtype=bf)
    for e in range(sh.E_local):
        w1[e] = torch.randn((sh.h, sh.d), generator=g, device=dev).mul_(sh.d ** -0.5).to(bf)
        w2[e] = torch.randn((sh.d, sh.h), generator=g, device=dev).mul_(sh.h ** -0.5).to(bf)
    return dict(xd=xd, w1=w1, w2=w2)


def to_numpy(t: torch.Tensor | None):
    """Host numpy view of a tensor; bf16 becomes its uint16 bit patterns."""
    if t is None:
        return None
    t = t.detach().to("cpu").contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view("uint16")
    return t.numpy()


def bf16_bits_to_f32(a):
    """Exact widening of uint16 bf16 bit patterns to float32 (numpy)."""
    import numpy as np
    return (np.asarray(a, dtype=np.uint32) << 16).view(np.float32)


def stats_std(w: Workload) -> dict:
    """Standard deviations used by the draw, for documentation and tests."""
    return dict(x=1.0, wg=1 / math.sqrt(w.d), w1=1 / math.sqrt(w.d), w2=1 / math.sqrt(w.h))
