"""Whole-layer parity on seeded random shapes.

Each case draws a layer shape from a fixed seed: token count, model and
hidden widths (ragged against the 256-wide GEMM tiles and the 64-wide
k-tiles, including single and odd k-tile counts), expert count (above 256
too, where every token takes the wave-per-token router), top-k, capacity
factor, activation dtype, routing mode (capacity, dropless or re-routing),
the Zipf gate bias and non-zero expert biases.  Every output is compared
with the oracle at every slot (routing, slots and drops bit-exact, each row
of the expert outputs and of y within three times the dtype's bar), with
and without the dispatch buffer, so the expert GEMMs run both their
gathered and their buffered A rows, both m-tile heights and the strip rows,
and the near-tie router sees many shapes.  The shapes are listed in the
test ids.
"""
import numpy as np
import pytest
import torch

import moe_workloads as mw
from parity_util import check_layer, run_layer

pytestmark = pytest.mark.gpu


def _draw(seed: int) -> tuple[mw.Workload, bool, bool]:
    rng = np.random.default_rng(1000 + seed)
    bf16 = seed % 5 != 4
    q = 64 if bf16 else 4
    d = int(q * rng.integers(1, 9 if bf16 else 65))
    h = int(q * rng.integers(1, 11 if bf16 else 97))
    E = int(rng.choice([1, 2, 3, 7, 16, 33, 64, 130, 256, 300]))
    k = int(rng.integers(1, min(8, E) + 1))
    S = int(rng.integers(1, 2500))
    cf = float(rng.choice([0.5, 1.0, 1.25, 2.0]))
    mode = rng.choice(["capacity", "dropless", "reroute"], p=[0.5, 0.25, 0.25])
    if mode == "reroute" and k >= E:
        mode = "capacity"
    w = mw.Workload(f"rand{seed}", S=S, d=d, h=h, E=E, k=k, capacity_factor=cf,
                    dtype="bf16" if bf16 else "f32", seed=500 + seed,
                    gate_bias="zipf1.2" if rng.random() < 0.3 else None,
                    dropless=mode == "dropless", reroute=mode == "reroute")
    return w, bool(rng.random() < 0.5), bool(rng.random() < 0.5)


CASES = [_draw(i) for i in range(32)]


def _id(case):
    w, bias, buf = case
    mode = "dropless" if w.dropless else ("reroute" if w.reroute else "capacity")
    return (f"{w.name}-{w.dtype}-S{w.S}-d{w.d}-h{w.h}-E{w.E}-k{w.k}-cf{w.capacity_factor}-{mode}"
            f"{'-zipf' if w.gate_bias else ''}{'-bias' if bias else ''}{'-buf' if buf else ''}")


@pytest.mark.parametrize("case", CASES, ids=[_id(c) for c in CASES])
def test_random_shape_layer_parity(case):
    w, ffn_bias, dispatch_buffer = case
    print(f"\n[random] {_id(case)}", flush=True)
    inputs = mw.generate(w, "cuda")
    if ffn_bias:
        g = torch.Generator(device="cuda").manual_seed(w.seed)
        dt = w.torch_dtype
        inputs["b1"] = (0.2 * torch.randn((w.E, w.h), generator=g, device="cuda")).to(dt)
        inputs["b2"] = (0.2 * torch.randn((w.E, w.d), generator=g, device="cuda")).to(dt)
    inputs, layer = run_layer(w, inputs, dispatch_buffer=dispatch_buffer)
    rep = check_layer(w, inputs, layer, full=True)
    print("  " + " ".join(f"{k}={v:.4g}" if isinstance(v, float) else f"{k}={v}"
                          for k, v in rep.items()), flush=True)
