"""GPU parity of overflow re-routing against the CPU oracle.

With re-routing, an assignment that overflows its expert's capacity is
offered to the token's next-ranked experts (the j-th dropped rank of a token
to its (k+j)-th ranked expert) and taken while that expert has room, after
every real assignment, virtual rank by virtual rank, tokens in order.  The
layer's topk_idx then names the serving expert, slot its row there, and
counts gains row k (accepted offers per expert).  Bars as for the capacity
layer: serving indices, rows and counts bit-exact given the GPU's fp32
logits; dispatch rows bit copies; expert outputs and y within relative
Frobenius error 1e-5 (fp32) / 1e-2 (bf16); losses within 1e-5 (unchanged by
re-routing: they belong to the router's own top-k).
"""
import numpy as np
import pytest
import torch

import moe_workloads as mw
import oracle
import sparse_moe_layer_wg_amd as moe
from parity_util import check_layer, run_layer
from sparse_moe_layer_wg_amd.layer import MoELayer
from test_gpu_backward import _with_biases, check_backward, run_backward

pytestmark = pytest.mark.gpu


def _print(name, rep):
    print(f"\n[{name}] " + " ".join(f"{k}={v:.4g}" if isinstance(v, float) else f"{k}={v}"
                                   for k, v in rep.items()), flush=True)


REROUTE_MID = [
    # zipf gate bias: hot experts overflow, cold ones have room for the offers
    mw.Workload("rr_skew_bf16", S=1000, d=256, h=384, E=16, k=2, capacity_factor=1.0,
                dtype="bf16", seed=61, gate_bias="zipf1.2", reroute=True),
    mw.Workload("rr_top8_bf16", S=700, d=192, h=320, E=40, k=8, capacity_factor=0.75,
                dtype="bf16", seed=62, gate_bias="zipf1.2", reroute=True),
    mw.Workload("rr_f32", S=333, d=96, h=160, E=6, k=2, capacity_factor=0.8, dtype="f32",
                seed=63, gate_bias="zipf1.2", reroute=True),
    # E = 80 > 64 experts: the ranking spans two lanes per expert slot
    mw.Workload("rr_e80_bf16", S=900, d=128, h=256, E=80, k=2, capacity_factor=1.0,
                dtype="bf16", seed=64, gate_bias="zipf1.2", reroute=True),
]


@pytest.mark.parametrize("w", REROUTE_MID, ids=lambda w: w.name)
@pytest.mark.parametrize("dispatch_buffer", [True, False], ids=["xd", "fused"])
def test_reroute_layer_full_parity(w, dispatch_buffer):
    """Whole moe_layer_forward with re-routing against the oracle at every
    row; the workloads overflow, so offers are made, taken and refused."""
    print(f"\n[reroute] {w} xd={dispatch_buffer}", flush=True)
    inputs, layer = run_layer(w, dispatch_buffer=dispatch_buffer)
    assert tuple(layer.counts.shape) == (w.k + 1, w.E)
    rep = check_layer(w, inputs, layer, full=True)
    r = oracle.route(layer.logits.cpu().numpy(), w.k, layer.C, True)
    rep["offers_refused"] = int((r["slot"] < 0).sum())
    _print(w.name, rep)
    assert rep["rerouted"] > 0


@pytest.mark.parametrize("w", REROUTE_MID[:2], ids=lambda w: w.name)
def test_reroute_moves_only_dropped_assignments(w):
    """Against the same layer without re-routing: kept assignments keep
    their expert and row, the losses and weights are the same, counts rows
    0..k-1 are the same, every re-routed assignment was dropped before, and
    no expert goes over its capacity."""
    inputs, rr = run_layer(w, dispatch_buffer=False)
    _, plain = run_layer(w.with_(reroute=False), inputs=inputs, dispatch_buffer=False)
    kept = plain.slot >= 0
    assert torch.equal(rr.topk_idx[kept], plain.topk_idx[kept])
    assert torch.equal(rr.slot[kept], plain.slot[kept])
    assert torch.equal(rr.losses, plain.losses) and torch.equal(rr.topk_w, plain.topk_w)
    assert torch.equal(rr.counts[:w.k], plain.counts)
    moved = rr.topk_idx != plain.topk_idx
    assert not torch.any(moved & kept)
    assert torch.equal(moved, (rr.slot >= 0) & ~kept)
    occ = oracle.occupancy(rr.counts.cpu().numpy(), rr.C, w.k)
    assert (occ <= rr.C).all()
    assert int(rr.counts[w.k].sum()) == int(moved.sum())


@pytest.mark.parametrize("w", [REROUTE_MID[0], REROUTE_MID[2]], ids=lambda w: w.name)
def test_reroute_stage_entry_points(w):
    """moe_gate, moe_dispatch, moe_expert_ffn and moe_combine called one by
    one with re-routing reproduce moe_layer_forward bit for bit."""
    print(f"\n[rr stages] {w}", flush=True)
    inputs, ref = run_layer(w, dispatch_buffer=True)
    cfg = ref.cfg
    at = w.torch_dtype
    S, d, E, k, C = w.S, w.d, w.E, w.k, ref.C
    dev = "cuda"
    ws = torch.empty(moe.workspace_bytes(cfg), dtype=torch.uint8, device=dev)
    lg = torch.empty((S, E), dtype=torch.float32, device=dev)
    idx = torch.empty((S, k), dtype=torch.int32, device=dev)
    tw = torch.empty((S, k), dtype=torch.float32, device=dev)
    slot = torch.empty((S, k), dtype=torch.int32, device=dev)
    counts = torch.empty((k + 1, E), dtype=torch.int32, device=dev)
    losses = torch.empty(2, dtype=torch.float32, device=dev)
    moe.gate(cfg, inputs["x"], inputs["wg"], inputs["bg"], lg, idx, tw, slot, counts, losses, ws)
    xd = torch.zeros((E, C, d), dtype=at, device=dev)
    moe.dispatch(cfg, inputs["x"], idx, slot, xd)
    out = torch.zeros((E, C, d), dtype=at, device=dev)
    moe.expert_ffn(cfg, xd, counts, inputs["w1"], inputs["b1"], inputs["w2"], inputs["b2"], out,
                   ws)
    y = torch.empty((S, d), dtype=at, device=dev)
    moe.combine(cfg, out, idx, slot, tw, y)
    torch.cuda.synchronize()
    occ = oracle.occupancy(counts.cpu().numpy(), C, k)
    filled = torch.from_numpy(np.arange(C)[None, :] < occ[:, None]).cuda()
    for a, b in ((idx, ref.topk_idx), (slot, ref.slot), (counts, ref.counts),
                 (losses, ref.losses), (y, ref.y)):
        assert torch.equal(a, b)
    assert torch.equal(xd[filled], ref.xd[filled]) and torch.equal(out[filled], ref.out[filled])
    # the routing from given logits (MOE_GATE_LOGITS_IN) is the same
    idx2, slot2, counts2 = torch.empty_like(idx), torch.empty_like(slot), torch.empty_like(counts)
    moe.gate(cfg, None, None, None, lg, idx2, torch.empty_like(tw), slot2, counts2,
             torch.empty_like(losses), ws, logits_in=True)
    torch.cuda.synchronize()
    assert torch.equal(idx2, idx) and torch.equal(slot2, slot) and torch.equal(counts2, counts)


def test_reroute_degenerate_cases():
    """k = E leaves no alternative expert: re-routing changes nothing and
    counts row k is zero.  A capacity no expert reaches drops nothing, so no
    offer is made."""
    for w, name in ((mw.Workload("rr_k_eq_e", S=500, d=64, h=128, E=2, k=2, capacity_factor=0.5,
                                 dtype="bf16", seed=65, reroute=True), "k=E"),
                    (mw.Workload("rr_roomy", S=400, d=64, h=128, E=8, k=2, capacity_factor=4.0,
                                 dtype="bf16", seed=66, reroute=True), "no drops")):
        inputs, rr = run_layer(w, dispatch_buffer=False)
        _, plain = run_layer(w.with_(reroute=False), inputs=inputs, dispatch_buffer=False)
        assert int(rr.counts[w.k].abs().sum()) == 0, name
        for a, b in ((rr.topk_idx, plain.topk_idx), (rr.slot, plain.slot), (rr.y, plain.y),
                     (rr.counts[:w.k], plain.counts)):
            assert torch.equal(a, b), name
        rep = check_layer(w, inputs, rr, full=True)
        _print(w.name, rep)


def test_reroute_tiny_capacity():
    """Capacity 1: almost every assignment overflows and the few free rows
    of cold experts are fought over by many offers."""
    w = mw.Workload("rr_c1", S=300, d=64, h=128, E=24, k=2, capacity_factor=1.0, dtype="bf16",
                    seed=67, gate_bias="zipf1.2", reroute=True)
    inputs = mw.generate(w, "cuda")
    cfg = moe.config(w.S, w.d, w.h, w.E, w.k, capacity=1, dtype=w.dtype, reroute=True)
    layer = MoELayer.from_inputs(cfg, inputs, keep=True, dispatch_buffer=True)
    layer.forward(inputs["x"])
    torch.cuda.synchronize()
    assert layer.C == 1
    rep = check_layer(w, inputs, layer, full=True)
    _print(w.name, rep)


@pytest.mark.parametrize("w", REROUTE_MID[:2], ids=lambda w: w.name)
def test_reroute_backward_full_parity(w):
    """Every gradient with re-routing against the oracle's: re-routed
    assignments feed their serving expert's weights while their weight's
    gradient reaches the logits of the router's own top-k."""
    print(f"\n[rr bwd] {w}", flush=True)
    inputs = _with_biases(w, mw.generate(w, "cuda"), w.seed + 100)
    inputs, layer = run_layer(w, inputs, dispatch_buffer=False)
    g = torch.Generator(device="cuda").manual_seed(w.seed + 200)
    dy = torch.randn((w.S, w.d), generator=g, device="cuda").to(torch.bfloat16)
    grads = run_backward(w, inputs, layer, dy, g_aux=0.7, g_z=0.3)
    check_backward(w, inputs, layer, grads, dy, 0.7, 0.3)


def test_reroute_full_size_whole():
    """The skewed full-size workload with re-routing, in the benchmark's
    launch configuration: routing and rows exact, every filled expert-output
    row and every row of y against the oracle, each row on its own."""
    w = mw.get("skewed_bf16").with_(reroute=True, name="skewed_bf16_reroute")
    print(f"\n[rr full] {w}", flush=True)
    inputs, layer = run_layer(w, dispatch_buffer=False)
    rep = check_layer(w, inputs, layer, full=True)
    _print(w.name, rep)
    assert rep["rerouted"] > 0
    del layer, inputs
    torch.cuda.empty_cache()


def test_reroute_forward_replays_in_a_hip_graph():
    """The re-routing pass enqueues kernels only, so a re-routing forward can
    be captured in a HIP graph: every replay, with new token values and eager
    work between replays, equals an eager run bit for bit."""
    w = REROUTE_MID[0]
    inputs = mw.generate(w, "cuda")
    cfg = moe.config(w.S, w.d, w.h, w.E, w.k, w.capacity_factor, dtype=w.dtype, reroute=True)
    eager = MoELayer.from_inputs(cfg, inputs, keep=True, dispatch_buffer=False)
    graphed = MoELayer.from_inputs(cfg, inputs, keep=True, dispatch_buffer=False)
    x_static = inputs["x"].clone()
    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        graphed.forward(x_static)          # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        graphed.forward(x_static)
    g = torch.Generator(device="cuda").manual_seed(6)
    for rep in range(4):
        x_new = torch.randn((w.S, w.d), generator=g, device="cuda").to(torch.bfloat16)
        x_static.copy_(x_new)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        eager.forward(x_new)
        torch.cuda.synchronize()
        assert int(eager.counts[w.k].sum()) > 0, "the inputs must make re-routing happen"
        for name in ("y", "topk_idx", "slot", "counts", "losses", "logits"):
            assert torch.equal(getattr(graphed, name), getattr(eager, name)), (rep, name)


# S, E, k, C: ragged S, E not a multiple of 64, tiny and large E, capacity 1
REROUTE_ROUTE_CASES = [
    (1, 2, 1, 1), (63, 3, 2, 5), (65, 8, 2, 16), (1000, 65, 3, 40), (777, 128, 2, 9),
    (2048, 256, 8, 70), (300, 1000, 4, 2), (129, 2048, 8, 1), (500, 9, 7, 60),
    # scanned rows of k * ceil(S/64) > 2048 entries (two chunks)
    (20000, 16, 8, 900),
]


@pytest.mark.parametrize("S,E,k,C", REROUTE_ROUTE_CASES)
def test_reroute_route_from_logits_bit_exact(S, E, k, C):
    """moe_gate with re-routing and MOE_GATE_LOGITS_IN on logits full of ties
    (small integers and +-0): serving experts, rows and the counts with
    their extra row equal the oracle's bit for bit, so alternative experts
    are ranked exactly as the router ranks (logit descending, index
    ascending, -0 equal to +0)."""
    print(f"\n[rr route] S={S} E={E} k={k} C={C}", flush=True)
    rng = np.random.default_rng(S * 7919 + E + 1)
    lg = rng.integers(-3, 4, (S, E)).astype(np.float32) / 2
    lg[rng.random((S, E)) < 0.05] = -0.0
    cfg = moe.config(S, 64, 64, E, k, capacity=C, dtype="bf16", reroute=True)
    dev = torch.device("cuda")
    L = torch.from_numpy(lg).to(dev)
    idx = torch.empty((S, k), dtype=torch.int32, device=dev)
    tw = torch.empty((S, k), dtype=torch.float32, device=dev)
    slot = torch.empty((S, k), dtype=torch.int32, device=dev)
    counts = torch.empty((k + 1, E), dtype=torch.int32, device=dev)
    losses = torch.empty(2, dtype=torch.float32, device=dev)
    ws = torch.empty(moe.workspace_bytes(cfg), dtype=torch.uint8, device=dev)
    moe.gate(cfg, None, None, None, L, idx, tw, slot, counts, losses, ws, logits_in=True)
    torch.cuda.synchronize()
    r = oracle.route(lg, k, C, reroute=True)
    assert np.array_equal(idx.cpu().numpy(), r["serve"])
    assert np.array_equal(slot.cpu().numpy(), r["slot"])
    assert np.array_equal(counts.cpu().numpy(), r["counts"])
    moved = int((r["serve"] != r["idx"]).sum())
    print(f"[rr route] re-routed {moved}, still dropped {int((r['slot'] < 0).sum())}", flush=True)
