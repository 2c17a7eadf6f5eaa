"""GPU parity of the dropless (unbounded-capacity) layer against the CPU oracle.

Dropless routing keeps every assignment: the dispatch buffer and the expert
output are compact [S*k, d] expert segments (expert order, then rank, then
token) and ``slot`` holds each assignment's global row.  Bars as for the
capacity-limited layer: routing indices, rows and counts bit-exact given the
GPU's fp32 logits; dispatch rows bit copies; expert outputs and y within
relative Frobenius error 1e-5 (fp32) / 1e-2 (bf16) of the oracle's dense
top-k sum; aux and z within relative error 1e-5.  The dropless layer performs
the capacity layer's arithmetic, so with an unreachable capacity the two
agree bit for bit.
"""
import numpy as np
import pytest
import torch

import moe_workloads as mw
import oracle
import sparse_moe_layer_wg_amd as moe
from parity_util import TOL, as_f64, check_layer, rel_fro, run_layer

pytestmark = pytest.mark.gpu


def _print(name, rep):
    print(f"\n[{name}] " + " ".join(f"{k}={v:.4g}" if isinstance(v, float) else f"{k}={v}"
                                   for k, v in rep.items()), flush=True)


DROPLESS_MID = [
    mw.Workload("dl_mid_bf16", S=1000, d=256, h=512, E=16, k=2, capacity_factor=1.0,
                dtype="bf16", seed=11, dropless=True),
    mw.Workload("dl_mid_bf16_top8", S=700, d=192, h=320, E=40, k=8, capacity_factor=1.0,
                dtype="bf16", seed=12, dropless=True),
    # zipf gate bias: the hot experts take several hundred rows (strip and
    # multi-tile segments) while cold ones are empty or nearly so
    mw.Workload("dl_mid_bf16_skew", S=900, d=128, h=256, E=32, k=2, capacity_factor=1.0,
                dtype="bf16", seed=13, gate_bias="zipf1.2", dropless=True),
    mw.Workload("dl_mid_f32", S=333, d=96, h=160, E=6, k=2, capacity_factor=1.0, dtype="f32",
                seed=14, ffn_bias="zeros", dropless=True),
]


@pytest.mark.parametrize("w", DROPLESS_MID, ids=lambda w: w.name)
@pytest.mark.parametrize("dispatch_buffer", [True, False], ids=["xd", "fused"])
def test_dropless_layer_full_parity(w, dispatch_buffer):
    """Whole dropless moe_layer_forward against the oracle at every row, with
    and without the dispatch buffer (without it, bf16 layers gather rows
    from x inside the first expert GEMM)."""
    print(f"\n[dropless] {w} xd={dispatch_buffer}", flush=True)
    inputs, layer = run_layer(w, dispatch_buffer=dispatch_buffer)
    assert tuple(layer.out.shape) == (w.S * w.k, w.d)
    rep = check_layer(w, inputs, layer, full=True)
    _print(w.name, rep)


@pytest.mark.parametrize("w", DROPLESS_MID[:3], ids=lambda w: w.name)
def test_dropless_equals_unreachable_capacity(w):
    """Dropless and capacity routing with C = S run the same arithmetic on
    the same rows: y and every expert output row agree bit for bit."""
    print(f"\n[dl=pad] {w}", flush=True)
    inputs, dl = run_layer(w, dispatch_buffer=False)
    cfg = moe.config(w.S, w.d, w.h, w.E, w.k, capacity=w.S, dtype=w.dtype)
    from sparse_moe_layer_wg_amd.layer import MoELayer
    pad = MoELayer.from_inputs(cfg, inputs, keep=True, dispatch_buffer=False)
    pad.forward(inputs["x"])
    torch.cuda.synchronize()
    assert torch.equal(dl.y, pad.y)
    assert torch.equal(dl.topk_idx, pad.topk_idx) and torch.equal(dl.losses, pad.losses)
    assert (pad.slot >= 0).all()
    rows = dl.slot.long().reshape(-1)
    assert torch.equal(dl.out[rows], pad.out[pad.topk_idx.long().reshape(-1),
                                             pad.slot.long().reshape(-1)])


@pytest.mark.parametrize("w", [DROPLESS_MID[0], DROPLESS_MID[3]], ids=lambda w: w.name)
def test_dropless_stage_entry_points(w):
    """moe_gate, moe_dispatch, moe_expert_ffn and moe_combine called one by
    one on a dropless config reproduce moe_layer_forward bit for bit."""
    print(f"\n[dl stages] {w}", flush=True)
    inputs, ref = run_layer(w, dispatch_buffer=True)
    cfg = ref.cfg
    at = w.torch_dtype
    S, d, E, k = w.S, w.d, w.E, w.k
    dev = "cuda"
    ws = torch.empty(moe.workspace_bytes(cfg), dtype=torch.uint8, device=dev)
    lg = torch.empty((S, E), dtype=torch.float32, device=dev)
    idx = torch.empty((S, k), dtype=torch.int32, device=dev)
    tw = torch.empty((S, k), dtype=torch.float32, device=dev)
    slot = torch.empty((S, k), dtype=torch.int32, device=dev)
    counts = torch.empty((k, E), dtype=torch.int32, device=dev)
    losses = torch.empty(2, dtype=torch.float32, device=dev)
    moe.gate(cfg, inputs["x"], inputs["wg"], inputs["bg"], lg, idx, tw, slot, counts, losses, ws)
    rows = moe.dispatch_rows(cfg)
    assert rows == S * k
    xd = torch.zeros((rows, d), dtype=at, device=dev)
    moe.dispatch(cfg, inputs["x"], idx, slot, xd)
    out = torch.zeros((rows, d), dtype=at, device=dev)
    moe.expert_ffn(cfg, xd, counts, inputs["w1"], inputs["b1"], inputs["w2"], inputs["b2"], out,
                   ws)
    y = torch.empty((S, d), dtype=at, device=dev)
    moe.combine(cfg, out, idx, slot, tw, y)
    torch.cuda.synchronize()
    for a, b in ((slot, ref.slot), (counts, ref.counts), (losses, ref.losses), (xd, ref.xd),
                 (out, ref.out), (y, ref.y)):
        assert torch.equal(a, b)
    # every row is written exactly once: rows are a permutation of 0..S*k-1
    assert torch.equal(torch.sort(slot.reshape(-1))[0],
                       torch.arange(S * k, dtype=torch.int32, device=dev))


# Segment lengths around the 32-row sub-tile, the 256-row m-tile and the
# 32-row strip boundaries, with empty experts between them.
SEG_LENS = [0, 1, 31, 33, 64, 65, 256, 257, 288, 289, 0, 300, 544, 545, 600, 0, 129]


@pytest.mark.parametrize("dtype,d,h", [("bf16", 256, 384), ("bf16", 320, 320),
                                       ("f32", 68, 132)])
def test_dropless_expert_ffn_ragged_segments(dtype, d, h):
    """moe_expert_ffn on compact segments of ragged lengths (empty, partial
    tile, strip and multi-tile): every row matches the oracle's FFN of its
    expert and no row outside the segments exists to be touched."""
    print(f"\n[dl ffn] {dtype} d={d} h={h}", flush=True)
    torch.manual_seed(3)
    at = torch.bfloat16 if dtype == "bf16" else torch.float32
    n = np.array(SEG_LENS, np.int64)
    E, S = len(n), int(n.sum())
    cfg = moe.config(S, d, h, E, 1, dtype=dtype, dropless=True)
    assert moe.dispatch_rows(cfg) == S
    counts = torch.from_numpy(n[None, :].astype(np.int32)).cuda()
    xd = torch.randn((S, d), device="cuda").to(at)
    w1 = (torch.randn((E, h, d), device="cuda") / d ** 0.5).to(at)
    w2 = (torch.randn((E, d, h), device="cuda") / h ** 0.5).to(at)
    b1 = (0.1 * torch.randn((E, h), device="cuda")).to(at)
    b2 = (0.1 * torch.randn((E, d), device="cuda")).to(at)
    out = torch.full((S, d), 7.0, device="cuda").to(at)
    ws = torch.empty(moe.workspace_bytes(cfg), dtype=torch.uint8, device="cuda")
    moe.expert_ffn(cfg, xd, counts, w1, b1, w2, b2, out, ws)
    torch.cuda.synchronize()
    o = as_f64(out)
    seg = np.concatenate([[0], np.cumsum(n)[:-1]])
    host = [mw.to_numpy(t) for t in (xd, w1, b1, w2, b2)]
    for e in range(E):
        if n[e] == 0:
            continue
        rows = slice(seg[e], seg[e] + n[e])
        want = oracle.expert_ffn(host[0][None, rows], np.array([n[e]], np.int32),
                                 host[1][e:e + 1], host[2][e:e + 1], host[3][e:e + 1],
                                 host[4][e:e + 1])[0]
        assert rel_fro(o[rows], want) <= TOL[dtype], e
        row_err = np.linalg.norm(o[rows] - want, axis=1) / \
            np.maximum(np.linalg.norm(want, axis=1), 1e-30)
        assert row_err.max() <= 3 * TOL[dtype], (e, row_err.max())


def test_dropless_empty_input():
    """S = 0 with dropless routing: no rows, zero counts and losses."""
    cfg = moe.config(0, 64, 64, 4, 2, dtype="bf16", dropless=True)
    assert moe.dispatch_rows(cfg) == 0
    dev = "cuda"
    z = lambda *s, dt=torch.bfloat16: torch.empty(s, dtype=dt, device=dev)
    counts = torch.full((2, 4), 5, dtype=torch.int32, device=dev)
    losses = torch.full((2,), 5.0, device=dev)
    ws = torch.empty(max(moe.workspace_bytes(cfg), 256), dtype=torch.uint8, device=dev)
    moe.layer_forward(cfg, z(0, 64), z(4, 64, dt=torch.float32), None, z(4, 64, 64), None,
                      z(4, 64, 64), None, z(0, 64), ws, counts=counts, losses=losses)
    torch.cuda.synchronize()
    assert counts.abs().sum().item() == 0 and losses.abs().sum().item() == 0


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["skewed_bf16", "deepseek_bf16"])
def test_dropless_full_size_whole(name):
    """Full-size shapes with dropless routing in the benchmark's launch
    configuration (gather fused into the first expert GEMM): routing and rows
    checked exactly, and every compact expert-output row and every row of y
    against the oracle, each row on its own.  On the skewed workload capacity
    routing would drop a large share of assignments; here none is (the
    hottest expert takes thousands of rows)."""
    w = mw.get(name).with_(dropless=True, name=name + "_dropless")
    print(f"\n[dl full] {w}", flush=True)
    inputs, layer = run_layer(w, dispatch_buffer=False)
    rep = check_layer(w, inputs, layer, full=True)
    rep["max_segment"] = int(layer.counts.sum(0).max().item())
    _print(w.name, rep)
    del layer, inputs
    torch.cuda.empty_cache()
