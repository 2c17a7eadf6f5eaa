"""GPU parity of the HIP MoE layer against the CPU oracle, through the C ABI.

Every input is seeded and synthetic (moe_workloads).  Bars: routing indices,
slots, counts and drop masks bit-exact given identical fp32 logits; ordered
top-k agreement with the oracle's own logits >= 99.99% of tokens; dispatch
buffers bit-exact; expert outputs and y within relative Frobenius error 1e-5
(fp32) / 1e-2 (bf16); aux and z within relative error 1e-5.
"""
import numpy as np
import pytest
import torch

import moe_workloads as mw
import oracle
import sparse_moe_layer_wg_amd as moe
from parity_util import TOL, as_f64, check_layer, rel_fro, run_layer

pytestmark = pytest.mark.gpu


def _dev_ws(cfg):
    return torch.empty(moe.workspace_bytes(cfg), dtype=torch.uint8, device="cuda")


def _print(name, rep):
    print(f"\n[{name}] " + " ".join(f"{k}={v:.4g}" if isinstance(v, float) else f"{k}={v}"
                                   for k, v in rep.items()), flush=True)


# --------------------------------------------------------------------- routing
ROUTE_CASES = [
    # S, E, k, C   (ragged S, E not a multiple of 64, tiny and large E)
    (1, 1, 1, 1), (63, 3, 2, 5), (64, 8, 2, 16), (65, 8, 2, 16), (1000, 65, 3, 40),
    (777, 128, 2, 9), (2048, 256, 8, 70), (300, 1000, 4, 2), (129, 2048, 8, 1), (500, 7, 7, 500),
    # histogram rows of k * ceil(S/64) > 2048 entries: the slot scan's second chunk
    (20000, 16, 8, 2000), (70000, 40, 2, 3000),
]


@pytest.mark.parametrize("S,E,k,C", ROUTE_CASES)
def test_route_from_logits_bit_exact(S, E, k, C):
    """moe_gate with MOE_GATE_LOGITS_IN on logits full of ties (small integers
    and +-0): indices, slots and counts equal the oracle's bit for bit."""
    print(f"\n[route] S={S} E={E} k={k} C={C}", flush=True)
    rng = np.random.default_rng(S * 7919 + E)
    lg = rng.integers(-3, 4, (S, E)).astype(np.float32) / 2
    lg[rng.random((S, E)) < 0.05] = -0.0
    cfg = moe.config(S, 64, 64, E, k, capacity=C, dtype="bf16")
    dev = torch.device("cuda")
    L = torch.from_numpy(lg).to(dev)
    idx = torch.empty((S, k), dtype=torch.int32, device=dev)
    tw = torch.empty((S, k), dtype=torch.float32, device=dev)
    slot = torch.empty((S, k), dtype=torch.int32, device=dev)
    counts = torch.empty((k, E), dtype=torch.int32, device=dev)
    losses = torch.empty(2, dtype=torch.float32, device=dev)
    moe.gate(cfg, None, None, None, L, idx, tw, slot, counts, losses, _dev_ws(cfg), logits_in=True)
    torch.cuda.synchronize()
    r = oracle.route(lg, k, C)
    assert np.array_equal(idx.cpu().numpy(), r["idx"])
    assert np.array_equal(slot.cpu().numpy(), r["slot"])
    assert np.array_equal(counts.cpu().numpy(), r["counts"])
    assert rel_fro(tw.cpu().numpy(), r["w"]) <= 1e-5
    lo = losses.cpu().numpy()
    assert abs(lo[0] - r["aux"]) <= 1e-5 * abs(r["aux"])
    assert abs(lo[1] - r["z"]) <= 1e-5 * max(abs(r["z"]), 1e-30)
    # the logits were an input and are unchanged
    assert np.array_equal(L.cpu().numpy(), lg)


# --------------------------------------------------------------------- permute
@pytest.mark.parametrize("dtype,S,d,E,k,cf", [("bf16", 333, 192, 12, 2, 0.7),
                                              ("f32", 100, 68, 5, 3, 0.5),
                                              ("bf16", 64, 7168 // 8, 256, 8, 1.5)])
def test_dispatch_and_combine(dtype, S, d, E, k, cf):
    """moe_dispatch is a bit copy into [E,C,d]; moe_combine matches the oracle."""
    print(f"\n[permute] {dtype} S={S} d={d} E={E} k={k} cf={cf}", flush=True)
    torch.manual_seed(0)
    rng = np.random.default_rng(1)
    cfg = moe.config(S, d, 64, E, k, cf, dtype=dtype)
    C = moe.capacity(cfg)
    assert C == oracle.capacity(S, E, k, cf)
    lg = rng.standard_normal((S, E)).astype(np.float32)
    r = oracle.route(lg, k, C)
    at = torch.bfloat16 if dtype == "bf16" else torch.float32
    x = torch.randn(S, d, device="cuda").to(at)
    idx = torch.from_numpy(r["idx"]).cuda()
    slot = torch.from_numpy(r["slot"]).cuda()
    xd = torch.zeros((E, C, d), dtype=at, device="cuda")
    moe.dispatch(cfg, x, idx, slot, xd)
    out = torch.randn((E, C, d), device="cuda").to(at)
    tw = torch.from_numpy(r["w"].astype(np.float32)).cuda()
    y = torch.empty((S, d), dtype=at, device="cuda")
    moe.combine(cfg, out, idx, slot, tw, y)
    torch.cuda.synchronize()
    xd_or = oracle.dispatch(mw.to_numpy(x), r["idx"], r["slot"], E, C)
    assert np.array_equal(mw.to_numpy(xd), xd_or)      # empties zero on both sides here
    y_or = oracle.combine(as_f64(out), r["idx"], r["slot"], r["w"].astype(np.float32), S)
    assert rel_fro(as_f64(y), y_or) <= TOL[dtype]
    assert np.all(as_f64(y)[(r["slot"] < 0).all(axis=1)] == 0)


# --------------------------------------------------------------------- expert FFN
# 256-row m-tiles take up to 32 more rows in an expert's last tile: 256..288
# rows run as one tile, 289 as 256 + 33, 544 as 256 + 288, 545 as three.
STRIP_OCC = [256, 257, 270, 288, 289, 300, 544, 545, 600, 0]
# Small and nearly empty last m-tiles around the 32-row sub-tile and strip
# boundaries, with K and N (320) not multiples of the 256-wide tiles.
SMALL_OCC = [1, 31, 33, 63, 64, 65, 289, 320, 321, 352, 0]


@pytest.mark.parametrize("dtype,E,C,d,h,bias", [("bf16", 5, 300, 256, 384, True),
                                                ("bf16", 3, 130, 128, 64, False),
                                                ("bf16", 10, 600, 128, 192, True),
                                                ("bf16", 11, 400, 320, 320, True),
                                                ("f32", 4, 70, 68, 132, True)])
def test_expert_ffn_ragged_occupancy(dtype, E, C, d, h, bias):
    """moe_expert_ffn over ragged occupancies (empty, partial tile, full C,
    every boundary of the extra rows an expert's last m-tile may take, small
    last tiles with K and N not multiples of 256); every filled row is also
    checked on its own."""
    print(f"\n[ffn] {dtype} E={E} C={C} d={d} h={h} bias={bias}", flush=True)
    torch.manual_seed(2)
    at = torch.bfloat16 if dtype == "bf16" else torch.float32
    k = 1
    cfg = moe.config(E * C, d, h, E, k, capacity=C, dtype=dtype)
    occ = np.array(STRIP_OCC if E == len(STRIP_OCC) else
                   SMALL_OCC if E == len(SMALL_OCC) else [C, 0, 1, C - 1, 129][:E], np.int32)
    counts = torch.from_numpy(occ[None, :].copy()).cuda()
    xd = torch.randn((E, C, d), device="cuda").to(at)
    w1 = (torch.randn((E, h, d), device="cuda") / d ** 0.5).to(at)
    w2 = (torch.randn((E, d, h), device="cuda") / h ** 0.5).to(at)
    b1 = (0.1 * torch.randn((E, h), device="cuda")).to(at) if bias else None
    b2 = (0.1 * torch.randn((E, d), device="cuda")).to(at) if bias else None
    out = torch.full((E, C, d), 7.0, device="cuda").to(at)
    moe.expert_ffn(cfg, xd, counts, w1, b1, w2, b2, out, _dev_ws(cfg))
    torch.cuda.synchronize()
    out_or = oracle.expert_ffn(mw.to_numpy(xd), occ, mw.to_numpy(w1), mw.to_numpy(b1),
                               mw.to_numpy(w2), mw.to_numpy(b2))
    filled = np.arange(C)[None, :] < occ[:, None]
    o = as_f64(out)
    assert rel_fro(o[filled], out_or[filled]) <= TOL[dtype]
    row_err = np.linalg.norm(o[filled] - out_or[filled], axis=1) / \
        np.maximum(np.linalg.norm(out_or[filled], axis=1), 1e-30)
    assert row_err.max() <= 3 * TOL[dtype], row_err.max()
    assert np.all(o[~filled] == 7.0)                   # rows past occupancy untouched


# --------------------------------------------------------------------- whole layer
MID = [
    mw.Workload("mid_bf16", S=1000, d=256, h=512, E=16, k=2, capacity_factor=1.0, dtype="bf16",
                seed=11),
    mw.Workload("mid_bf16_top8", S=700, d=192, h=320, E=40, k=8, capacity_factor=1.5,
                dtype="bf16", seed=12),
    mw.Workload("mid_bf16_skew", S=900, d=128, h=256, E=32, k=2, capacity_factor=1.0,
                dtype="bf16", seed=13, gate_bias="zipf1.2"),
    mw.Workload("mid_f32_bias", S=333, d=96, h=160, E=6, k=2, capacity_factor=0.8, dtype="f32",
                seed=14, ffn_bias="zeros"),
    # degenerate routing: top-1 (every renormalised weight is 1) and a single
    # expert that keeps only the first C = S/2 tokens
    mw.Workload("mid_bf16_top1", S=517, d=128, h=192, E=8, k=1, capacity_factor=1.0,
                dtype="bf16", seed=15),
    mw.Workload("mid_bf16_one_expert", S=300, d=64, h=128, E=1, k=1, capacity_factor=0.5,
                dtype="bf16", seed=16),
]


@pytest.mark.parametrize("w", [mw.get("tiny_fp32")] + MID, ids=lambda w: w.name)
def test_layer_full_parity(w):
    """Whole moe_layer_forward against the oracle at every slot."""
    print(f"\n[layer] {w}", flush=True)
    inputs, layer = run_layer(w)
    rep = check_layer(w, inputs, layer, full=True)
    _print(w.name, rep)


def test_layer_with_ffn_biases_bf16():
    """Non-zero expert biases take the bias path of both GEMMs."""
    w = mw.Workload("bias_bf16", S=500, d=128, h=192, E=8, k=2, capacity_factor=1.25,
                    dtype="bf16", seed=21)
    inputs = mw.generate(w, "cuda")
    g = torch.Generator(device="cuda").manual_seed(99)
    inputs["b1"] = (0.2 * torch.randn((w.E, w.h), generator=g, device="cuda")).to(torch.bfloat16)
    inputs["b2"] = (0.2 * torch.randn((w.E, w.d), generator=g, device="cuda")).to(torch.bfloat16)
    inputs, layer = run_layer(w, inputs)
    _print(w.name, check_layer(w, inputs, layer, full=True))


def test_empty_input():
    """S = 0: nothing to route; counts and losses are zero."""
    cfg = moe.config(0, 64, 64, 4, 2, 1.0, dtype="bf16")
    dev = "cuda"
    z = lambda *s, dt=torch.bfloat16: torch.empty(s, dtype=dt, device=dev)
    counts = torch.full((2, 4), 5, dtype=torch.int32, device=dev)
    losses = torch.full((2,), 5.0, device=dev)
    moe.layer_forward(cfg, z(0, 64), z(4, 64, dt=torch.float32), None, z(4, 64, 64), None,
                      z(4, 64, 64), None, z(0, 64), _dev_ws(cfg), counts=counts, losses=losses)
    torch.cuda.synchronize()
    assert counts.abs().sum().item() == 0 and losses.abs().sum().item() == 0


def test_deterministic_repeat():
    """Two runs are bit-identical in routing, slots, drops, losses and y."""
    w = MID[0]
    inputs, layer = run_layer(w)
    first = [t.clone() for t in (layer.topk_idx, layer.slot, layer.losses, layer.y, layer.logits)]
    layer.forward(inputs["x"])
    torch.cuda.synchronize()
    for a, b in zip(first, (layer.topk_idx, layer.slot, layer.losses, layer.y, layer.logits)):
        assert torch.equal(a, b)


@pytest.mark.parametrize("w", [w for w in MID if w.dtype == "bf16"], ids=lambda w: w.name)
def test_fused_gather_matches_dispatch_buffer(w):
    """Without a dispatch buffer the first expert GEMM gathers rows from x:
    y, out and every routing output equal the unfused run bit for bit, and
    the fused run passes the full oracle check."""
    print(f"\n[fused] {w}", flush=True)
    inputs, ref = run_layer(w)
    _, fused = run_layer(w, inputs, dispatch_buffer=False)
    assert fused.xd is None
    occ = np.minimum(ref.counts.cpu().numpy().sum(0), ref.C)
    filled = torch.from_numpy(np.arange(ref.C)[None, :] < occ[:, None]).cuda()
    assert torch.equal(ref.out[filled], fused.out[filled])
    for a, b in ((ref.y, fused.y), (ref.slot, fused.slot), (ref.topk_idx, fused.topk_idx),
                 (ref.losses, fused.losses)):
        assert torch.equal(a, b)
    _print(w.name + "_fused", check_layer(w, inputs, fused, full=True))


# --------------------------------------------------------------------- full sizes
@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["balanced_bf16", "skewed_bf16", "large_bf16", "deepseek_bf16"])
def test_full_size_whole(name):
    """Full-size workloads in the benchmark's launch configuration (no dispatch
    buffer: the gather is fused into the first expert GEMM): all routing
    checked exactly, and every filled expert-output row and every row of y
    against the oracle, each row on its own as well as the whole tensor."""
    import time
    w = mw.get(name)
    print(f"\n[full] {w}", flush=True)
    inputs, layer = run_layer(w, dispatch_buffer=False)
    t0 = time.perf_counter()
    rep = check_layer(w, inputs, layer, full=True)
    rep["oracle_s"] = time.perf_counter() - t0
    _print(name, rep)
    del layer, inputs
    torch.cuda.empty_cache()


# Many more GEMM tiles than compute units (512 per forward GEMM against 256
# CUs), so every persistent block claims several tiles in a row: the tile
# counters, the claim of the next tile during an epilogue and the reuse of
# LDS between tiles all run, and every row is checked.
MANY_TILES = mw.Workload("many_tiles_bf16", S=8192, d=2048, h=2048, E=16, k=2,
                         capacity_factor=1.0, dtype="bf16", seed=17)


@pytest.mark.timeout(600)
def test_many_tiles_whole():
    print(f"\n[many tiles] {MANY_TILES}", flush=True)
    inputs, layer = run_layer(MANY_TILES, dispatch_buffer=False)
    _print(MANY_TILES.name, check_layer(MANY_TILES, inputs, layer, full=True))


# --------------------------------------------------------------------- near-tie refinement
def test_duplicated_router_rows_exact_ties():
    """Router rows duplicated in pairs: every token has exactly tied logits,
    so every token goes through the fp64 re-evaluation; ties must resolve to
    the lower expert index exactly as in the oracle."""
    w = mw.Workload("dup_rows", S=2000, d=512, h=128, E=64, k=4, capacity_factor=1.0,
                    dtype="bf16", seed=31)
    inputs = mw.generate(w, "cuda")
    inputs["wg"] = inputs["wg"][0::2].repeat_interleave(2, dim=0).contiguous()
    inputs, layer = run_layer(w, inputs)
    rep = check_layer(w, inputs, layer, full=True)
    _print(w.name, rep)
    idx = layer.topk_idx.cpu().numpy()
    # the lower index of each tied pair always comes first
    for r in range(w.k - 1):
        pair = (idx[:, r] // 2 == idx[:, r + 1] // 2)
        assert np.all(idx[pair, r] < idx[pair, r + 1])


@pytest.mark.parametrize("scale", [1.0, 100.0])
def test_near_tie_pairs_exact_at_any_input_scale(scale):
    """Router rows in nearly tied pairs (row 2i+1 = row 2i + 7e-8 * N(0,1)
    noise, so a token's two best experts are usually a pair whose logits
    differ by about 7e-8 |x_s|) and x scaled by `scale`.  At scale 100 those
    differences (about 1.6e-4) are as small as the fp32 GEMM's error there;
    the refinement margin grows with |x_s| and max_j |w_j|, so every such
    decision is re-evaluated in fp64 and the ordered top-k equals the
    oracle's from its own logits for every token."""
    w = mw.Workload("near_pairs", S=4000, d=512, h=128, E=64, k=2, capacity_factor=1.0,
                    dtype="bf16", seed=33)
    inputs = mw.generate(w, "cuda")
    g = torch.Generator(device="cuda").manual_seed(34)
    base = inputs["wg"][0::2]
    twin = base + 7e-8 * torch.randn(base.shape, generator=g, device="cuda")
    inputs["wg"] = torch.stack([base, twin], dim=1).reshape(w.E, w.d).contiguous()
    inputs["x"] = (inputs["x"].float() * scale).to(torch.bfloat16)
    inputs, layer = run_layer(w, inputs, dispatch_buffer=False)
    rep = check_layer(w, inputs, layer, full=True)
    _print(f"near_pairs_x{scale:g}", rep)
    assert rep["topk_mismatches"] == 0, rep
    idx = layer.topk_idx.cpu().numpy()
    rep_pairs = float(np.mean(idx[:, 0] // 2 == idx[:, 1] // 2))
    print(f"  tokens whose top-2 is a tied pair: {rep_pairs:.3f}", flush=True)
    assert rep_pairs > 0.5


@pytest.mark.parametrize("E,k", [(8, 2), (64, 2), (40, 8)])
def test_zero_router_closed_form(E, k):
    """All-zero router weight: every logit is 0, so the top-k is (0..k-1) with
    weights 1/k, aux = 1, z = (ln E)^2 and the first C tokens of each rank are
    kept.  E = 64 drives the re-evaluation through its longest-chain path."""
    S, d, h = 300, 64, 64
    cf = 1.0
    w = mw.Workload("zero_router", S=S, d=d, h=h, E=E, k=k, capacity_factor=cf, dtype="bf16",
                    seed=41)
    inputs = mw.generate(w, "cuda")
    inputs["wg"].zero_()
    inputs, layer = run_layer(w, inputs)
    C = layer.C
    idx = layer.topk_idx.cpu().numpy()
    assert np.all(idx == np.arange(k)[None, :])
    assert np.allclose(layer.topk_w.cpu().numpy(), 1.0 / k, rtol=1e-6)
    s = np.arange(S)
    for r in range(k):
        assert np.array_equal(layer.slot.cpu().numpy()[:, r], np.where(s < C, s, -1))
    aux, z = layer.losses.cpu().numpy()
    assert abs(aux - 1.0) <= 1e-5 and abs(z - np.log(E) ** 2) <= 1e-5 * np.log(E) ** 2
    _print(f"zero_router_E{E}", check_layer(w, inputs, layer, full=True))


# --------------------------------------------------------------------- graph capture
def test_layer_forward_replays_in_a_hip_graph():
    """moe_layer_forward enqueues kernels only (no allocation, copy, memset or
    host synchronisation), so it can be captured in a HIP graph.  The graph is
    replayed several times, with eager work and synchronisations between the
    replays and new token values each time, and every replay equals an eager
    run on the same inputs bit for bit."""
    from sparse_moe_layer_wg_amd.layer import MoELayer
    w = MID[0]
    inputs = mw.generate(w, "cuda")
    eager = MoELayer.from_inputs(moe.config(w.S, w.d, w.h, w.E, w.k, w.capacity_factor,
                                            dtype=w.dtype), inputs, keep=True,
                                 dispatch_buffer=False)
    graphed = MoELayer.from_inputs(eager.cfg, inputs, keep=True, dispatch_buffer=False)
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
    g = torch.Generator(device="cuda").manual_seed(5)
    for rep in range(4):
        x_new = torch.randn((w.S, w.d), generator=g, device="cuda").to(torch.bfloat16)
        x_static.copy_(x_new)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        eager.forward(x_new)
        torch.cuda.synchronize()
        for name in ("y", "topk_idx", "slot", "counts", "losses", "logits"):
            assert torch.equal(getattr(graphed, name), getattr(eager, name)), (rep, name)
