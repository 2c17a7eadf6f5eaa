"""GPU parity of the layer's backward pass (moe_layer_backward) against the
fp64 CPU oracle, through the C ABI.

The forward runs on the GPU; the oracle's backward takes the GPU's fp32
logits, so both sides differentiate the same routing.  Bars: every gradient
within relative Frobenius error 1e-2 of the oracle (bf16 operands and
outputs, fp32 accumulation; the router side sees the forward's bf16 expert
outputs); exact zeros where the loss does not depend on an input; repeated
runs bit-identical.
"""
import numpy as np
import pytest
import torch

import moe_workloads as mw
import oracle
import sparse_moe_layer_wg_amd as moe
from parity_util import as_f64, rel_fro, row_rel, run_layer

pytestmark = pytest.mark.gpu

TOL = 1e-2


def _print(name, rep):
    print(f"\n[{name}] " + " ".join(f"{k}={v:.4g}" if isinstance(v, float) else f"{k}={v}"
                                   for k, v in rep.items()), flush=True)


def _with_biases(w, inputs, seed):
    g = torch.Generator(device="cuda").manual_seed(seed)
    inputs["b1"] = (0.2 * torch.randn((w.E, w.h), generator=g, device="cuda")).to(torch.bfloat16)
    inputs["b2"] = (0.2 * torch.randn((w.E, w.d), generator=g, device="cuda")).to(torch.bfloat16)
    return inputs


def run_backward(w, inputs, layer, dy, g_aux, g_z, want_biases=True, hidden=None):
    cfg = layer.cfg
    E, d, h = w.E, w.d, w.h
    dev = "cuda"
    at = torch.bfloat16
    grads = dict(
        dx=torch.full((w.S, d), 3.0, dtype=at, device=dev),
        dwg=torch.full((E, d), 3.0, dtype=torch.float32, device=dev),
        dbg=torch.full((E,), 3.0, dtype=torch.float32, device=dev) if want_biases else None,
        dw1=torch.full((E, h, d), 3.0, dtype=at, device=dev),
        db1=torch.full((E, h), 3.0, dtype=at, device=dev) if want_biases else None,
        dw2=torch.full((E, d, h), 3.0, dtype=at, device=dev),
        db2=torch.full((E, d), 3.0, dtype=at, device=dev) if want_biases else None,
    )
    ws = torch.empty(moe.backward_workspace_bytes(cfg), dtype=torch.uint8, device=dev)
    moe.layer_backward(cfg, inputs["x"], inputs["wg"], inputs["w1"], inputs["b1"], inputs["w2"],
                       layer.logits, layer.topk_idx, layer.topk_w, layer.slot, layer.counts,
                       layer.out, dy, grads["dx"], grads["dwg"], grads["dw1"], grads["dw2"], ws,
                       db_gate=grads["dbg"], db1=grads["db1"], db2=grads["db2"], g_aux=g_aux,
                       g_z=g_z, hidden=hidden)
    torch.cuda.synchronize()
    return grads


def check_backward(w, inputs, layer, grads, dy, g_aux, g_z):
    host = {n: mw.to_numpy(t) for n, t in inputs.items()}
    ref = oracle.layer_backward(host["x"], host["wg"], host["w1"], host["b1"], host["w2"],
                                host["b2"], w.k, layer.C, layer.logits.cpu().numpy(),
                                mw.to_numpy(dy), g_aux, g_z, reroute=w.reroute)
    rep = {}
    for key in ("dx", "dwg", "dbg", "dw1", "db1", "dw2", "db2"):
        if grads[key] is None:
            continue
        rep[key] = rel_fro(as_f64(grads[key]), ref[key])
    _print(w.name, rep)
    for key, err in rep.items():
        assert err <= TOL, (key, rep)
    return rep


BWD = [
    mw.Workload("bwd_mid", S=1000, d=256, h=512, E=16, k=2, capacity_factor=1.0, dtype="bf16",
                seed=51),
    mw.Workload("bwd_top8", S=600, d=192, h=320, E=40, k=8, capacity_factor=1.5, dtype="bf16",
                seed=52),
    # hot experts overflow: many drops, ragged rows, empty experts
    mw.Workload("bwd_skew", S=900, d=128, h=256, E=32, k=2, capacity_factor=1.0, dtype="bf16",
                seed=53, gate_bias="zipf1.2"),
    mw.Workload("bwd_dropless_skew", S=700, d=128, h=320, E=24, k=2, capacity_factor=1.0,
                dtype="bf16", seed=54, gate_bias="zipf1.2", dropless=True),
    # degenerate routing: with top-1 the renormalised weight is the constant 1,
    # so only the aux and z terms reach the router; with one expert the aux
    # loss is constant too and only z remains
    mw.Workload("bwd_top1", S=517, d=128, h=192, E=8, k=1, capacity_factor=1.0, dtype="bf16",
                seed=55),
    mw.Workload("bwd_one_expert", S=300, d=64, h=128, E=1, k=1, capacity_factor=0.5,
                dtype="bf16", seed=56),
]


@pytest.mark.parametrize("w", BWD, ids=lambda w: w.name)
def test_backward_full_parity(w):
    """Every gradient of the layer against the oracle's, with non-zero FFN
    biases and both loss weights non-zero."""
    print(f"\n[bwd] {w}", flush=True)
    inputs = _with_biases(w, mw.generate(w, "cuda"), w.seed + 100)
    inputs, layer = run_layer(w, inputs, dispatch_buffer=False)
    g = torch.Generator(device="cuda").manual_seed(w.seed + 200)
    dy = torch.randn((w.S, w.d), generator=g, device="cuda").to(torch.bfloat16)
    grads = run_backward(w, inputs, layer, dy, g_aux=0.7, g_z=0.3)
    check_backward(w, inputs, layer, grads, dy, 0.7, 0.3)


def _block_rel_max(a, b, bm=256, bn=256):
    """Largest relative error over [bm, bn] blocks of the last two axes (the
    weight-gradient GEMMs' output tiles); a zero block must be exactly zero."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    worst = 0.0
    M, N = a.shape[-2], a.shape[-1]
    for i in range(0, M, bm):
        for j in range(0, N, bn):
            da = a[..., i:i + bm, j:j + bn].reshape(a.shape[0], -1) if a.ndim == 3 else \
                a[i:i + bm, j:j + bn].reshape(1, -1)
            db = b[..., i:i + bm, j:j + bn].reshape(b.shape[0], -1) if b.ndim == 3 else \
                b[i:i + bm, j:j + bn].reshape(1, -1)
            worst = max(worst, float(row_rel(da, db).max()))
    return worst


def _whole_backward(w, inputs, layer, grads, dy, g_aux, g_z):
    """Every gradient against the oracle's: each whole tensor within the bar,
    each row of dx, db1, db2 and each 256 x 256 output tile of dW1 and dW2
    within 3x the bar (dx rows above it must be explained by a ReLU kink)."""
    import time
    host = {n: mw.to_numpy(t) for n, t in inputs.items()}
    t0 = time.perf_counter()
    ref = oracle.layer_backward(host["x"], host["wg"], host["w1"], host["b1"], host["w2"],
                                host["b2"], w.k, layer.C, layer.logits.cpu().numpy(),
                                mw.to_numpy(dy), g_aux, g_z)
    rep = {"oracle_s": time.perf_counter() - t0}
    for key in ("dx", "dwg", "dbg", "dw1", "db1", "dw2", "db2"):
        if grads[key] is not None:
            rep[key] = rel_fro(as_f64(grads[key]), ref[key])
    rows = row_rel(as_f64(grads["dx"]), ref["dx"])
    rep["dw1_tile_max"] = _block_rel_max(as_f64(grads["dw1"]), ref["dw1"])
    rep["dw2_tile_max"] = _block_rel_max(as_f64(grads["dw2"]), ref["dw2"])
    for key in ("db1", "db2"):
        if grads[key] is not None:
            rep[key + "_row_max"] = float(row_rel(as_f64(grads[key]), ref[key]).max())
    # dx rows: a hidden pre-activation within fp32 rounding of zero can land
    # on the other side of the ReLU in the GPU's fp32 accumulation than in
    # the oracle's fp64, and that unit's whole W1 row then enters dx or not
    # (about 1/sqrt(active units) of the row, ~3% at d_ff = 2048).  A row
    # above the per-row bar must hold such a unit (|u| within 1e-5 of the
    # pre-activations' rms); such rows must be rare and stay below 0.1.
    over = np.nonzero(rows > 3 * TOL)[0]
    slot = layer.slot.cpu().numpy()
    idx = layer.topk_idx.cpu().numpy()
    for s in over:
        assert rows[s] <= 0.1, (s, rows[s])
        assert _near_kink(host, idx[s], slot[s], s), (s, rows[s])
    assert len(over) <= max(2, w.S // 1000), len(over)
    rep["dx_rows_over_bar"] = int(len(over))
    rep["dx_row_max_else"] = float(np.delete(rows, over).max())
    _print(w.name + "_bwd", rep)
    for key, err in rep.items():
        if key not in ("dx_rows_over_bar", "oracle_s"):
            assert err <= (3 * TOL if key.endswith(("_max", "_else")) else TOL), (key, rep)
    return rep


@pytest.mark.timeout(600)
def test_backward_many_tiles_whole():
    """A backward with many more tiles than compute units (the forward GEMMs
    512 tiles each, the weight gradients 1024): every gradient against the
    oracle, each row of dx and each 256 x 256 output tile of dW1 and dW2 on
    its own as well as the whole tensors."""
    from test_gpu_parity import MANY_TILES as w
    print(f"\n[bwd many tiles] {w}", flush=True)
    inputs = _with_biases(w, mw.generate(w, "cuda"), w.seed + 100)
    inputs, layer = run_layer(w, inputs, dispatch_buffer=False)
    g = torch.Generator(device="cuda").manual_seed(w.seed + 200)
    dy = torch.randn((w.S, w.d), generator=g, device="cuda").to(torch.bfloat16)
    grads = run_backward(w, inputs, layer, dy, g_aux=0.7, g_z=0.3)
    _whole_backward(w, inputs, layer, grads, dy, 0.7, 0.3)


@pytest.mark.timeout(900)
def test_backward_balanced_full_size_whole():
    """The balanced full-size workload in the training benchmark's
    configuration (fused gather, the benchmark's loss weights): every
    gradient against the oracle, whole and row by row / tile by tile."""
    w = mw.get("balanced_bf16")
    print(f"\n[bwd full whole] {w}", flush=True)
    inputs, layer = run_layer(w, dispatch_buffer=False)
    g = torch.Generator(device="cuda").manual_seed(w.seed + 1000)
    dy = torch.randn((w.S, w.d), generator=g, device="cuda").to(torch.bfloat16)
    grads = run_backward(w, inputs, layer, dy, 0.01, 0.001)
    _whole_backward(w, inputs, layer, grads, dy, 0.01, 0.001)
    del layer, inputs, grads
    torch.cuda.empty_cache()


def _near_kink(host, idx_s, slot_s, s, rel=1e-5):
    """Whether token s has, in one of its kept experts, a hidden
    pre-activation u = W1_e x_s + b1_e (fp64) within rel * rms(u) of zero."""
    f64 = lambda a: (np.asarray(a).astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    x = f64(host["x"][s])
    for e, c in zip(idx_s, slot_s):
        if c < 0:
            continue
        u = f64(host["w1"][e]) @ x
        if host["b1"] is not None:
            u += f64(host["b1"][e])
        if np.abs(u).min() <= rel * np.sqrt(np.mean(u * u)):
            return True
    return False


def test_backward_saved_hidden_matches_recompute():
    """A forward that keeps its hidden activations, and a backward that reuses
    them, give the same forward outputs and the same gradients, bit for bit,
    as the recomputing backward; the saved buffer is left unchanged."""
    from sparse_moe_layer_wg_amd.layer import MoELayer
    for w in (BWD[0], BWD[3]):
        inputs = _with_biases(w, mw.generate(w, "cuda"), w.seed + 100)
        inputs, plain = run_layer(w, inputs, dispatch_buffer=False)
        cfg = plain.cfg
        kept = MoELayer.from_inputs(cfg, inputs, keep=True, dispatch_buffer=False,
                                    keep_hidden=True)
        kept.forward(inputs["x"])
        torch.cuda.synchronize()
        assert torch.equal(kept.y, plain.y)
        # expert outputs of the filled rows (padded rows are never written)
        if w.dropless:
            assert torch.equal(kept.out, plain.out)
        else:
            occ = np.minimum(plain.counts.cpu().numpy().sum(0), plain.C)
            filled = torch.from_numpy(np.arange(plain.C)[None, :] < occ[:, None]).cuda()
            assert torch.equal(kept.out[filled], plain.out[filled])
        saved = kept.hidden.clone()
        g = torch.Generator(device="cuda").manual_seed(w.seed + 300)
        dy = torch.randn((w.S, w.d), generator=g, device="cuda").to(torch.bfloat16)
        a = run_backward(w, inputs, plain, dy, 0.4, 0.2)
        b = run_backward(w, inputs, kept, dy, 0.4, 0.2, hidden=kept.hidden)
        for key in a:
            assert torch.equal(a[key], b[key]), (w.name, key)
        # bit patterns: rows past an expert's occupancy are never written and
        # hold whatever the allocation held, NaN patterns included
        assert torch.equal(kept.hidden.view(torch.int16), saved.view(torch.int16))


def test_backward_zero_upstream_gives_exact_zeros():
    """dy = 0 and zero loss weights: every gradient is exactly zero."""
    w = BWD[0]
    inputs, layer = run_layer(w, dispatch_buffer=False)
    dy = torch.zeros((w.S, w.d), dtype=torch.bfloat16, device="cuda")
    grads = run_backward(w, inputs, layer, dy, 0.0, 0.0)
    for key, t in grads.items():
        if t is not None:
            assert not torch.any(t != 0), key


def test_backward_deterministic():
    """Two backward calls are bit-identical."""
    w = BWD[2]
    inputs, layer = run_layer(w, dispatch_buffer=False)
    g = torch.Generator(device="cuda").manual_seed(7)
    dy = torch.randn((w.S, w.d), generator=g, device="cuda").to(torch.bfloat16)
    a = run_backward(w, inputs, layer, dy, 0.5, 0.5)
    b = run_backward(w, inputs, layer, dy, 0.5, 0.5)
    for key in a:
        if a[key] is not None:
            assert torch.equal(a[key], b[key]), key


def test_backward_empty_input():
    """S = 0: every weight gradient is zero."""
    cfg = moe.config(0, 64, 128, 4, 2, dtype="bf16")
    dev = "cuda"
    z = lambda *s, dt=torch.bfloat16: torch.zeros(s, dtype=dt, device=dev)
    grads = dict(dwg=torch.full((4, 64), 3.0, device=dev), dbg=torch.full((4,), 3.0, device=dev),
                 dw1=torch.full((4, 128, 64), 3.0, device=dev).to(torch.bfloat16),
                 db1=torch.full((4, 128), 3.0, device=dev).to(torch.bfloat16),
                 dw2=torch.full((4, 64, 128), 3.0, device=dev).to(torch.bfloat16),
                 db2=torch.full((4, 64), 3.0, device=dev).to(torch.bfloat16))
    ws = torch.empty(max(moe.backward_workspace_bytes(cfg), 256), dtype=torch.uint8, device=dev)
    moe.layer_backward(cfg, z(0, 64), z(4, 64, dt=torch.float32), z(4, 128, 64), None,
                       z(4, 64, 128), z(0, 4, dt=torch.float32), z(0, 2, dt=torch.int32),
                       z(0, 2, dt=torch.float32), z(0, 2, dt=torch.int32),
                       z(2, 4, dt=torch.int32), z(0, 64), z(0, 64), z(0, 64), grads["dwg"],
                       grads["dw1"], grads["dw2"], ws, db_gate=grads["dbg"], db1=grads["db1"],
                       db2=grads["db2"], g_aux=1.0, g_z=1.0)
    torch.cuda.synchronize()
    for key, t in grads.items():
        assert not torch.any(t != 0), key


@pytest.mark.parametrize("name,ntok,reroute", [("deepseek_bf16", 6, False),
                                               ("skewed_bf16", 16, True)])
def test_backward_full_size_sampled(name, ntok, reroute):
    """Full-size workloads in the training benchmark's configuration (fused
    gather in the forward, the benchmark's loss weights).  dx rows of sampled
    tokens and sampled entries of dW1, dW2, db1, db2 are computed one by one
    by the oracle; the router gradients dWg (sampled columns) and dbg come
    from the oracle's logit gradient for all tokens, given the forward's
    expert outputs.  The skewed workload runs with overflow re-routing."""
    w = mw.get(name).with_(reroute=reroute)
    print(f"\n[bwd full] {w}", flush=True)
    inputs, layer = run_layer(w, dispatch_buffer=False)
    g = torch.Generator(device="cuda").manual_seed(w.seed + 1000)
    dy = torch.randn((w.S, w.d), generator=g, device="cuda").to(torch.bfloat16)
    g_aux, g_z = 0.01, 0.001
    grads = run_backward(w, inputs, layer, dy, g_aux, g_z)
    host = {n: mw.to_numpy(t) for n, t in inputs.items()}
    lg = layer.logits.cpu().numpy()
    dy_h = mw.to_numpy(dy)
    rng = np.random.default_rng(w.seed)
    tok = np.sort(rng.choice(w.S, ntok, replace=False))
    counts = layer.counts.cpu().numpy()
    nonempty = np.nonzero(counts.sum(0) > 0)[0]
    ents = []
    for kind, na, nb in ((1, w.h, w.d), (2, w.d, w.h), (3, w.h, 1), (4, w.d, 1)):
        for _ in range(48):
            ents.append((kind, int(rng.choice(nonempty)), int(rng.integers(na)),
                         int(rng.integers(nb))))
    rows, vals = oracle.backward_entries(host["x"], host["wg"], host["w1"], host["b1"],
                                         host["w2"], host["b2"], w.k, layer.C, lg, dy_h, g_aux,
                                         g_z, tok, ents, reroute=w.reroute)
    rep = {"dx_rows": rel_fro(as_f64(grads["dx"][torch.from_numpy(tok).cuda()]), rows)}
    gpu = {1: as_f64(grads["dw1"]), 2: as_f64(grads["dw2"]), 3: as_f64(grads["db1"]),
           4: as_f64(grads["db2"])}
    for kind, key in ((1, "dw1"), (2, "dw2"), (3, "db1"), (4, "db2")):
        sel = [i for i, e in enumerate(ents) if e[0] == kind]
        got = [gpu[kind][ents[i][1], ents[i][2], ents[i][3]] if kind <= 2 else
               gpu[kind][ents[i][1], ents[i][2]] for i in sel]
        rep[key] = rel_fro(got, vals[sel])

    # router: the logit gradient for every token from the forward's own
    # expert outputs (dw = dy . out row), then dbg and sampled dWg columns
    r = oracle.route(lg, w.k, layer.C, w.reroute)
    out = layer.out.reshape(-1, w.d)
    slot, idx = r["slot"], r["serve"]
    dwk = np.zeros((w.S, w.k))
    for s0 in range(0, w.S, 1024):
        sl = slice(s0, min(w.S, s0 + 1024))
        for rr in range(w.k):
            keep = slot[sl, rr] >= 0
            u = idx[sl, rr].astype(np.int64) * layer.C + slot[sl, rr]
            u_t = torch.from_numpy(np.where(keep, u, 0)).cuda()
            o = as_f64(out[u_t])
            dwk[sl, rr] = np.where(keep, np.einsum("ij,ij->i", o, dy_h_f64(dy_h[sl])), 0.0)
    dl = oracle.router_backward(lg, r["idx"], r["w"], dwk, counts[:w.k], g_aux, g_z)
    rep["dbg"] = rel_fro(as_f64(grads["dbg"]), dl.sum(0))
    cols = np.sort(rng.choice(w.d, 128, replace=False))
    x64 = dy_h_f64(host["x"][:, cols])
    rep["dwg_cols"] = rel_fro(as_f64(grads["dwg"])[:, cols], dl.T @ x64)
    _print(name + "_bwd", rep)
    for key, err in rep.items():
        assert err <= TOL, (key, rep)
    del layer, inputs, grads
    torch.cuda.empty_cache()


def dy_h_f64(a):
    """bf16 bit patterns (uint16) as float64."""
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_backward_replays_in_a_hip_graph():
    """moe_layer_backward enqueues kernels only, so a forward + backward step
    can be captured in a HIP graph: every replay, with new upstream
    gradients and eager work between replays, equals an eager step bit for
    bit."""
    from sparse_moe_layer_wg_amd.layer import MoELayer
    w = BWD[0]
    inputs = _with_biases(w, mw.generate(w, "cuda"), w.seed + 100)
    cfg = moe.config(w.S, w.d, w.h, w.E, w.k, w.capacity_factor, dtype=w.dtype)
    layers = [MoELayer.from_inputs(cfg, inputs, keep=True, dispatch_buffer=False,
                                   keep_hidden=True) for _ in range(2)]
    dys = [torch.zeros((w.S, w.d), dtype=torch.bfloat16, device="cuda") for _ in range(2)]
    grads = [None, None]

    def step(i):
        layers[i].forward(inputs["x"])
        grads[i] = run_backward_nosync(w, inputs, layers[i], dys[i], 0.7, 0.3,
                                       hidden=layers[i].hidden, out=grads[i])

    stream = torch.cuda.Stream()
    stream.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(stream):
        step(1)                              # warm-up outside the capture (allocates)
    torch.cuda.current_stream().wait_stream(stream)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(1)
    g = torch.Generator(device="cuda").manual_seed(9)
    for rep in range(3):
        dy = torch.randn((w.S, w.d), generator=g, device="cuda").to(torch.bfloat16)
        dys[1].copy_(dy)
        dys[0].copy_(dy)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        step(0)
        torch.cuda.synchronize()
        for key in grads[0]:
            if key != "ws" and grads[0][key] is not None:   # (ws: scratch)
                assert torch.equal(grads[0][key], grads[1][key]), (rep, key)


def run_backward_nosync(w, inputs, layer, dy, g_aux, g_z, hidden=None, out=None):
    """moe_layer_backward into the buffers of `out` (allocated when None),
    without a host synchronisation (so that it can be captured)."""
    cfg = layer.cfg
    E, d, h = w.E, w.d, w.h
    dev, at = "cuda", torch.bfloat16
    if out is None:
        out = dict(dx=torch.empty((w.S, d), dtype=at, device=dev),
                   dwg=torch.empty((E, d), dtype=torch.float32, device=dev),
                   dbg=torch.empty((E,), dtype=torch.float32, device=dev),
                   dw1=torch.empty((E, h, d), dtype=at, device=dev),
                   db1=torch.empty((E, h), dtype=at, device=dev),
                   dw2=torch.empty((E, d, h), dtype=at, device=dev),
                   db2=torch.empty((E, d), dtype=at, device=dev),
                   ws=torch.empty(moe.backward_workspace_bytes(cfg), dtype=torch.uint8,
                                  device=dev))
    moe.layer_backward(cfg, inputs["x"], inputs["wg"], inputs["w1"], inputs["b1"], inputs["w2"],
                       layer.logits, layer.topk_idx, layer.topk_w, layer.slot, layer.counts,
                       layer.out, dy, out["dx"], out["dwg"], out["dw1"], out["dw2"], out["ws"],
                       db_gate=out["dbg"], db1=out["db1"], db2=out["db2"], g_aux=g_aux, g_z=g_z,
                       hidden=hidden)
    return out
