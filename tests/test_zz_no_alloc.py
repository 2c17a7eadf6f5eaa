"""moe_gate_noalloc (the router entry point that uses the library's static
device scratch instead of a caller workspace) against moe_gate, through the
C ABI: two calls in a row, the second on a smaller input, each compared with
moe_gate on the same inputs (routing, slots, counts bit for bit; weights,
losses and logits bit for bit too, since both run the same kernels) and with
the oracle's routing from the same logits."""
import numpy as np
import pytest
import torch

import moe_workloads as mw
import oracle
import sparse_moe_layer_wg_amd as moe

pytestmark = pytest.mark.gpu


def _outputs(cfg):
    dev = "cuda"
    S, E, k = cfg.S, cfg.E, cfg.k
    return dict(logits=torch.full((S, E), 5.0, device=dev),
                topk_idx=torch.full((S, k), -7, dtype=torch.int32, device=dev),
                topk_w=torch.full((S, k), 5.0, device=dev),
                slot=torch.full((S, k), -7, dtype=torch.int32, device=dev),
                counts=torch.full((cfg.count_rows, E), -7, dtype=torch.int32, device=dev),
                losses=torch.full((2,), 5.0, device=dev))


def _run(w, reroute=False):
    print(f"\n[noalloc] {w} reroute={reroute}", flush=True)
    inp = mw.generate(w, "cuda")
    cfg = moe.config(w.S, w.d, w.h, w.E, w.k, w.capacity_factor, dtype=w.dtype,
                     reroute=reroute)
    ref, got = _outputs(cfg), _outputs(cfg)
    ws = torch.empty(moe.workspace_bytes(cfg), dtype=torch.uint8, device="cuda")
    moe.gate(cfg, inp["x"], inp["wg"], inp["bg"], ref["logits"], ref["topk_idx"],
             ref["topk_w"], ref["slot"], ref["counts"], ref["losses"], ws)
    moe.gate_noalloc(cfg, inp["x"], inp["wg"], inp["bg"], got["logits"], got["topk_idx"],
                     got["topk_w"], got["slot"], got["counts"], got["losses"])
    torch.cuda.synchronize()
    for name in ref:
        assert torch.equal(ref[name], got[name]), name
    r = oracle.route(got["logits"].cpu().numpy(), w.k, moe.capacity(cfg), reroute)
    assert np.array_equal(got["topk_idx"].cpu().numpy(), r["serve"])
    assert np.array_equal(got["slot"].cpu().numpy(), r["slot"])
    assert np.array_equal(got["counts"].cpu().numpy(), r["counts"])
    return got


def test_noalloc_gate_two_calls_second_smaller():
    big = mw.get("balanced_bf16")
    small = mw.Workload("noalloc_small", S=1000, d=256, h=256, E=16, k=2, capacity_factor=1.0,
                        dtype="bf16", seed=61)
    _run(big)
    _run(small)


def test_noalloc_gate_logits_kept_in_scratch_and_reroute():
    """logits NULL (kept in the static scratch), then re-routing on a skewed
    shape whose drops are offered to other experts."""
    w = mw.get("deepseek_bf16")
    inp = mw.generate(w, "cuda")
    cfg = moe.config(w.S, w.d, w.h, w.E, w.k, w.capacity_factor, dtype=w.dtype)
    ref, got = _outputs(cfg), _outputs(cfg)
    ws = torch.empty(moe.workspace_bytes(cfg), dtype=torch.uint8, device="cuda")
    moe.gate(cfg, inp["x"], inp["wg"], None, None, ref["topk_idx"], ref["topk_w"], ref["slot"],
             ref["counts"], ref["losses"], ws)
    moe.gate_noalloc(cfg, inp["x"], inp["wg"], None, None, got["topk_idx"], got["topk_w"],
                     got["slot"], got["counts"], got["losses"])
    torch.cuda.synchronize()
    for name in ("topk_idx", "topk_w", "slot", "counts", "losses"):
        assert torch.equal(ref[name], got[name]), name
    _run(mw.Workload("noalloc_skew", S=3000, d=256, h=256, E=32, k=2, capacity_factor=1.0,
                     dtype="bf16", seed=62, gate_bias="zipf1.2"), reroute=True)
