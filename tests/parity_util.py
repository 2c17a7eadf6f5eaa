"""Helpers shared by the GPU parity tests: run the HIP layer on a workload and
compare every output with the CPU oracle.

Bars (see the module docstrings of the tests): routing indices, slots,
counts and drop masks bit-exact given the GPU's fp32 logits; end-to-end
ordered top-k agreement with the oracle's own logits >= 99.99% of tokens;
dispatch buffers bit-exact; expert outputs and y within relative Frobenius
error 1e-5 (fp32) or 1e-2 (bf16) of the oracle run on the GPU's routing;
losses within relative error 1e-5.
"""
from __future__ import annotations

import numpy as np
import torch

import moe_workloads as mw
import oracle
import sparse_moe_layer_wg_amd as moe
from sparse_moe_layer_wg_amd.layer import MoELayer

TOL = {"f32": 1e-5, "bf16": 1e-2}
LOSS_TOL = 1e-5
AGREEMENT = 0.9999


def rel_fro(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


def as_f64(t) -> np.ndarray:
    """Device/host tensor (fp32 or bf16) as a float64 numpy array."""
    return t.detach().to("cpu", torch.float64).numpy() if isinstance(t, torch.Tensor) \
        else np.asarray(t, np.float64)


def cfg_of(w: mw.Workload):
    return moe.config(w.S, w.d, w.h, w.E, w.k, w.capacity_factor, dtype=w.dtype,
                      dropless=w.dropless, reroute=w.reroute)


def run_layer(w: mw.Workload, inputs=None, dispatch_buffer=True):
    """Generate inputs on the GPU and run moe_layer_forward keeping every
    output (without the dispatch buffer when ``dispatch_buffer`` is False:
    then bf16 layers gather token rows inside the first expert GEMM)."""
    inputs = inputs or mw.generate(w, "cuda")
    layer = MoELayer.from_inputs(cfg_of(w), inputs, keep=True, dispatch_buffer=dispatch_buffer)
    layer.forward(inputs["x"])
    torch.cuda.synchronize()
    return inputs, layer


def check_layer(w: mw.Workload, inputs, layer, full: bool, n_sample: int = 96, seed: int = 0,
                report: dict | None = None):
    """Compare one finished layer run with the oracle.  ``full`` runs the
    oracle over every slot; otherwise rows are sampled.  A dropless layer is
    routed with a capacity of S (never reached) and its slots are the compact
    rows of the oracle's (expert, rank, token) order.  With re-routing the
    layer's topk_idx names each assignment's serving expert (the oracle's
    ``serve``) and counts has the extra row of accepted offers."""
    rep = {} if report is None else report
    S, E, k = w.S, w.E, w.k
    C = layer.C
    if w.dropless:
        assert C == S
    tol = TOL[w.dtype]

    # routing from the GPU's own fp32 logits: integer outputs bit-exact
    r = oracle.route(layer.logits.cpu().numpy(), k, C, w.reroute)
    idx = layer.topk_idx.cpu().numpy()
    slot = layer.slot.cpu().numpy()
    assert np.array_equal(idx, r["serve"]), "top-k (serving) indices differ from the oracle"
    if w.dropless:
        assert (r["slot"] >= 0).all()
        assert np.array_equal(slot, oracle.compact_rows(r["idx"], E)), \
            "dropless rows differ from the oracle"
        return _check_dropless(w, inputs, layer, r, full, n_sample, seed, rep)
    assert np.array_equal(slot, r["slot"]), "slots / drop mask differ from the oracle"
    host = _check_routing_outputs(w, inputs, layer, r, rep)
    rep["drops"] = int((slot < 0).sum())

    if w.reroute:
        rep["rerouted"] = int((r["serve"] != r["idx"]).sum())
    occ = oracle.occupancy(r["counts"], C, k)
    xd_gpu = layer.xd
    out_gpu = layer.out
    y_gpu = as_f64(layer.y)
    if full:
        xd_or = oracle.dispatch(host["x"], r["serve"], r["slot"], E, C)
        filled = np.arange(C)[None, :] < occ[:, None]
        if xd_gpu is not None:
            xd_h = mw.to_numpy(xd_gpu)
            assert np.array_equal(xd_h[filled], xd_or[filled]), "dispatch buffer is not a bit copy"
        out_or = oracle.expert_ffn(xd_or, occ, host["w1"], host["b1"], host["w2"], host["b2"])
        rep["out_rel"] = rel_fro(as_f64(out_gpu)[filled], out_or[filled])
        assert rep["out_rel"] <= tol, rep
        y_or = oracle.combine(out_or, r["serve"], r["slot"], r["w"], S)
        rep["y_rel"] = rel_fro(y_gpu, y_or)
        assert rep["y_rel"] <= tol, rep
        dropped_all = (r["slot"] < 0).all(axis=1)
        assert np.all(y_gpu[dropped_all] == 0)
        return rep

    # sampled: tokens, including some with drops, checked row by row
    rng = np.random.default_rng(seed)
    tok = rng.choice(S, size=min(n_sample, S), replace=False)
    with_drop = np.nonzero((r["slot"] < 0).any(axis=1))[0]
    if with_drop.size:
        tok = np.unique(np.concatenate([tok, rng.choice(with_drop, size=min(16, with_drop.size),
                                                        replace=False)]))
    tok = np.sort(tok)
    # dispatch rows of the sampled tokens are bit copies of x
    for s in (tok[:32] if xd_gpu is not None else []):
        for rr in range(k):
            c = r["slot"][s, rr]
            if c >= 0:
                row = mw.to_numpy(xd_gpu[r["serve"][s, rr], c])
                assert np.array_equal(row, host["x"][s]), "dispatch row differs"
    y_or = oracle.token_output(tok, host["x"], host["w1"], host["b1"], host["w2"], host["b2"],
                               r["serve"], r["slot"], r["w"])
    rep["y_rel"] = rel_fro(y_gpu[tok], y_or)
    assert rep["y_rel"] <= tol, rep
    return rep


def _check_routing_outputs(w, inputs, layer, r, rep):
    """Counts, weights and losses given the GPU's logits, and end-to-end top-k
    agreement with the oracle's own logits."""
    host = {n: mw.to_numpy(t) for n, t in inputs.items()}
    counts = layer.counts.cpu().numpy()
    losses = layer.losses.cpu().numpy()
    assert np.array_equal(counts, r["counts"]), "per-rank counts differ from the oracle"
    rep["w_rel"] = rel_fro(layer.topk_w.cpu().numpy(), r["w"])
    assert rep["w_rel"] <= 1e-5
    rep["aux"], rep["z"] = float(losses[0]), float(losses[1])
    assert abs(losses[0] - r["aux"]) <= LOSS_TOL * abs(r["aux"]), (losses[0], r["aux"])
    assert abs(losses[1] - r["z"]) <= LOSS_TOL * abs(r["z"]), (losses[1], r["z"])
    lg = layer.logits.cpu().numpy()
    lg_or = oracle.logits(host["x"], host["wg"], host["bg"])
    rep["logit_max_abs_err"] = float(np.abs(lg.astype(np.float64) - lg_or).max())
    # The router re-evaluates in fp64 every top-k decision closer than
    # tau = 32 * sqrt(d) * 2^-24; that is exact only while the logit error
    # stays well below tau / 2.
    tau = 32.0 * np.sqrt(w.d) * 2.0 ** -24
    rep["logit_err_over_tau"] = rep["logit_max_abs_err"] / tau
    assert rep["logit_err_over_tau"] < 0.25, rep
    r_or = oracle.route(lg_or, w.k, layer.C, w.reroute)
    agree = np.all(layer.topk_idx.cpu().numpy() == r_or["serve"], axis=1)
    rep["topk_agreement"] = float(agree.mean())
    rep["topk_mismatches"] = int((~agree).sum())
    assert rep["topk_agreement"] >= AGREEMENT, rep
    return host


def _check_dropless(w, inputs, layer, r, full, n_sample, seed, rep):
    """Dropless run: every assignment kept; compact [S*k,d] buffers."""
    tol = TOL[w.dtype]
    host = _check_routing_outputs(w, inputs, layer, r, rep)
    rep["drops"] = 0
    rows = oracle.compact_rows(r["idx"], w.E)
    y_gpu = as_f64(layer.y)
    if full:
        res = oracle.layer_dropless(host["x"], host["wg"], host["bg"], host["w1"], host["b1"],
                                    host["w2"], host["b2"], w.k, lg=layer.logits.cpu().numpy())
        assert np.array_equal(res["rows"], rows)
        if layer.xd is not None:
            assert np.array_equal(mw.to_numpy(layer.xd), res["xd_rows"]), \
                "compact dispatch buffer is not a bit copy"
        rep["out_rel"] = rel_fro(as_f64(layer.out), res["out_rows"])
        assert rep["out_rel"] <= tol, rep
        rep["y_rel"] = rel_fro(y_gpu, res["y"])
        assert rep["y_rel"] <= tol, rep
        return rep
    rng = np.random.default_rng(seed)
    tok = np.sort(rng.choice(w.S, size=min(n_sample, w.S), replace=False))
    if layer.xd is not None:
        for s in tok[:32]:
            for rr in range(w.k):
                assert np.array_equal(mw.to_numpy(layer.xd[rows[s, rr]]), host["x"][s])
    y_or = oracle.token_output(tok, host["x"], host["w1"], host["b1"], host["w2"], host["b2"],
                               r["idx"], r["slot"], r["w"])
    rep["y_rel"] = rel_fro(y_gpu[tok], y_or)
    assert rep["y_rel"] <= tol, rep
    return rep
