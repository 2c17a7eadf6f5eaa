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
# every single row (of y, of the expert outputs) within this multiple of the
# whole-tensor bar: a lost, doubled or misplaced GEMM tile shows up in the
# rows it covers even where the whole-tensor error would stay below the bar
ROW_FACTOR = 3.0
LOSS_TOL = 1e-5
AGREEMENT = 0.9999


def rel_fro(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (nb if nb > 0 else 1.0))


def row_rel(a, b) -> np.ndarray:
    """Relative error of every row (last axis) of a against b.  A row that is
    zero in b must be exactly zero in a (error 0, else inf)."""
    a = np.asarray(a, np.float64).reshape(-1, np.shape(a)[-1])
    b = np.asarray(b, np.float64).reshape(-1, np.shape(b)[-1])
    num = np.linalg.norm(a - b, axis=1)
    den = np.linalg.norm(b, axis=1)
    safe = np.where(den > 0, den, 1.0)
    return np.where(den > 0, num / safe, np.where(num == 0, 0.0, np.inf))


def check_rows(rep: dict, key: str, a, b, tol: float):
    """Whole-tensor relative Frobenius error and the largest row error, both
    recorded in rep and asserted against tol and ROW_FACTOR * tol."""
    rep[key + "_rel"] = rel_fro(a, b)
    rows = row_rel(a, b)
    rep[key + "_row_max"] = float(rows.max()) if rows.size else 0.0
    rep[key + "_rows"] = int(rows.size)
    assert rep[key + "_rel"] <= tol, rep
    assert rep[key + "_row_max"] <= ROW_FACTOR * tol, rep


def expert_ffn_chunked(xd, occ, w1, b1, w2, b2, chunk_flop: float = 1.5e12) -> np.ndarray:
    """oracle.expert_ffn over groups of experts, printing a line after each
    group (a full-size check runs the oracle for minutes)."""
    import time
    E, C, d = xd.shape
    h = w1.shape[1]
    out = np.zeros((E, C, d), np.float64)
    t0 = time.perf_counter()
    e0 = 0
    while e0 < E:
        e1, fl = e0, 0.0
        while e1 < E and (e1 == e0 or fl + 4.0 * d * h * occ[e1] <= chunk_flop):
            fl += 4.0 * d * h * occ[e1]
            e1 += 1
        out[e0:e1] = oracle.expert_ffn(xd[e0:e1], occ[e0:e1], w1[e0:e1],
                                       None if b1 is None else b1[e0:e1], w2[e0:e1],
                                       None if b2 is None else b2[e0:e1])
        if E > 1:
            print(f"  oracle experts {e0}..{e1 - 1} of {E}: {time.perf_counter() - t0:.1f} s",
                  flush=True)
        e0 = e1
    return out


def router_margin(x, wg, bg) -> np.ndarray:
    """Per-token refinement margin of the router, as the library defines it:
    tau_s = 32 * 2^-24 * (|x_s| * max_j |wg_j| + max_j |bg_j| / 8)."""
    x = np.asarray(x)
    x64 = ((x.astype(np.uint32) << 16).view(np.float32) if x.dtype == np.uint16 else x)
    x64 = x64.astype(np.float64)
    wmax = np.sqrt((np.asarray(wg, np.float64) ** 2).sum(axis=1).max())
    bmax = 0.0 if bg is None else float(np.abs(np.asarray(bg, np.float64)).max())
    return 32.0 * 2.0 ** -24 * (np.sqrt((x64 ** 2).sum(axis=1)) * wmax + bmax / 8.0)


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
        out_or = expert_ffn_chunked(xd_or, occ, host["w1"], host["b1"], host["w2"], host["b2"])
        del xd_or
        check_rows(rep, "out", as_f64(out_gpu)[filled], out_or[filled], tol)
        y_or = oracle.combine(out_or, r["serve"], r["slot"], r["w"], S)
        del out_or
        check_rows(rep, "y", y_gpu, y_or, tol)
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
    check_rows(rep, "y", y_gpu[tok], y_or, tol)
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
    err = np.abs(lg.astype(np.float64) - lg_or)
    rep["logit_max_abs_err"] = float(err.max()) if err.size else 0.0
    # The router re-evaluates in fp64 every top-k decision of token s closer
    # than its margin tau_s; that is exact only while the logit error stays
    # well below tau_s / 2.
    tau = router_margin(host["x"], host["wg"], host["bg"])
    # (a zero margin means exact logits: an all-zero router and no bias)
    emax = err.max(axis=1) if err.size else np.zeros(0)
    ratio = np.where(tau > 0, emax / np.where(tau > 0, tau, 1.0), np.where(emax == 0, 0.0, np.inf))
    rep["logit_err_over_tau"] = float(ratio.max()) if ratio.size else 0.0
    assert rep["logit_err_over_tau"] < 0.25, rep
    r_or = oracle.route(lg_or, w.k, layer.C, w.reroute)
    agree = np.all(layer.topk_idx.cpu().numpy() == r_or["serve"], axis=1)
    rep["topk_agreement"] = float(agree.mean())
    rep["topk_mismatches"] = int((~agree).sum())
    assert rep["topk_agreement"] >= AGREEMENT, rep
    return host


def dropless_whole(w, host, layer, r, rows, rep, tol):
    """Every compact expert-output row and every row of y of a dropless run
    against the oracle, without the oracle's [E, S, d] buffers (too large at
    full size): each group of experts' rows go through oracle.expert_ffn as
    compact [n_e, d] blocks, and y is the routing weights' sum of those rows
    (the combine step's definition)."""
    import time
    S, k, E, d = w.S, w.k, w.E, w.d
    n = np.bincount(r["idx"].reshape(-1), minlength=E)
    seg = np.concatenate([[0], np.cumsum(n)[:-1]])
    x = host["x"]
    out_or = np.zeros((S * k, d), np.float64)
    tok_of_row = np.empty(S * k, np.int64)
    tok_of_row[rows.reshape(-1)] = np.repeat(np.arange(S), k)
    t0 = time.perf_counter()
    e0 = 0
    while e0 < E:
        e1, fl = e0, 0.0
        while e1 < E and (e1 == e0 or fl + 4.0 * d * w.h * n[e1] <= 1.5e12):
            fl += 4.0 * d * w.h * n[e1]
            e1 += 1
        m = int(n[e0:e1].max()) if e1 > e0 else 0
        if m > 0:
            xd = np.zeros((e1 - e0, m, d), x.dtype)
            for e in range(e0, e1):
                xd[e - e0, :n[e]] = x[tok_of_row[seg[e]:seg[e] + n[e]]]
            o = oracle.expert_ffn(xd, n[e0:e1].astype(np.int32), host["w1"][e0:e1],
                                  None if host["b1"] is None else host["b1"][e0:e1],
                                  host["w2"][e0:e1],
                                  None if host["b2"] is None else host["b2"][e0:e1])
            for e in range(e0, e1):
                out_or[seg[e]:seg[e] + n[e]] = o[e - e0, :n[e]]
        print(f"  oracle experts {e0}..{e1 - 1} of {E}: {time.perf_counter() - t0:.1f} s",
              flush=True)
        e0 = e1
    check_rows(rep, "out", as_f64(layer.out), out_or, tol)
    y_or = np.zeros((S, d), np.float64)
    for rr in range(k):
        y_or += r["w"][:, rr:rr + 1].astype(np.float64) * out_or[rows[:, rr]]
    check_rows(rep, "y", as_f64(layer.y), y_or, tol)
    return rep


def _check_dropless(w, inputs, layer, r, full, n_sample, seed, rep):
    """Dropless run: every assignment kept; compact [S*k,d] buffers."""
    tol = TOL[w.dtype]
    host = _check_routing_outputs(w, inputs, layer, r, rep)
    rep["drops"] = 0
    rows = oracle.compact_rows(r["idx"], w.E)
    y_gpu = as_f64(layer.y)
    # the oracle's padded [E, S, d] fp64 buffers above 2 GiB: compact blocks
    if full and 8 * w.S * w.E * w.d > (1 << 31):
        return dropless_whole(w, host, layer, r, rows, rep, tol)
    if full:
        res = oracle.layer_dropless(host["x"], host["wg"], host["bg"], host["w1"], host["b1"],
                                    host["w2"], host["b2"], w.k, lg=layer.logits.cpu().numpy())
        assert np.array_equal(res["rows"], rows)
        if layer.xd is not None:
            assert np.array_equal(mw.to_numpy(layer.xd), res["xd_rows"]), \
                "compact dispatch buffer is not a bit copy"
        check_rows(rep, "out", as_f64(layer.out), res["out_rows"], tol)
        check_rows(rep, "y", y_gpu, res["y"], tol)
        return rep
    rng = np.random.default_rng(seed)
    tok = np.sort(rng.choice(w.S, size=min(n_sample, w.S), replace=False))
    if layer.xd is not None:
        for s in tok[:32]:
            for rr in range(w.k):
                assert np.array_equal(mw.to_numpy(layer.xd[rows[s, rr]]), host["x"][s])
    y_or = oracle.token_output(tok, host["x"], host["w1"], host["b1"], host["w2"], host["b2"],
                               r["idx"], r["slot"], r["w"])
    check_rows(rep, "y", y_gpu[tok], y_or, tol)
    return rep
