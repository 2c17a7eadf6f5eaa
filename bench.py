"""Benchmark of the MI355X GShard MoE-layer forward (one GPU).

One step = one moe_layer_forward over one batch of S synthetic tokens: router
logits, softmax, top-k, capacity slots, dispatch (for bf16, a row gather fused
into the first expert GEMM), both expert GEMMs, combine, aux loss and z-loss.  Inputs are resident in HBM before timing starts.

Prints ONE JSON line.  ``value`` = tokens per second of the whole layer.
The expert GEMMs are timed by HIP events recorded around them on the launch
stream inside the timed region; a per-stage breakdown comes from a few
extra steps with every stage boundary recorded.  ``roofline`` describes the
slowest kernel (an expert GEMM); ``cpu_baseline`` times the CPU oracle on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

import moe_workloads as mw  # noqa: E402
import sparse_moe_layer_wg_amd as moe  # noqa: E402
from sparse_moe_layer_wg_amd.layer import MoELayer  # noqa: E402

METRIC = "MoE-layer tokens/s (gate+dispatch+FFN+combine); % bf16 MFMA peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_PEAK_TFLOPS = {"bf16": 2500.0, "f32": 157.3}   # dense, TFLOP/s
STAGES = ["gate_logits", "route", "slot_scan", "slot_positions", "dispatch", "expert_gemm1",
          "expert_gemm2", "combine"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    # default: the largest single-GPU workload, where the expert GEMMs are
    # bound by the matrix cores rather than by streaming the weights
    ap.add_argument("--workload", default="large_bf16", choices=mw.ORDER)
    ap.add_argument("--dropless", action="store_true",
                    help="no capacity limit: compact [S*k,d] expert segments, no drops")
    ap.add_argument("--reroute", action="store_true",
                    help="offer dropped assignments to the tokens' next-ranked experts")
    ap.add_argument("--backward", action="store_true",
                    help="time a training step: forward + moe_layer_backward")
    ap.add_argument("--ep-share", default=None, choices=list(mw.EP_SHARES),
                    help="time the expert FFN at one GPU's expert-parallel share instead")
    ap.add_argument("--vendor-gemm", action="store_true",
                    help="time the expert FFN at uniform occupancy (S*k/E rows per expert) "
                         "against the same GEMMs through hipBLASLt (torch.bmm)")
    ap.add_argument("--copy-reference", action="store_true",
                    help="time plain device-to-device copies (read + write) of 64 MiB to "
                         "1 GiB: the HBM rate a streaming kernel can reach on this GPU")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--copy-calibration-mb", type=int, default=0,
                    help="after timing, run one plain device copy of this many MiB "
                         "(reference kernel for the FETCH_SIZE/WRITE_SIZE counters)")
    return ap.parse_args()


def source_sha(name: str) -> str:
    import hashlib
    path = os.path.join(ROOT, "sparse_moe_layer_wg_amd", "csrc", name)
    return hashlib.sha256(open(path, "rb").read()).hexdigest()


def measured_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` from the committed counter summary
    (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy of known size), or None
    when there is none or the kernel's source file has changed since the
    counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        entries = json.load(open(path))
    except ValueError:
        return None
    for ent in entries:
        if ent.get("workload") == workload and ent.get("kernel") == kernel:
            if ent.get("source_sha256") != source_sha(ent.get("source", "gemm.hip")):
                return None
            return float(ent["fetch_bytes"]) + float(ent["write_bytes"])
    return None


def algorithmic_work(w: mw.Workload, occ: np.ndarray, kept: int) -> dict:
    """Bytes and FLOPs the method must move / do, per launch of each kernel.
    GEMM weights count only for experts with at least one filled slot."""
    es = 2 if w.dtype == "bf16" else 4
    nonempty = int((occ > 0).sum())
    S, d, h, E, k = w.S, w.d, w.h, w.E, w.k
    return {
        "expert_gemm1": dict(flops=2.0 * kept * d * h,
                             bytes=nonempty * h * d * es + kept * d * es + kept * h * es),
        "expert_gemm2": dict(flops=2.0 * kept * d * h,
                             bytes=nonempty * d * h * es + kept * h * es + kept * d * es),
        "dispatch": dict(flops=0.0, bytes=S * d * es + kept * d * es),
        "combine": dict(flops=2.0 * kept * d, bytes=kept * d * es + S * d * es),
        "gate_logits": dict(flops=2.0 * S * d * E, bytes=S * d * es + E * d * 4 + S * E * 4),
    }


ROTATE_BYTES = 512 * 2 ** 20


def rotated(t: torch.Tensor, budget: int = ROTATE_BYTES) -> list:
    """Identical copies of t at distinct addresses, enough that one pass over
    them (at least 512 MiB) exceeds the 256 MB last-level cache: step i reads
    copy i % len, so no step finds its inputs left in cache by the previous
    one."""
    n = max(1, min(16, -(-budget // max(1, t.numel() * t.element_size()))))
    return [t] + [t.clone() for _ in range(n - 1)]


def filled_rows(counts: np.ndarray, C: int, k: int) -> np.ndarray:
    """Rows each expert holds: min(assignments, C), plus the accepted
    re-routed assignments when counts carries that extra row."""
    occ = np.minimum(counts[:k].sum(0), C)
    return occ + counts[k] if counts.shape[0] > k else occ


def host_cpu() -> dict:
    """The host the CPU baseline runs on: CPU model (lscpu), OMP_NUM_THREADS
    and the number of cores this process may run on."""
    import subprocess
    model = None
    try:
        out = subprocess.run(["lscpu"], capture_output=True, text=True, timeout=10).stdout
        for line in out.splitlines():
            if line.startswith("Model name:"):
                model = line.split(":", 1)[1].strip()
                break
    except (OSError, subprocess.SubprocessError):
        pass
    if model is None:
        try:
            for line in open("/proc/cpuinfo"):
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
        except OSError:
            pass
    return {"cpu_model": model, "omp_num_threads": os.environ.get("OMP_NUM_THREADS"),
            "affinity_cores": len(os.sched_getaffinity(0)), "os_cpu_count": os.cpu_count()}


def oracle_threads() -> int:
    """Threads the OpenMP oracle runs with: OMP_NUM_THREADS when set, else
    libgomp's default, one per core in the affinity mask."""
    return int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))


def cpu_baseline(w: mw.Workload, inputs: dict, target_s: float, backward=False) -> dict:
    import oracle
    host = {n: mw.to_numpy(t) for n, t in inputs.items()}
    dy = host["x"][::-1].copy()     # any fixed upstream gradient of the right shape

    def run(n):
        C = n if w.dropless else oracle.capacity(n, w.E, w.k, w.capacity_factor)
        t0 = time.perf_counter()
        if backward:
            lg = oracle.logits(host["x"][:n], host["wg"], host["bg"])
            oracle.layer(host["x"][:n], host["wg"], host["bg"], host["w1"], host["b1"],
                         host["w2"], host["b2"], w.k, max(C, 1), lg=lg, reroute=w.reroute)
            oracle.layer_backward(host["x"][:n], host["wg"], host["w1"], host["b1"], host["w2"],
                                  host["b2"], w.k, max(C, 1), lg, dy[:n], 0.01, 0.001,
                                  reroute=w.reroute)
        elif w.dropless:
            oracle.layer_dropless(host["x"][:n], host["wg"], host["bg"], host["w1"], host["b1"],
                                  host["w2"], host["b2"], w.k)
        else:
            oracle.layer(host["x"][:n], host["wg"], host["bg"], host["w1"], host["b1"],
                         host["w2"], host["b2"], w.k, C, reroute=w.reroute)
        return time.perf_counter() - t0

    n0 = min(w.S, 256)
    t0 = run(n0)
    n = int(min(w.S, max(n0, n0 * target_s / max(t0, 1e-3))))
    n = max(64, (n // 64) * 64) if n >= 64 else n
    t = run(n) if n != n0 else t0
    return {"value": n / t, "unit": "tokens/s", "cores": oracle_threads(), "kind": "oracle",
            "host": host_cpu(),
            "sample": f"first {n} of the {w.S} tokens of the same workload (same E, d, h, k, "
                      + ("dropless routing" if w.dropless else
                         "capacity_factor; C scaled with the sample"
                         + (", overflow re-routing" if w.reroute else ""))
                      + "), full fp64 oracle layer from logits to y"
                      + (" plus its backward" if backward else "") + f", {t:.1f} s"}


def main():
    a = parse()
    if a.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {a.gpus} is not supported "
              f"(the layer has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if a.ep_share:
        out = bench_ep_share(a, mw.EP_SHARES[a.ep_share])
        if a.copy_calibration_mb > 0:
            out["copy_calibration_bytes"] = calibration_copy(a.copy_calibration_mb)
        print(json.dumps(out), flush=True)
        return
    if a.copy_reference:
        print(json.dumps(bench_copy_reference(a)), flush=True)
        return
    w = mw.get(a.workload)
    if a.vendor_gemm:
        print(json.dumps(bench_vendor_gemm(a, w)), flush=True)
        return
    if a.dropless and a.reroute:
        print("--dropless drops nothing: --reroute does not apply", file=sys.stderr)
        sys.exit(2)
    if a.dropless:
        w = w.with_(dropless=True, name=w.name + "_dropless")
    if a.reroute:
        w = w.with_(reroute=True, name=w.name + "_reroute")
    inputs = mw.generate(w, "cuda")
    cfg = moe.config(w.S, w.d, w.h, w.E, w.k, w.capacity_factor, dtype=w.dtype,
                     dropless=w.dropless, reroute=w.reroute)
    if a.backward:
        out = bench_training(a, w, inputs, cfg)
        if a.copy_calibration_mb > 0:
            out["copy_calibration_bytes"] = calibration_copy(a.copy_calibration_mb)
        if not a.no_cpu_baseline:
            out["cpu_baseline"] = cpu_baseline(w, inputs, a.cpu_seconds, backward=True)
        print(json.dumps(out), flush=True)
        return
    layer = MoELayer.from_inputs(cfg, inputs, keep=False)
    x = inputs["x"]
    xs = rotated(x)
    stream = torch.cuda.current_stream()

    def make_events(which):
        evs = [torch.cuda.Event(enable_timing=True) if i in which else None
               for i in range(moe.MOE_NUM_STAGE_EVENTS)]
        for e in evs:
            if e is not None:
                e.record(stream)
        return evs

    for i in range(a.warmup):
        layer.forward(xs[i % len(xs)])
    # Inside the timed steps only the boundaries of the two expert GEMMs are
    # recorded (each recorded event costs a few microseconds between two
    # kernels); the full per-stage breakdown comes from separate steps below.
    gemm_bounds = (5, 6, 7)
    step_events = [make_events(gemm_bounds) for _ in range(a.steps)]
    torch.cuda.synchronize()

    # step boundaries: bounds[0] opens the timed region, bounds[i+1] closes
    # step i (the last one closes the region)
    bounds = [torch.cuda.Event(enable_timing=True) for _ in range(a.steps + 1)]
    wall0 = time.perf_counter()
    bounds[0].record(stream)
    for i in range(a.steps):
        layer.forward(xs[i % len(xs)], events=step_events[i])
        bounds[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = bounds[0].elapsed_time(bounds[-1])
    ms = total_ms / a.steps
    step_ms = [bounds[i].elapsed_time(bounds[i + 1]) for i in range(a.steps)]
    gemm_us = {
        "expert_gemm1": float(np.mean([ev[5].elapsed_time(ev[6]) * 1000.0 for ev in step_events])),
        "expert_gemm2": float(np.mean([ev[6].elapsed_time(ev[7]) * 1000.0 for ev in step_events])),
    }

    # per-stage breakdown: extra fully instrumented steps after the timed ones
    n_inst = min(a.steps, 10)
    inst_events = [make_events(range(moe.MOE_NUM_STAGE_EVENTS)) for _ in range(n_inst)]
    torch.cuda.synchronize()
    for i in range(n_inst):
        layer.forward(xs[i % len(xs)], events=inst_events[i])
    torch.cuda.synchronize()
    stage_us = {}
    for si, name in enumerate(STAGES):
        vals = [ev[si].elapsed_time(ev[si + 1]) * 1000.0 for ev in inst_events]
        stage_us[name] = float(np.mean(vals))

    # routing statistics of this batch (from a keep=True run)
    probe = MoELayer.from_inputs(cfg, inputs, keep=True)
    probe.forward(x)
    torch.cuda.synchronize()
    counts = probe.counts.cpu().numpy()
    occ = filled_rows(counts, probe.C, w.k)
    kept = int(occ.sum())
    aux, z = (float(v) for v in probe.losses.cpu().numpy())
    drops = int((probe.slot < 0).sum().item())
    del probe

    work = algorithmic_work(w, occ, kept)
    dom = max(("expert_gemm1", "expert_gemm2"), key=lambda n: gemm_us[n])
    t = gemm_us[dom] * 1e-6
    fl, by = work[dom]["flops"], work[dom]["bytes"]
    t_mfma = fl / (MFMA_PEAK_TFLOPS[w.dtype] * 1e12)
    t_hbm = by / (HBM_PEAK_GBS * 1e9)
    if t_hbm >= t_mfma:
        roof = {"bound": "hbm", "achieved": by / t / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": fl / t / 1e12, "peak": MFMA_PEAK_TFLOPS[w.dtype],
                "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(w.name, dom)
    roof["kernel"] = dom
    roof["algorithmic_flops"] = fl
    roof["algorithmic_bytes"] = by
    roof["avg_launch_us"] = gemm_us[dom]

    ffn_s = (gemm_us["expert_gemm1"] + gemm_us["expert_gemm2"]) * 1e-6
    ffn_flops = work["expert_gemm1"]["flops"] + work["expert_gemm2"]["flops"]
    # bf16 layers without a dispatch buffer gather token rows inside the first
    # expert GEMM (x under 4 GiB): the dispatch stage is then empty.
    fused = w.dtype == "bf16" and w.S * w.d * 2 < 2 ** 32
    stage_frac = {}
    for n in ("gate_logits", "dispatch", "combine", "expert_gemm1", "expert_gemm2"):
        if n == "dispatch" and fused:
            stage_frac[n] = "fused into expert_gemm1"
            continue
        ts = gemm_us.get(n, stage_us[n]) * 1e-6
        # the stage's roofline time: its algorithmic bytes at the HBM peak or
        # its matrix work at the MFMA peak, whichever is longer (the bf16
        # router runs three MFMAs per product for its exact weight split)
        mf = work[n]["flops"] * (3 if n == "gate_logits" and w.dtype == "bf16" else 1)
        t_b = work[n]["bytes"] / (HBM_PEAK_GBS * 1e9)
        t_f = mf / (MFMA_PEAK_TFLOPS[w.dtype] * 1e12)
        stage_frac[n] = {"GB_s": work[n]["bytes"] / ts / 1e9,
                         "TFLOP_s": work[n]["flops"] / ts / 1e12,
                         "bound": "hbm" if t_b >= t_f else "mfma",
                         "roofline_frac": max(t_b, t_f) / ts}

    out = {
        "metric": METRIC,
        "value": w.S / (ms / 1000.0),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms,
        "ms_per_step_median": float(np.median(step_ms)),
        "ms_per_step_min": float(np.min(step_ms)),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "S": w.S, "d_model": w.d, "d_ff": w.h, "E": w.E,
                   "k": w.k, "capacity_factor": None if w.dropless else w.capacity_factor,
                   "C": None if w.dropless else probe_C(cfg), "dropless": w.dropless,
                   "reroute": w.reroute, "seed": w.seed},
        "roofline": roof,
        "ffn_mfma_frac": ffn_flops / ffn_s / (MFMA_PEAK_TFLOPS[w.dtype] * 1e12),
        "gemm_us": gemm_us,
        "stage_us": stage_us,
        "stage_us_note": f"{n_inst} extra steps with every stage boundary recorded "
                         f"(each recorded event adds queue time between two kernels)",
        "stage_rates": stage_frac,
        "routing": {"kept": kept, "dropped": drops, "nonempty_experts": int((occ > 0).sum()),
                    "rerouted": int(counts[w.k].sum()) if w.reroute else 0,
                    "aux": aux, "z": z},
        "wall_s": wall,
        "input_copies": len(xs),
    }
    if a.copy_calibration_mb > 0:
        out["copy_calibration_bytes"] = calibration_copy(a.copy_calibration_mb)
    if not a.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, inputs, a.cpu_seconds)
    print(json.dumps(out), flush=True)


def calibration_copy(mib: int) -> int:
    """One plain device copy of `mib` MiB: the reference kernel of known size
    for the FETCH_SIZE / WRITE_SIZE counters."""
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    return n


def probe_C(cfg):
    return moe.capacity(cfg)


def bench_ep_share(a, sh) -> dict:
    """One step = moe_expert_ffn over the rows one GPU of an expert-parallel
    layer receives (compact expert segments, as the dispatch all-to-all would
    deliver them): both expert GEMMs over E_local experts."""
    counts = mw.ep_share_counts(sh)
    rows = int(counts.sum())
    inp = mw.generate_ep_share(sh, rows, "cuda")
    cfg = moe.config(rows, sh.d, sh.h, sh.E_local, 1, dtype="bf16", dropless=True)
    out = torch.empty((rows, sh.d), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(moe.workspace_bytes(cfg), dtype=torch.uint8, device="cuda")
    cnt = torch.from_numpy(counts[None, :].astype(np.int32)).cuda()

    xs = rotated(inp["xd"])

    def step(i):
        moe.expert_ffn(cfg, xs[i % len(xs)], cnt, inp["w1"], None, inp["w2"], None, out, ws)

    for i in range(a.warmup):
        step(i)
    stream = torch.cuda.current_stream()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(a.steps)]
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record(stream)
    for i in range(a.steps):
        evs[i][0].record(stream)
        step(i)
        evs[i][1].record(stream)
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = t0.elapsed_time(t1) / a.steps
    ffn_us = float(np.mean([b.elapsed_time(e) * 1000.0 for b, e in evs]))
    flops = 2 * 2.0 * rows * sh.d * sh.h
    by = 2 * sh.E_local * sh.d * sh.h * 2 + rows * (2 * sh.d + 2 * sh.h) * 2
    t = ffn_us * 1e-6
    if by / (HBM_PEAK_GBS * 1e9) >= flops / (MFMA_PEAK_TFLOPS["bf16"] * 1e12):
        roof = {"bound": "hbm", "achieved": by / t / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": flops / t / 1e12, "peak": MFMA_PEAK_TFLOPS["bf16"],
                "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    t1, t2 = (measured_traffic(sh.name, k) for k in ("expert_gemm1", "expert_gemm2"))
    roof["traffic"] = t1 + t2 if t1 is not None and t2 is not None else None
    roof["kernel"] = "expert_gemm1+expert_gemm2 (one moe_expert_ffn call)"
    roof["algorithmic_flops"] = flops
    roof["algorithmic_bytes"] = by
    roof["avg_launch_us"] = ffn_us
    out_d = {
        "metric": "expert-FFN rows/s on one GPU's expert-parallel share",
        "value": rows / (ms / 1000.0),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": sh.name, "sources": sh.sources, "tokens_per_source": sh.S,
                   "E_total": sh.E_total, "k": sh.k, "E_local": sh.E_local, "d_model": sh.d,
                   "d_ff": sh.h, "rows": rows, "seed": sh.seed},
        "roofline": roof,
        "wall_s": wall,
        "input_copies": len(xs),
    }
    if not a.no_cpu_baseline:
        import oracle
        w1h, w2h = mw.to_numpy(inp["w1"]), mw.to_numpy(inp["w2"])
        seg = np.concatenate([[0], np.cumsum(counts)[:-1]])

        def run(m):   # the first m rows of every local expert
            idx = (seg[:, None] + np.arange(m)[None, :]).reshape(-1)
            xs = mw.to_numpy(inp["xd"][torch.from_numpy(idx).cuda()]).reshape(sh.E_local, m, sh.d)
            t_0 = time.perf_counter()
            oracle.expert_ffn(xs, np.full(sh.E_local, m, np.int32), w1h, None, w2h, None)
            return time.perf_counter() - t_0
        m0 = 2
        t_m0 = run(m0)
        m = int(min(counts.min(), max(m0, m0 * a.cpu_seconds / max(t_m0, 1e-3))))
        tc = run(m) if m != m0 else t_m0
        out_d["cpu_baseline"] = {"value": sh.E_local * m / tc, "unit": "rows/s",
                                 "cores": oracle_threads(), "kind": "oracle",
                                 "host": host_cpu(),
                                 "sample": f"the first {m} rows of each of the {sh.E_local} local "
                                           f"experts through the fp64 oracle FFN, {tc:.1f} s"}
    return out_d


def bench_copy_reference(a) -> dict:
    """Plain device copies (torch copy_, read + write) of several sizes:
    median of `steps` timed copies after `warmup`, bytes counted both ways."""
    out = {"metric": "device-to-device copy rate (read + write bytes)", "unit": "TB/s",
           "steps": a.steps, "warmup": a.warmup, "copies": {}}
    stream = torch.cuda.current_stream()
    for mib in (64, 256, 1024):
        src = torch.empty(mib << 20, dtype=torch.uint8, device="cuda")
        src.fill_(1)
        dst = torch.empty_like(src)
        for _ in range(a.warmup):
            dst.copy_(src)
        ts = []
        for _ in range(a.steps):
            b = torch.cuda.Event(enable_timing=True)
            e = torch.cuda.Event(enable_timing=True)
            b.record(stream)
            dst.copy_(src)
            e.record(stream)
            torch.cuda.synchronize()
            ts.append(b.elapsed_time(e) * 1000.0)
        us = float(np.median(ts))
        out["copies"][f"{mib}MiB"] = {"us": us, "TB_s": 2.0 * (mib << 20) / us / 1e6}
        del src, dst
    return out


def bench_vendor_gemm(a, w: mw.Workload) -> dict:
    """Both expert GEMMs at uniform occupancy, m = ceil(S*k/E) rows per
    expert: moe_expert_ffn (this library) against torch.bmm, which runs
    hipBLASLt, on the same operands (the weights transposed once, outside the
    timed region, into the [K,N] layout bmm takes contiguously; ReLU between
    the two products).  Median of `steps` timed calls after `warmup`."""
    S, d, h, E, k = w.S, w.d, w.h, w.E, w.k
    m = -(-S * k // E)
    inp = mw.generate(w, "cuda")
    w1, w2 = inp["w1"], inp["w2"]
    g = torch.Generator(device="cuda").manual_seed(w.seed + 7)
    xd = torch.randn((E, m, d), generator=g, device="cuda").to(w.torch_dtype)
    cfg = moe.config(E * m, d, h, E, 1, capacity=m, dtype=w.dtype)
    cnt = torch.full((1, E), m, dtype=torch.int32, device="cuda")
    out = torch.empty((E, m, d), dtype=w.torch_dtype, device="cuda")
    ws = torch.empty(moe.workspace_bytes(cfg), dtype=torch.uint8, device="cuda")
    w1t = w1.transpose(1, 2).contiguous()      # [E,d,h]
    w2t = w2.transpose(1, 2).contiguous()      # [E,h,d]
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(a.warmup):
            fn()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(a.steps)]
        torch.cuda.synchronize()
        for b, e in evs:
            b.record(stream)
            fn()
            e.record(stream)
        torch.cuda.synchronize()
        return float(np.median([b.elapsed_time(e) * 1000.0 for b, e in evs]))

    ours = timed(lambda: moe.expert_ffn(cfg, xd, cnt, w1, None, w2, None, out, ws))
    hbuf = torch.empty((E, m, h), dtype=w.torch_dtype, device="cuda")
    obuf = torch.empty((E, m, d), dtype=w.torch_dtype, device="cuda")
    g1 = timed(lambda: torch.bmm(xd, w1t, out=hbuf))
    g2 = timed(lambda: torch.bmm(hbuf, w2t, out=obuf))
    relu = timed(lambda: hbuf.relu_())
    # the two paths agree (same operands, fp32 accumulation in both)
    torch.bmm(xd, w1t, out=hbuf)
    hbuf.relu_()
    torch.bmm(hbuf, w2t, out=obuf)
    moe.expert_ffn(cfg, xd, cnt, w1, None, w2, None, out, ws)
    torch.cuda.synchronize()
    diff = float((out.float() - obuf.float()).norm() / obuf.float().norm())
    flops = 2 * 2.0 * E * m * d * h
    return {"metric": "expert FFN at uniform occupancy: moe_expert_ffn vs hipBLASLt (torch.bmm)",
            "config": {"workload": w.name, "E": E, "rows_per_expert": m, "d_model": d, "d_ff": h},
            "steps": a.steps, "warmup": a.warmup,
            "moe_expert_ffn_us": ours,
            "hipblaslt_gemm1_us": g1, "hipblaslt_gemm2_us": g2, "relu_us": relu,
            "hipblaslt_gemms_us": g1 + g2,
            "moe_expert_ffn_tflops": flops / ours / 1e6,
            "hipblaslt_tflops": flops / (g1 + g2) / 1e6,
            "rel_diff": diff}


BWD_STAGES = ["setup", "recompute_h", "combine_router_bwd", "wgrad2", "dgrad2", "wgrad1",
              "dgrad1", "router_dx_dw"]
BWD_GEMMS = ("wgrad2", "dgrad2", "wgrad1", "dgrad1")   # H is saved: no recompute


def bench_training(a, w: mw.Workload, inputs: dict, cfg) -> dict:
    """One step = moe_layer_forward (keeping the routing, expert outputs and
    hidden activations) + moe_layer_backward of sum(dy*y) + 0.01*aux +
    0.001*z."""
    # the forward keeps the expert hidden activations for the backward
    layer = MoELayer.from_inputs(cfg, inputs, keep=True, dispatch_buffer=False, keep_hidden=True)
    x = inputs["x"]
    S, d, h, E = w.S, w.d, w.h, w.E
    dev, at = "cuda", w.torch_dtype
    g = torch.Generator(device=dev).manual_seed(w.seed + 1000)
    dy = torch.randn((S, d), generator=g, device=dev).to(at)
    bws = torch.empty(moe.backward_workspace_bytes(cfg), dtype=torch.uint8, device=dev)
    gr = dict(dx=torch.empty((S, d), dtype=at, device=dev),
              dwg=torch.empty((E, d), dtype=torch.float32, device=dev),
              dbg=torch.empty((E,), dtype=torch.float32, device=dev),
              dw1=torch.empty((E, h, d), dtype=at, device=dev),
              db1=torch.empty((E, h), dtype=at, device=dev),
              dw2=torch.empty((E, d, h), dtype=at, device=dev),
              db2=torch.empty((E, d), dtype=at, device=dev))
    stream = torch.cuda.current_stream()

    xs, dys = rotated(x), rotated(dy)

    def step(i, bwd_events=None):
        x, dy = xs[i % len(xs)], dys[i % len(dys)]
        layer.forward(x)
        moe.layer_backward(cfg, x, inputs["wg"], inputs["w1"], inputs["b1"], inputs["w2"],
                           layer.logits, layer.topk_idx, layer.topk_w, layer.slot, layer.counts,
                           layer.out, dy, gr["dx"], gr["dwg"], gr["dw1"], gr["dw2"], bws,
                           db_gate=gr["dbg"], db1=gr["db1"], db2=gr["db2"], g_aux=0.01,
                           g_z=0.001, hidden=layer.hidden, events=bwd_events)

    def make_events():
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(moe.MOE_NUM_BWD_EVENTS)]
        for e in evs:
            e.record(stream)
        return evs

    for i in range(a.warmup):
        step(i)
    evs = [make_events() for _ in range(a.steps)]
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record(stream)
    for i in range(a.steps):
        step(i, evs[i])
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = t0.elapsed_time(t1) / a.steps
    stage_us = {n: float(np.mean([ev[i].elapsed_time(ev[i + 1]) * 1000.0 for ev in evs]))
                for i, n in enumerate(BWD_STAGES)}
    bwd_ms = float(np.mean([ev[0].elapsed_time(ev[-1]) for ev in evs]))

    counts = layer.counts.cpu().numpy()
    occ = filled_rows(counts, layer.C, w.k)
    kept = int(occ.sum())
    nonempty = int((occ > 0).sum())
    es = 2
    flops = 2.0 * kept * d * h
    act = kept * (d + h) * es
    work = {
        "recompute_h": dict(flops=flops, bytes=nonempty * h * d * es + kept * (d + h) * es),
        # weight gradients: every expert's [d,h] gradient is written
        "wgrad2": dict(flops=flops, bytes=E * d * h * es + act),
        "wgrad1": dict(flops=flops, bytes=E * d * h * es + act),
        # data gradients: weights of non-empty experts read once, rows in and out
        "dgrad2": dict(flops=flops, bytes=nonempty * d * h * es + act + kept * h * es),
        "dgrad1": dict(flops=flops, bytes=nonempty * d * h * es + act),
    }
    dom = max(BWD_GEMMS, key=lambda n: stage_us[n])
    t = stage_us[dom] * 1e-6
    fl, by = work[dom]["flops"], work[dom]["bytes"]
    if by / (HBM_PEAK_GBS * 1e9) >= fl / (MFMA_PEAK_TFLOPS[w.dtype] * 1e12):
        roof = {"bound": "hbm", "achieved": by / t / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s"}
    else:
        roof = {"bound": "mfma", "achieved": fl / t / 1e12, "peak": MFMA_PEAK_TFLOPS[w.dtype],
                "unit": "TFLOP/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic(w.name + "_training", dom)
    roof["kernel"] = dom
    roof["algorithmic_flops"] = fl
    roof["algorithmic_bytes"] = by
    roof["avg_launch_us"] = stage_us[dom]
    gemm_s = sum(stage_us[n] for n in BWD_GEMMS) * 1e-6
    return {
        "metric": "MoE-layer training tokens/s (forward + backward)",
        "value": S / (ms / 1000.0),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": w.name, "pass": "forward+backward", "hidden": "saved",
                   "S": S, "d_model": d,
                   "d_ff": h, "E": E, "k": w.k,
                   "capacity_factor": None if w.dropless else w.capacity_factor,
                   "C": None if w.dropless else layer.C, "dropless": w.dropless,
                   "reroute": w.reroute, "seed": w.seed},
        "roofline": roof,
        "backward_ms": bwd_ms,
        "backward_stage_us": stage_us,
        "backward_gemm_mfma_frac": len(BWD_GEMMS) * flops / gemm_s /
        (MFMA_PEAK_TFLOPS[w.dtype] * 1e12),
        "routing": {"kept": kept, "nonempty_experts": nonempty},
        "wall_s": wall,
        "input_copies": len(xs),
    }


if __name__ == "__main__":
    main()
