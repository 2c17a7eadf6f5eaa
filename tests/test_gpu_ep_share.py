"""The expert FFN at one GPU's expert-parallel share of the DeepSeek-shaped
layout (256 experts over 8 GPUs: 32 local experts, rows from every source GPU,
about 2048 rows per expert), through the C ABI.

The received rows sit in compact expert segments: the layout of the dropless
mode, and the layout an expert-major receive buffer of the dispatch all-to-all
has.  Inputs are seeded and synthetic (moe_workloads.ep_share_counts /
generate_ep_share).  Rows checked: one random row of every 32-row block of
every expert segment (the expert GEMMs' sub-tile height), so every m-tile of
every segment is covered, plus the first and last row of each segment.  Bar:
relative Frobenius error 1e-2 against the fp64 oracle, each row within 3e-2.
"""
import numpy as np
import pytest
import torch

import moe_workloads as mw
import oracle
import sparse_moe_layer_wg_amd as moe
from parity_util import TOL, as_f64, rel_fro, row_rel

pytestmark = pytest.mark.gpu


def test_ep_share_expert_ffn_every_subtile():
    sh = mw.EP_SHARES["deepseek_ep8_share"]
    counts = mw.ep_share_counts(sh)
    rows = int(counts.sum())
    print(f"\n[ep share] {sh} rows={rows}", flush=True)
    inp = mw.generate_ep_share(sh, rows, "cuda")
    cfg = moe.config(rows, sh.d, sh.h, sh.E_local, 1, dtype="bf16", dropless=True)
    assert moe.dispatch_rows(cfg) == rows
    out = torch.full((rows, sh.d), 7.0, device="cuda").to(torch.bfloat16)
    ws = torch.empty(moe.workspace_bytes(cfg), dtype=torch.uint8, device="cuda")
    cnt = torch.from_numpy(counts[None, :].astype(np.int32)).cuda()
    moe.expert_ffn(cfg, inp["xd"], cnt, inp["w1"], None, inp["w2"], None, out, ws)
    torch.cuda.synchronize()

    seg = np.concatenate([[0], np.cumsum(counts)[:-1]])
    rng = np.random.default_rng(0)
    picks = []
    for e in range(sh.E_local):
        n = int(counts[e])
        mine = [0, n - 1]
        for b0 in range(0, n, 32):
            mine.append(int(rng.integers(b0, min(n, b0 + 32))))
        picks.append(np.unique(np.array(mine, np.int64)) + seg[e])
    m = max(len(p) for p in picks)
    occ = np.array([len(p) for p in picks], np.int32)
    flat = np.concatenate(picks)
    xs_rows = mw.to_numpy(inp["xd"][torch.from_numpy(flat).cuda()])
    xs = np.zeros((sh.E_local, m, sh.d), xs_rows.dtype)
    o = 0
    for e in range(sh.E_local):
        xs[e, :occ[e]] = xs_rows[o:o + occ[e]]
        o += occ[e]
    want = oracle.expert_ffn(xs, occ, mw.to_numpy(inp["w1"]), None, mw.to_numpy(inp["w2"]), None)
    want = np.concatenate([want[e, :occ[e]] for e in range(sh.E_local)])
    got = as_f64(out[torch.from_numpy(flat).cuda()])
    err = rel_fro(got, want)
    row_err = row_rel(got, want)
    print(f"[ep share] rows checked={flat.size} rel_fro={err:.4g} max_row={row_err.max():.4g}",
          flush=True)
    assert err <= TOL["bf16"] and row_err.max() <= 3 * TOL["bf16"]
