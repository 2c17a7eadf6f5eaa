"""The expert FFN at one GPU's expert-parallel share of the DeepSeek-shaped
layout (256 experts over 8 GPUs: 32 local experts, rows from every source GPU,
about 2048 rows per expert), through the C ABI.

The received rows sit in compact expert segments: the layout of the dropless
mode, and the layout an expert-major receive buffer of the dispatch all-to-all
has.  Inputs are seeded and synthetic (moe_workloads.ep_share_counts /
generate_ep_share).  Bar: sampled rows within relative Frobenius error 1e-2
of the fp64 oracle (each row within 3e-2), and rows at every segment boundary
included.
"""
import numpy as np
import pytest
import torch

import moe_workloads as mw
import oracle
import sparse_moe_layer_wg_amd as moe
from parity_util import TOL, as_f64, rel_fro

pytestmark = pytest.mark.gpu


def test_ep_share_expert_ffn_sampled():
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
    m = 4
    pick = np.empty((sh.E_local, m), np.int64)
    for e in range(sh.E_local):
        inner = rng.choice(np.arange(1, counts[e] - 1), size=m - 2, replace=False)
        pick[e] = np.concatenate([[0, counts[e] - 1], inner]) + seg[e]
    xs = mw.to_numpy(inp["xd"][torch.from_numpy(pick.reshape(-1)).cuda()])
    xs = xs.reshape(sh.E_local, m, sh.d)
    want = oracle.expert_ffn(xs, np.full(sh.E_local, m, np.int32), mw.to_numpy(inp["w1"]), None,
                             mw.to_numpy(inp["w2"]), None)
    got = as_f64(out[torch.from_numpy(pick.reshape(-1)).cuda()]).reshape(sh.E_local, m, sh.d)
    err = rel_fro(got, want)
    row_err = (np.linalg.norm((got - want).reshape(-1, sh.d), axis=1) /
               np.linalg.norm(want.reshape(-1, sh.d), axis=1))
    print(f"[ep share] rel_fro={err:.4g} max_row={row_err.max():.4g}", flush=True)
    assert err <= TOL["bf16"] and row_err.max() <= 3 * TOL["bf16"]
