"""Pins of the oracle's backward pass.

The oracle's gradients are hand-derived formulas in C.  They are checked here
against torch fp64 autograd of the forward, written from the layer's
definition in torch ops with the routing (top-k set, slots) held fixed, and
against central finite differences of that forward.  Routing comes from a
brute-force top-k and slot count, not from the oracle.  Biases are non-zero,
h != d, drops are present, and both loss weights are non-zero, so a dropped
term, a wrong sign or a transposed operand in any gradient fails a check.
"""
import math

import numpy as np
import pytest
import torch

import oracle


def brute_route(lg, k, C):
    """Top-k by full sort (logit descending, index ascending); slots rank by
    rank, tokens in order, dropped (-1) at C or more."""
    S, E = lg.shape
    idx = np.array([sorted(range(E), key=lambda j: (-float(lg[s, j]), j))[:k] for s in range(S)],
                   np.int64).reshape(S, k)
    slot = np.full((S, k), -1, np.int64)
    cnt = np.zeros(E, np.int64)
    for r in range(k):
        for s in range(S):
            e = idx[s, r]
            slot[s, r] = cnt[e] if cnt[e] < C else -1
            cnt[e] += 1
    first = np.bincount(idx[:, 0], minlength=E)
    return idx, slot, first


def torch_loss(x, wg, bg, w1, b1, w2, b2, dy, idx, slot, first, g_aux, g_z):
    """L = sum(dy * y) + g_aux * aux + g_z * z for a fixed routing, fp64."""
    S, E = x.shape[0], wg.shape[0]
    lg = x @ wg.T + bg
    # routing precision: the logits are rounded to fp32 once (identity for
    # the gradient)
    lg = lg + (lg.to(torch.float32).to(torch.float64) - lg).detach()
    p = torch.softmax(lg, dim=1)
    lse = torch.logsumexp(lg, dim=1)
    ii = torch.from_numpy(idx)
    wsel = torch.softmax(torch.gather(lg, 1, ii), dim=1)   # renormalised top-k weights
    y = torch.zeros_like(x[:, :w2.shape[1]])
    for s in range(S):
        for r in range(idx.shape[1]):
            if slot[s, r] < 0:
                continue
            e = idx[s, r]
            a = torch.relu(w1[e] @ x[s] + b1[e])
            y[s] = y[s] + wsel[s, r] * (w2[e] @ a + b2[e])
    f = torch.from_numpy(first.astype(np.float64)) / S
    aux = E * torch.sum(f * p.mean(dim=0))
    z = torch.mean(lse ** 2)
    return torch.sum(dy * y) + g_aux * aux + g_z * z


def make(S, d, h, E, seed, dtype=np.float32):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((S, d)).astype(np.float32)
    wg = (rng.standard_normal((E, d)) / math.sqrt(d)).astype(np.float32)
    bg = (0.3 * rng.standard_normal(E)).astype(np.float32)
    w1 = (rng.standard_normal((E, h, d)) / math.sqrt(d)).astype(np.float32)
    b1 = (0.2 * rng.standard_normal((E, h))).astype(np.float32)
    w2 = (rng.standard_normal((E, d, h)) / math.sqrt(h)).astype(np.float32)
    b2 = (0.2 * rng.standard_normal((E, d))).astype(np.float32)
    dy = rng.standard_normal((S, d)).astype(np.float32)
    return x, wg, bg, w1, b1, w2, b2, dy


def bf16_bits(a):
    """Round-to-nearest-even fp32 -> bf16 bit patterns, and their fp32 values."""
    u = np.ascontiguousarray(a, np.float32).view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    return r, (r.astype(np.uint32) << 16).view(np.float32)


CASES = [
    # S, d, h, E, k, cf, g_aux, g_z, seed
    (24, 6, 10, 4, 2, 0.75, 0.7, 0.3, 1),     # drops
    (20, 5, 7, 5, 3, 1.0, -1.3, 0.9, 2),      # k = 3, drops
    (16, 4, 9, 3, 1, 2.0, 0.5, -0.4, 3),      # k = 1
    (12, 8, 6, 4, 2, None, 1.1, 0.2, 4),      # dropless: C = S
]


@pytest.mark.parametrize("S,d,h,E,k,cf,g_aux,g_z,seed", CASES)
def test_backward_matches_autograd(S, d, h, E, k, cf, g_aux, g_z, seed):
    x, wg, bg, w1, b1, w2, b2, dy = make(S, d, h, E, seed)
    C = S if cf is None else oracle.capacity(S, E, k, cf)
    lg = oracle.logits(x, wg, bg)
    idx, slot, first = brute_route(lg, k, C)
    if cf is not None and cf < 1.5:
        assert (slot < 0).any()
    g = oracle.layer_backward(x, wg, w1, b1, w2, b2, k, C, lg, dy, g_aux, g_z)
    # the oracle's routing for the same logits fixes the same assignments
    assert np.array_equal(oracle.route(lg, k, C)["idx"], idx)

    t = {n: torch.tensor(v.astype(np.float64), requires_grad=n != "dy")
         for n, v in dict(x=x, wg=wg, bg=bg, w1=w1, b1=b1, w2=w2, b2=b2, dy=dy).items()}
    L = torch_loss(t["x"], t["wg"], t["bg"], t["w1"], t["b1"], t["w2"], t["b2"], t["dy"], idx,
                   slot, first, g_aux, g_z)
    L.backward()
    for name, key in (("x", "dx"), ("wg", "dwg"), ("bg", "dbg"), ("w1", "dw1"), ("b1", "db1"),
                      ("w2", "dw2"), ("b2", "db2")):
        want = t[name].grad.numpy()
        assert np.allclose(g[key], want, rtol=1e-10, atol=1e-12), key
    # gradient of the top-k weights: dy . expert output, zero when dropped
    assert np.all(g["dw"][slot < 0] == 0)


def test_backward_central_differences():
    """A few entries of every gradient against (L(t+e) - L(t-e)) / 2e of the
    fixed-routing forward (no autograd involved)."""
    S, d, h, E, k, cf, g_aux, g_z = 18, 5, 8, 4, 2, 0.75, 0.8, 0.6
    x, wg, bg, w1, b1, w2, b2, dy = make(S, d, h, E, 7)
    C = oracle.capacity(S, E, k, cf)
    lg = oracle.logits(x, wg, bg)
    idx, slot, first = brute_route(lg, k, C)
    g = oracle.layer_backward(x, wg, w1, b1, w2, b2, k, C, lg, dy, g_aux, g_z)
    base = {n: torch.tensor(v.astype(np.float64))
            for n, v in dict(x=x, wg=wg, bg=bg, w1=w1, b1=b1, w2=w2, b2=b2, dy=dy).items()}

    def L(over):
        a = dict(base, **over)
        # no fp32 rounding of the logits here: a perturbation of 1e-6 would
        # be lost in it; the rounding is the identity for the gradient anyway
        lg64 = a["x"] @ a["wg"].T + a["bg"]
        p = torch.softmax(lg64, 1)
        lse = torch.logsumexp(lg64, 1)
        wsel = torch.softmax(torch.gather(lg64, 1, torch.from_numpy(idx)), 1)
        tot = 0.0
        for s in range(S):
            for r in range(k):
                if slot[s, r] < 0:
                    continue
                e = idx[s, r]
                o = a["w2"][e] @ torch.relu(a["w1"][e] @ a["x"][s] + a["b1"][e]) + a["b2"][e]
                tot = tot + wsel[s, r] * torch.dot(a["dy"][s], o)
        f = torch.from_numpy(first.astype(np.float64)) / S
        return float(tot + g_aux * E * torch.sum(f * p.mean(0)) + g_z * torch.mean(lse ** 2))

    rng = np.random.default_rng(0)
    eps = 1e-6
    for name, key in (("x", "dx"), ("wg", "dwg"), ("bg", "dbg"), ("w1", "dw1"), ("b1", "db1"),
                      ("w2", "dw2"), ("b2", "db2")):
        for _ in range(4):
            pos = tuple(int(rng.integers(n)) for n in base[name].shape)
            hi, lo = base[name].clone(), base[name].clone()
            hi[pos] += eps
            lo[pos] -= eps
            num = (L({name: hi}) - L({name: lo})) / (2 * eps)
            assert abs(num - g[key][pos]) <= 1e-6 * max(1.0, abs(num)), (key, pos, num,
                                                                         g[key][pos])


def test_backward_bf16_inputs_widen_exactly():
    """bf16 activations give the gradients of their exact fp32 values."""
    S, d, h, E, k = 14, 6, 8, 4, 2
    x, wg, bg, w1, b1, w2, b2, dy = make(S, d, h, E, 9)
    bits = [bf16_bits(a) for a in (x, w1, b1, w2, b2, dy)]
    C = oracle.capacity(S, E, k, 1.0)
    lg = oracle.logits(bits[0][0], wg, bg)
    gb = oracle.layer_backward(bits[0][0], wg, *[b[0] for b in bits[1:5]], k, C, lg,
                               bits[5][0], 0.5, 0.5)
    gf = oracle.layer_backward(bits[0][1], wg, *[b[1] for b in bits[1:5]], k, C, lg,
                               bits[5][1], 0.5, 0.5)
    for key in gb:
        assert np.array_equal(gb[key], gf[key]), key


def test_no_loss_weight_no_router_gradient_from_losses():
    """With g_aux = g_z = 0 and dy = 0 every gradient is exactly zero; with
    only g_z the logit gradient is (2/S) lse p, a closed form."""
    S, d, h, E, k = 10, 4, 6, 5, 2
    x, wg, bg, w1, b1, w2, b2, dy = make(S, d, h, E, 11)
    C = oracle.capacity(S, E, k, 1.0)
    lg = oracle.logits(x, wg, bg)
    zero = np.zeros_like(dy)
    g = oracle.layer_backward(x, wg, w1, b1, w2, b2, k, C, lg, zero, 0.0, 0.0)
    for key in g:
        assert not np.any(g[key]), key
    g = oracle.layer_backward(x, wg, w1, b1, w2, b2, k, C, lg, zero, 0.0, 1.0)
    l64 = torch.from_numpy(lg.astype(np.float64))
    want = 2.0 / S * torch.logsumexp(l64, 1)[:, None] * torch.softmax(l64, 1)
    assert np.allclose(g["dl"], want.numpy(), rtol=1e-13, atol=0)
    assert np.allclose(g["dbg"], want.numpy().sum(0), rtol=1e-12, atol=1e-15)


def test_entries_match_full_backward():
    """The one-by-one entries (full-size checks) equal the full backward's,
    and the router function equals its logit gradient."""
    S, d, h, E, k = 30, 6, 10, 5, 2
    x, wg, bg, w1, b1, w2, b2, dy = make(S, d, h, E, 13)
    C = oracle.capacity(S, E, k, 0.8)
    lg = oracle.logits(x, wg, bg)
    g = oracle.layer_backward(x, wg, w1, b1, w2, b2, k, C, lg, dy, 0.6, 0.4)
    rng = np.random.default_rng(1)
    tok = rng.choice(S, 7, replace=False)
    ents = [(1, int(rng.integers(E)), int(rng.integers(h)), int(rng.integers(d))) for _ in range(9)]
    ents += [(2, int(rng.integers(E)), int(rng.integers(d)), int(rng.integers(h))) for _ in range(9)]
    ents += [(3, int(rng.integers(E)), int(rng.integers(h)), 0) for _ in range(5)]
    ents += [(4, int(rng.integers(E)), int(rng.integers(d)), 0) for _ in range(5)]
    rows, vals = oracle.backward_entries(x, wg, w1, b1, w2, b2, k, C, lg, dy, 0.6, 0.4, tok, ents)
    assert np.allclose(rows, g["dx"][tok], rtol=1e-12, atol=1e-13)
    full = {1: g["dw1"], 2: g["dw2"], 3: g["db1"], 4: g["db2"]}
    want = [full[kd][e, a, b] if kd <= 2 else full[kd][e, a] for kd, e, a, b in ents]
    assert np.allclose(vals, want, rtol=1e-12, atol=1e-13)
    r = oracle.route(lg, k, C)
    dl = oracle.router_backward(lg, r["idx"], r["w"], g["dw"], r["counts"], 0.6, 0.4)
    assert np.allclose(dl, g["dl"], rtol=1e-13, atol=1e-15)
