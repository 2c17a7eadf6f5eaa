"""Pins of the oracle's overflow re-routing (oracle_reroute) and of the layer
and backward with it.

Reading (the pages name the option and give no rule): the j-th dropped
assignment of a token (in rank order) is offered to the token's (k+j)-th
ranked expert; offers are taken virtual rank by virtual rank, tokens in order,
while the expert holds fewer than C rows; an assignment keeps its weight.
The brute force below restates that rule in plain Python from a full sort of
each token's logits, independently of the C code.
"""
import numpy as np
import pytest
import torch

import oracle
from test_oracle_backward_pins import make


def ranking(row):
    return sorted(range(len(row)), key=lambda j: (-float(row[j]), j))


def brute_reroute(lg, k, C):
    S, E = lg.shape
    order = [ranking(lg[s]) for s in range(S)]
    idx = np.array([o[:k] for o in order], np.int64).reshape(S, k)
    slot = np.full((S, k), -1, np.int64)
    cnt = [0] * E          # rows kept per expert
    for r in range(k):
        for s in range(S):
            e = idx[s, r]
            if cnt[e] < C:
                slot[s, r] = cnt[e]
                cnt[e] += 1
    serve = idx.copy()
    offers = {}
    for s in range(S):
        dropped = [r for r in range(k) if slot[s, r] < 0]
        for j, r in enumerate(dropped):
            if k + j < E:
                offers[(j, s)] = (r, order[s][k + j])
    acc = [0] * E
    for j in range(k):
        for s in range(S):
            if (j, s) not in offers:
                continue
            r, e = offers[(j, s)]
            if cnt[e] < C:
                serve[s, r] = e
                slot[s, r] = cnt[e]
                cnt[e] += 1
                acc[e] += 1
    return idx, serve, slot, np.array(acc)


# (12, 5, 2, 2, 162): a token's second offer and another token's first offer
# compete for one expert, so taking offers token by token (instead of virtual
# rank by virtual rank) gives a different result
@pytest.mark.parametrize("S,E,k,C,seed", [(20, 5, 2, 3, 0), (33, 6, 3, 4, 1), (40, 4, 2, 6, 2),
                                          (17, 9, 4, 2, 3), (25, 3, 2, 9, 4), (30, 8, 1, 2, 5),
                                          (12, 5, 2, 2, 162)])
def test_reroute_matches_brute_force(S, E, k, C, seed):
    rng = np.random.default_rng(seed)
    lg = rng.integers(-3, 4, (S, E)).astype(np.float32) / 2   # many ties
    r = oracle.route(lg, k, C, reroute=True)
    idx, serve, slot, acc = brute_reroute(lg, k, C)
    assert np.array_equal(r["idx"], idx)
    assert np.array_equal(r["serve"], serve)
    assert np.array_equal(r["slot"], slot)
    assert np.array_equal(r["counts"][k], acc)
    plain = oracle.route(lg, k, C)
    assert np.array_equal(r["counts"][:k], plain["counts"])   # f_j, aux unchanged
    assert r["aux"] == plain["aux"] and r["z"] == plain["z"]


def test_reroute_invariants():
    rng = np.random.default_rng(7)
    S, E, k, C = 300, 12, 3, 40
    lg = (rng.standard_normal((S, E)) + np.linspace(2, -2, E)).astype(np.float32)
    r = oracle.route(lg, k, C, reroute=True)
    plain = oracle.route(lg, k, C)
    kept = r["slot"] >= 0
    # every expert's rows are slots 0..occ-1, each used once, occ <= C
    for e in range(E):
        sl = np.sort(r["slot"][kept & (r["serve"] == e)])
        assert np.array_equal(sl, np.arange(len(sl))) and len(sl) <= C
    assert np.array_equal(oracle.occupancy(r["counts"], C, k),
                          np.bincount(r["serve"][kept], minlength=E))
    # a token's serving experts are distinct; moved ones lie outside its top-k
    for s in range(S):
        srv = r["serve"][s][kept[s]]
        assert len(set(srv)) == len(srv)
        moved = kept[s] & (r["serve"][s] != r["idx"][s])
        assert not set(r["serve"][s][moved]) & set(r["idx"][s])
    # assignments kept by the capacity pass are unchanged; more are kept
    was = plain["slot"] >= 0
    assert np.array_equal(r["slot"][was], plain["slot"][was])
    assert np.array_equal(r["serve"][was], plain["idx"][was])
    assert kept.sum() > was.sum()


def test_reroute_without_drops_is_identity():
    rng = np.random.default_rng(8)
    lg = rng.standard_normal((50, 6)).astype(np.float32)
    r = oracle.route(lg, 2, 50, reroute=True)
    assert np.array_equal(r["serve"], r["idx"]) and (r["slot"] >= 0).all()
    assert not r["counts"][2].any()


def test_reroute_zero_router_closed_form():
    """All logits equal: the ranking is 0, 1, ..., E-1.  Tokens s < C keep
    experts 0..k-1; tokens C <= s < 2C have every rank dropped and re-routed,
    rank r to expert k + r, slot s - C; later tokens stay dropped."""
    S, E, k, C = 70, 8, 3, 25
    r = oracle.route(np.zeros((S, E), np.float32), k, C, reroute=True)
    s = np.arange(S)
    for rank in range(k):
        want_e = np.where(s < C, rank, k + rank)
        want_slot = np.where(s < C, s, np.where(s < 2 * C, s - C, -1))
        assert np.array_equal(r["slot"][:, rank], want_slot)
        assert np.array_equal(r["serve"][s < 2 * C, rank], want_e[s < 2 * C])
    assert np.array_equal(r["counts"][k], [0] * k + [C] * k + [0] * (E - 2 * k))


def test_reroute_layer_and_backward():
    """Forward: y is the dense sum over served assignments with the original
    weights.  Backward: torch autograd of that forward, the weights being the
    softmax of the top-k logits and the FFN that of the serving expert."""
    S, d, h, E, k = 24, 6, 10, 5, 2
    x, wg, bg, w1, b1, w2, b2, dy = make(S, d, h, E, 21)
    C = oracle.capacity(S, E, k, 0.6)
    lg = oracle.logits(x, wg, bg)
    res = oracle.layer(x, wg, bg, w1, b1, w2, b2, k, C, lg=lg, reroute=True)
    moved = (res["slot"] >= 0) & (res["serve"] != res["idx"])
    assert moved.any()
    tok = np.arange(S)
    yt = oracle.token_output(tok, x, w1, b1, w2, b2, res["serve"], res["slot"], res["w"])
    assert np.allclose(res["y"], yt, rtol=1e-12, atol=1e-12)

    g = oracle.layer_backward(x, wg, w1, b1, w2, b2, k, C, lg, dy, 0.7, 0.3, reroute=True)
    t = {n: torch.tensor(v.astype(np.float64), requires_grad=n != "dy")
         for n, v in dict(x=x, wg=wg, bg=bg, w1=w1, b1=b1, w2=w2, b2=b2, dy=dy).items()}
    first = np.bincount(res["idx"][:, 0], minlength=E)
    # torch_loss evaluates expert idx[s, r] for kept assignments: give it the
    # serving experts there, and the top-k for the weights
    lgt = t["x"] @ t["wg"].T + t["bg"]
    lgt = lgt + (lgt.to(torch.float32).to(torch.float64) - lgt).detach()
    wsel = torch.softmax(torch.gather(lgt, 1, torch.from_numpy(res["idx"].astype(np.int64))), 1)
    y = torch.zeros((S, d), dtype=torch.float64)
    for s in range(S):
        for r in range(k):
            if res["slot"][s, r] < 0:
                continue
            e = res["serve"][s, r]
            a = torch.relu(t["w1"][e] @ t["x"][s] + t["b1"][e])
            y[s] = y[s] + wsel[s, r] * (t["w2"][e] @ a + t["b2"][e])
    p = torch.softmax(lgt, 1)
    lse = torch.logsumexp(lgt, 1)
    f = torch.from_numpy(first.astype(np.float64)) / S
    L = torch.sum(t["dy"] * y) + 0.7 * E * torch.sum(f * p.mean(0)) + 0.3 * torch.mean(lse ** 2)
    L.backward()
    for name, key in (("x", "dx"), ("wg", "dwg"), ("bg", "dbg"), ("w1", "dw1"), ("b1", "db1"),
                      ("w2", "dw2"), ("b2", "db2")):
        assert np.allclose(g[key], t[name].grad.numpy(), rtol=1e-10, atol=1e-12), key
