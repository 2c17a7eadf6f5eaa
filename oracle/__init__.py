"""TEST INFRASTRUCTURE -- ctypes binding of the fp64 CPU oracle.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports it, and it imports nothing from the product.

The oracle is a plain, slow implementation of the forward pass of a GShard
mixture-of-experts feed-forward layer (gate, top-k with renormalised weights,
capacity-limited slots, dispatch, expert ReLU FFN, combine, auxiliary loss and
z-loss); ``moe_oracle.c`` documents each step and the passage it follows.

Arrays are numpy.  An activation array is ``float32`` (fp32) or ``uint16``
(raw bf16 bit patterns); both are widened exactly inside the oracle.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "moe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

F32 = 0
BF16 = 1

_lib = None


def build() -> str:
    """Compile ``moe_oracle.c`` into ``liboracle.so`` (gcc, OpenMP)."""
    tmp = _LIB_PATH + ".tmp"
    subprocess.check_call(
        ["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"]
    )
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    # MOE_ORACLE_LIBRARY: a separately built copy of the same source (the
    # sanitizer test loads an instrumented build this way)
    override = os.environ.get("MOE_ORACLE_LIBRARY")
    if override:
        lib = ctypes.CDLL(override)
    else:
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
    vp = ctypes.c_void_p
    i32 = ctypes.c_int
    lib.oracle_capacity.argtypes = [i32, i32, i32, ctypes.c_double]
    lib.oracle_capacity.restype = i32
    lib.oracle_logits.argtypes = [i32, i32, i32, vp, i32, vp, vp, vp]
    lib.oracle_route.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.oracle_dispatch.argtypes = [i32, i32, i32, i32, i32, vp, i32, vp, vp, vp]
    lib.oracle_expert_ffn.argtypes = [i32, i32, i32, i32, vp, vp, i32, vp, vp, vp, vp, vp]
    lib.oracle_combine.argtypes = [i32, i32, i32, i32, i32, vp, vp, vp, vp, vp]
    lib.oracle_token_output.argtypes = [i32, vp, i32, i32, i32, vp, i32, vp, vp, vp, vp, vp, vp, vp, vp]
    f64 = ctypes.c_double
    lib.oracle_layer_backward.argtypes = [i32] * 7 + [vp, i32, vp, vp, vp, vp, vp, vp, vp, f64, f64] \
        + [vp] * 9
    lib.oracle_reroute.argtypes = [i32, i32, i32, i32, vp, vp, vp, vp, vp]
    lib.oracle_router_backward.argtypes = [i32, i32, i32, vp, vp, vp, vp, vp, f64, f64, vp]
    lib.oracle_backward_entries.argtypes = [i32] * 7 + [vp, i32, vp, vp, vp, vp, vp, vp, vp] \
        + [f64, f64, i32, vp, vp, i32, vp, vp, vp, vp, vp]
    for name in ("oracle_logits", "oracle_route", "oracle_dispatch", "oracle_expert_ffn",
                 "oracle_combine", "oracle_token_output", "oracle_layer_backward",
                 "oracle_router_backward", "oracle_backward_entries", "oracle_reroute"):
        getattr(lib, name).restype = None
    _lib = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _act(a: np.ndarray) -> tuple[np.ndarray, int]:
    a = np.ascontiguousarray(a)
    if a.dtype == np.float32:
        return a, F32
    if a.dtype == np.uint16:
        return a, BF16
    raise TypeError(f"activation arrays are float32 or uint16 (bf16 bits), got {a.dtype}")


def _same_dtype(ref: int, *arrays):
    out = []
    for a in arrays:
        if a is None:
            out.append(None)
            continue
        a, dt = _act(a)
        if dt != ref:
            raise TypeError("all activation arrays must share one dtype")
        out.append(a)
    return out


def capacity(S: int, E: int, k: int, capacity_factor: float) -> int:
    """C = ceil(capacity_factor * k * S / E)."""
    return int(_load().oracle_capacity(S, E, k, float(capacity_factor)))


def logits(x: np.ndarray, wg: np.ndarray, bg: np.ndarray | None = None) -> np.ndarray:
    """fp32 router logits x . Wg^T + bg, accumulated in fp64."""
    x, dt = _act(x)
    S, d = x.shape
    wg = np.ascontiguousarray(wg, dtype=np.float32)
    E = wg.shape[0]
    assert wg.shape == (E, d)
    if bg is not None:
        bg = np.ascontiguousarray(bg, dtype=np.float32)
        assert bg.shape == (E,)
    out = np.empty((S, E), dtype=np.float32)
    _load().oracle_logits(S, d, E, _ptr(x), dt, _ptr(wg), _ptr(bg), _ptr(out))
    return out


def route(lg: np.ndarray, k: int, C: int, reroute: bool = False) -> dict:
    """Softmax, top-k, renormalised weights, capacity slots, counts, losses.
    ``serve`` is the expert serving each assignment: ``idx``, except that
    with ``reroute`` dropped assignments move to alternative experts
    (oracle_reroute); ``counts`` then gains a row k with the offers each
    expert accepted."""
    lg = np.ascontiguousarray(lg, dtype=np.float32)
    S, E = lg.shape
    assert 1 <= k <= E and C >= 1
    idx = np.empty((S, k), np.int32)
    w = np.empty((S, k), np.float64)
    slot = np.empty((S, k), np.int32)
    counts = np.empty((k, E), np.int32)
    lse = np.empty((S,), np.float64)
    psum = np.empty((E,), np.float64)
    losses = np.empty((2,), np.float64)
    _load().oracle_route(S, E, k, C, _ptr(lg), _ptr(idx), _ptr(w), _ptr(slot), _ptr(counts),
                         _ptr(lse), _ptr(psum), _ptr(losses))
    serve = idx
    if reroute:
        serve = np.empty_like(idx)
        acc = np.empty(E, np.int32)
        _load().oracle_reroute(S, E, k, C, _ptr(lg), _ptr(idx), _ptr(serve), _ptr(slot), _ptr(acc))
        counts = np.vstack([counts, acc[None, :]])
    return dict(idx=idx, serve=serve, w=w, slot=slot, counts=counts, lse=lse, psum=psum,
                aux=float(losses[0]), z=float(losses[1]))


def occupancy(counts: np.ndarray, C: int, k: int | None = None) -> np.ndarray:
    """Filled slots per expert: min(assignments, C), plus the accepted
    re-routed offers (row k of counts) when counts has k + 1 rows."""
    k = counts.shape[0] if k is None else k
    occ = np.minimum(counts[:k].sum(axis=0), C)
    if counts.shape[0] > k:
        occ = occ + counts[k]
    return occ.astype(np.int32)


def dispatch(x: np.ndarray, idx: np.ndarray, slot: np.ndarray, E: int, C: int) -> np.ndarray:
    """[E,C,d] buffer of dispatched rows (zero where no token was placed)."""
    x, dt = _act(x)
    S, d = x.shape
    k = idx.shape[1]
    idx = np.ascontiguousarray(idx, np.int32)
    slot = np.ascontiguousarray(slot, np.int32)
    xd = np.empty((E, C, d), dtype=x.dtype)
    _load().oracle_dispatch(S, d, E, C, k, _ptr(x), dt, _ptr(idx), _ptr(slot), _ptr(xd))
    return xd


def expert_ffn(xd, occ, w1, b1, w2, b2) -> np.ndarray:
    """fp64 expert outputs [E,C,d] for filled slots (zero elsewhere)."""
    xd, dt = _act(xd)
    E, C, d = xd.shape
    h = w1.shape[1]
    w1, b1, w2, b2 = _same_dtype(dt, w1, b1, w2, b2)
    assert w1.shape == (E, h, d) and w2.shape == (E, d, h)
    occ = np.ascontiguousarray(occ, np.int32)
    out = np.empty((E, C, d), np.float64)
    _load().oracle_expert_ffn(E, C, d, h, _ptr(occ), _ptr(xd), dt, _ptr(w1), _ptr(b1),
                              _ptr(w2), _ptr(b2), _ptr(out))
    return out


def combine(out: np.ndarray, idx, slot, w, S: int) -> np.ndarray:
    """fp64 layer output y [S,d] = sum of kept w * expert output rows."""
    out = np.ascontiguousarray(out, np.float64)
    E, C, d = out.shape
    k = idx.shape[1]
    idx = np.ascontiguousarray(idx, np.int32)
    slot = np.ascontiguousarray(slot, np.int32)
    w = np.ascontiguousarray(w, np.float64)
    y = np.empty((S, d), np.float64)
    _load().oracle_combine(S, d, E, C, k, _ptr(out), _ptr(idx), _ptr(slot), _ptr(w), _ptr(y))
    return y


def token_output(tokens, x, w1, b1, w2, b2, idx, slot, w) -> np.ndarray:
    """fp64 y rows for the given tokens, computed per token without buffers."""
    x, dt = _act(x)
    S, d = x.shape
    h = w1.shape[1]
    k = idx.shape[1]
    w1, b1, w2, b2 = _same_dtype(dt, w1, b1, w2, b2)
    tokens = np.ascontiguousarray(tokens, np.int64)
    assert tokens.size == 0 or (tokens.min() >= 0 and tokens.max() < S)
    idx = np.ascontiguousarray(idx, np.int32)
    slot = np.ascontiguousarray(slot, np.int32)
    w = np.ascontiguousarray(w, np.float64)
    y = np.empty((tokens.size, d), np.float64)
    _load().oracle_token_output(tokens.size, _ptr(tokens), d, h, k, _ptr(x), dt, _ptr(w1),
                                _ptr(b1), _ptr(w2), _ptr(b2), _ptr(idx), _ptr(slot), _ptr(w),
                                _ptr(y))
    return y


def compact_rows(idx: np.ndarray, E: int) -> np.ndarray:
    """Dropless layout: the row of each assignment (s, r) in compact expert
    segments.  Assignments are numbered 0..S*k-1 in the order (expert, rank,
    token): expert segments back to back in expert order, and inside a
    segment the slot order of capacity routing (every first choice before
    any second choice, tokens in order).  A reading of the paper card
    "GShard: Scaling Giant Models with Conditional Computation and Automatic
    Sharding", method paragraph (dropless routing, as in MegaBlocks, keeps
    every assignment); the pages fix no layout.  A plain sort."""
    idx = np.asarray(idx)
    S, k = idx.shape
    assert S == 0 or (idx.min() >= 0 and idx.max() < E)
    tok = np.repeat(np.arange(S), k)
    rank = np.tile(np.arange(k), S)
    order = np.lexsort((tok, rank, idx.reshape(-1)))  # last key is the primary one
    rows = np.empty(S * k, np.int64)
    rows[order] = np.arange(S * k)
    return rows.reshape(S, k)


def layer_dropless(x, wg, bg, w1, b1, w2, b2, k: int, lg: np.ndarray | None = None) -> dict:
    """Whole forward pass with no capacity limit (every assignment kept):
    y[s] = sum_r w[s,r] FFN_{idx[s,r]}(x[s]), the dense top-k sum.  Routing,
    weights and losses are those of capacity routing (a capacity of S cannot
    be reached, as a token's k experts are distinct).  Also returns the
    compact layout: ``rows`` [S,k] and the expert outputs ``out_rows``
    [S*k,d] (fp64) and dispatched inputs ``xd_rows`` [S*k,d] in row order."""
    x_act, _ = _act(x)
    S = x_act.shape[0]
    if lg is None:
        lg = logits(x, wg, bg)
    E = lg.shape[1]
    res = layer(x, wg, bg, w1, b1, w2, b2, k, max(S, 1), lg=lg)
    assert (res["slot"] >= 0).all()
    rows = compact_rows(res["idx"], E)
    d = x_act.shape[1]
    out_rows = np.zeros((S * k, d), np.float64)
    xd_rows = np.zeros((S * k, d), x_act.dtype)
    flat = rows.reshape(-1)
    out_rows[flat] = res["out"][res["idx"].reshape(-1), res["slot"].reshape(-1)]
    xd_rows[flat] = np.repeat(x_act, k, axis=0)
    res.update(rows=rows, out_rows=out_rows, xd_rows=xd_rows)
    return res


def layer(x, wg, bg, w1, b1, w2, b2, k: int, C: int, lg: np.ndarray | None = None,
          reroute: bool = False) -> dict:
    """Whole forward pass.  With ``lg`` given, routing starts from those fp32
    logits instead of computing them (used to compare against a device that
    produced the logits itself)."""
    if lg is None:
        lg = logits(x, wg, bg)
    r = route(lg, k, C, reroute)
    E = lg.shape[1]
    S = lg.shape[0]
    xd = dispatch(x, r["serve"], r["slot"], E, C)
    occ = occupancy(r["counts"], C, k)
    out = expert_ffn(xd, occ, w1, b1, w2, b2)
    y = combine(out, r["serve"], r["slot"], r["w"], S)
    r.update(logits=lg, xd=xd, occ=occ, out=out, y=y)
    return r


def layer_backward(x, wg, w1, b1, w2, b2, k: int, C: int, lg: np.ndarray, dy: np.ndarray,
                   g_aux: float = 0.0, g_z: float = 0.0, reroute: bool = False) -> dict:
    """fp64 gradients of L = sum(dy * y) + g_aux * aux + g_z * z with the
    routing that the fp32 logits ``lg`` select (capacity C; C = S for
    dropless routing, which no expert can exceed).  Returns dx [S,d],
    dwg [E,d], dbg [E], dw1 [E,h,d], db1 [E,h], dw2 [E,d,h], db2 [E,d],
    dl [S,E] (gradient of the logits) and dw [S,k] (of the top-k weights)."""
    x, dt = _act(x)
    S, d = x.shape
    h = w1.shape[1]
    lg = np.ascontiguousarray(lg, dtype=np.float32)
    E = lg.shape[1]
    w1, b1, w2, b2, dy = _same_dtype(dt, w1, b1, w2, b2, dy)
    assert w1.shape == (E, h, d) and w2.shape == (E, d, h) and dy.shape == (S, d)
    wg = np.ascontiguousarray(wg, dtype=np.float32)
    assert wg.shape == (E, d) and 1 <= k <= E and C >= 1
    out = dict(dx=np.empty((S, d)), dwg=np.empty((E, d)), dbg=np.empty(E),
               dw1=np.empty((E, h, d)), db1=np.empty((E, h)), dw2=np.empty((E, d, h)),
               db2=np.empty((E, d)), dl=np.empty((S, E)), dw=np.empty((S, k)))
    _load().oracle_layer_backward(
        S, d, h, E, k, C, int(reroute), _ptr(x), dt, _ptr(wg), _ptr(lg), _ptr(w1), _ptr(b1), _ptr(w2),
        _ptr(b2), _ptr(dy), float(g_aux), float(g_z),
        *[_ptr(out[n]) for n in ("dx", "dwg", "dbg", "dw1", "db1", "dw2", "db2", "dl", "dw")])
    return out


def router_backward(lg: np.ndarray, idx, w, dw, counts, g_aux: float, g_z: float) -> np.ndarray:
    """fp64 gradient of the logits [S,E] from the top-k weight gradient dw
    [S,k] (any source, e.g. dot products with given expert outputs), the aux
    loss and the z-loss."""
    lg = np.ascontiguousarray(lg, dtype=np.float32)
    S, E = lg.shape
    k = idx.shape[1]
    idx = np.ascontiguousarray(idx, np.int32)
    w = np.ascontiguousarray(w, np.float64)
    dw = np.ascontiguousarray(dw, np.float64)
    counts = np.ascontiguousarray(counts, np.int32)
    assert idx.shape == w.shape == dw.shape == (S, k) and counts.shape == (k, E)
    dl = np.empty((S, E))
    _load().oracle_router_backward(S, E, k, _ptr(lg), _ptr(idx), _ptr(w), _ptr(dw), _ptr(counts),
                                   float(g_aux), float(g_z), _ptr(dl))
    return dl


def backward_entries(x, wg, w1, b1, w2, b2, k: int, C: int, lg, dy, g_aux, g_z, tokens,
                     entries, reroute: bool = False) -> tuple[np.ndarray, np.ndarray]:
    """dx rows of ``tokens`` and weight-gradient ``entries`` [(kind, e, a, b)]
    (kind 1 dW1[e,a,b], 2 dW2[e,a,b], 3 db1[e,a], 4 db2[e,a]) computed one by
    one, for full-size checks."""
    x, dt = _act(x)
    S, d = x.shape
    h = w1.shape[1]
    lg = np.ascontiguousarray(lg, dtype=np.float32)
    E = lg.shape[1]
    w1, b1, w2, b2, dy = _same_dtype(dt, w1, b1, w2, b2, dy)
    wg = np.ascontiguousarray(wg, dtype=np.float32)
    tokens = np.ascontiguousarray(tokens, np.int64)
    ent = np.ascontiguousarray(np.asarray(entries, np.int32).reshape(-1, 4))
    kind, ee, ea, eb = (np.ascontiguousarray(ent[:, c]) for c in range(4))
    dx_rows = np.empty((tokens.size, d))
    vals = np.empty(len(ent))
    _load().oracle_backward_entries(
        S, d, h, E, k, C, int(reroute), _ptr(x), dt, _ptr(wg), _ptr(lg), _ptr(w1), _ptr(b1), _ptr(w2),
        _ptr(b2), _ptr(dy), float(g_aux), float(g_z), tokens.size, _ptr(tokens), _ptr(dx_rows),
        len(ent), _ptr(kind), _ptr(ee), _ptr(ea), _ptr(eb), _ptr(vals))
    return dx_rows, vals
