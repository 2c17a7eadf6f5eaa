"""ctypes binding of ``libmoe.so`` (the C ABI declared in ``include/moe.h``).

Functions take torch tensors on the GPU, check their dtype, device, size and
contiguity (the C ABI receives raw pointers and cannot), and pass
``data_ptr()`` plus the current HIP stream.  Nothing is computed here.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_PKG, "libmoe.so")

MOE_F32 = 0
MOE_BF16 = 1
MOE_GATE_LOGITS_IN = 1
MOE_CFG_DROPLESS = 1
MOE_CFG_REROUTE = 2
MOE_NUM_STAGE_EVENTS = 9
MOE_NUM_BWD_EVENTS = 9

MOE_STATIC_SCRATCH_BYTES = 32 << 20

_STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_UNSUPPORTED",
           3: "MOE_ERR_WORKSPACE", 4: "MOE_ERR_HIP", 5: "MOE_ERR_SCRATCH_LIMIT"}


class MoeError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_STATUS.get(status, status)}")


class MoeConfig(ctypes.Structure):
    _fields_ = [
        ("S", ctypes.c_int32),
        ("d_model", ctypes.c_int32),
        ("d_ff", ctypes.c_int32),
        ("E", ctypes.c_int32),
        ("k", ctypes.c_int32),
        ("capacity", ctypes.c_int32),
        ("capacity_factor", ctypes.c_double),
        ("act_dtype", ctypes.c_int32),
        ("flags", ctypes.c_uint32),
    ]

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.act_dtype == MOE_BF16 else torch.float32

    @property
    def dropless(self) -> bool:
        return bool(self.flags & MOE_CFG_DROPLESS)

    @property
    def reroute(self) -> bool:
        return bool(self.flags & MOE_CFG_REROUTE)

    @property
    def count_rows(self) -> int:
        """Rows of counts: k, or k + 1 with re-routing."""
        return self.k + (1 if self.reroute else 0)


def config(S, d_model, d_ff, E, k, capacity_factor=1.0, capacity=0, dtype="bf16",
           dropless=False, reroute=False) -> MoeConfig:
    """Layer shape.  ``dropless``: no capacity limit; xd/out are compact
    [S*k, d] expert segments and ``slot`` holds global rows.  ``reroute``:
    dropped assignments are offered to the tokens' next-ranked experts."""
    dt = {"bf16": MOE_BF16, "f32": MOE_F32, torch.bfloat16: MOE_BF16,
          torch.float32: MOE_F32}[dtype]
    return MoeConfig(int(S), int(d_model), int(d_ff), int(E), int(k), int(capacity),
                     float(capacity_factor), dt,
                     (MOE_CFG_DROPLESS if dropless else 0) | (MOE_CFG_REROUTE if reroute else 0))


_lib = None


def library():
    """Load ``libmoe.so``, building it first when it is missing or was built
    from sources other than the ones in the tree (a digest of csrc/ and
    include/ is stored beside the library); a failed build raises."""
    global _lib
    if _lib is not None:
        return _lib
    from . import _build
    if not _build.is_current(library_path, library_path + ".srcsha"):
        _build.build()
    if not _build.is_current(library_path, library_path + ".srcsha"):
        raise RuntimeError(f"HIP library {library_path} is missing or stale and could not be "
                           f"built from the sources")
    lib = ctypes.CDLL(library_path)
    vp, cfgp = ctypes.c_void_p, ctypes.POINTER(MoeConfig)
    lib.moe_capacity.argtypes = [cfgp]
    lib.moe_capacity.restype = ctypes.c_int32
    lib.moe_dispatch_rows.argtypes = [cfgp]
    lib.moe_dispatch_rows.restype = ctypes.c_int64
    lib.moe_workspace_bytes.argtypes = [cfgp, ctypes.POINTER(ctypes.c_size_t)]
    lib.moe_status_string.argtypes = [ctypes.c_int32]
    lib.moe_status_string.restype = ctypes.c_char_p
    lib.moe_gate.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_uint32, vp,
                             ctypes.c_size_t, vp]
    lib.moe_gate_noalloc.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                     ctypes.c_uint32, vp]
    lib.moe_dispatch.argtypes = [cfgp, vp, vp, vp, vp, vp]
    lib.moe_expert_ffn.argtypes = [cfgp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.moe_combine.argtypes = [cfgp, vp, vp, vp, vp, vp, vp]
    lib.moe_layer_forward.argtypes = [cfgp] + [vp] * 18 + [ctypes.c_size_t, vp, vp]
    lib.moe_backward_workspace_bytes.argtypes = [cfgp, ctypes.POINTER(ctypes.c_size_t)]
    f32 = ctypes.c_float
    lib.moe_layer_backward.argtypes = [cfgp] + [vp] * 13 + [f32, f32] + [vp] * 8 + \
        [ctypes.c_size_t, vp, vp]
    for f in ("moe_workspace_bytes", "moe_gate", "moe_gate_noalloc", "moe_dispatch", "moe_expert_ffn",
              "moe_combine", "moe_layer_forward", "moe_backward_workspace_bytes",
              "moe_layer_backward"):
        getattr(lib, f).restype = ctypes.c_int32
    _lib = lib
    return lib


def _check(status: int, where: str):
    if status != 0:
        raise MoeError(status, where)


def capacity(cfg: MoeConfig) -> int:
    return int(library().moe_capacity(ctypes.byref(cfg)))


def dispatch_rows(cfg: MoeConfig) -> int:
    """Rows of xd/out: E*C, or S*k for a dropless config."""
    return int(library().moe_dispatch_rows(ctypes.byref(cfg)))


def workspace_bytes(cfg: MoeConfig) -> int:
    n = ctypes.c_size_t(0)
    _check(library().moe_workspace_bytes(ctypes.byref(cfg), ctypes.byref(n)),
           "moe_workspace_bytes")
    return int(n.value)


def _stream(stream):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _arg(t, name, dtype, numel, required=True):
    """data_ptr of a checked tensor (None -> NULL)."""
    if t is None:
        if required:
            raise ValueError(f"{name} is required")
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() != numel:
        raise ValueError(f"{name} must have {numel} elements, got {t.numel()}")
    return ctypes.c_void_p(t.data_ptr())


def _ws(ws):
    if ws is None:
        raise ValueError("workspace is required")
    if ws.device.type != "cuda" or not ws.is_contiguous():
        raise ValueError("workspace must be a contiguous GPU tensor")
    return ctypes.c_void_p(ws.data_ptr()), ws.numel() * ws.element_size()


def _events(events, n):
    """ctypes array of n hipEvent_t handles (None entries -> NULL), or None."""
    if events is None:
        return None
    if len(events) != n:
        raise ValueError(f"events must hold {n} events")
    handles = [None if e is None else e.cuda_event for e in events]
    if not all(h for e, h in zip(events, handles) if e is not None):
        raise ValueError("events must be created (recorded once) before use")
    return (ctypes.c_void_p * n)(*handles)


def gate(cfg, x, w_gate, gate_bias, logits, topk_idx, topk_w, slot, counts, losses, ws,
         logits_in=False, stream=None):
    """Router, top-k and capacity slots (``moe_gate``)."""
    S, d, E, k = cfg.S, cfg.d_model, cfg.E, cfg.k
    at = cfg.torch_dtype
    wsp, wsb = _ws(ws)
    st = library().moe_gate(
        ctypes.byref(cfg),
        _arg(x, "x", at, S * d, required=not logits_in),
        _arg(w_gate, "w_gate", torch.float32, E * d, required=not logits_in),
        _arg(gate_bias, "gate_bias", torch.float32, E, required=False),
        _arg(logits, "logits", torch.float32, S * E, required=logits_in),
        _arg(topk_idx, "topk_idx", torch.int32, S * k),
        _arg(topk_w, "topk_w", torch.float32, S * k),
        _arg(slot, "slot", torch.int32, S * k),
        _arg(counts, "counts", torch.int32, cfg.count_rows * E),
        _arg(losses, "losses", torch.float32, 2),
        MOE_GATE_LOGITS_IN if logits_in else 0, wsp, wsb, _stream(stream))
    _check(st, "moe_gate")


def gate_noalloc(cfg, x, w_gate, gate_bias, logits, topk_idx, topk_w, slot, counts, losses,
                 logits_in=False, stream=None):
    """``moe_gate`` on the library's static scratch (``moe_gate_noalloc``): no
    workspace argument, nothing allocated."""
    S, d, E, k = cfg.S, cfg.d_model, cfg.E, cfg.k
    at = cfg.torch_dtype
    st = library().moe_gate_noalloc(
        ctypes.byref(cfg),
        _arg(x, "x", at, S * d, required=not logits_in),
        _arg(w_gate, "w_gate", torch.float32, E * d, required=not logits_in),
        _arg(gate_bias, "gate_bias", torch.float32, E, required=False),
        _arg(logits, "logits", torch.float32, S * E, required=logits_in),
        _arg(topk_idx, "topk_idx", torch.int32, S * k),
        _arg(topk_w, "topk_w", torch.float32, S * k),
        _arg(slot, "slot", torch.int32, S * k),
        _arg(counts, "counts", torch.int32, cfg.count_rows * E),
        _arg(losses, "losses", torch.float32, 2),
        MOE_GATE_LOGITS_IN if logits_in else 0, _stream(stream))
    _check(st, "moe_gate_noalloc")


def dispatch(cfg, x, topk_idx, slot, xd, stream=None):
    """Permute token rows into [E,C,d] or compact [S*k,d] (``moe_dispatch``)."""
    R = dispatch_rows(cfg)
    at = cfg.torch_dtype
    st = library().moe_dispatch(
        ctypes.byref(cfg), _arg(x, "x", at, cfg.S * cfg.d_model),
        _arg(topk_idx, "topk_idx", torch.int32, cfg.S * cfg.k),
        _arg(slot, "slot", torch.int32, cfg.S * cfg.k),
        _arg(xd, "xd", at, R * cfg.d_model), _stream(stream))
    _check(st, "moe_dispatch")


def expert_ffn(cfg, xd, counts, w1, b1, w2, b2, out, ws, stream=None):
    """Expert ReLU FFNs over filled slots (``moe_expert_ffn``)."""
    R = dispatch_rows(cfg)
    E, d, h = cfg.E, cfg.d_model, cfg.d_ff
    at = cfg.torch_dtype
    wsp, wsb = _ws(ws)
    st = library().moe_expert_ffn(
        ctypes.byref(cfg), _arg(xd, "xd", at, R * d),
        _arg(counts, "counts", torch.int32, cfg.count_rows * E),
        _arg(w1, "w1", at, E * h * d), _arg(b1, "b1", at, E * h, required=False),
        _arg(w2, "w2", at, E * d * h), _arg(b2, "b2", at, E * d, required=False),
        _arg(out, "out", at, R * d), wsp, wsb, _stream(stream))
    _check(st, "moe_expert_ffn")


def combine(cfg, out, topk_idx, slot, topk_w, y, stream=None):
    """Gate-weighted combine back to token order (``moe_combine``)."""
    R = dispatch_rows(cfg)
    at = cfg.torch_dtype
    S, k = cfg.S, cfg.k
    st = library().moe_combine(
        ctypes.byref(cfg), _arg(out, "out", at, R * cfg.d_model),
        _arg(topk_idx, "topk_idx", torch.int32, S * k), _arg(slot, "slot", torch.int32, S * k),
        _arg(topk_w, "topk_w", torch.float32, S * k), _arg(y, "y", at, S * cfg.d_model),
        _stream(stream))
    _check(st, "moe_combine")


def layer_forward(cfg, x, w_gate, gate_bias, w1, b1, w2, b2, y, ws, logits=None,
                  topk_idx=None, topk_w=None, slot=None, counts=None, losses=None, xd=None,
                  out=None, hidden=None, events=None, stream=None):
    """Whole forward pass (``moe_layer_forward``).  ``events``: None or a list
    of MOE_NUM_STAGE_EVENTS entries, each None (boundary not recorded) or a
    torch.cuda.Event already created."""
    R = dispatch_rows(cfg)
    S, d, h, E, k = cfg.S, cfg.d_model, cfg.d_ff, cfg.E, cfg.k
    at = cfg.torch_dtype
    wsp, wsb = _ws(ws)
    ev = _events(events, MOE_NUM_STAGE_EVENTS)
    st = library().moe_layer_forward(
        ctypes.byref(cfg), _arg(x, "x", at, S * d), _arg(w_gate, "w_gate", torch.float32, E * d),
        _arg(gate_bias, "gate_bias", torch.float32, E, required=False),
        _arg(w1, "w1", at, E * h * d), _arg(b1, "b1", at, E * h, required=False),
        _arg(w2, "w2", at, E * d * h), _arg(b2, "b2", at, E * d, required=False),
        _arg(y, "y", at, S * d),
        _arg(logits, "logits", torch.float32, S * E, required=False),
        _arg(topk_idx, "topk_idx", torch.int32, S * k, required=False),
        _arg(topk_w, "topk_w", torch.float32, S * k, required=False),
        _arg(slot, "slot", torch.int32, S * k, required=False),
        _arg(counts, "counts", torch.int32, cfg.count_rows * E, required=False),
        _arg(losses, "losses", torch.float32, 2, required=False),
        _arg(xd, "xd", at, R * d, required=False),
        _arg(out, "out", at, R * d, required=False),
        _arg(hidden, "hidden", at, R * h, required=False),
        wsp, wsb, ev, _stream(stream))
    _check(st, "moe_layer_forward")


def backward_workspace_bytes(cfg: MoeConfig) -> int:
    n = ctypes.c_size_t(0)
    _check(library().moe_backward_workspace_bytes(ctypes.byref(cfg), ctypes.byref(n)),
           "moe_backward_workspace_bytes")
    return int(n.value)


def layer_backward(cfg, x, w_gate, w1, b1, w2, logits, topk_idx, topk_w, slot, counts, out, dy,
                   dx, dw_gate, dw1, dw2, ws, db_gate=None, db1=None, db2=None, g_aux=0.0,
                   g_z=0.0, hidden=None, events=None, stream=None):
    """Gradients of sum(dy*y) + g_aux*aux + g_z*z (``moe_layer_backward``).
    ``events``: None or MOE_NUM_BWD_EVENTS entries (None or created events)."""
    R = dispatch_rows(cfg)
    S, d, h, E, k = cfg.S, cfg.d_model, cfg.d_ff, cfg.E, cfg.k
    at = cfg.torch_dtype
    wsp, wsb = _ws(ws)
    st = library().moe_layer_backward(
        ctypes.byref(cfg), _arg(x, "x", at, S * d), _arg(w_gate, "w_gate", torch.float32, E * d),
        _arg(w1, "w1", at, E * h * d), _arg(b1, "b1", at, E * h, required=False),
        _arg(w2, "w2", at, E * d * h), _arg(logits, "logits", torch.float32, S * E),
        _arg(topk_idx, "topk_idx", torch.int32, S * k),
        _arg(topk_w, "topk_w", torch.float32, S * k), _arg(slot, "slot", torch.int32, S * k),
        _arg(counts, "counts", torch.int32, cfg.count_rows * E), _arg(out, "out", at, R * d),
        _arg(hidden, "hidden", at, R * h, required=False), _arg(dy, "dy", at, S * d),
        float(g_aux), float(g_z), _arg(dx, "dx", at, S * d),
        _arg(dw_gate, "dw_gate", torch.float32, E * d),
        _arg(db_gate, "db_gate", torch.float32, E, required=False),
        _arg(dw1, "dw1", at, E * h * d), _arg(db1, "db1", at, E * h, required=False),
        _arg(dw2, "dw2", at, E * d * h), _arg(db2, "db2", at, E * d, required=False),
        wsp, wsb, _events(events, MOE_NUM_BWD_EVENTS), _stream(stream))
    _check(st, "moe_layer_backward")
