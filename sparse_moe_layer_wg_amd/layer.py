"""Convenience owner of one MoE layer's device buffers.

``MoELayer`` keeps the weights, allocates the workspace and the optional
outputs once, and calls ``moe_layer_forward``.  It only allocates torch
tensors and forwards pointers; all computation happens in ``libmoe.so``.
"""
from __future__ import annotations

import torch

from . import _lib


class MoELayer:
    def __init__(self, cfg: _lib.MoeConfig, w_gate, gate_bias, w1, b1, w2, b2,
                 keep: bool = True, device="cuda", dispatch_buffer: bool = True,
                 keep_hidden: bool = False):
        self.cfg = cfg
        self.C = _lib.capacity(cfg)
        # rows of the dispatch buffer / expert output: [E,C] padded, or S*k
        # compact expert segments for a dropless config
        self.rows = _lib.dispatch_rows(cfg)
        rshape = (cfg.S * cfg.k,) if cfg.dropless else (cfg.E, self.C)
        self.w_gate, self.gate_bias = w_gate, gate_bias
        self.w1, self.b1, self.w2, self.b2 = w1, b1, w2, b2
        dev = torch.device(device)
        S, d, E, k = cfg.S, cfg.d_model, cfg.E, cfg.k
        at = cfg.torch_dtype
        self.ws = torch.empty(_lib.workspace_bytes(cfg), dtype=torch.uint8, device=dev)
        self.y = torch.empty((S, d), dtype=at, device=dev)
        self.keep = keep
        if keep:
            self.logits = torch.empty((S, E), dtype=torch.float32, device=dev)
            self.topk_idx = torch.empty((S, k), dtype=torch.int32, device=dev)
            self.topk_w = torch.empty((S, k), dtype=torch.float32, device=dev)
            self.slot = torch.empty((S, k), dtype=torch.int32, device=dev)
            self.counts = torch.empty((cfg.count_rows, E), dtype=torch.int32, device=dev)
            self.losses = torch.empty((2,), dtype=torch.float32, device=dev)
            # Without a dispatch buffer the first expert GEMM gathers token
            # rows straight from x (bf16); with one, x is first permuted into it.
            self.xd = torch.empty((*rshape, d), dtype=at, device=dev) if dispatch_buffer \
                else None
            self.out = torch.empty((*rshape, d), dtype=at, device=dev)
            # the expert hidden activations, kept for the backward pass
            self.hidden = torch.empty((*rshape, cfg.d_ff), dtype=at, device=dev) \
                if keep_hidden else None
        else:
            self.hidden = None
            self.logits = self.topk_idx = self.topk_w = self.slot = None
            self.counts = self.losses = self.xd = self.out = None
            self.losses = torch.empty((2,), dtype=torch.float32, device=dev)

    @classmethod
    def from_inputs(cls, cfg, inputs: dict, keep=True, dispatch_buffer=True, keep_hidden=False):
        return cls(cfg, inputs["wg"], inputs["bg"], inputs["w1"], inputs["b1"], inputs["w2"],
                   inputs["b2"], keep=keep, device=inputs["x"].device,
                   dispatch_buffer=dispatch_buffer, keep_hidden=keep_hidden)

    def forward(self, x, y=None, events=None, stream=None):
        y = self.y if y is None else y
        _lib.layer_forward(self.cfg, x, self.w_gate, self.gate_bias, self.w1, self.b1, self.w2,
                           self.b2, y, self.ws, logits=self.logits, topk_idx=self.topk_idx,
                           topk_w=self.topk_w, slot=self.slot, counts=self.counts,
                           losses=self.losses, xd=self.xd, out=self.out, hidden=self.hidden,
                           events=events, stream=stream)
        return y
