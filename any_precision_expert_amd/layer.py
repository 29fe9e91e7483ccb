"""Glue for driving one MoE layer through the C ABI from Python.

Registers a layer's blocks (parent codes are packed by the library's host
packer) and holds the device buffers of one token batch.  Only argument
marshalling: route, permute and the FFN run in libpw.so.
"""
from __future__ import annotations

from typing import Optional

import numpy as np

from . import EXPERT_SHARED, MODULE_DOWN, MODULE_GATE_UP, QMAX, Context


def register_layer(ctx: Context, layer: int, weights) -> None:
    """weights: object with .gate_up/.down lists of blocks (code8, luts, q) and
    optional .shared_gate_up/.shared_down (registered at width 8)."""
    for e, (gu, dn) in enumerate(zip(weights.gate_up, weights.down)):
        ctx.register_code_block(layer, e, MODULE_GATE_UP, gu.code8, gu.luts, gu.q)
        ctx.register_code_block(layer, e, MODULE_DOWN, dn.code8, dn.luts, dn.q)
    if getattr(weights, "shared_gate_up", None) is not None:
        ctx.register_code_block(layer, EXPERT_SHARED, MODULE_GATE_UP, weights.shared_gate_up.code8,
                                weights.shared_gate_up.luts, QMAX)
        ctx.register_code_block(layer, EXPERT_SHARED, MODULE_DOWN, weights.shared_down.code8,
                                weights.shared_down.luts, QMAX)


class Batch:
    """Device buffers for T tokens of one layer (torch tensors on `device`)."""

    def __init__(self, ctx: Context, T: int, device="cuda:0"):
        import torch
        d = ctx.desc
        self.ctx, self.T = ctx, T
        self.logits = torch.zeros((T, d.num_experts), dtype=torch.float32, device=device)
        self.x = torch.zeros((T, d.hidden), dtype=torch.float16, device=device)
        self.idx = torch.zeros((T, d.top_k), dtype=torch.int32, device=device)
        self.w = torch.zeros((T, d.top_k), dtype=torch.float32, device=device)
        self.offsets = torch.zeros((d.num_experts + 1,), dtype=torch.int32, device=device)
        self.sorted = torch.zeros((max(T * d.top_k, 1),), dtype=torch.int32, device=device)
        self.y = torch.zeros((T, d.hidden), dtype=torch.float16, device=device)
        ws = ctx.workspace_size(T)
        self.ws = torch.empty((max(ws, 256),), dtype=torch.uint8, device=device)
        self.ws_bytes = ws

    def load(self, logits: np.ndarray, x: np.ndarray) -> None:
        import torch
        self.logits.copy_(torch.from_numpy(np.ascontiguousarray(logits, dtype=np.float32)))
        self.x.copy_(torch.from_numpy(np.ascontiguousarray(x, dtype=np.float16)))

    def route(self, stream=None, fused: bool = True) -> None:
        if fused:
            self.ctx.route_permute(self.logits, self.T, self.idx, self.w, self.offsets, self.sorted, stream)
        else:
            self.ctx.route_topk(self.logits, self.T, self.idx, self.w, stream)
            self.ctx.permute_by_expert(self.idx, self.T, self.offsets, self.sorted, stream)

    def ffn(self, layer: int, stream=None, x=None, y=None) -> None:
        self.ctx.moe_ffn_bitplane(layer, self.x if x is None else x, self.T, self.idx, self.w,
                                  self.offsets, self.sorted, self.y if y is None else y, self.ws,
                                  self.ws_bytes, stream)

    def step(self, layer: int, stream=None, separate: bool = False) -> None:
        """One pass of the hot path: route -> permute -> FFN -> combine, as one
        pw_moe_layer call (routing inside the gate_up launch for decode-sized
        batches) or, with `separate`, as pw_route_permute + pw_moe_ffn_bitplane."""
        if separate:
            self.route(stream)
            self.ffn(layer, stream)
            return
        self.ctx.moe_layer(layer, self.logits, self.x, self.T, self.idx, self.w, self.offsets, self.sorted,
                           self.y, self.ws, self.ws_bytes, stream)
