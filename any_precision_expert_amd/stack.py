"""Multi-layer decode driver with committed-width changes between steps.

Drives an L-layer MoE stack through the C ABI: each step runs, for every
layer, top-k routing -> permutation -> fused FFN on that layer's activations;
every `commit_every` steps a commit event changes the widths of a fraction of
the routed blocks (planner.plan_event) with pw_set_committed_bits, whose
plane/LUT reloads run on a side copy stream.  Widths change only between
steps ("commit at safe boundaries", PagedWeight pages, Core components 3).

Device buffers: all steps' activations are staged up front; routing outputs
are kept per (step, layer) so the routing mass can be read back at commit
events without copies on the hot path.  Only argument marshalling happens
here; the work runs in libpw.so.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np

from . import Context, plan_widths
from .planner import RoutingMass, apply_event, plan_event


class StackDriver:
    def __init__(self, ctx: Context, q_init: np.ndarray, logits: np.ndarray, x: np.ndarray,
                 commit_every: int = 8, fraction: float = 0.2, device="cuda:0",
                 byte_targets: Optional[Sequence[int]] = None, sensitivity: Optional[np.ndarray] = None,
                 plan_params: Optional[dict] = None):
        """q_init: int [L][E][2] routed widths; logits: fp32 [S][L][T][E];
        x: fp16 [S][L][T][H] (staged to the device once).

        Without byte_targets, each event changes `fraction` of the routed
        blocks by one bit (plan_event, host routing mass).  With byte_targets
        (one routed-byte target per event), the device routing-mass
        accumulator feeds the greedy planner (pw_plan_widths) with the given
        per-block sensitivity [L][E][2] and plan_params, and the event commits
        every width the planner changes."""
        import torch
        d = ctx.desc
        S, L, T, E = logits.shape
        self.ctx, self.S, self.L, self.T, self.E, self.k = ctx, S, L, T, E, d.top_k
        self.q = np.array(q_init, dtype=np.int64)
        self.mass = RoutingMass(L, E)
        self.commit_every, self.fraction = commit_every, fraction
        self.logits = torch.from_numpy(np.ascontiguousarray(logits, np.float32)).to(device)
        self.x = torch.from_numpy(np.ascontiguousarray(x, np.float16)).to(device)
        self.idx = torch.zeros((S, L, T, self.k), dtype=torch.int32, device=device)
        self.w = torch.zeros((S, L, T, self.k), dtype=torch.float32, device=device)
        self.offsets = torch.zeros((L, E + 1), dtype=torch.int32, device=device)
        self.sorted = torch.zeros((L, T * self.k), dtype=torch.int32, device=device)
        self.y = torch.zeros((L, T, d.hidden), dtype=torch.float16, device=device)
        self.ws_bytes = ctx.workspace_size(T)
        self.ws = torch.empty((max(self.ws_bytes, 256),), dtype=torch.uint8, device=device)
        self.compute = torch.cuda.Stream()
        self.copy = torch.cuda.Stream()
        self.mass_upto = 0
        self.events = []  # (step, lowered?, n blocks, bytes resident after)
        self.byte_targets = None if byte_targets is None else [int(b) for b in byte_targets]
        self.sensitivity = None if sensitivity is None else np.asarray(sensitivity, np.float32)
        self.plan_params = dict(plan_params or {})
        self.plans = []  # budget mode: (step, target, planned routed bytes, widths after)
        if self.byte_targets is not None:
            ctx.routing_mass_enable(True)
            ctx.routing_mass_reset(self.compute)
        torch.cuda.synchronize()  # staged buffers ready before the side streams use them

    def layer_step(self, s: int, l: int) -> None:
        c, st = self.ctx, self.compute
        c.moe_layer(l, self.logits[s, l], self.x[s, l], self.T, self.idx[s, l], self.w[s, l], self.offsets[l],
                    self.sorted[l], self.y[l], self.ws, self.ws_bytes, st)

    def step(self, s: int) -> None:
        for l in range(self.L):
            self.layer_step(s, l)

    def commit_event(self, s: int) -> None:
        """Before step s: accumulate routing mass of the finished steps, plan
        and commit one event (odd events lower, even events raise; or, with
        byte targets, whatever the planner changes)."""
        if self.byte_targets is not None:
            self._budget_event(s)
            return
        self.compute.synchronize()
        idx = self.idx[self.mass_upto:s].cpu().numpy()
        w = self.w[self.mass_upto:s].cpu().numpy()
        for l in range(self.L):
            self.mass.add(l, idx[:, l], w[:, l])
        self.mass_upto = s
        k = s // self.commit_every
        lower = (k % 2) == 1
        n = int(round(self.fraction * self.L * self.E * 2))
        ids, newq = plan_event(self.mass.m, self.q, lower, n)
        self.ctx.set_committed_bits(ids, newq, self.compute, self.copy)
        apply_event(self.q, ids, newq, self.E)
        self.events.append((s, lower, int(ids.size), self.ctx.resident_bytes()))

    def _budget_event(self, s: int) -> None:
        d = self.ctx.desc
        k = s // self.commit_every
        target = self.byte_targets[(k - 1) % len(self.byte_targets)]
        mass = self.ctx.routing_mass(self.compute)  # after the finished steps
        newq, total = plan_widths(d.hidden, d.inter, self.q.astype(np.uint8), mass, self.sensitivity, target,
                                  **self.plan_params)
        ch = np.argwhere(newq != self.q)
        ids = np.array([self.ctx.block_id(int(l), int(e), int(m)) for l, e, m in ch], dtype=np.int32)
        vals = np.array([newq[l, e, m] for l, e, m in ch], dtype=np.uint8)
        if ids.size:
            self.ctx.set_committed_bits(ids, vals, self.compute, self.copy)
        lowered = bool(np.sum(newq.astype(np.int64) - self.q) < 0)
        self.q = newq.astype(np.int64)
        self.events.append((s, lowered, int(ids.size), self.ctx.resident_bytes()))
        self.plans.append((s, target, total, self.q.copy()))

    def is_event(self, s: int) -> bool:
        return s > 0 and s % self.commit_every == 0

    def run(self, steps: Optional[int] = None, on_layer=None) -> None:
        """All steps; on_layer(s, l) (if given) is called after each layer's
        work is enqueued (for checks; it may synchronise)."""
        for s in range(self.S if steps is None else steps):
            if self.is_event(s):
                self.commit_event(s)
            for l in range(self.L):
                self.layer_step(s, l)
                if on_layer is not None:
                    on_layer(s, l)
