"""Multi-layer decode driver with width changes committed at step boundaries.

Drives an L-layer MoE stack through the C ABI: each step runs, for every
layer, top-k routing -> permutation -> fused FFN on that layer's inputs.
Widths change only between steps ("commit at safe boundaries", PagedWeight
pages, "Technical summary: PagedWeight", Core components 3), in one of three
modes:

* "async" (the pages' design): at an event the driver snapshots the device
  routing mass (an asynchronous copy behind the finished steps), enqueues the
  event's step at the widths in force, then waits only for the snapshot, lets
  the library choose the blocks (pw_plan_event, or pw_retarget for a byte
  target) and requests the new widths (pw_request_widths): the plane and LUT
  copies run on a side stream while the steps go on.  Before every step,
  pw_commit_ready commits whatever has landed, so a request takes effect at
  the first step boundary after its copies, and the compute stream never
  waits for the copy stream.
* "blocking": the event commits with pw_set_committed_bits before the
  event's step (the compute stream waits for the copies).
* "none": no width changes.

Every step's committed widths are logged (q_log) so the oracle can replay
each (step, layer) at the widths it ran with.  The work runs in libpw.so;
this module only marshals buffers and holds the schedule.
"""
from __future__ import annotations

import time
from typing import Callable, Optional, Sequence

import numpy as np

from . import Context, plan_event


class StackDriver:
    def __init__(self, ctx: Context, q_init: np.ndarray, logits: np.ndarray, x: np.ndarray,
                 commit_every: int = 8, fraction: float = 0.2, device="cuda:0",
                 byte_targets: Optional[Sequence[int]] = None, sensitivity: Optional[np.ndarray] = None,
                 plan_params: Optional[dict] = None, mode: str = "async",
                 target_fn: Optional[Callable[[int], int]] = None, request_lead: int = 0):
        """q_init: int [L][E][2] routed widths as registered; logits: fp32
        [S][L][T][E]; x: fp16 [S][L][T][H] (staged to the device once).

        Events come every `commit_every` steps.  Without byte_targets or
        target_fn, an event moves `fraction` of the routed blocks one bit
        (odd events lower, even events raise; least routing mass first).
        With byte_targets (one routed-byte target per event, cycled) the
        event plans the widths for that target (pw_plan_widths on the device
        routing mass with the per-block `sensitivity` [L][E][2] and
        plan_params).  target_fn(step) -> routed-byte target replaces the
        event schedule by a memory-target trigger: whenever the target
        changes, the widths are re-planned for it (async mode only).
        request_lead (async mode): the host enqueues this many further steps
        before it plans and issues an event's request, so the host time of
        the request overlaps work already queued on the GPU (the widths the
        steps use are unaffected: commits happen only at step boundaries
        after the request's copies land)."""
        import torch
        d = ctx.desc
        S, L, T, E = logits.shape
        if mode not in ("async", "blocking", "none"):
            raise ValueError("mode must be async, blocking or none")
        if target_fn is not None and mode != "async":
            raise ValueError("a memory-target trigger needs the async mode")
        self.ctx, self.S, self.L, self.T, self.E, self.k = ctx, S, L, T, E, d.top_k
        self.mode = mode
        self.q = np.array(q_init, dtype=np.int64)      # committed routed widths [L][E][2]
        self.qd = self.q.copy()                         # desired widths (committed or requested)
        self.commit_every, self.fraction = commit_every, fraction
        self.byte_targets = None if byte_targets is None else [int(b) for b in byte_targets]
        self.sensitivity = None if sensitivity is None else np.asarray(sensitivity, np.float32)
        self.plan_params = dict(plan_params or {})
        self.target_fn = target_fn
        self.request_lead = max(0, int(request_lead))
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
        self.mass_snap = torch.zeros((L * E,), dtype=torch.float64).pin_memory()
        self.q_log = []       # committed widths [L][E][2] each step ran with
        self.events = []      # (step, lowered?, n blocks requested or committed, resident bytes after the call)
        self.plans = []       # budget / target modes: (step, target, planned routed bytes)
        self.commits = []     # (step boundary, blocks committed there)
        self.requests = []    # async: (step, n blocks, H2D bytes, start / end events on the copy stream)
        self.last_target = None
        self.host_s = {"request": 0.0, "commit": 0.0, "plan": 0.0}  # host time in library calls
        ctx.routing_mass_enable(True)
        ctx.routing_mass_reset(self.compute)
        self.graphs = None
        torch.cuda.synchronize()  # staged buffers ready before the side streams use them

    # ------------------------------------------------------------ steps
    def layer_step(self, s: int, l: int) -> None:
        self.ctx.moe_layer(l, self.logits[s, l], self.x[s, l], self.T, self.idx[s, l], self.w[s, l],
                           self.offsets[l], self.sorted[l], self.y[l], self.ws, self.ws_bytes, self.compute)

    def capture_graphs(self) -> None:
        """One HIP graph per step (its L layer calls).  Kernels read widths from
        the device page table, so width commits between replays stay valid."""
        import torch
        with torch.cuda.stream(self.compute):
            for l in range(self.L):
                self.layer_step(0, l)
        torch.cuda.synchronize()
        self.graphs = []
        for s in range(self.S):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=self.compute):
                for l in range(self.L):
                    self.layer_step(s, l)
            self.graphs.append(g)
        torch.cuda.synchronize()

    def enqueue_step(self, s: int, on_layer=None) -> None:
        import torch
        if self.graphs is not None and on_layer is None:
            with torch.cuda.stream(self.compute):
                self.graphs[s].replay()
            return
        for l in range(self.L):
            self.layer_step(s, l)
            if on_layer is not None:
                on_layer(s, l)

    # ------------------------------------------------------------ events
    def is_event(self, s: int) -> bool:
        if self.mode == "none" or self.target_fn is not None:
            return False
        return s > 0 and s % self.commit_every == 0

    def _refresh_committed(self) -> None:
        qc = self.ctx.committed_widths()
        self.q = qc[:, :self.E, :].astype(np.int64)

    def _snapshot(self):
        """Routing mass behind the work enqueued so far (asynchronous)."""
        import torch
        self.ctx.routing_mass_copy(self.mass_snap, self.compute)
        ev = torch.cuda.Event()
        ev.record(self.compute)
        return ev

    def _mass(self, ev) -> np.ndarray:
        ev.synchronize()
        return self.mass_snap.numpy().reshape(self.L, self.E).copy()

    def _choose(self, s: int, mass: np.ndarray):
        """(ids, new widths, lowered?) of an event before step s."""
        skip = (self.qd != self.q).astype(np.uint8)  # blocks with a request in flight
        if self.byte_targets is None:
            k = s // self.commit_every
            lower = (k % 2) == 1
            n = int(round(self.fraction * self.L * self.E * 2))
            ids, newq = plan_event(self.qd, mass, lower, n, skip)
            return ids, newq, lower
        raise AssertionError("byte targets are planned by _budget_event")

    def _budget_event(self, s: int, mass: np.ndarray, target: int) -> None:
        before = self.qd.copy()
        n, total = self.ctx.retarget(target, mass, self._sens(), self.copy, **self.plan_params)
        self._record_request(s, n, before)
        self.plans.append((s, target, total))

    def _sens(self) -> np.ndarray:
        if self.sensitivity is None:
            return np.ones((self.L, self.E, 2), np.float32)
        return self.sensitivity

    def _record_request(self, s: int, n: int, before: np.ndarray) -> None:
        """After requests were issued: desired widths from the library, the
        event logged."""
        for l in range(self.L):
            for e in range(self.E):
                for m in (0, 1):
                    if n:
                        self.qd[l, e, m] = self.ctx.block_state(self.ctx.block_id(l, e, m))[1]
        lowered = bool(np.sum(self.qd - before) < 0)
        self.events.append((s, lowered, int(n), self.ctx.resident_bytes()))

    def _request(self, s: int, ids: np.ndarray, newq: np.ndarray, lowered: bool) -> None:
        import torch
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        start.record(self.copy)
        t0 = time.perf_counter()
        if ids.size:
            self.ctx.request_widths(ids, newq, self.copy)
        self.host_s["request"] += time.perf_counter() - t0
        end.record(self.copy)
        h2d = 0
        for b, qn in zip(ids.tolist(), newq.tolist()):
            m, e, l = b & 1, (b >> 1) % (self.E + 1), (b >> 1) // (self.E + 1)
            self.qd[l, e, m] = qn
            h2d += self._move_bytes(m, int(self.q[l, e, m]), int(qn))
        self.requests.append((s, int(ids.size), h2d, start, end))
        self.events.append((s, lowered, int(ids.size), self.ctx.resident_bytes()))

    def _move_bytes(self, module: int, q_old: int, q_new: int) -> int:
        """Host-to-device bytes of a width change: the planes gained plus the new LUT."""
        d = self.ctx.desc
        R, K = (2 * d.inter, d.hidden) if module == 0 else (d.hidden, d.inter)
        planes = max(0, q_new - q_old) * R * K // 8
        return planes + R * (1 << q_new) * 2

    def _blocking_event(self, s: int) -> None:
        self.compute.synchronize()
        mass = self.ctx.routing_mass(self.compute)
        if self.byte_targets is not None:
            target = self.byte_targets[(s // self.commit_every - 1) % len(self.byte_targets)]
            from . import plan_widths
            d = self.ctx.desc
            newq, total = plan_widths(d.hidden, d.inter, self.q.astype(np.uint8), mass, self._sens(), target,
                                      **self.plan_params)
            ch = np.argwhere(newq != self.q)
            ids = np.array([self.ctx.block_id(int(l), int(e), int(m)) for l, e, m in ch], dtype=np.int32)
            vals = np.array([newq[l, e, m] for l, e, m in ch], dtype=np.uint8)
            lowered = bool(np.sum(newq.astype(np.int64) - self.q) < 0)
            self.plans.append((s, target, total))
        else:
            ids, vals, lowered = self._choose(s, mass)
        if ids.size:
            self.ctx.set_committed_bits(ids, vals, self.compute, self.copy)
        self._refresh_committed()
        self.qd = self.q.copy()
        self.events.append((s, lowered, int(ids.size), self.ctx.resident_bytes()))

    # ------------------------------------------------------------ the run
    def boundary(self, s: int) -> None:
        """Safe boundary before step s: commit the requests whose copies landed."""
        if self.mode == "async":
            t0 = time.perf_counter()
            n = self.ctx.commit_ready(self.compute)
            self.host_s["commit"] += time.perf_counter() - t0
            if n:
                self._refresh_committed()
                self.commits.append((s, n))

    def _async_event(self, s: int, snap, target) -> None:
        mass = self._mass(snap)  # the GPU runs the steps enqueued since meanwhile
        if target is not None:
            self.last_target = target
            self._budget_event(s, mass, target)
        elif self.byte_targets is not None:
            tgt = self.byte_targets[(s // self.commit_every - 1) % len(self.byte_targets)]
            self._budget_event(s, mass, tgt)
        else:
            t0 = time.perf_counter()
            ids, newq, lowered = self._choose(s, mass)
            self.host_s["plan"] += time.perf_counter() - t0
            self._request(s, ids, newq, lowered)

    def run(self, steps: Optional[int] = None, on_layer=None) -> None:
        """All steps; on_layer(s, l) (if given) is called after each layer's
        work is enqueued (for checks; it may synchronise)."""
        n_steps = self.S if steps is None else steps
        deferred = []  # async events (step, snapshot event, trigger target or None) not yet requested
        for s in range(n_steps):
            self.boundary(s)
            if self.mode == "blocking" and self.is_event(s):
                self._blocking_event(s)
            target = self.target_fn(s) if self.target_fn is not None else None
            trigger = target is not None and target != self.last_target
            if trigger:
                self.last_target = target
            if self.mode == "async" and (self.is_event(s) or trigger):
                deferred.append((s, self._snapshot(), target if trigger else None))
            self.q_log.append(self.q.copy())
            self.enqueue_step(s, on_layer)
            while deferred and s >= deferred[0][0] + self.request_lead:
                self._async_event(*deferred.pop(0))
        while deferred:
            self._async_event(*deferred.pop(0))

    def drain(self) -> None:
        """Wait for outstanding copies and commit them (end of a run)."""
        self.copy.synchronize()
        self.boundary(self.S)
