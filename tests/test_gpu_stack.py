"""The 24-layer Qwen-shaped decode stack (batch 4, 64 steps, Zipf routing)
with a commit event every 8 steps that lowers or raises by one bit the 20% of
routed blocks with the least routing mass.  The events run the pages'
asynchronous design: the library chooses the blocks from the device routing
mass, the plane / LUT copies run on a side stream while the steps go on, and
each request is committed at the first step boundary after its copies land.
Routing, permutation and y are checked against the fp64 oracle at the widths
logged for each checked step: every layer at the first and last steps and at
every step where a commit took effect, sampled layers around every event.
Also: the budget planner's blocking events, and a memory-target trigger
driven by a synthetic KV-cache schedule."""
import copy

import numpy as np
import pytest

import pw_synth
from tests.gpu_util import compare, say

pytestmark = pytest.mark.gpu

SAMPLE_LAYERS = (0, 5, 11, 17, 23)
EVENT_STEPS = (7, 8, 9, 15, 16, 17, 24, 31, 32, 40, 47, 48, 55, 56)


@pytest.fixture(scope="module", autouse=True)
def _gpu(require_gpu):
    import any_precision_expert_amd as pw
    pw.lib()


def _with_q(w, q):
    w2 = copy.copy(w)
    w2.gate_up = [copy.copy(b) for b in w.gate_up]
    w2.down = [copy.copy(b) for b in w.down]
    for e in range(len(w2.gate_up)):
        w2.gate_up[e].q, w2.down[e].q = int(q[e, 0]), int(q[e, 1])
    return w2


def _gpu_out(drv, s, l, T, k):
    return dict(idx=drv.idx[s, l].cpu().numpy(), w=drv.w[s, l].cpu().numpy(),
                offsets=drv.offsets[l].cpu().numpy(), sorted=drv.sorted[l].cpu().numpy()[:T * k],
                y=drv.y[l].cpu().numpy().astype(np.float64))


def test_config4_stack_with_async_commit_events():
    import torch
    import oracle
    import any_precision_expert_amd as pw
    from any_precision_expert_amd.layer import register_layer
    from any_precision_expert_amd.stack import StackDriver
    spec = pw_synth.CONFIGS[4]
    shape, T = spec.shape, spec.tokens[0]
    L, S = spec.layers, spec.steps
    seed = pw_synth.config_seed(4)
    ctx = pw.Context(0, L, shape.E, shape.H, shape.I, shape.top_k, shape.I_shared, keep_host_masters=True)
    weights, q0 = [], np.zeros((L, shape.E, 2), np.int64)
    try:
        for l in range(L):
            w = pw_synth.make_weights(shape, seed, l, spec.q_policy, spec.logits)
            register_layer(ctx, l, w)
            q0[l] = [[g.q, d.q] for g, d in zip(w.gate_up, w.down)]
            weights.append(w)
        say("registered %d layers, resident %.2f GB" % (L, ctx.resident_bytes() / 1e9))
        logits = np.zeros((S, L, T, shape.E), np.float32)
        x = np.zeros((S, L, T, shape.H), np.float16)
        for s in range(S):
            for l in range(L):
                a = pw_synth.make_activations(shape, T, seed, l, s, spec.logits, weights[l].rank)
                logits[s, l], x[s, l] = a.logits, a.x
        drv = StackDriver(ctx, q0, logits, x, commit_every=spec.extra["commit_every"],
                          fraction=spec.extra["commit_fraction"], mode="async")
        worst, checked = [0.0, 0.0], []

        def check(s, l):
            commit_step = bool(drv.commits) and drv.commits[-1][0] == s
            if not (s in (0, S - 1) or commit_step or (l in SAMPLE_LAYERS and s in EVENT_STEPS)):
                return
            drv.compute.synchronize()
            acts = pw_synth.Activations(x=x[s, l], logits=logits[s, l])
            ref = oracle.moe_layer(_with_q(weights[l], drv.q_log[s][l]), acts)
            rel, mx = compare(_gpu_out(drv, s, l, T, shape.top_k), ref, label="step %d layer %d" % (s, l))
            worst[0], worst[1] = max(worst[0], rel), max(worst[1], mx)
            checked.append((s, l))

        drv.run(on_layer=check)
        drv.drain()
        torch.cuda.synchronize()
        for ev in drv.events:
            say("event before step %d: %s, %d blocks requested" % (ev[0], "lower" if ev[1] else "raise", ev[2]))
        say("commits at step boundaries: %s" % drv.commits)
        assert len(drv.events) == 7
        # every event moves 20% of the routed blocks (576 of 2880) unless some
        # were still in transfer from the previous event (skipped, logged)
        for ev in drv.events:
            assert 0 < ev[2] <= 576
        assert sum(n for _, n in drv.commits) == sum(ev[2] for ev in drv.events)
        # widths changed only at step boundaries, one bit per event per block
        changes = [np.abs(drv.q_log[s + 1] - drv.q_log[s]).sum() for s in range(S - 1)]
        commit_steps = {c[0] for c in drv.commits}
        assert all(c == 0 for s, c in enumerate(changes) if (s + 1) not in commit_steps)
        # the host view of the committed widths matches the library's
        assert np.array_equal(ctx.committed_widths()[:, :shape.E, :], drv.q)
        assert np.array_equal(drv.q, drv.qd)
        say("worst rel_l2 %.3e max_abs %.3e over %d checks" % (worst[0], worst[1], len(checked)))
        assert len({l for s, l in checked if s == S - 1}) == L
    finally:
        ctx.close()


def test_budget_planner_stack():
    """Three Zipf-routed layers (H=256, I=256, 16 experts, top-2, batch 8),
    16 steps, an event every 4 steps with a routed-byte target (the bytes of
    every block at 4, then 7, then 5 bits): the device routing mass feeds
    pw_plan_widths and the event commits its widths before its step
    (pw_set_committed_bits, the blocking form).  Checks: committed widths and resident
    bytes equal the plan, the plan fits its target, hot experts stay at or
    above their floor, and every step matches the oracle at the widths
    committed for it."""
    import torch
    import oracle
    import oracle.plan as op
    import any_precision_expert_amd as pw
    from any_precision_expert_amd.layer import register_layer
    from any_precision_expert_amd.stack import StackDriver
    shape = pw_synth.LayerShape(H=256, I=256, E=16, top_k=2)
    L, S, T, seed = 3, 16, 8, 4242
    ctx = pw.Context(0, L, shape.E, shape.H, shape.I, shape.top_k, shape.I_shared, keep_host_masters=True)
    try:
        ws, q0, ranks = [], np.zeros((L, shape.E, 2), np.int64), []
        for l in range(L):
            w = pw_synth.make_weights(shape, seed, l, "zipf_tiers", "zipf")
            register_layer(ctx, l, w)
            q0[l] = [[g.q, d.q] for g, d in zip(w.gate_up, w.down)]
            ws.append(w)
            ranks.append(w.rank)
        init = ctx.resident_bytes()
        logits = np.zeros((S, L, T, shape.E), np.float32)
        x = np.zeros((S, L, T, shape.H), np.float16)
        for s in range(S):
            for l in range(L):
                a = pw_synth.make_activations(shape, T, seed, l, s, "zipf", ranks[l])
                logits[s, l], x[s, l] = a.logits, a.x
        sens = np.random.default_rng(seed).uniform(0.5, 1.5, size=(L, shape.E, 2)).astype(np.float32)
        params = dict(q_min=3, q_max=8, hot_floor=6, hot_share=0.15, hot_mult=4.0, mass_eps=1e-3)
        def uniform_bytes(qq):
            return L * shape.E * sum(op.block_bytes(*op.block_shape(m, shape.H, shape.I), qq) for m in (0, 1))
        assert init == sum(op.block_bytes(*op.block_shape(m, shape.H, shape.I), int(q0[l, e, m]))
                           for l in range(L) for e in range(shape.E) for m in (0, 1))
        targets = [uniform_bytes(4), uniform_bytes(7), uniform_bytes(5)]
        drv = StackDriver(ctx, q0, logits, x, commit_every=4, byte_targets=targets, sensitivity=sens,
                          plan_params=params, mode="blocking")
        mass_host = np.zeros((L, shape.E))
        worst = [0.0]

        def check(s, l):
            drv.compute.synchronize()
            k = shape.top_k
            gpu = dict(idx=drv.idx[s, l].cpu().numpy(), w=drv.w[s, l].cpu().numpy(),
                       offsets=drv.offsets[l].cpu().numpy(), sorted=drv.sorted[l].cpu().numpy()[:T * k],
                       y=drv.y[l].cpu().numpy().astype(np.float64))
            acts = pw_synth.Activations(x=x[s, l], logits=logits[s, l])
            rel, _ = compare(gpu, oracle.moe_layer(_with_q(ws[l], drv.q_log[s][l]), acts),
                             label="step %d layer %d" % (s, l))
            worst[0] = max(worst[0], rel)

        drv.run(on_layer=check)
        torch.cuda.synchronize()
        assert len(drv.plans) == 3
        for (s, target, total), ev in zip(drv.plans, drv.events):
            q = drv.q_log[s]  # the widths the event committed, used from step s on
            say("event before step %d: target %.2f MB, planned %.2f MB, resident %.2f MB, %d blocks changed"
                % (s, target / 1e6, total / 1e6, ev[3] / 1e6, ev[2]))
            assert total <= target and ev[3] == total  # algorithmic bytes = storage for these shapes
            # hot experts (share of their layer's mass up to this event) keep the floor
            for l in range(L):
                mass_host[l] = 0.0
                for s2 in range(s):
                    idx, gw = oracle.route_topk(logits[s2, l], shape.top_k)
                    row = list(mass_host[l])
                    op.routing_mass_add(row, idx.tolist(), gw.tolist())
                    mass_host[l] = row
                share = mass_host[l] / mass_host[l].sum()
                for e in np.nonzero(share >= params["hot_share"] + 1e-6)[0]:
                    assert np.all(q[l, e] >= params["hot_floor"]), (l, e)
        for l in range(L):
            for e in range(shape.E):
                for m in (0, 1):
                    assert ctx.committed_bits(ctx.block_id(l, e, m)) == drv.q[l, e, m]
        say("worst rel_l2 %.3e over %d checks" % (worst[0], S * L))
    finally:
        ctx.close()


def test_memory_target_trigger_with_async_commits():
    """A synthetic KV-cache schedule sets the routed-weight budget: the
    budget shrinks twice (KV growing) and then grows (KV freed).  Each change
    triggers pw_retarget (pw_plan_widths on the device routing mass, then
    pw_request_widths); the commits happen at step boundaries after the
    copies land.  Checks: every step matches the oracle at its logged widths;
    while a raise is in flight its new planes report IN_TRANSFER or READY and
    the planes above the desired width CPU; the final widths fit the last
    budget; after every block is lowered to 3 bits, trimming returns the
    freed plane chunks to the device."""
    import torch
    import oracle
    import oracle.plan as op
    import any_precision_expert_amd as pw
    from any_precision_expert_amd.layer import register_layer
    from any_precision_expert_amd.stack import StackDriver
    shape = pw_synth.LayerShape(H=256, I=256, E=16, top_k=2)
    L, S, T, seed = 3, 24, 8, 4343
    ctx = pw.Context(0, L, shape.E, shape.H, shape.I, shape.top_k, shape.I_shared, keep_host_masters=True)
    try:
        ws, q0 = [], np.zeros((L, shape.E, 2), np.int64)
        for l in range(L):
            w = pw_synth.make_weights(shape, seed, l, "zipf_tiers", "zipf")
            register_layer(ctx, l, w)
            q0[l] = [[g.q, d.q] for g, d in zip(w.gate_up, w.down)]
            ws.append(w)
        logits = np.zeros((S, L, T, shape.E), np.float32)
        x = np.zeros((S, L, T, shape.H), np.float16)
        for s in range(S):
            for l in range(L):
                a = pw_synth.make_activations(shape, T, seed, l, s, "zipf", ws[l].rank)
                logits[s, l], x[s, l] = a.logits, a.x

        def uniform_bytes(qq):
            return L * shape.E * sum(op.block_bytes(*op.block_shape(m, shape.H, shape.I), qq) for m in (0, 1))

        # device memory for the routed weights = a fixed budget minus a KV cache
        # that grows by a third of the 8-bit -> 4-bit difference at steps 5 and
        # 10, then is freed at step 18
        budget = uniform_bytes(8)
        kv = lambda s: (min(s, 14) // 5) * (uniform_bytes(8) - uniform_bytes(4)) // 3 if s < 18 else 0
        target_fn = lambda s: budget - kv(s)
        sens = np.random.default_rng(seed).uniform(0.5, 1.5, size=(L, shape.E, 2)).astype(np.float32)
        params = dict(q_min=3, q_max=8, hot_floor=6, hot_share=0.15, hot_mult=4.0, mass_eps=1e-3)
        drv = StackDriver(ctx, q0, logits, x, sensitivity=sens, plan_params=params, mode="async",
                          target_fn=target_fn)
        seen_states = []
        worst = [0.0]

        def check(s, l):
            drv.compute.synchronize()
            if l == 0:  # page states of a block with a request in flight, if any
                pend = np.argwhere(drv.qd != drv.q)
                if pend.size:
                    le, ee, mm = (int(v) for v in pend[0])
                    st = ctx.plane_states(ctx.block_id(le, ee, mm))
                    seen_states.append((int(drv.q[le, ee, mm]), int(drv.qd[le, ee, mm]), st.tolist()))
            acts = pw_synth.Activations(x=x[s, l], logits=logits[s, l])
            rel, _ = compare(_gpu_out(drv, s, l, T, shape.top_k),
                             oracle.moe_layer(_with_q(ws[l], drv.q_log[s][l]), acts), label="step %d layer %d" % (s, l))
            worst[0] = max(worst[0], rel)

        drv.run(on_layer=check)
        drv.drain()
        torch.cuda.synchronize()
        for p in drv.plans:
            say("trigger before step %d: target %.2f MB, planned %.2f MB" % (p[0], p[1] / 1e6, p[2] / 1e6))
        say("commits: %s" % drv.commits)
        assert [p[0] for p in drv.plans] == sorted({0, 5, 10, 18} & {s for s in range(S)})
        assert all(p[2] <= p[1] for p in drv.plans)
        final = sum(op.block_bytes(*op.block_shape(m, shape.H, shape.I), int(drv.q[l, e, m]))
                    for l in range(L) for e in range(shape.E) for m in (0, 1))
        assert final <= target_fn(S - 1) and final == drv.plans[-1][2]
        assert np.array_equal(ctx.committed_widths()[:, :shape.E, :], drv.q)
        # page states seen while a request was in flight
        assert seen_states, "no request was observed in flight"
        for qc, qd, st in seen_states:
            assert all(v == pw.PLANE_GPU for v in st[:qc])
            if qd > qc:
                assert all(v in (pw.PLANE_IN_TRANSFER, pw.PLANE_READY) for v in st[qc:qd])
            assert all(v == pw.PLANE_CPU for v in st[max(qc, qd):8])
            assert st[8] in (pw.PLANE_IN_TRANSFER, pw.PLANE_READY)
        # dropping the top planes of every block and trimming returns their
        # chunks to the device: device free memory grows by what trim reports
        ids = [ctx.block_id(l, e, m) for l in range(L) for e in range(shape.E) for m in (0, 1)]
        ctx.set_committed_bits(ids, [3] * len(ids))
        torch.cuda.synchronize()
        stats = ctx.pool_stats()
        free0 = torch.cuda.mem_get_info()[0]
        freed = ctx.trim()
        free1 = torch.cuda.mem_get_info()[0]
        after = ctx.pool_stats()
        say("pool %s, trim freed %.2f MB, device free +%.2f MB, after %s"
            % (stats, freed / 1e6, (free1 - free0) / 1e6, after))
        assert freed > 0 and after["held"] == stats["held"] - freed
        assert after["waiting"] == 0 and after["resident"] == stats["resident"]
        assert after["resident"] == sum(op.block_bytes(*op.block_shape(m, shape.H, shape.I), 3)
                                        for l in range(L) for e in range(shape.E) for m in (0, 1))
        assert free1 - free0 >= freed // 2  # the device sees (most of) the memory back
        say("worst rel_l2 %.3e over %d checks" % (worst[0], S * L))
    finally:
        ctx.close()
