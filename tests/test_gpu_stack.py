"""The 24-layer Qwen-shaped decode stack (batch 4, 64 steps, Zipf routing)
with a commit event every 8 steps that lowers or raises by one bit the 20% of
routed blocks with the least routing mass.  Routing, permutation and y are
checked against the fp64 oracle at the widths committed for each checked
step, on sampled layers and on the steps around every commit event."""
import copy

import numpy as np
import pytest

import pw_synth
from tests.gpu_util import compare, say

pytestmark = pytest.mark.gpu

CHECK_LAYERS = (0, 11, 23)
CHECK_STEPS = (0, 7, 8, 9, 15, 16, 17, 24, 31, 32, 40, 47, 48, 55, 56, 63)


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


def test_config4_stack_with_commit_events():
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
    kept, q0, ranks = {}, np.zeros((L, shape.E, 2), np.int64), []
    try:
        for l in range(L):
            w = pw_synth.make_weights(shape, seed, l, spec.q_policy, spec.logits)
            register_layer(ctx, l, w)
            q0[l] = [[g.q, d.q] for g, d in zip(w.gate_up, w.down)]
            ranks.append(w.rank)
            if l in CHECK_LAYERS:
                kept[l] = w
        say("registered %d layers, resident %.2f GB" % (L, ctx.resident_bytes() / 1e9))
        logits = np.zeros((S, L, T, shape.E), np.float32)
        x = np.zeros((S, L, T, shape.H), np.float16)
        for s in range(S):
            for l in range(L):
                a = pw_synth.make_activations(shape, T, seed, l, s, spec.logits, ranks[l])
                logits[s, l], x[s, l] = a.logits, a.x
        drv = StackDriver(ctx, q0, logits, x, commit_every=spec.extra["commit_every"],
                          fraction=spec.extra["commit_fraction"])
        preps = {l: None for l in CHECK_LAYERS}
        worst = [0.0, 0.0]

        def check(s, l):
            if l not in CHECK_LAYERS or s not in CHECK_STEPS:
                return
            drv.compute.synchronize()
            k = shape.top_k
            gpu = dict(idx=drv.idx[s, l].cpu().numpy(), w=drv.w[s, l].cpu().numpy(),
                       offsets=drv.offsets[l].cpu().numpy(), sorted=drv.sorted[l].cpu().numpy()[:T * k],
                       y=drv.y[l].cpu().numpy().astype(np.float64))
            wq = _with_q(kept[l], drv.q[l])
            acts = pw_synth.Activations(x=x[s, l], logits=logits[s, l])
            rel, mx = compare(gpu, oracle.moe_layer(wq, acts), label="step %d layer %d" % (s, l))
            worst[0], worst[1] = max(worst[0], rel), max(worst[1], mx)

        drv.run(on_layer=check)
        torch.cuda.synchronize()
        for ev in drv.events:
            say("event before step %d: %s %d blocks, resident %.2f GB" % (ev[0], "lower" if ev[1] else "raise",
                                                                          ev[2], ev[3] / 1e9))
        assert len(drv.events) == 7
        assert all(ev[2] == 576 for ev in drv.events)
        # lowering frees device memory, raising takes it back
        res = [ev[3] for ev in drv.events]
        assert res[0] < res[1] and res[2] < res[1]
        # the host view of the committed widths matches the planner's copy
        for l in CHECK_LAYERS:
            for e in range(shape.E):
                for m in (0, 1):
                    assert ctx.committed_bits(ctx.block_id(l, e, m)) == drv.q[l, e, m]
        say("worst rel_l2 %.3e max_abs %.3e over %d checks" % (worst[0], worst[1],
                                                              len(CHECK_LAYERS) * len(CHECK_STEPS)))
    finally:
        ctx.close()


def test_budget_planner_stack():
    """Three Zipf-routed layers (H=256, I=256, 16 experts, top-2, batch 8),
    16 steps, an event every 4 steps with a routed-byte target (the bytes of
    every block at 4, then 7, then 5 bits): the device routing mass feeds pw_plan_widths and
    the event commits its widths.  Checks: committed widths and resident
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
                          plan_params=params)
        mass_host = np.zeros((L, shape.E))
        worst = [0.0]

        def check(s, l):
            drv.compute.synchronize()
            k = shape.top_k
            gpu = dict(idx=drv.idx[s, l].cpu().numpy(), w=drv.w[s, l].cpu().numpy(),
                       offsets=drv.offsets[l].cpu().numpy(), sorted=drv.sorted[l].cpu().numpy()[:T * k],
                       y=drv.y[l].cpu().numpy().astype(np.float64))
            acts = pw_synth.Activations(x=x[s, l], logits=logits[s, l])
            rel, _ = compare(gpu, oracle.moe_layer(_with_q(ws[l], drv.q[l]), acts), label="step %d layer %d" % (s, l))
            worst[0] = max(worst[0], rel)

        drv.run(on_layer=check)
        torch.cuda.synchronize()
        assert len(drv.plans) == 3
        for (s, target, total, q), ev in zip(drv.plans, drv.events):
            say("event before step %d: target %.2f MB, planned %.2f MB, resident %.2f MB, %d blocks changed"
                % (s, target / 1e6, total / 1e6, ev[3] / 1e6, ev[2]))
            assert total <= target and ev[3] == total
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
