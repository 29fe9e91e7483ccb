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
