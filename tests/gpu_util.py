"""Helpers for the GPU parity tests: run one layer through the C ABI and
compare with the fp64 oracle."""
from __future__ import annotations

import sys

import numpy as np

import any_precision_expert_amd as pw
import oracle
from any_precision_expert_amd.layer import Batch, register_layer

RTOL_L2 = 1e-3   # relative L2 error bound on y
ATOL_MAX = 1e-2  # max abs error bound on y
W_ATOL = 1e-6    # gate weights (fp32 softmax vs fp64), diagnostic


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def make_ctx(shape, layers=1, keep_host_masters=True):
    return pw.Context(0, layers, shape.E, shape.H, shape.I, shape.top_k, shape.I_shared, keep_host_masters)


def run_gpu(ctx, layer, acts, separate=False):
    """One layer step; outputs are pre-filled with a poison value so that a
    result the path fails to write shows up."""
    import torch
    T = acts.x.shape[0]
    b = Batch(ctx, T)
    b.load(acts.logits, acts.x)
    for t in (b.idx, b.offsets, b.sorted):
        t.fill_(-7)
    b.w.fill_(-7.0)
    b.y.fill_(-7.0)
    b.step(layer, separate=separate)
    torch.cuda.synchronize()
    return dict(idx=b.idx.cpu().numpy(), w=b.w.cpu().numpy(), offsets=b.offsets.cpu().numpy(),
                sorted=b.sorted.cpu().numpy()[:T * ctx.desc.top_k],
                y=b.y.cpu().numpy().astype(np.float64))


def y_errors(y, ref):
    rel = float(np.linalg.norm(y - ref) / max(np.linalg.norm(ref), 1e-300))
    mx = float(np.max(np.abs(y - ref))) if y.size else 0.0
    return rel, mx


def compare(gpu, ref, tokens=None, label=""):
    assert np.array_equal(gpu["idx"], ref["idx"]), label + " routing indices differ"
    assert np.array_equal(gpu["offsets"], ref["offsets"]), label + " expert offsets differ"
    assert np.array_equal(gpu["sorted"], ref["sorted"]), label + " permutation differs"
    assert np.max(np.abs(gpu["w"] - ref["w"])) <= W_ATOL, label + " gate weights differ"
    y = gpu["y"] if tokens is None else gpu["y"][np.asarray(tokens)]
    rel, mx = y_errors(y, ref["y"])
    say("%s rel_l2=%.3e max_abs=%.3e" % (label, rel, mx))
    assert rel <= RTOL_L2 and mx <= ATOL_MAX, "%s y: rel_l2 %.3e max_abs %.3e" % (label, rel, mx)
    return rel, mx


def check_layer(weights, acts, tokens=None, label="", ctx=None, layer=0):
    own = ctx is None
    if own:
        ctx = make_ctx(weights.shape)
        register_layer(ctx, 0, weights)
    try:
        gpu = run_gpu(ctx, layer, acts)
    finally:
        if own:
            ctx.close()
    ref = oracle.moe_layer(weights, acts, tokens=tokens)
    return compare(gpu, ref, tokens, label)
