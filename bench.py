"""Benchmark of the fused mixed-precision MoE expert path on one MI355X.

Workload: one Qwen1.5-MoE-A2.7B-shaped MoE layer in decode (H=2048, 60 routed
experts with I=1408, top-4, one shared expert with I=5632 at 8 bits, 4 tokens
per batch), Zipf(1.1)-biased routing, routed blocks at mixed widths 3..8 tiered
by routing rank.  All inputs are seeded synthetic arrays (pw_synth).

A step is one pass of the whole hot path over one batch: top-k routing ->
permutation by expert -> gate_up (bit-plane gather, LUT decode, SiLU*mul) ->
down -> gate-weighted combine.  Steps rotate over `--layers` distinct copies
of the layer's weights so the working set exceeds the 256 MB MALL; the timed
region replays a HIP graph of those steps (no host launch overhead), with the
inputs already resident in HBM.

Prints ONE JSON line.  `roofline` is for the dominant kernel (gate_up):
algorithmic bytes per launch / its mean duration from HIP events recorded
around every launch on the launch stream.  `cpu_baseline` times the fp64 CPU
oracle on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
CFG = 1


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def block_bytes(R, K, q):
    """Algorithmic bytes of one block at width q: its q planes + LUT_q."""
    return R * K * q // 8 + R * (1 << q) * 2


def step_bytes(shape, wq, offsets, T):
    """Algorithmic bytes of one layer step, split by kernel."""
    H, I, Is, k, E = shape.H, shape.I, shape.I_shared, shape.top_k, shape.E
    active = [e for e in range(E) if offsets[e + 1] > offsets[e]]
    gu = sum(block_bytes(2 * I, H, int(wq[e, 0])) for e in active)
    dn = sum(block_bytes(H, I, int(wq[e, 1])) for e in active)
    if Is:
        gu += block_bytes(2 * Is, H, 8)
        dn += block_bytes(H, Is, 8)
    rows_h = T * k * I + (T * Is if Is else 0)
    rows_d = (T * k + (T if Is else 0)) * H
    gate_up = gu + T * H * 2 + rows_h * 4          # planes+LUT, x in, h (hi+lo fp16) out
    down = dn + rows_h * 4 + rows_d * 4            # planes+LUT, h in, per-assignment d out
    path = gu + dn + T * H * 2 + T * H * 2 + T * E * 4  # weights + x + y + logits
    return dict(gate_up=gate_up, down=down, path=path, weights=gu + dn, active=len(active))


def cpu_baseline(weights, acts_list, budget_s):
    import oracle
    P = oracle.PreparedLayer(weights)
    n_tok, secs, batches = 0, 0.0, 0
    while secs < budget_s and batches < len(acts_list) * 50:
        a = acts_list[batches % len(acts_list)]
        dt, _ = oracle.timed_layer(P, a)
        secs += dt
        n_tok += a.x.shape[0]
        batches += 1
    return dict(value=n_tok / secs, unit="tokens/s", cores=oracle.num_threads(), kind="oracle",
                sample="%d batches of %d tokens of the same Qwen-shaped layer (route, permute, "
                       "all routed experts + shared expert, combine) in fp64; %.1f s"
                       % (batches, acts_list[0].x.shape[0], secs))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=800)
    ap.add_argument("--warmup", type=int, default=80)
    ap.add_argument("--layers", type=int, default=8, help="distinct weight copies rotated per step")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-graph", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this path has no multi-GPU mode (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import any_precision_expert_amd as pw
    import pw_synth
    from any_precision_expert_amd.layer import Batch

    assert torch.cuda.is_available(), "bench needs a GPU"
    spec = pw_synth.CONFIGS[CFG]
    shape, T = spec.shape, spec.tokens[0]
    seed = pw_synth.config_seed(CFG)
    L = args.layers
    t0 = time.time()
    w = pw_synth.make_weights(shape, seed, 0, spec.q_policy, spec.logits)
    wq = np.array([[g.q, d.q] for g, d in zip(w.gate_up, w.down)])
    acts = [pw_synth.make_activations(shape, T, seed, 0, s, spec.logits, w.rank) for s in range(L)]
    log("generated weights in %.1fs" % (time.time() - t0))

    ctx = pw.Context(0, L, shape.E, shape.H, shape.I, shape.top_k, shape.I_shared,
                     keep_host_masters=False)
    t0 = time.time()
    blocks = [(e, pw.MODULE_GATE_UP, w.gate_up[e]) for e in range(shape.E)] + \
             [(e, pw.MODULE_DOWN, w.down[e]) for e in range(shape.E)] + \
             [(pw.EXPERT_SHARED, pw.MODULE_GATE_UP, w.shared_gate_up),
              (pw.EXPERT_SHARED, pw.MODULE_DOWN, w.shared_down)]
    for e, m, b in blocks:
        planes, luts = pw.pack_bitplanes(b.code8), pw.concat_luts(b.luts)
        q = b.q if e != pw.EXPERT_SHARED else 8
        for l in range(L):
            ctx.register_block(l, e, m, planes, luts, q)
    log("registered %d layer copies in %.1fs, resident %.2f GB"
        % (L, time.time() - t0, ctx.resident_bytes() / 1e9))

    batches = []
    for l in range(L):
        b = Batch(ctx, T)
        b.load(acts[l].logits, acts[l].x)
        batches.append(b)
    stream = torch.cuda.Stream()

    def run_steps(n, first=0):
        for i in range(first, first + n):
            batches[i % L].step(i % L, stream)

    with torch.cuda.stream(stream):
        run_steps(L)
    torch.cuda.synchronize()
    offsets = [b.offsets.cpu().numpy() for b in batches]
    sb = [step_bytes(shape, wq, o, T) for o in offsets]

    # graph of L consecutive steps (one per layer copy)
    graph = None
    if not args.no_graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            run_steps(L)
        torch.cuda.synchronize()

    def timed(n_steps):
        reps = max(1, n_steps // L)
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        ev0.record(stream)
        w0 = time.perf_counter()
        for _ in range(reps):
            if graph is not None:
                graph.replay()
            else:
                run_steps(L)
        ev1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
        return reps * L, ev0.elapsed_time(ev1) / 1e3, wall

    with torch.cuda.stream(stream):
        timed(args.warmup)
        n, gpu_s, wall_s = timed(args.steps)
    ms_per_step = gpu_s / n * 1e3
    tok_s = T * n / gpu_s
    mean_b = {k: float(np.mean([s[k] for s in sb])) for k in sb[0]}
    log("timed %d steps: %.4f ms/step (wall %.4f ms/step), %.0f tokens/s/layer, path %.1f GB/s"
        % (n, ms_per_step, wall_s / n * 1e3, tok_s, mean_b["path"] / (ms_per_step * 1e-3) / 1e9))

    # per-kernel durations: HIP events around every launch, on the launch stream
    ctx.profile_enable(True)
    with torch.cuda.stream(stream):
        run_steps(min(args.steps, 1600))
    torch.cuda.synchronize()
    kern = {}
    for name in ("route", "permute", "gate_up", "down", "combine"):
        ms, cnt = ctx.profile_read(name)
        kern[name] = dict(mean_us=ms / max(cnt, 1) * 1e3, launches=cnt)
    ctx.profile_enable(False)
    for name, d in kern.items():
        log("  %-8s %8.2f us  x%d" % (name, d["mean_us"], d["launches"]))
    gu_us = kern["gate_up"]["mean_us"]
    dn_us = kern["down"]["mean_us"]
    gu_gbps = mean_b["gate_up"] / (gu_us * 1e-6) / 1e9
    dn_gbps = mean_b["down"] / (dn_us * 1e-6) / 1e9
    log("  gate_up %.1f GB/s, down %.1f GB/s (algorithmic)" % (gu_gbps, dn_gbps))

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(w, acts, args.cpu_seconds)
        log("cpu oracle: %.1f tokens/s on %d threads" % (cpu["value"], cpu["cores"]))

    out = {
        "metric": "routed tokens/s per MoE layer at mixed 3-8 bit + achieved HBM GB/s vs peak",
        "value": round(tok_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": n,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16xf16->f32 (LUT-decoded 3-8 bit codes)",
        "data": "synthetic",
        "config": {"workload": spec.name, "H": shape.H, "I": shape.I, "E": shape.E, "top_k": shape.top_k,
                   "I_shared": shape.I_shared, "tokens_per_batch": T, "layer_copies": L,
                   "q": "routed blocks tiered by Zipf rank (8 / 5-6 / 3-4), shared at 8",
                   "graph": graph is not None},
        "path_gbps": round(mean_b["path"] / (ms_per_step * 1e-3) / 1e9, 1),
        "path_bytes_per_step": int(mean_b["path"]),
        "active_experts_per_step": mean_b["active"],
        "kernels_us": {k: round(v["mean_us"], 3) for k, v in kern.items()},
        "roofline": {"bound": "hbm", "kernel": "gate_up", "achieved": round(gu_gbps, 1),
                     "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(gu_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": None, "bytes_per_launch": int(mean_b["gate_up"]),
                     "down_achieved": round(dn_gbps, 1)},
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    ctx.close()


if __name__ == "__main__":
    main()
