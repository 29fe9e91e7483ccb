"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Bit-exact: routing indices, expert offsets, the permutation, decoded child
codes and dequantised fp16 weights.  Within tolerance: y (relative L2 <= 1e-3,
max abs <= 1e-2) and the fp32 gate weights (<= 1e-6 from fp64).
"""
import numpy as np
import pytest

import pw_synth
from tests.gpu_util import check_layer, compare, make_ctx, run_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu(require_gpu):
    import any_precision_expert_amd as pw
    pw.lib()  # loud failure if the library is missing


# ------------------------------------------------------------------ decode

# Every decode path an FFN kernel runs, pinned bit for bit: the codes and the
# fp16 weights produced by the FFN's own decode routines (pw_debug_decode) must
# equal the oracle's code8 >> (8 - q) and LUT_q[row][code] ("Technical summary:
# PagedWeight", Core components 1).  Paths: the decode contraction's 128-row
# tiles (gate_up whole tiles; q = 3 two-set pair tables, q = 4 single tables,
# q >= 5 bit transpose) and 64-row tiles (gate_up half tiles, down; q <= 4 pair
# tables), 64-row tiles of 16- and 32-token passes (single tables at q = 4), and the
# prefill decoder (per-lane rotate form).  Shapes: ragged row
# tiles, ragged K (a last chunk of 1 or 3 words) and several chunks per K-wave.
DECODE_SHAPES = {"ragged": (352, 224), "multi_chunk": (1056, 608)}


@pytest.mark.parametrize("shape", sorted(DECODE_SHAPES))
@pytest.mark.parametrize("q", [3, 4, 5, 6, 7, 8])
def test_ffn_decode_paths_bit_exact(q, shape):
    import torch
    import any_precision_expert_amd as pw
    import oracle
    H, I = DECODE_SHAPES[shape]
    w, _ = pw_synth.make_small(H=H, I=I, E=2, top_k=1, T=1, seed=100 + q + 10 * H, q_fixed=q)
    ctx = make_ctx(w.shape)
    paths = {"tile128": pw.DECODE_PATH_TILE128, "tile64": pw.DECODE_PATH_TILE64,
             "prefill": pw.DECODE_PATH_PREFILL, "tile64_wide": pw.DECODE_PATH_TILE64_WIDE}
    try:
        for e in range(2):
            for m, blk in ((pw.MODULE_GATE_UP, w.gate_up[e]), (pw.MODULE_DOWN, w.down[e])):
                ctx.register_code_block(0, e, m, blk.code8, blk.luts, blk.q)
                bid = ctx.block_id(0, e, m)
                want_codes = oracle.decode_codes(blk.code8, q)
                want_w = oracle.decode_block(blk)
                for name, path in paths.items():
                    say("decode q=%d %s expert %d module %d path %s" % (q, shape, e, m, name))
                    codes = torch.full(blk.code8.shape, 255, dtype=torch.uint8, device="cuda")
                    wts = torch.full(blk.code8.shape, -7.0, dtype=torch.float16, device="cuda")
                    ctx.debug_decode(bid, path, codes, wts)
                    torch.cuda.synchronize()
                    got_c = codes.cpu().numpy()
                    got_w = wts.cpu().numpy().astype(np.float64)
                    bad = np.argwhere(got_c != want_codes)
                    assert bad.size == 0, "%s: %d codes differ, first at %s" % (name, len(bad), bad[0])
                    bad = np.argwhere(got_w != want_w)
                    assert bad.size == 0, "%s: %d weights differ, first at %s" % (name, len(bad), bad[0])
                # the two single-output exports run the decode contraction's tile
                out = torch.zeros(blk.code8.shape, dtype=torch.uint8, device="cuda")
                ctx.debug_decode_codes(bid, out)
                wout = torch.zeros(blk.code8.shape, dtype=torch.float16, device="cuda")
                ctx.debug_dequant(bid, wout)
                torch.cuda.synchronize()
                assert np.array_equal(out.cpu().numpy(), want_codes)
                assert np.array_equal(wout.cpu().numpy().astype(np.float64), want_w)
    finally:
        ctx.close()


# ------------------------------------------------------------------ routing

# Expert counts around the 64-lane groups of the wave-per-token top-k (E = 33,
# 63, 64), the one-token-per-lane top-k up to 32 experts (E = 1..32, k up to
# 8) and exact ties on every fourth token.
@pytest.mark.parametrize("T,E,k", [(1, 4, 2), (16, 4, 2), (37, 60, 4), (300, 8, 2), (4096, 8, 2),
                                   (64, 256, 8), (5, 7, 7), (1000, 1, 1), (9, 16, 3), (23, 17, 5),
                                   (50, 33, 2), (40, 63, 6), (31, 64, 8), (70, 32, 4), (200, 12, 8)])
def test_route_and_permute_bit_exact(T, E, k):
    import torch
    import oracle
    rng = np.random.default_rng(T * 31 + E)
    logits = rng.normal(size=(T, E)).astype(np.float32)
    logits[::4] = np.round(logits[::4] * 2) / 2  # exact ties
    H, I = 64, 32
    ctx = make_ctx(pw_synth.LayerShape(H=H, I=I, E=E, top_k=k))
    try:
        lg = torch.from_numpy(logits).cuda()
        idx = torch.zeros((T, k), dtype=torch.int32, device="cuda")
        wt = torch.zeros((T, k), dtype=torch.float32, device="cuda")
        offs = torch.zeros((E + 1,), dtype=torch.int32, device="cuda")
        srt = torch.zeros((T * k,), dtype=torch.int32, device="cuda")
        ridx, rw = oracle.route_topk(logits, k)
        roff, rsrt = oracle.permute(ridx, E)
        # the two calls, then the fused call (one workgroup for T * k <= 4096)
        for fused in (False, True):
            for b in (idx, wt, offs, srt):
                b.fill_(-7)
            if fused:
                ctx.route_permute(lg, T, idx, wt, offs, srt)
            else:
                ctx.route_topk(lg, T, idx, wt)
                ctx.permute_by_expert(idx, T, offs, srt)
            torch.cuda.synchronize()
            assert np.array_equal(idx.cpu().numpy(), ridx), "fused=%s" % fused
            assert np.max(np.abs(wt.cpu().numpy() - rw)) <= 1e-6, "fused=%s" % fused
            assert np.array_equal(offs.cpu().numpy(), roff), "fused=%s" % fused
            assert np.array_equal(srt.cpu().numpy(), rsrt), "fused=%s" % fused
    finally:
        ctx.close()


# ------------------------------------------------------------------ FFN, small shapes

@pytest.mark.parametrize("q", [3, 4, 5, 6, 7, 8])
def test_ffn_each_width(q):
    w, a = pw_synth.make_small(H=352, I=224, E=6, top_k=3, T=7, I_shared=96, seed=200 + q, q_fixed=q)
    check_layer(w, a, label="q=%d" % q)


@pytest.mark.parametrize("T", [1, 2, 5, 9, 33, 45])  # 45: ~18 tokens per expert, three passes, kept plane loads
def test_ffn_mixed_widths_ragged(T):
    w, a = pw_synth.make_small(H=352, I=224, E=5, top_k=2, T=T, seed=300 + T)
    check_layer(w, a, label="mixed T=%d" % T)


# Each tokens-per-pass width of the decode contraction against the oracle, and
# the multi-pass cases (units holding more tokens than a pass, plane loads kept
# in the cache): 8 (128-row gate_up tiles, routing in the gate_up launch), 16
# and 32 (64-row tiles; 32: two waves share one activation slice).
@pytest.mark.parametrize("T,Is,width", [(9, 0, 8), (20, 0, 16), (33, 0, 32), (100, 0, 32),
                                        (12, 96, 16), (40, 96, 32), (70, 96, 32)])
def test_ffn_each_pass_width(T, Is, width):
    import any_precision_expert_amd as pw
    assert pw.decode_tokens_per_pass(T, 2, 5, Is) == width
    w, a = pw_synth.make_small(H=352, I=224, E=5, top_k=2, T=T, I_shared=Is, seed=700 + T)
    check_layer(w, a, label="T=%d Is=%d pass=%d" % (T, Is, width))
    ctx = make_ctx(w.shape)
    try:
        from any_precision_expert_amd.layer import register_layer
        register_layer(ctx, 0, w)
        g1 = run_gpu(ctx, 0, a)
        g2 = run_gpu(ctx, 0, a, separate=True)
        assert np.array_equal(g1["y"], g2["y"]), "layer call and separate calls differ"
    finally:
        ctx.close()


# Forced pass widths (pw_set_tokens_per_pass) on one layer: 8- and 32-token
# passes run the same K split on the same tiles, so y is bit-identical; every
# width stays within tolerance of the oracle.
@pytest.mark.parametrize("T,Is", [(40, 0), (70, 0), (20, 96), (45, 96)])
def test_forced_pass_widths(T, Is):
    import oracle
    from any_precision_expert_amd.layer import register_layer
    w, a = pw_synth.make_small(H=352, I=224, E=8, top_k=2, T=T, I_shared=Is, seed=800 + T + Is)
    ref = oracle.moe_layer(w, a)
    ctx = make_ctx(w.shape)
    try:
        register_layer(ctx, 0, w)
        import any_precision_expert_amd as pw
        assert pw.lib().pw_set_tokens_per_pass(ctx.h, 12) == pw.PW_ERR_INVALID
        ys = {}
        for tp in (8, 16, 32, 0):
            ctx.set_tokens_per_pass(tp)
            g = run_gpu(ctx, 0, a)
            compare(g, ref, label="T=%d Is=%d forced %d" % (T, Is, tp))
            ys[tp] = g["y"]
        assert np.array_equal(ys[8], ys[32]), "8- and 32-token passes differ"
    finally:
        ctx.close()


def test_ffn_single_expert_all_tokens():
    w, a = pw_synth.make_small(H=256, I=128, E=1, top_k=1, T=11, seed=401)
    check_layer(w, a, label="E=1")


def test_ffn_all_tokens_to_one_expert():
    w, a = pw_synth.make_small(H=256, I=128, E=8, top_k=2, T=13, seed=402)
    a.logits[:, 3] += 100.0
    check_layer(w, a, label="hot expert")


def test_ffn_k_equals_E_and_large_tiles():
    w, a = pw_synth.make_small(H=1024, I=512, E=4, top_k=4, T=6, I_shared=256, seed=403)
    check_layer(w, a, label="k=E")


# ------------------------------------------------------------------ prefill GEMM path (T >= 256)

@pytest.mark.parametrize("q", [3, 4, 5, 6, 7, 8])
def test_prefill_each_width(q):
    """128-row x 512-token MFMA tiles over weights decoded into LDS; ragged
    rows (I = 352 is not a multiple of 64), ragged K and partial token tiles."""
    w, a = pw_synth.make_small(H=416, I=352, E=4, top_k=2, T=300, I_shared=160, seed=700 + q, q_fixed=q)
    check_layer(w, a, label="prefill q=%d" % q)


def test_prefill_mixed_widths_hot_expert():
    """Mixed widths and one expert with every token: 600 tokens -> one token
    tile for that expert and a tail of 88 on the decode kernels, empty
    experts skipped."""
    w, a = pw_synth.make_small(H=256, I=192, E=6, top_k=2, T=600, seed=710)
    a.logits[:, 4] += 100.0
    check_layer(w, a, label="prefill hot expert")


def test_prefill_ragged_token_tiles():
    """Token counts per expert just past a 512-token tile and at the 64-token
    boundary of a wave's range: tails of 1, 64 and 65 tokens past the last
    whole tile (fewer than 96: taken by the decode kernels on the tails), an
    expert with none, and a shared expert whose third tile holds 130 tokens."""
    counts = [513, 576, 65, 0]
    T = sum(counts)
    w, a = pw_synth.make_small(H=256, I=192, E=4, top_k=1, T=T, I_shared=96, seed=720)
    target = np.repeat(np.arange(4), counts)
    np.random.default_rng(720).shuffle(target)
    a.logits[np.arange(T), target] += 100.0
    check_layer(w, a, label="prefill ragged tiles")


def test_prefill_ragged_gemm_tiles():
    """Tails of 96 tokens or more stay GEMM tiles: last tiles holding 97, 129
    (two whole 64-token wave ranges and one token) and 511 tokens, whose waves
    past the last token skip their matrix work, beside an expert with a tail
    of 95 on the decode kernels."""
    counts = [512 + 97, 129, 511, 95]
    T = sum(counts)
    w, a = pw_synth.make_small(H=256, I=192, E=4, top_k=1, T=T, seed=721)
    target = np.repeat(np.arange(4), counts)
    np.random.default_rng(721).shuffle(target)
    a.logits[np.arange(T), target] += 100.0
    check_layer(w, a, label="prefill ragged GEMM tiles")


def test_prefill_tails_many_experts():
    """A 300-token batch over 70 experts (top-2: a few tokens each, so every
    expert's tokens are a tail taken by the decode kernels, whose slot search
    then spans two groups of 64 experts) beside a shared expert on its GEMM
    tiles."""
    w, a = pw_synth.make_small(H=256, I=128, E=70, top_k=2, T=300, I_shared=64, seed=730)
    check_layer(w, a, label="prefill tails, 70 experts")


def test_zero_tokens_enqueues_nothing():
    import torch
    w, a = pw_synth.make_small(H=64, I=32, E=2, top_k=1, T=1, seed=404)
    from any_precision_expert_amd.layer import register_layer
    ctx = make_ctx(w.shape)
    try:
        register_layer(ctx, 0, w)
        assert ctx.workspace_size(0) == 0
        y = torch.full((1, 64), 7.0, dtype=torch.float16, device="cuda")
        ctx.route_topk(0, 0, 0, 0)
        ctx.moe_ffn_bitplane(0, 0, 0, 0, 0, 0, 0, y, 0, 0)
        torch.cuda.synchronize()
        assert torch.all(y == 7.0)
    finally:
        ctx.close()


# ------------------------------------------------------------------ the workload configurations

def test_config0_toy():
    w, a = pw_synth.make_config(0)
    check_layer(w, a, label="cfg0")


def test_config1_qwen_decode():
    w, a = pw_synth.make_config(1)
    check_layer(w, a, label="cfg1")


@pytest.fixture(scope="module")
def mixtral():
    import any_precision_expert_amd as pw
    from any_precision_expert_amd.layer import register_layer
    spec = pw_synth.CONFIGS[2]
    w = pw_synth.make_weights(spec.shape, pw_synth.config_seed(2), 0, spec.q_policy, spec.logits)
    ctx = make_ctx(w.shape)
    register_layer(ctx, 0, w)
    yield w, ctx
    ctx.close()


@pytest.mark.parametrize("T", [1, 4, 16, 64])
def test_config2_mixtral_decode(mixtral, T):
    w, ctx = mixtral
    spec = pw_synth.CONFIGS[2]
    a = pw_synth.make_activations(spec.shape, T, pw_synth.config_seed(2), 0, 0, spec.logits)
    check_layer(w, a, label="cfg2 T=%d" % T, ctx=ctx)  # every token of the batch


def stratified_tokens(idx, offsets, sorted_assign, k, seed, tile=512, wave_range=64):
    """Tokens that cover every cell of the prefill GEMM: for each expert, one
    random assignment in each (512-token tile, 64-token wave range) of its
    sorted assignment list, plus the expert's first and last assignment; the
    token of each chosen assignment."""
    rng = np.random.default_rng(seed)
    picks = set()
    for e in range(len(offsets) - 1):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if hi <= lo:
            continue
        picks.update((lo, hi - 1))
        for start in range(lo, hi, wave_range):
            end = min(hi, start + wave_range)
            picks.add(int(rng.integers(start, end)))
    return sorted({int(sorted_assign[p]) // k for p in picks})


def test_config3_mixtral_prefill_stratified():
    """Every (expert, 512-token tile, 64-token wave range) cell of the
    Mixtral-shaped prefill layer (4096 tokens) holds a compared token, and so do
    each expert's first and last assignments (the ragged last tiles)."""
    import oracle
    w, a = pw_synth.make_config(3)
    idx, _ = oracle.route_topk(a.logits, w.shape.top_k)
    offsets, srt = oracle.permute(idx, w.shape.E)
    tokens = stratified_tokens(idx, offsets, srt, w.shape.top_k, seed=3)
    say("cfg3: %d stratified tokens" % len(tokens))
    check_layer(w, a, tokens=tokens, label="cfg3 prefill")


# ------------------------------------------------------------------ a user-supplied model config

@pytest.fixture(scope="module")
def user_config():
    """A MoE shape read from a model-config file (nested text_config, two
    shared experts, H = 1120 = 8.75 chunks, 24 experts top-6)."""
    import os
    from any_precision_expert_amd.layer import register_layer
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "configs", "example_moe_config.json")
    spec = pw_synth.model_config_spec(path)
    w = pw_synth.make_weights(spec.shape, pw_synth.USER_CONFIG_SEED, 0, spec.q_policy, spec.logits)
    ctx = make_ctx(w.shape)
    register_layer(ctx, 0, w)
    yield spec, w, ctx
    ctx.close()


@pytest.mark.parametrize("T", [1, 4, 16, 300])
def test_user_model_config_layer(user_config, T):
    spec, w, ctx = user_config
    a = pw_synth.make_activations(spec.shape, T, pw_synth.USER_CONFIG_SEED, 0, T, spec.logits, w.rank)
    tokens = None if T <= 16 else sorted({0, T - 1} | set(range(1, T, 37)))
    check_layer(w, a, tokens=tokens, label="%s T=%d" % (spec.name, T), ctx=ctx)


# ------------------------------------------------------------------ one call per layer

@pytest.fixture(scope="module")
def qwen():
    from any_precision_expert_amd.layer import register_layer
    spec = pw_synth.CONFIGS[1]
    w = pw_synth.make_weights(spec.shape, pw_synth.config_seed(1), 0, spec.q_policy, spec.logits)
    ctx = make_ctx(w.shape)
    register_layer(ctx, 0, w)
    yield w, ctx
    ctx.close()


@pytest.mark.parametrize("T", [1, 4, 16, 17])
def test_layer_call_equals_separate_calls_qwen(qwen, T):
    """pw_moe_layer (routing inside the gate_up launch up to T*k = 64, the
    separate launches above) gives bit for bit the outputs of pw_route_permute
    + pw_moe_ffn_bitplane, and both match the oracle."""
    from tests.gpu_util import run_gpu
    import oracle
    w, ctx = qwen
    spec = pw_synth.CONFIGS[1]
    a = pw_synth.make_activations(spec.shape, T, pw_synth.config_seed(1), 0, 3, spec.logits, w.rank)
    sep = run_gpu(ctx, 0, a, separate=True)
    one = run_gpu(ctx, 0, a)
    for key in ("idx", "w", "offsets", "sorted", "y"):
        assert np.array_equal(one[key], sep[key]), "T=%d: %s differs from the separate calls" % (T, key)
    compare(one, oracle.moe_layer(w, a), label="layer call T=%d" % T)


@pytest.mark.parametrize("T", [4, 16])
def test_decode_calls_repeatable(qwen, T):
    """Two batches run alternately 40 times each (every fourth call with the
    separate routing launches), y poisoned before every call: every y equals
    the first bit for bit, and the first matches the oracle."""
    import torch
    import oracle
    from any_precision_expert_amd.layer import Batch
    w, ctx = qwen
    spec = pw_synth.CONFIGS[1]
    acts = [pw_synth.make_activations(spec.shape, T, pw_synth.config_seed(1), 0, 20 + i, spec.logits, w.rank)
            for i in range(2)]
    batches = []
    for a in acts:
        b = Batch(ctx, T)
        b.load(a.logits, a.x)
        batches.append(b)
    outs = [[], []]
    for rep in range(40):
        for i, b in enumerate(batches):
            b.y.fill_(-7.0)
            b.step(0, separate=(rep % 4 == 3))
            outs[i].append(b.y.clone())
    torch.cuda.synchronize()
    for i in range(2):
        first = outs[i][0].cpu().numpy()
        for rep, y in enumerate(outs[i][1:], 1):
            assert np.array_equal(y.cpu().numpy().view(np.uint16), first.view(np.uint16)), \
                "batch %d, call %d: y differs from the first call" % (i, rep)
        b = batches[i]
        gpu = dict(idx=b.idx.cpu().numpy(), w=b.w.cpu().numpy(), offsets=b.offsets.cpu().numpy(),
                   sorted=b.sorted.cpu().numpy()[:T * ctx.desc.top_k], y=first.astype(np.float64))
        compare(gpu, oracle.moe_layer(w, acts[i]), label="repeated T=%d batch %d" % (T, i))


@pytest.mark.parametrize("T", [4, 16])
def test_graph_replays_repeatable(qwen, T):
    """pw_moe_layer captured in a HIP graph (two batches sharing one
    workspace) and replayed six times, with eager calls on the same workspace
    (in-launch and separate routing) between the replays: every replay's y
    equals the eager result bit for bit."""
    import torch
    from any_precision_expert_amd.layer import Batch
    w, ctx = qwen
    spec = pw_synth.CONFIGS[1]
    acts = [pw_synth.make_activations(spec.shape, T, pw_synth.config_seed(1), 0, 40 + i, spec.logits, w.rank)
            for i in range(2)]
    batches = []
    for a in acts:
        b = Batch(ctx, T)
        b.load(a.logits, a.x)
        batches.append(b)
    batches[1].ws = batches[0].ws  # one workspace for both
    stream = torch.cuda.Stream()
    with torch.cuda.stream(stream):
        for b in batches:
            b.step(0, stream)
    torch.cuda.synchronize()
    want = [b.y.clone() for b in batches]
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for b in batches:
            b.step(0, stream)
    torch.cuda.synchronize()
    for rep in range(6):
        for b in batches:
            b.y.fill_(-7.0)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            graph.replay()
        torch.cuda.synchronize()
        for i, b in enumerate(batches):
            assert torch.equal(b.y.view(torch.int16), want[i].view(torch.int16)), "replay %d batch %d" % (rep, i)
        with torch.cuda.stream(stream):
            batches[rep % 2].step(0, stream, separate=(rep % 3 == 2))
        torch.cuda.synchronize()
        assert torch.equal(batches[rep % 2].y.view(torch.int16), want[rep % 2].view(torch.int16)), "eager %d" % rep


@pytest.mark.parametrize("T", [16, 300])
def test_layer_call_equals_separate_calls_toy(T):
    from any_precision_expert_amd.layer import register_layer
    from tests.gpu_util import run_gpu
    w, a = pw_synth.make_config(0)
    if T != a.x.shape[0]:
        spec = pw_synth.CONFIGS[0]
        a = pw_synth.make_activations(spec.shape, T, pw_synth.config_seed(0), 0, 1, spec.logits)
    ctx = make_ctx(w.shape)
    try:
        register_layer(ctx, 0, w)
        sep = run_gpu(ctx, 0, a, separate=True)
        one = run_gpu(ctx, 0, a)
    finally:
        ctx.close()
    for key in ("idx", "w", "offsets", "sorted", "y"):
        assert np.array_equal(one[key], sep[key]), "T=%d: %s differs from the separate calls" % (T, key)


# ------------------------------------------------------------------ routing mass (Core components 2)

def test_routing_mass_accumulates_like_the_oracle():
    """Mass over pw_moe_layer calls on two layers (in-launch routing at T = 16,
    the separate launches at T = 5 with a prefill-sized T = 300) against the
    oracle's fp64 routing; rerunning the same calls gives the same bits; reset
    zeroes it.  Also pins the byte model the planner uses against the
    library's own resident-byte count."""
    import oracle
    import oracle.plan as op
    from any_precision_expert_amd.layer import Batch, register_layer
    import torch
    spec = pw_synth.CONFIGS[0]
    shape, seed = spec.shape, pw_synth.config_seed(0)
    w = pw_synth.make_weights(shape, seed, 0, spec.q_policy, spec.logits)
    ctx = make_ctx(shape, layers=2)
    try:
        for l in range(2):
            register_layer(ctx, l, w)
        want_bytes = 2 * sum(op.block_bytes(*op.block_shape(m, shape.H, shape.I), int(b.q))
                             for m, blocks in ((0, w.gate_up), (1, w.down)) for b in blocks)
        assert ctx.resident_bytes() == want_bytes
        calls = [(0, 16), (1, 16), (0, 300), (1, 5), (0, 16)]
        runs = []
        for rep in range(2):
            ctx.routing_mass_enable(True)
            ctx.routing_mass_reset()
            expected = [[0.0] * shape.E for _ in range(2)]
            for step, (layer, T) in enumerate(calls):
                a = pw_synth.make_activations(shape, T, seed, layer, step, spec.logits)
                b = Batch(ctx, T)
                b.load(a.logits, a.x)
                b.step(layer)
                idx, gw = oracle.route_topk(a.logits, shape.top_k)
                op.routing_mass_add(expected[layer], idx.tolist(), gw.tolist())
            torch.cuda.synchronize()
            got = ctx.routing_mass()
            say("routing mass max |gpu - oracle| = %.3e" % np.max(np.abs(got - np.array(expected))))
            assert np.max(np.abs(got - np.array(expected))) <= 1e-6 * sum(T for _, T in calls)
            runs.append(got)
        assert np.array_equal(runs[0], runs[1])
        ctx.routing_mass_reset()
        ctx.routing_mass_enable(False)
        assert np.all(ctx.routing_mass() == 0.0)
    finally:
        ctx.close()
