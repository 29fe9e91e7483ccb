"""GPU tests of committed-width changes (pw_set_committed_bits): lowering
frees planes, raising reloads planes and LUTs from the pinned host masters on
a copy stream, the new widths apply exactly to work enqueued after the call,
and bad requests change nothing.  Outputs are checked against the fp64 oracle
evaluated at the widths committed for that work."""
import copy

import numpy as np
import pytest

import pw_synth
from tests.gpu_util import compare, make_ctx, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu(require_gpu):
    import any_precision_expert_amd as pw
    pw.lib()


def _layer(seed=500, T=6):
    return pw_synth.make_small(H=256, I=160, E=5, top_k=2, T=T, I_shared=64, seed=seed)


def _run(ctx, acts, stream=None):
    import torch
    from any_precision_expert_amd.layer import Batch
    b = Batch(ctx, acts.x.shape[0])
    b.load(acts.logits, acts.x)
    b.step(0, stream)
    return b


def _fetch(b):
    import torch
    torch.cuda.synchronize()
    T = b.T
    return dict(idx=b.idx.cpu().numpy(), w=b.w.cpu().numpy(), offsets=b.offsets.cpu().numpy(),
                sorted=b.sorted.cpu().numpy()[:T * b.ctx.desc.top_k], y=b.y.cpu().numpy().astype(np.float64))


def _with_q(w, qs):
    w2 = copy.copy(w)
    w2.gate_up = [copy.copy(b) for b in w.gate_up]
    w2.down = [copy.copy(b) for b in w.down]
    for e, (qg, qd) in enumerate(qs):
        w2.gate_up[e].q, w2.down[e].q = int(qg), int(qd)
    return w2


def test_lower_then_raise_matches_oracle_and_frees_memory():
    import oracle
    import torch
    import any_precision_expert_amd as pw
    from any_precision_expert_amd.layer import register_layer
    w, a = _layer()
    ctx = make_ctx(w.shape)
    try:
        register_layer(ctx, 0, w)
        q0 = [(b.q, d.q) for b, d in zip(w.gate_up, w.down)]
        res0 = ctx.resident_bytes()
        compare(_fetch(_run(ctx, a)), oracle.moe_layer(w, a), label="initial")
        ids = [ctx.block_id(0, e, m) for e in range(w.shape.E) for m in (0, 1)]
        # lower every routed block to 3
        ctx.set_committed_bits(ids, [3] * len(ids))
        assert all(ctx.committed_bits(i) == 3 for i in ids)
        y3 = _fetch(_run(ctx, a))
        compare(y3, oracle.moe_layer(_with_q(w, [(3, 3)] * w.shape.E), a), label="lowered")
        assert ctx.resident_bytes() < res0
        # debug decode sees the new width
        bid = ctx.block_id(0, 1, pw.MODULE_DOWN)
        out = torch.zeros(w.down[1].code8.shape, dtype=torch.uint8, device="cuda")
        ctx.debug_decode_codes(bid, out)
        torch.cuda.synchronize()
        assert np.array_equal(out.cpu().numpy(), w.down[1].code8 >> 5)
        # raise every routed block to 8 (planes and LUT_8 reloaded from the host masters)
        copy_stream = torch.cuda.Stream()
        ctx.set_committed_bits(ids, [8] * len(ids), torch.cuda.current_stream(), copy_stream)
        y8 = _fetch(_run(ctx, a))
        compare(y8, oracle.moe_layer(_with_q(w, [(8, 8)] * w.shape.E), a), label="raised")
        # back to the initial widths
        ctx.set_committed_bits(ids, [q for e in q0 for q in e])
        compare(_fetch(_run(ctx, a)), oracle.moe_layer(w, a), label="restored")
    finally:
        ctx.close()


def test_new_widths_apply_only_to_later_work():
    """Enqueue a step, change widths, enqueue another step -- no host sync in
    between: the first sees the old widths, the second the new ones."""
    import oracle
    import torch
    from any_precision_expert_amd.layer import Batch, register_layer
    w, a = _layer(seed=501)
    ctx = make_ctx(w.shape)
    try:
        register_layer(ctx, 0, w)
        torch.cuda.synchronize()
        s = torch.cuda.current_stream()
        cs = torch.cuda.Stream()
        b1 = Batch(ctx, a.x.shape[0])
        b2 = Batch(ctx, a.x.shape[0])
        b1.load(a.logits, a.x)
        b2.load(a.logits, a.x)
        torch.cuda.synchronize()
        ids = [ctx.block_id(0, e, m) for e in range(w.shape.E) for m in (0, 1)]
        qa = [5 if i % 2 else 8 for i in range(len(ids))]
        qb = [4 if i % 3 else 7 for i in range(len(ids))]
        ctx.set_committed_bits(ids, qa, s, cs)
        torch.cuda.synchronize()
        for _ in range(3):  # several rounds without a host sync
            b1.step(0, s)
            ctx.set_committed_bits(ids, qb, s, cs)
            b2.step(0, s)
            ctx.set_committed_bits(ids, qa, s, cs)
        r1, r2 = _fetch(b1), _fetch(b2)
        pa = list(zip(qa[0::2], qa[1::2]))
        pb = list(zip(qb[0::2], qb[1::2]))
        compare(r1, oracle.moe_layer(_with_q(w, pa), a), label="before change")
        compare(r2, oracle.moe_layer(_with_q(w, pb), a), label="after change")
    finally:
        ctx.close()


def test_bad_requests_change_nothing():
    import any_precision_expert_amd as pw
    from any_precision_expert_amd.layer import register_layer
    w, a = _layer(seed=502)
    ctx = make_ctx(w.shape)
    try:
        register_layer(ctx, 0, w)
        ids = [ctx.block_id(0, 0, 0), ctx.block_id(0, 1, 1)]
        before = [ctx.committed_bits(i) for i in ids]
        res = ctx.resident_bytes()
        for bad_ids, bad_q in (([ids[0], ids[0]], [4, 5]),      # duplicate id
                               ([ids[0], 10 ** 6], [4, 5]),      # unknown id
                               ([ids[0], ids[1]], [2, 5]),       # q below 3
                               ([ids[0], ids[1]], [4, 9])):      # q above 8
            with pytest.raises(pw.PwError) as ei:
                ctx.set_committed_bits(bad_ids, bad_q)
            assert ei.value.status == pw.PW_ERR_INVALID
            assert [ctx.committed_bits(i) for i in ids] == before
            assert ctx.resident_bytes() == res
    finally:
        ctx.close()


def test_no_host_masters_means_no_width_changes():
    import any_precision_expert_amd as pw
    from any_precision_expert_amd.layer import register_layer
    w, a = _layer(seed=503)
    ctx = make_ctx(w.shape, keep_host_masters=False)
    try:
        register_layer(ctx, 0, w)
        bid = ctx.block_id(0, 2, 0)
        q = ctx.committed_bits(bid)
        with pytest.raises(pw.PwError) as ei:
            ctx.set_committed_bits([bid], [3 if q != 3 else 4])
        assert ei.value.status == pw.PW_ERR_STATE
        assert ctx.committed_bits(bid) == q
        ctx.set_committed_bits([bid], [q])  # unchanged width: a no-op, accepted
    finally:
        ctx.close()


def test_requested_widths_commit_only_after_their_copies_land():
    """pw_request_widths starts the moves on a copy stream held back by a
    spinning kernel: the blocks report IN_TRANSFER, pw_commit_ready commits
    nothing and a step on the compute stream runs (without waiting for the
    copy stream) at the old widths.  Once the copy stream has drained the
    blocks report READY, pw_commit_ready commits all of them and the next step
    runs at the new widths.  A second request for a pending block, and a
    pw_set_committed_bits on it, are refused with STATE."""
    import oracle
    import torch
    import any_precision_expert_amd as pw
    from any_precision_expert_amd.layer import register_layer
    w, a = _layer(seed=503)
    ctx = make_ctx(w.shape)
    try:
        register_layer(ctx, 0, w)
        torch.cuda.synchronize()
        q0 = [(b.q, d.q) for b, d in zip(w.gate_up, w.down)]
        ids = [ctx.block_id(0, e, m) for e in range(w.shape.E) for m in (0, 1)]
        want = [3 if q0[e][m] > 5 else 8 for e in range(w.shape.E) for m in (0, 1)]
        from any_precision_expert_amd.layer import Batch
        compute, copy_stream = torch.cuda.Stream(), torch.cuda.Stream()
        batches = []
        for _ in range(2):
            bb = Batch(ctx, a.x.shape[0])
            bb.load(a.logits, a.x)
            batches.append(bb)
        torch.cuda.synchronize()
        with torch.cuda.stream(copy_stream):
            torch.cuda._sleep(200_000_000)  # keeps the copies queued behind it for a while
        ctx.request_widths(ids, want, copy_stream)
        states = [ctx.block_state(i) for i in ids]
        assert all(st == pw.PAGE_IN_TRANSFER for (_, _, st) in states)
        assert [qd for (_, qd, _) in states] == want
        assert ctx.commit_ready(compute) == 0
        with pytest.raises(pw.PwError):
            ctx.request_widths(ids[:1], [4], copy_stream)
        with pytest.raises(pw.PwError):
            ctx.set_committed_bits(ids[:1], [4], compute, copy_stream)
        batches[0].step(0, compute)
        compute.synchronize()
        # the library adds no wait of the compute stream on the copy stream;
        # whether the step finished while the copies were still held back also
        # depends on the two streams landing on different hardware queues
        # (4 per process), which the library does not control: logged only
        say("copy stream still busy after the step: %s" % (not copy_stream.query()))
        compare(_fetch(batches[0]), oracle.moe_layer(w, a), label="old widths while moving")
        assert all(ctx.block_state(i)[0] == q for i, q in zip(ids, [q0[e][m] for e in range(w.shape.E)
                                                                    for m in (0, 1)]))
        copy_stream.synchronize()
        assert all(ctx.block_state(i)[2] == pw.PAGE_READY for i in ids)
        assert ctx.commit_ready(compute) == len(ids)
        assert all(ctx.block_state(i) == (q, q, pw.PAGE_RESIDENT) for i, q in zip(ids, want))
        batches[1].step(0, compute)
        pairs = list(zip(want[0::2], want[1::2]))
        compare(_fetch(batches[1]), oracle.moe_layer(_with_q(w, pairs), a), label="new widths after commit")
    finally:
        ctx.close()


def test_copy_and_update_events_are_recycled():
    """60 request / commit cycles on two blocks: the HIP events behind the
    copies and the page-table updates are reused once nothing waits on them,
    so the context creates a handful, not one or two per cycle; widths and
    resident bytes follow the last commit."""
    import torch
    import any_precision_expert_amd as pw
    from any_precision_expert_amd.layer import register_layer
    w, a = _layer(seed=507)
    ctx = make_ctx(w.shape)
    try:
        register_layer(ctx, 0, w)
        ids = [ctx.block_id(0, 0, 0), ctx.block_id(0, 1, 1)]
        compute, copy_stream = torch.cuda.Stream(), torch.cuda.Stream()
        ctx.set_committed_bits(ids, [8, 3], compute, copy_stream)
        torch.cuda.synchronize()
        ev0 = ctx.pool_stats()["events"]
        for i in range(60):
            q = [4, 7] if i % 2 == 0 else [5, 6]  # always differs from the committed pair
            ctx.request_widths(ids, q, copy_stream)
            copy_stream.synchronize()
            assert ctx.commit_ready(compute) == 2
            compute.synchronize()
            assert [ctx.committed_bits(b) for b in ids] == q
        created = ctx.pool_stats()["events"] - ev0
        say("events created over 60 cycles: %d" % created)
        assert created <= 8
    finally:
        ctx.close()


def test_staged_copies_beyond_the_chunk_ring():
    """One pw_request_widths raising twelve Mixtral-sized blocks (6 experts x
    gate_up / down, H = 4096, I = 14336) from q = 3 to 8 moves ~760 MB of
    planes and LUTs through the library's staging (16 chunks of 32 MB), so
    chunks are reused within the call after their scatter completes.  After
    the commit every block decodes to its parent codes bit for bit (code8 >>
    (8 - q) at q = 8, "Technical summary: PagedWeight", Core components 1)."""
    import torch
    import any_precision_expert_amd as pw
    E, H, I = 6, 4096, 14336
    ctx = pw.Context(0, 1, E, H, I, 2, 0)
    try:
        rng = np.random.default_rng(901)
        codes = {}
        for e in range(E):
            for m in (0, 1):
                R, K = (2 * I, H) if m == 0 else (H, I)
                c = rng.integers(0, 256, size=(R, K), dtype=np.uint8)
                luts = {k: np.zeros((R, 1 << k), np.float16) for k in range(3, 9)}  # unused by the check
                ctx.register_block(0, e, m, pw.pack_bitplanes(c), pw.concat_luts(luts), 3)
                codes[(e, m)] = c
        ids = [ctx.block_id(0, e, m) for e in range(E) for m in (0, 1)]
        compute, copy_stream = torch.cuda.Stream(), torch.cuda.Stream()
        torch.cuda.synchronize()
        ctx.request_widths(ids, [8] * len(ids), copy_stream)
        copy_stream.synchronize()
        assert ctx.commit_ready(compute) == len(ids)
        compute.synchronize()
        for (e, m), c in codes.items():
            out = torch.empty(c.shape, dtype=torch.uint8, device="cuda")
            ctx.debug_decode_codes(ctx.block_id(0, e, m), out)
            torch.cuda.synchronize()
            assert np.array_equal(out.cpu().numpy(), c), "expert %d module %d" % (e, m)
        say("staged raise of %d blocks: resident %.2f GB" % (len(ids), ctx.resident_bytes() / 1e9))
    finally:
        ctx.close()


def test_close_with_staged_copies_in_flight():
    """pw_destroy right after pw_request_widths, with the staged gathers, DMAs
    and scatters of ~500 MB still queued (no synchronisation, no commit): the
    context waits for them before it frees the staging and its gather
    threads, and a new context on the same device then runs a layer that
    matches the oracle."""
    import torch
    import any_precision_expert_amd as pw
    E, H, I = 4, 4096, 14336
    ctx = pw.Context(0, 1, E, H, I, 2, 0)
    closed = False
    try:
        rng = np.random.default_rng(902)
        for e in range(E):
            for m in (0, 1):
                R, K = (2 * I, H) if m == 0 else (H, I)
                c = rng.integers(0, 256, size=(R, K), dtype=np.uint8)
                luts = {k: np.zeros((R, 1 << k), np.float16) for k in range(3, 9)}
                ctx.register_block(0, e, m, pw.pack_bitplanes(c), pw.concat_luts(luts), 3)
        ids = [ctx.block_id(0, e, m) for e in range(E) for m in (0, 1)]
        copy_stream = torch.cuda.Stream()
        torch.cuda.synchronize()
        ctx.request_widths(ids, [8] * len(ids), copy_stream)
        ctx.close()
        closed = True
    finally:
        if not closed:
            ctx.close()
    torch.cuda.synchronize()
    import oracle
    from any_precision_expert_amd.layer import register_layer
    w, a = _layer(seed=903)
    ctx2 = make_ctx(w.shape)
    try:
        register_layer(ctx2, 0, w)
        compare(_fetch(_run(ctx2, a)), oracle.moe_layer(w, a), label="after closing with copies in flight")
    finally:
        ctx2.close()
