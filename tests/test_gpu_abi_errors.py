"""Argument checks of the FFN entry points on a real device.

Each bad call must return its status before anything is enqueued, so the
outputs (pre-filled with a poison value) stay untouched and a following good
call still matches the oracle.  Cases: workspace smaller than
pw_workspace_size, misaligned x / y / workspace, a routed or shared block not
registered (STATE), and the prefill path's 4 GiB bound on x and h.
"""
import ctypes

import numpy as np
import pytest

import pw_synth
from tests.gpu_util import compare, make_ctx, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu(require_gpu):
    import any_precision_expert_amd as pw
    pw.lib()


def _ffn_status(ctx, layer, x, T, b, y, ws, ws_bytes):
    """Raw status of pw_moe_ffn_bitplane (pointers as integers)."""
    import any_precision_expert_amd as pw
    import torch
    return pw.lib().pw_moe_ffn_bitplane(ctx.h, layer, x, T, b.idx.data_ptr(), b.w.data_ptr(),
                                        b.offsets.data_ptr(), b.sorted.data_ptr(), y, ws, ws_bytes,
                                        torch.cuda.current_stream().cuda_stream)


def test_bad_workspace_and_alignment_enqueue_nothing():
    import torch
    import any_precision_expert_amd as pw
    import oracle
    from any_precision_expert_amd.layer import Batch, register_layer
    w, a = pw_synth.make_small(H=256, I=128, E=4, top_k=2, T=5, I_shared=64, seed=901)
    ctx = make_ctx(w.shape)
    try:
        register_layer(ctx, 0, w)
        T = a.x.shape[0]
        b = Batch(ctx, T)
        b.load(a.logits, a.x)
        b.route()
        need = ctx.workspace_size(T)
        ws = torch.empty(need + 512, dtype=torch.uint8, device="cuda")
        xs = torch.zeros(T * 256 + 64, dtype=torch.float16, device="cuda")
        xs[:T * 256].copy_(b.x.view(-1))
        ys = torch.full((T * 256 + 64,), -7.0, dtype=torch.float16, device="cuda")
        x0, y0, w0 = xs.data_ptr(), ys.data_ptr(), ws.data_ptr()
        assert x0 % 256 == 0 and y0 % 256 == 0 and w0 % 256 == 0
        cases = [
            ("workspace one byte short", x0, y0, w0, need - 1, pw.PW_ERR_INVALID),
            ("x 2-byte aligned", x0 + 2, y0, w0, need, pw.PW_ERR_INVALID),
            ("y 8-byte aligned", x0, y0 + 8, w0, need, pw.PW_ERR_INVALID),
            ("workspace 128-byte aligned", x0, y0, w0 + 128, need, pw.PW_ERR_INVALID),
            ("null workspace", x0, y0, 0, need, pw.PW_ERR_INVALID),
            ("layer out of range", x0, y0, w0, need, pw.PW_ERR_INVALID),
        ]
        for label, x, y, wsp, nb, want in cases:
            layer = 1 if label == "layer out of range" else 0
            st = _ffn_status(ctx, layer, x, T, b, y, wsp, nb)
            say("%s: status %d (%s)" % (label, st, pw.last_error()))
            assert st == want, label
            assert pw.last_error(), label
        torch.cuda.synchronize()
        assert torch.all(ys == -7.0), "a rejected call wrote y"
        # the same buffers with a valid call
        assert _ffn_status(ctx, 0, x0, T, b, y0, w0, need) == pw.PW_OK
        torch.cuda.synchronize()
        ref = oracle.moe_layer(w, a)
        gpu = dict(idx=b.idx.cpu().numpy(), w=b.w.cpu().numpy(), offsets=b.offsets.cpu().numpy(),
                   sorted=b.sorted.cpu().numpy()[:T * w.shape.top_k],
                   y=ys[:T * 256].view(T, 256).cpu().numpy().astype(np.float64))
        compare(gpu, ref, label="after rejected calls")
    finally:
        ctx.close()


@pytest.mark.parametrize("missing", ["routed_down", "shared_gate_up"])
def test_unregistered_block_is_a_state_error(missing):
    import torch
    import any_precision_expert_amd as pw
    from any_precision_expert_amd.layer import Batch
    w, a = pw_synth.make_small(H=128, I=64, E=3, top_k=1, T=4, I_shared=64, seed=902)
    ctx = make_ctx(w.shape)
    try:
        for e in range(3):
            ctx.register_code_block(0, e, pw.MODULE_GATE_UP, w.gate_up[e].code8, w.gate_up[e].luts, w.gate_up[e].q)
            if not (missing == "routed_down" and e == 2):
                ctx.register_code_block(0, e, pw.MODULE_DOWN, w.down[e].code8, w.down[e].luts, w.down[e].q)
        if missing != "shared_gate_up":
            ctx.register_code_block(0, pw.EXPERT_SHARED, pw.MODULE_GATE_UP, w.shared_gate_up.code8,
                                    w.shared_gate_up.luts, 8)
        ctx.register_code_block(0, pw.EXPERT_SHARED, pw.MODULE_DOWN, w.shared_down.code8, w.shared_down.luts, 8)
        T = a.x.shape[0]
        b = Batch(ctx, T)
        b.load(a.logits, a.x)
        b.route()
        b.y.fill_(-7.0)
        st = _ffn_status(ctx, 0, b.x.data_ptr(), T, b, b.y.data_ptr(), b.ws.data_ptr(), b.ws_bytes)
        say("missing %s: status %d (%s)" % (missing, st, pw.last_error()))
        assert st == pw.PW_ERR_STATE
        with pytest.raises(pw.PwError) as ei:
            b.step(0)
        assert ei.value.status == pw.PW_ERR_STATE
        torch.cuda.synchronize()
        assert torch.all(b.y == -7.0)
    finally:
        ctx.close()


def test_prefill_four_gib_bound():
    """T = 65536 tokens with top-8 routing and I = 4096: the prefill path's
    fp16 h (T * 9 rows of 4096) spans 4.5 GiB, beyond its 32-bit byte
    offsets, so the call is refused (split the batch) before anything is
    enqueued.  The workspace check comes first: one byte short, the same
    call fails on the workspace instead."""
    import torch
    import any_precision_expert_amd as pw
    ctx = pw.Context(0, 1, 8, 64, 4096, 8, 0)
    try:
        T = 65536
        need = ctx.workspace_size(T)
        assert need > 4 * 2 ** 30
        # pointers are only checked for alignment: nothing is read or written
        small = torch.zeros(4096, dtype=torch.int32, device="cuda")
        p = small.data_ptr()
        S = torch.cuda.current_stream().cuda_stream
        st = pw.lib().pw_moe_ffn_bitplane(ctx.h, 0, p, T, p, p, p, p, p, p, need, S)
        msg = pw.last_error()
        say("T=%d: status %d (%s)" % (T, st, msg))
        assert st == pw.PW_ERR_INVALID and "4 GiB" in msg
        st = pw.lib().pw_moe_ffn_bitplane(ctx.h, 0, p, T, p, p, p, p, p, p, need - 1, S)
        assert st == pw.PW_ERR_INVALID and "workspace" in pw.last_error()
        torch.cuda.synchronize()
        assert torch.all(small == 0)
    finally:
        ctx.close()
