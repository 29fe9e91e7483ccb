"""pw_moe_layer_noalloc (the allocation-free layer call, whose workspace is a
library-held device buffer per GPU) against pw_moe_layer with a caller
workspace: identical routing outputs and y, bit for bit, on two calls in a
row, the second with a smaller batch, and y within tolerance of the oracle;
a batch whose workspace exceeds the held buffer is refused."""
import numpy as np
import pytest

import pw_synth
from tests.gpu_util import compare, make_ctx, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu(require_gpu):
    import any_precision_expert_amd as pw
    pw.lib()


def _outputs(b):
    T, k = b.T, b.ctx.desc.top_k
    return dict(idx=b.idx.cpu().numpy(), w=b.w.cpu().numpy(), offsets=b.offsets.cpu().numpy(),
                sorted=b.sorted.cpu().numpy()[:T * k], y=b.y.cpu().numpy())


def test_noalloc_layer_equals_layer_call():
    import torch
    import any_precision_expert_amd as pw
    import oracle
    from any_precision_expert_amd.layer import Batch, register_layer
    spec = pw_synth.CONFIGS[1]
    shape, seed = spec.shape, pw_synth.config_seed(1)
    w = pw_synth.make_weights(shape, seed, 0, spec.q_policy, spec.logits)
    ctx = make_ctx(shape)
    try:
        register_layer(ctx, 0, w)
        for call, T in enumerate((16, 4)):
            say("noalloc call %d: T=%d" % (call, T))
            a = pw_synth.make_activations(shape, T, seed, 0, 50 + call, spec.logits, w.rank)
            ref_b, na_b = Batch(ctx, T), Batch(ctx, T)
            for b in (ref_b, na_b):
                b.load(a.logits, a.x)
                for t in (b.idx, b.offsets, b.sorted):
                    t.fill_(-7)
                b.w.fill_(-7.0)
                b.y.fill_(-7.0)
            ref_b.step(0)
            ctx.moe_layer_noalloc(0, na_b.logits, na_b.x, T, na_b.idx, na_b.w, na_b.offsets, na_b.sorted, na_b.y)
            torch.cuda.synchronize()
            want, got = _outputs(ref_b), _outputs(na_b)
            for key in want:
                assert np.array_equal(got[key].view(np.uint8), want[key].view(np.uint8)), \
                    "call %d (T=%d): %s differs from pw_moe_layer" % (call, T, key)
            got["y"] = got["y"].astype(np.float64)
            compare(got, oracle.moe_layer(w, a), label="noalloc T=%d" % T)
        # a batch whose workspace is larger than the held buffer is refused
        T = 256
        assert ctx.workspace_size(T) > pw.STATIC_SCRATCH_BYTES
        b = Batch(ctx, T)
        b.y.fill_(-7.0)
        with pytest.raises(pw.PwError) as ei:
            ctx.moe_layer_noalloc(0, b.logits, b.x, T, b.idx, b.w, b.offsets, b.sorted, b.y)
        assert ei.value.status == pw.PW_ERR_INVALID
        torch.cuda.synchronize()
        assert torch.all(b.y == -7.0)
    finally:
        ctx.close()
