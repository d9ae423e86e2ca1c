"""The forward entry point without allocation (moe_forward_bf16_noalloc), called
through the C-ABI, against moe_forward_bf16 with a caller workspace: bitwise the
same outputs on two calls in a row (the second with fewer tokens, so the static
workspace holds the first call's contents), and a clear error for a shape whose
workspace exceeds the static array."""
import ctypes

import pytest
import torch

from gpu_util import say, to_dev
from synth import Shape, make_inputs

pytestmark = pytest.mark.gpu


def _forward_both(shape, seed):
    from mixture_experts_layer_plan_amd import LayerBuffers, binding as B
    inp = to_dev(make_inputs(shape, seed=seed, device="cpu", with_dy=False))
    b = LayerBuffers(shape.T, shape.H, shape.I, shape.E, shape.k, shape.I_shared, "bf16",
                     backward=False)
    B.moe_route(b.s, inp["logits"], b.topk_idx, b.topk_w)
    B.moe_plan(b.s, b.topk_idx, b.plan)
    sh = [inp.get(n) for n in ("s_gate", "s_up", "s_down")]
    B.moe_forward_bf16(b.s, b.plan, inp["x"], b.topk_w, inp["w_gate"], inp["w_up"],
                       inp["w_down"], *sh, b.y, b.saved, b.ws_fwd)
    y_ref, saved_ref = b.y.clone(), b.saved.clone()
    b.y.fill_(float("nan"))
    b.saved.fill_(255)
    B.moe_forward_bf16_noalloc(b.s, b.plan, inp["x"], b.topk_w, inp["w_gate"], inp["w_up"],
                               inp["w_down"], *sh, b.y, b.saved)
    torch.cuda.synchronize()
    return y_ref, saved_ref, b.y, b.saved


def test_noalloc_forward_matches_forward_twice():
    big = Shape(T=400, H=512, I=256, E=16, k=4, I_shared=256, zipf_s=1.2)
    small = Shape(T=77, H=512, I=256, E=16, k=4, I_shared=256, zipf_s=1.2)
    for n, shape in (("first", big), ("second, smaller", small)):
        say(f"noalloc forward, {n} call: {shape}")
        y_ref, s_ref, y, s = _forward_both(shape, seed=11 if n == "first" else 12)
        assert torch.equal(y, y_ref), n
        assert torch.equal(s, s_ref), n


def test_noalloc_forward_rejects_workspace_beyond_the_static_array():
    from mixture_experts_layer_plan_amd import binding as B
    s = B.shape(4096, 7168, 2048, 256, 8, 2048)
    assert B.moe_workspace_bytes(s, B.MOE_BF16, False) > B.MOE_NOALLOC_SCRATCH_BYTES
    FAKE = 0x10000
    rc = B.lib().moe_forward_bf16_noalloc(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                          FAKE, FAKE, FAKE, FAKE, FAKE, None)
    assert rc == 4
    with pytest.raises(B.MoeError):
        B._call("moe_forward_bf16_noalloc", ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                FAKE, FAKE, FAKE, FAKE, FAKE, None)
