"""CPU checks of the MXFP8 code-choice allowance of tests/tolerance.py: it is zero
without arithmetic error, it marks exactly the elements that sit at a rounding
midpoint or whose block maximum sits at a scale boundary, and it covers an fp32
emulation of the kernels' intermediates (A, B, h, dh', dA, dB computed in fp32
from the same quantised operands, then quantised) against the fp64 oracle on the
layer shape whose y once exceeded the per-element bound on the GPU."""
import numpy as np
import pytest
import torch

from oracle import moe_mx
from oracle.mx import mx_roundtrip
from synth import Shape, make_inputs
from tolerance import check, mx_layer_allowances, mx_value_spread


def test_spread_is_zero_without_error():
    v = np.random.default_rng(0).standard_normal((8, 96))
    assert not mx_value_spread(v, 0.0).any()


def test_spread_at_a_midpoint_and_at_a_scale_boundary():
    b = np.zeros((1, 32))
    b[0, 0], b[0, 1] = 1.0, 1.0625          # 1.0625 is the midpoint of 1.0 and 1.125
    s = mx_value_spread(b, 1e-9)
    assert s[0, 0] == 0.0 and s[0, 1] == 0.125
    b = np.full((1, 32), 0.5)
    b[0, 0] = 2.0 - 1e-12                    # saturates to 1.75 at scale 2^-8, 2.0 at 2^-7
    s = mx_value_spread(b, 1e-9)
    assert s[0, 0] == 0.25 and not s[0, 1:].any()


def _f32(a):
    return np.asarray(a, dtype=np.float32)


def _emulate_fp32(inp, c, E, H):
    """y and dx with every GEMM result and SwiGLU value computed in fp32 from the
    oracle's quantised operands (numpy float32 BLAS), the quantisers of the oracle
    applied to those fp32 values; combine and reverse-dispatch in fp64."""
    qc = c["qcache"]
    x = inp["x"].double().numpy()
    dy = inp["dy"].double().numpy()
    w = c["topk_w"]
    y = np.zeros_like(x)
    dx = np.zeros_like(x)
    for mb in c["minibatches"]:
        sl, plan = mb["slice"], mb["plan"]
        xq, dyq = moe_mx.q_rows(x[sl]), moe_mx.q_rows(dy[sl])
        for e in range(E):
            r0, r1 = int(plan["offsets"][e]), int(plan["offsets"][e + 1])
            if r1 == r0:
                continue
            st = plan["src_token"][r0:r1]
            g = _f32(w[sl][st, plan["src_slot"][r0:r1]])[:, None]
            A = _f32(xq[st]) @ _f32(qc.get("g_H", e)).T
            B = _f32(xq[st]) @ _f32(qc.get("u_H", e)).T
            sg = np.float32(1) / (np.float32(1) + np.exp(-A))
            sl_ = A * sg
            h = sl_ * B
            Y = moe_mx.q_rows(h.astype(np.float64)) @ qc.get("d_I", e).T
            d = _f32(dyq[st]) @ _f32(qc.get("d_H", e))
            dh = g * d
            dA = dh * B * (sg * (np.float32(1) + A * (np.float32(1) - sg)))
            dB = dh * sl_
            dX = moe_mx.q_rows(dA.astype(np.float64)) @ qc.get("g_I", e) \
                + moe_mx.q_rows(dB.astype(np.float64)) @ qc.get("u_I", e)
            np.add.at(y, sl.start + st, g.astype(np.float64) * Y)
            np.add.at(dx, sl.start + st, dX)
    return y, dx


@pytest.mark.parametrize("T_mb", [0, 512])
def test_allowance_covers_fp32_emulation(T_mb):
    counts = np.array([0, 1, 31, 32, 33, 127, 128, 129, 255, 256, 257, 300])
    shape = Shape(T=int(counts.sum()), H=256, I=256, E=len(counts), k=1, dtype="mxfp8")
    inp = make_inputs(shape, seed=7, device="cpu", with_dy=True)
    rng = np.random.default_rng(7)
    choice = rng.permutation(np.repeat(np.arange(shape.E), counts))
    L = 0.5 * rng.standard_normal((shape.T, shape.E)).astype(np.float32)
    L[np.arange(shape.T), choice] = 8.0
    inp["logits"] = torch.from_numpy(L)
    c = moe_mx.layer_forward_mx(inp["x"], inp["logits"], 1, inp["w_gate"], inp["w_up"],
                                inp["w_down"], T_mb=T_mb)
    g = moe_mx.layer_backward_mx(c, inp["dy"], keep_operands=True)
    y_al, dx_al = mx_layer_allowances(inp["x"], inp["dy"], c, g, shape.E)
    y32, dx32 = _emulate_fp32(inp, c, shape.E, shape.H)
    # the emulation does pick other codes than the oracle in some rows ...
    moved = np.linalg.norm(y32 - c["y"], axis=1) / np.maximum(np.linalg.norm(c["y"], axis=1), 1e-300)
    assert (moved > 1e-3).any()
    # ... and meets the per-element bound with the allowance
    check(y32, c["y"], "mxfp8", "y", allowance=y_al)
    check(dx32, g["dx"], "mxfp8", "dx", allowance=dx_al)
    # the allowance stays small against the bound itself on average
    for al, r in ((y_al, c["y"]), (dx_al, g["dx"])):
        bound = 5e-2 * np.maximum(np.abs(r), np.linalg.norm(r) / np.sqrt(r.size))
        assert np.mean(al / bound) < 0.25
