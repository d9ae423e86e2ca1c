"""GPU parity of the whole layer (forward and backward) against the fp64 oracle.

Small shapes that span several tiles with ragged tails are compared element by
element on every output; the full-size workloads are compared on sampled tokens,
sampled weight-gradient slices and exact properties (plan, routing, zero
gradients of empty experts, bitwise repeatability)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import digest, np_, say, shared_of, to_dev
from synth import CONFIGS, Shape, make_inputs
from tolerance import check

pytestmark = pytest.mark.gpu

SMALL = {
    "ragged_bf16": Shape(T=300, H=384, I=256, E=8, k=2),
    "skew_shared_bf16": Shape(T=517, H=256, I=384, E=16, k=4, I_shared=256, zipf_s=1.2),
    "dense_E1_bf16": Shape(T=129, H=256, I=128, E=1, k=1),
    "k_eq_E_bf16": Shape(T=70, H=128, I=128, E=4, k=4),
    "one_token_bf16": Shape(T=1, H=128, I=128, E=8, k=2, I_shared=128),
    "hot_expert_bf16": Shape(T=700, H=256, I=256, E=32, k=2, zipf_s=4.0),
    # two experts past the large-tile wgrad threshold (987 and 593 rows: ragged last
    # K tiles), one just under it (255), small ones and six without rows; M / 256 = 8
    "hot_wgrad_bf16": Shape(T=1024, H=2048, I=1024, E=16, k=2, zipf_s=2.0),
    "tiny_f32": CONFIGS["tiny_f32"],
    "ragged_f32": Shape(T=200, H=256, I=256, E=6, k=3, I_shared=128, dtype="f32"),
}


def gpu_run(shape: Shape, inp_dev: dict, backward=True, fused_forward=False):
    from mixture_experts_layer_plan_amd import LayerBuffers, run_layer
    b = LayerBuffers(shape.T, shape.H, shape.I, shape.E, shape.k, shape.I_shared,
                     dtype=shape.dtype, backward=backward, router_gemm=shape.router == "gemm",
                     fused_forward=fused_forward)
    run_layer(b, inp_dev, backward=backward)
    torch.cuda.synchronize()
    return b


def router_margin_ok(L, k):
    """Top-k decisions of fp32 router logits can only be compared where the
    k-th and (k+1)-th logits are further apart than the fp32 GEMM error."""
    s = -np.sort(-L, axis=1)
    if L.shape[1] == k:
        return np.ones(L.shape[0], bool)
    return (s[:, k - 1] - s[:, k]) > 1e-4


@pytest.mark.parametrize("name", list(SMALL))
def test_layer_small_all_outputs(name):
    shape = SMALL[name]
    say(f"layer {name}: {shape}")
    inp = make_inputs(shape, seed=0, device="cpu", with_dy=True)
    check_all_outputs(shape, inp)


# Row counts around the K-loop variants of the 256-row GEMMs (a tile of at most 64
# rows, at most 128, more) and the large-tile wgrad threshold (256), plus an expert
# without rows; with H = 128 the K loop is shorter than the deepest ring's prologue.
EXACT_COUNTS = [0, 1, 63, 64, 65, 127, 128, 129, 255, 256, 257, 320]


@pytest.mark.parametrize("H", [128, 768])
def test_layer_exact_row_counts(H):
    counts = np.array(EXACT_COUNTS)
    shape = Shape(T=int(counts.sum()), H=H, I=256, E=len(counts), k=1)
    say(f"layer exact counts {EXACT_COUNTS}: {shape}")
    inp = make_inputs(shape, seed=5, device="cpu", with_dy=True)
    # top-1 expert of token t fixed by a margin of 8 over N(0, 0.25) logits, the
    # experts' tokens interleaved in a seeded order
    rng = np.random.default_rng(5)
    choice = rng.permutation(np.repeat(np.arange(shape.E), counts))
    L = 0.5 * rng.standard_normal((shape.T, shape.E)).astype(np.float32)
    L[np.arange(shape.T), choice] = 8.0
    inp["logits"] = torch.from_numpy(L)
    c = check_all_outputs(shape, inp)
    np.testing.assert_array_equal(np.bincount(c["topk_idx"].ravel(), minlength=shape.E), counts)


def check_all_outputs(shape: Shape, inp: dict, fused_forward=False):
    """Run the layer forward + backward on the GPU and compare every output with
    the oracle; returns the oracle's forward cache."""
    kind = shape.dtype
    b = gpu_run(shape, to_dev(inp), fused_forward=fused_forward)
    c = oracle.layer_forward(inp["x"], inp.get("logits"), shape.k, inp["w_gate"], inp["w_up"],
                             inp["w_down"], shared=shared_of(inp), w_router=inp.get("w_router"))
    g = oracle.layer_backward(c, inp["dy"])
    if shape.router == "gemm":
        assert router_margin_ok(c["logits"], shape.k).all(), "seed has a near-tie in the router"
        check(b.logits, c["logits"], kind, "logits")
    np.testing.assert_array_equal(np_(b.topk_idx), c["topk_idx"])
    check(b.topk_w, c["topk_w"], "f32" if kind == "f32" else "bf16", "topk_w")
    pv = b.plan_views()
    np.testing.assert_array_equal(np_(pv["src_token"]), c["plan"]["src_token"])
    np.testing.assert_array_equal(np_(pv["pos"]), c["plan"]["pos"])
    check(b.y, c["y"], kind, "y")
    # saved Z = (A | B) of every routed row
    R, I = shape.R, shape.I
    Z = b.saved[: R * 2 * I * 4].view(torch.float32).view(R, 2 * I)
    check(Z[:, :I], c["A"], kind, "saved A")
    check(Z[:, I:], c["B"], kind, "saved B")
    check(b.dx, g["dx"], kind, "dx")
    check(b.d_topk_w, g["dg"], kind, "d_topk_w")
    check(b.d_logits, g["dlogits"], kind, "d_logits")
    for e in range(shape.E):
        for n in ("dw_gate", "dw_up", "dw_down"):
            check(getattr(b, n)[e], g[n][e], kind, f"{n}[{e}]")
    if shape.I_shared:
        for n in ("ds_gate", "ds_up", "ds_down"):
            check(getattr(b, n), g[n], kind, n)
    if shape.router == "gemm":
        check(b.dw_router, g["dw_router"], kind, "dw_router")
    assert int(b.plan_views()["err_flag"].item()) == 0
    return c


def test_layer_bitwise_repeatable_and_buffer_independent():
    shape = SMALL["skew_shared_bf16"]
    say("determinism: 3 runs, 2 buffer sets")
    inp = to_dev(make_inputs(shape, seed=1, device="cpu", with_dy=True))
    outs = []
    for rep in range(3):
        b = gpu_run(shape, inp)
        outs.append(digest(b.y, b.dx, b.dw_gate, b.dw_up, b.dw_down, b.ds_gate, b.ds_up, b.ds_down,
                           b.d_topk_w, b.d_logits, b.topk_idx, b.topk_w))
        del b
    assert outs[0] == outs[1] == outs[2]


@pytest.mark.parametrize("name", ["hot_wgrad_bf16", "skew_shared_bf16"])
def test_layer_bitwise_independent_of_persistent_grid(name):
    """Every output is bitwise the same whether the persistent kernels (the weight
    gradients) run one workgroup per CU of the whole chip or far fewer: each output
    element comes from one workgroup with a fixed K order."""
    from mixture_experts_layer_plan_amd import binding
    shape = SMALL[name]
    say(f"determinism over persistent grid sizes: {name}")
    inp = to_dev(make_inputs(shape, seed=2, device="cpu", with_dy=True))
    outs = []
    try:
        for cus in (0, 8, 40, 128):
            binding.moe_set_cu_budget(cus)
            b = gpu_run(shape, inp)
            outs.append(digest(b.y, b.dx, b.dw_gate, b.dw_up, b.dw_down, b.ds_gate, b.ds_up,
                               b.ds_down, b.d_topk_w, b.d_logits))
            del b
    finally:
        binding.moe_set_cu_budget(0)
    assert len(set(outs)) == 1, outs


@pytest.mark.parametrize("name", ["hot_wgrad_bf16", "skew_shared_bf16"])
def test_side_stream_bitwise_equal_serial(name):
    """The bf16 forward runs the shared expert's GEMMs, and the backward the dispatch
    replay of x and the up-projection weight gradients, on a second stream that each
    joins back into the caller's stream; while a kernel trace is set they enqueue
    everything on the caller's stream. Both give bitwise the same outputs, read right
    after the calls on the caller's stream, which the join has to order after the
    second stream's kernels."""
    from mixture_experts_layer_plan_amd import binding
    shape = SMALL[name]
    say(f"forward and backward on two streams vs one: {name}")
    inp = to_dev(make_inputs(shape, seed=4, device="cpu", with_dy=True))
    outs = []
    b = gpu_run(shape, inp)
    outs.append(digest(b.y, b.dx, b.dw_gate, b.dw_up, b.dw_down, b.ds_gate, b.ds_up,
                       b.ds_down, b.d_topk_w, b.d_logits))
    del b
    tr = binding.KernelTrace(capacity=256)
    try:
        with tr:
            b = gpu_run(shape, inp)
            outs.append(digest(b.y, b.dx, b.dw_gate, b.dw_up, b.dw_down, b.ds_gate,
                               b.ds_up, b.ds_down, b.d_topk_w, b.d_logits))
            del b
        names = [n for n, _ in tr.records()]
    finally:
        tr.close()
    assert any(n.startswith("gemm_wgrad_up") for n in names), names
    assert outs[0] == outs[1]


@pytest.mark.parametrize("name", ["skew_shared_bf16", "one_token_bf16", "hot_expert_bf16"])
def test_fused_forward_small_all_outputs(name):
    """MOE_FUSED_FORWARD (routed and shared expert GEMMs and the combine in one
    persistent launch with counter hand-off) against the oracle, every output."""
    shape = SMALL[name]
    say(f"fused forward, layer {name}: {shape}")
    inp = make_inputs(shape, seed=0, device="cpu", with_dy=True)
    check_all_outputs(shape, inp, fused_forward=True)


@pytest.mark.parametrize("name", ["hot_wgrad_bf16", "skew_shared_bf16", "ragged_bf16",
                                  "hot_expert_bf16", "one_token_bf16", "k_eq_E_bf16"])
def test_fused_forward_bitwise_equal_separate_launches(name):
    """MOE_FUSED_FORWARD gives bitwise the outputs of the separate launches, backward
    included (the saved pre-activations are the same), and leaves the plan's err flag
    at 0."""
    from mixture_experts_layer_plan_amd import LayerBuffers, run_layer
    shape = SMALL[name]
    say(f"fused forward vs two launches: {name}")
    inp = to_dev(make_inputs(shape, seed=3, device="cpu", with_dy=True))
    outs = []
    for fused in (False, True):
        b = LayerBuffers(shape.T, shape.H, shape.I, shape.E, shape.k, shape.I_shared, "bf16",
                         backward=True, fused_forward=fused)
        run_layer(b, inp, backward=True)
        torch.cuda.synchronize()
        outs.append(digest(b.y, b.saved, b.dx, b.dw_gate, b.dw_up, b.dw_down, b.d_topk_w))
        assert int(b.plan_views()["err_flag"].item()) == 0
    assert outs[0] == outs[1]


@pytest.mark.parametrize("name", ["kimi_bf16_fwd", "kimi_bf16_fwdbwd"])
def test_fused_forward_full_size_bitwise_equal(name):
    """At the full sizes (the second with the shared expert), forward only: y and
    the saved pre-activations bitwise those of the separate launches, twice."""
    from mixture_experts_layer_plan_amd import LayerBuffers, run_layer
    shape = CONFIGS[name]
    say(f"fused forward at full size {name}: inputs on the device")
    inp = make_inputs(shape, seed=4, device="cuda", with_dy=False)
    ref = None
    for fused in (False, True, True):
        say(f"fused forward at full size: fused = {fused}")
        b = LayerBuffers(shape.T, shape.H, shape.I, shape.E, shape.k, shape.I_shared, "bf16",
                         backward=False, fused_forward=fused)
        run_layer(b, inp, backward=False)
        torch.cuda.synchronize()
        assert int(b.plan_views()["err_flag"].item()) == 0
        if ref is None:
            ref = (b.y.clone(), b.saved.clone())
        else:
            assert torch.equal(b.y, ref[0]) and torch.equal(b.saved, ref[1])
        del b


def test_fused_forward_reused_buffers_fresh_tokens():
    """The fused forward run twice on the same buffers, the second time with every
    token's x moved to the next token (same routing, so the same rows, but new h and Y
    values in every row): bitwise the separate launches on the second input.  A GEMM2
    tile or combine item that read a line of h, Y or the shared rows left in its XCD's
    cache by the first launch would differ."""
    from mixture_experts_layer_plan_amd import LayerBuffers, run_layer
    shape = CONFIGS["kimi_bf16_fwdbwd"]
    say("fused forward, reused buffers, fresh tokens: inputs on the device")
    inp = make_inputs(shape, seed=6, device="cuda", with_dy=False)
    inp2 = dict(inp)
    inp2["x"] = torch.roll(inp["x"], 1, dims=0)
    outs = []
    for fused in (True, False):
        say(f"fused = {fused}")
        b = LayerBuffers(shape.T, shape.H, shape.I, shape.E, shape.k, shape.I_shared, "bf16",
                         backward=False, fused_forward=fused)
        if fused:
            run_layer(b, inp, backward=False)
            torch.cuda.synchronize()
            y1 = b.y.clone()
        run_layer(b, inp2, backward=False)
        torch.cuda.synchronize()
        assert int(b.plan_views()["err_flag"].item()) == 0
        outs.append((b.y.clone(), b.saved.clone()))
        del b
    assert not torch.equal(y1, outs[0][0])
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


# --------------------------------------------------------------- full sizes
class ExpertCache:
    """fp64 host copies of single experts of a device weight stack, on demand."""

    def __init__(self, w):
        self.w, self.c = w, {}

    def __getitem__(self, e):
        e = int(e)
        if e not in self.c:
            self.c[e] = self.w[e].to("cpu", torch.float64).numpy()
        return self.c[e]


def full_size(name, backward):
    shape = CONFIGS[name]
    say(f"full size {name}: generating inputs on the device")
    inp = make_inputs(shape, seed=0, device="cuda", with_dy=backward)
    say(f"full size {name}: running the layer")
    b = gpu_run(shape, inp, backward=backward)
    return shape, inp, b


def sampled_tokens(T, n=8):
    return np.unique(np.linspace(0, T - 1, n).astype(int))


@pytest.mark.parametrize("name", ["mid_bf16_fwd", "kimi_bf16_fwd"])
def test_full_size_forward_sampled(name):
    shape, inp, b = full_size(name, backward=False)
    L = np_(inp["logits"])
    idx, w = oracle.route(L, shape.k)
    np.testing.assert_array_equal(np_(b.topk_idx), idx)
    ref_plan = oracle.build_plan(idx, shape.E)
    pv = b.plan_views()
    for key in ("counts", "offsets", "src_token", "src_slot", "pos"):
        np.testing.assert_array_equal(np_(pv[key]), ref_plan[key], err_msg=key)
    Wg, Wu, Wd = ExpertCache(inp["w_gate"]), ExpertCache(inp["w_up"]), ExpertCache(inp["w_down"])
    toks = sampled_tokens(shape.T)
    got = np_(b.y.double())[toks]
    ref = np.stack([oracle.token_forward(inp["x"][t], idx[t], w[t], Wg, Wu, Wd) for t in toks])
    check(got, ref, "bf16", f"{name} y (sampled tokens)")


def test_full_size_forward_backward_sampled():
    name = "kimi_bf16_fwdbwd"
    shape, inp, b = full_size(name, backward=True)
    L = np_(inp["logits"])
    idx, w = oracle.route(L, shape.k)
    np.testing.assert_array_equal(np_(b.topk_idx), idx)
    plan = oracle.build_plan(idx, shape.E)
    pv = b.plan_views()
    for key in ("counts", "offsets", "src_token", "src_slot", "pos"):
        np.testing.assert_array_equal(np_(pv[key]), plan[key], err_msg=key)
    Wg, Wu, Wd = ExpertCache(inp["w_gate"]), ExpertCache(inp["w_up"]), ExpertCache(inp["w_down"])
    sh = shared_of(inp)
    toks = sampled_tokens(shape.T, 6)
    say(f"{name}: oracle on {len(toks)} sampled tokens")
    y_ref, dx_ref, dg_ref, dl_ref = [], [], [], []
    for t in toks:
        y_ref.append(oracle.token_forward(inp["x"][t], idx[t], w[t], Wg, Wu, Wd, shared=sh))
        dx_t, dg_t = oracle.token_backward(inp["x"][t], idx[t], w[t], inp["dy"][t], Wg, Wu, Wd,
                                           shared=sh)
        dx_ref.append(dx_t)
        dg_ref.append(dg_t)
        dl_ref.append(oracle.route_backward(idx[t:t + 1], w[t:t + 1], dg_t[None], shape.E)[0])
    check(np_(b.y.double())[toks], np.stack(y_ref), "bf16", "y (sampled)")
    check(np_(b.dx.double())[toks], np.stack(dx_ref), "bf16", "dx (sampled)")
    check(np_(b.d_topk_w)[toks], np.stack(dg_ref), "bf16", "d_topk_w (sampled)")
    check(np_(b.d_logits)[toks], np.stack(dl_ref), "bf16", "d_logits (sampled)")
    # weight-gradient slices of a hot, a median, a single-row and an empty expert
    counts = plan["counts"]
    order = np.argsort(-counts, kind="stable")
    picks = [int(order[0]), int(order[len(order) // 4])]
    ones = np.nonzero(counts == 1)[0]
    zeros = np.nonzero(counts == 0)[0]
    picks += [int(ones[0])] if len(ones) else []
    cols = [0, 777, shape.I - 1]
    x64 = inp["x"]
    for e in picks:
        seg = slice(plan["offsets"][e], plan["offsets"][e + 1])
        tok, slot = plan["src_token"][seg], plan["src_slot"][seg]
        say(f"{name}: dW slices of expert {e} ({counts[e]} rows)")
        ti = torch.as_tensor(tok, device="cuda")
        dg_, du_, dd_ = oracle.expert_weight_grad_slices(
            x64[ti], inp["dy"][ti], w[tok, slot], Wg[e], Wu[e], Wd[e], cols)
        check(np_(b.dw_gate[e].double())[cols], dg_, "bf16", f"dw_gate[{e}] rows")
        check(np_(b.dw_up[e].double())[cols], du_, "bf16", f"dw_up[{e}] rows")
        check(np_(b.dw_down[e].double())[:, cols], dd_, "bf16", f"dw_down[{e}] cols")
    for e in zeros[:3]:
        assert not b.dw_gate[int(e)].any() and not b.dw_up[int(e)].any() and not b.dw_down[int(e)].any()
    say(f"{name}: shared-expert gradient slices")
    ones_g = np.ones(shape.T)
    sg_, su_, sd_ = oracle.expert_weight_grad_slices(x64, inp["dy"], ones_g, sh[0], sh[1], sh[2],
                                                     cols)
    check(np_(b.ds_gate.double())[cols], sg_, "bf16", "ds_gate rows")
    check(np_(b.ds_up.double())[cols], su_, "bf16", "ds_up rows")
    check(np_(b.ds_down.double())[:, cols], sd_, "bf16", "ds_down cols")
    # bitwise repeatability at full size
    say(f"{name}: repeat for bitwise equality")
    d1 = digest(b.y, b.dx, b.d_topk_w, b.dw_gate, b.dw_down)
    from mixture_experts_layer_plan_amd import run_layer
    run_layer(b, inp, backward=True)
    torch.cuda.synchronize()
    assert digest(b.y, b.dx, b.d_topk_w, b.dw_gate, b.dw_down) == d1


def test_ep_share_forward_backward_sampled():
    """One GPU's share of an expert-parallel layer: 4 experts x 4096 rows (every token on
    every expert), so every weight gradient runs on the large-tile wgrad kernel with
    K = 4096; sampled tokens and weight-gradient slices of every expert."""
    name = "ep_share_bf16"
    shape, inp, b = full_size(name, backward=True)
    L = np_(inp["logits"])
    idx, w = oracle.route(L, shape.k)
    np.testing.assert_array_equal(np_(b.topk_idx), idx)
    plan = oracle.build_plan(idx, shape.E)
    assert (plan["counts"] == shape.T).all()
    Wg, Wu, Wd = ExpertCache(inp["w_gate"]), ExpertCache(inp["w_up"]), ExpertCache(inp["w_down"])
    toks = sampled_tokens(shape.T, 6)
    say(f"{name}: oracle on {len(toks)} sampled tokens")
    y_ref, dx_ref, dg_ref = [], [], []
    for t in toks:
        y_ref.append(oracle.token_forward(inp["x"][t], idx[t], w[t], Wg, Wu, Wd))
        dx_t, dg_t = oracle.token_backward(inp["x"][t], idx[t], w[t], inp["dy"][t], Wg, Wu, Wd)
        dx_ref.append(dx_t)
        dg_ref.append(dg_t)
    check(np_(b.y.double())[toks], np.stack(y_ref), "bf16", "y (sampled)")
    check(np_(b.dx.double())[toks], np.stack(dx_ref), "bf16", "dx (sampled)")
    check(np_(b.d_topk_w)[toks], np.stack(dg_ref), "bf16", "d_topk_w (sampled)")
    cols = [0, 1500, shape.I - 1]
    for e in range(shape.E):
        seg = slice(plan["offsets"][e], plan["offsets"][e + 1])
        tok, slot = plan["src_token"][seg], plan["src_slot"][seg]
        say(f"{name}: dW slices of expert {e}")
        ti = torch.as_tensor(tok, device="cuda")
        dg_, du_, dd_ = oracle.expert_weight_grad_slices(
            inp["x"][ti], inp["dy"][ti], w[tok, slot], Wg[e], Wu[e], Wd[e], cols)
        check(np_(b.dw_gate[e].double())[cols], dg_, "bf16", f"dw_gate[{e}] rows")
        check(np_(b.dw_up[e].double())[cols], du_, "bf16", f"dw_up[{e}] rows")
        check(np_(b.dw_down[e].double())[:, cols], dd_, "bf16", f"dw_down[{e}] cols")


def test_empty_batch_zeroes_weight_gradients():
    say("layer T=0: forward is a no-op, backward overwrites dW with zeros")
    from mixture_experts_layer_plan_amd import LayerBuffers, run_layer
    shape = Shape(T=0, H=256, I=128, E=4, k=2, I_shared=128)
    inp = to_dev(make_inputs(shape, seed=0, device="cpu", with_dy=True))
    b = LayerBuffers(0, 256, 128, 4, 2, 128, "bf16", backward=True)
    for t in (b.dw_gate, b.dw_up, b.dw_down, b.ds_gate, b.ds_up, b.ds_down):
        t.fill_(1.0)
    run_layer(b, inp, backward=True)
    torch.cuda.synchronize()
    for t in (b.dw_gate, b.dw_up, b.dw_down, b.ds_gate, b.ds_up, b.ds_down):
        assert not t.any()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_experts_without_rows_get_zero_gradients(dtype):
    # a Zipf(2.0) routing over 64 experts: a hot expert (>= 256 rows, the large-tile
    # wgrads), small ones, and experts without rows, whose gradient blocks the
    # small-tile wgrads overwrite with zeros in contiguous spans
    shape = Shape(T=512, H=256, I=128, E=64, k=2, zipf_s=2.0, dtype=dtype)
    say(f"layer {dtype}: dW of experts without rows overwritten with zeros, others written")
    from mixture_experts_layer_plan_amd import LayerBuffers, run_layer
    inp = to_dev(make_inputs(shape, seed=3, device="cpu", with_dy=True))
    b = LayerBuffers(shape.T, shape.H, shape.I, shape.E, shape.k, 0, dtype, backward=True)
    for t in (b.dw_gate, b.dw_up, b.dw_down):
        t.fill_(1.0)
    run_layer(b, inp, backward=True)
    torch.cuda.synchronize()
    counts = np.bincount(np_(b.topk_idx).ravel(), minlength=shape.E)
    empty = [e for e in range(shape.E) if counts[e] == 0]
    assert empty and counts.max() >= 256, counts
    for e in range(shape.E):
        for t in (b.dw_gate, b.dw_up, b.dw_down):
            if counts[e] == 0:
                assert not t[e].any(), e
            else:
                assert not (t[e] == 1.0).all(dim=-1).any(), e  # no row left as filled
