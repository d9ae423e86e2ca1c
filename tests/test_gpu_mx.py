"""GPU parity of the MXFP8 path: the quantisers bit-exact against the oracle's OCP
MX quantiser, the layer (forward + backward over a ring of minibatches) against
the MXFP8 oracle fed the same dequantised operands, and the properties that hold
at any size (row-local outputs independent of the minibatch size, bitwise
repeatability)."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import digest, np_, say, shared_of, to_dev
from oracle import moe_mx
from oracle.mx import mx_quantize
from synth import CONFIGS, Shape, make_inputs
from tolerance import check, mx_layer_allowances, one_flip_allowance

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    from mixture_experts_layer_plan_amd import binding
    return binding


def mx_input(rows, cols, seed):
    g = torch.Generator().manual_seed(seed)
    a = torch.randn((rows, cols), generator=g) * torch.exp(torch.randn((rows, 1), generator=g) * 3)
    a[0, :32] = 0.0                                   # an all-zero block
    a[1, :32] = -0.0
    a[2, 5] = 1e30                                    # a block dominated by one huge value
    a[3, :] = torch.randn(cols, generator=g) * 1e-38  # fp32 subnormal range
    return a.to(torch.bfloat16)


@pytest.mark.parametrize("rows,cols", [(64, 256), (96, 7168)])
def test_quantise_rows_bitexact(B, rows, cols):
    say(f"mx quantise rows {rows}x{cols}")
    a = mx_input(rows, cols, 1)
    q = torch.empty((rows, cols), dtype=torch.uint8, device="cuda")
    s = torch.empty((rows, cols // 32), dtype=torch.uint8, device="cuda")
    B.moe_quantize_mxfp8(a.cuda(), rows, cols, 1, q, s)
    torch.cuda.synchronize()
    rq, rs = mx_quantize(a.double().numpy(), axis=1)
    np.testing.assert_array_equal(np_(s), rs)
    np.testing.assert_array_equal(np_(q), rq)


@pytest.mark.parametrize("rows,cols", [(64, 256), (2048, 300)])
def test_quantise_cols_transposed_bitexact(B, rows, cols):
    say(f"mx quantise cols {rows}x{cols}")
    a = mx_input(rows, cols, 2)
    q = torch.empty((cols, rows), dtype=torch.uint8, device="cuda")
    s = torch.empty((cols, rows // 32), dtype=torch.uint8, device="cuda")
    B.moe_quantize_mxfp8(a.cuda(), rows, cols, 0, q, s)
    torch.cuda.synchronize()
    rq, rs = mx_quantize(a.double().numpy(), axis=0)
    np.testing.assert_array_equal(np_(q), rq.T)
    np.testing.assert_array_equal(np_(s), rs.T)


def rounding_edges_f32(n_blocks, seed):
    """fp32 blocks of 32 whose scaled values sit on the E4M3 grid, on every midpoint
    between neighbouring codes and one fp32 step either side of it, and between 448
    and 480 (saturated): block b has scale exponent X_b (its first value fixes amax
    in [2^8, 2^9) 2^X_b), including X_b = -125, whose smaller values are fp32
    subnormals."""
    rng = np.random.default_rng(seed)
    grid = oracle.mx.e4m3_decode(np.arange(127))            # codes 0 .. 126: 0 .. 448
    mids = (grid[:-1] + grid[1:]) / 2
    m32 = mids.astype(np.float32)
    cand = np.concatenate([grid, mids, np.nextafter(m32, np.float32(np.inf)).astype(np.float64),
                           np.nextafter(m32, np.float32(0)).astype(np.float64),
                           np.float32([450.0, 463.99, 464.0, 479.9]).astype(np.float64)])
    X = rng.integers(-30, 30, n_blocks)
    X[:4] = [-125, -120, 100, 0]
    blocks = rng.choice(cand, (n_blocks, 32)) * rng.choice([-1.0, 1.0], (n_blocks, 32))
    blocks[:, 0] = rng.choice(np.float32([256.0, 300.0, 448.0, 479.9]).astype(np.float64), n_blocks)
    a = (blocks * np.exp2(X.astype(np.float64))[:, None]).astype(np.float32)
    assert np.array_equal(a.astype(np.float64)[4:], (blocks * np.exp2(X[:, None]))[4:])
    return a


@pytest.mark.parametrize("axis", [1, 0])
def test_quantise_f32_rounding_edges_bitexact(B, axis):
    """The fp32 quantiser (the MXFP8 backward's dZ and g h) on values at and beside every
    E4M3 rounding midpoint, saturated values and fp32 subnormals, bit for bit."""
    say(f"mx quantise fp32 rounding edges, axis {axis}")
    a = rounding_edges_f32(4096, 11).reshape(64, 2048)   # blocks along the columns
    if axis == 0:
        a = np.ascontiguousarray(a.T)                     # blocks along the rows
    rows, cols = a.shape
    qs = (cols, rows) if axis == 0 else (rows, cols)
    q = torch.empty(qs, dtype=torch.uint8, device="cuda")
    s = torch.empty((qs[0], qs[1] // 32), dtype=torch.uint8, device="cuda")
    B.moe_quantize_mxfp8_f32(torch.from_numpy(a).cuda(), rows, cols, axis, q, s)
    torch.cuda.synchronize()
    rq, rs = mx_quantize(a.astype(np.float64), axis=axis)
    if axis == 0:
        rq, rs = rq.T, rs.T
    np.testing.assert_array_equal(np_(s), rs)
    np.testing.assert_array_equal(np_(q), rq)


def test_weight_quantisation_all_orientations(B):
    say("mx weight quantisation")
    E, I, H = 3, 128, 256
    shape = Shape(T=8, H=H, I=I, E=E, k=2)
    inp = make_inputs(shape, seed=3, device="cpu")
    s = B.shape(8, H, I, E, 2)
    wq = torch.empty(B.moe_mx_weights_bytes(s), dtype=torch.uint8, device="cuda")
    B.moe_quantize_weights_mxfp8(s, inp["w_gate"].cuda(), inp["w_up"].cuda(), inp["w_down"].cuda(), wq)
    torch.cuda.synchronize()
    buf = np_(wq)
    n = E * I * H
    off = 0

    def take(nbytes):
        nonlocal off
        v = buf[off:off + nbytes]
        off += -(-nbytes // 256) * 256
        return v

    wg, wu, wd = (inp[k].double().numpy() for k in ("w_gate", "w_up", "w_down"))
    expect = [(wg, 2, False), (wu, 2, False), (wd, 2, False), (wd, 1, True), (wg, 1, True),
              (wu, 1, True)]
    for arr, axis, transposed in expect:
        codes = take(n)
        scales = take(n // 32)
        rq, rs = mx_quantize(arr, axis=axis)
        if transposed:
            rq, rs = np.swapaxes(rq, 1, 2), np.swapaxes(rs, 1, 2)
        np.testing.assert_array_equal(codes, rq.reshape(-1))
        np.testing.assert_array_equal(scales, rs.reshape(-1))


def check_layer_outputs(b, inp, c, g, E):
    """y, dx, d_topk_w and d_logits element by element; y and dx with the allowance
    for the E4M3 codes of h and dZ that fp32 and fp64 values may round differently."""
    y_al, dx_al = mx_layer_allowances(inp["x"], inp["dy"], c, g, E)
    check(b.y, c["y"], "mxfp8", "y", allowance=y_al)
    check(b.dx, g["dx"], "mxfp8", "dx", allowance=dx_al)
    check(b.d_topk_w, g["dg"], "mxfp8", "d_topk_w")
    check(b.d_logits, g["dlogits"], "mxfp8", "d_logits")


def gpu_mx(shape, inp, T_mb):
    from mixture_experts_layer_plan_amd import LayerBuffers, run_layer
    b = LayerBuffers(shape.T, shape.H, shape.I, shape.E, shape.k, shape.I_shared, "mxfp8",
                     backward=True, T_minibatch=T_mb)
    run_layer(b, inp, backward=True)
    torch.cuda.synchronize()
    return b


SMALL_MX = {
    "ring3_ragged": (Shape(T=300, H=256, I=256, E=8, k=2, I_shared=128, dtype="mxfp8"), 128),
    "skew_ring": (Shape(T=512, H=384, I=256, E=16, k=4, I_shared=256, zipf_s=1.2, dtype="mxfp8"), 128),
    "one_minibatch": (Shape(T=200, H=256, I=128, E=6, k=3, dtype="mxfp8"), 0),
    # most experts receive no row in any of the three minibatches
    "sparse_experts": (Shape(T=96, H=256, I=128, E=16, k=2, zipf_s=3.0, dtype="mxfp8"), 32),
}


@pytest.mark.parametrize("name", list(SMALL_MX))
def test_mx_layer_small_all_outputs(name):
    shape, T_mb = SMALL_MX[name]
    say(f"mx layer {name}: {shape} T_mb={T_mb}")
    inp = make_inputs(shape, seed=0, device="cpu", with_dy=True)
    b = gpu_mx(shape, to_dev(inp), T_mb)
    c = moe_mx.layer_forward_mx(inp["x"], inp["logits"], shape.k, inp["w_gate"], inp["w_up"],
                                inp["w_down"], shared=shared_of(inp), T_mb=T_mb)
    g = moe_mx.layer_backward_mx(c, inp["dy"], keep_operands=True)
    np.testing.assert_array_equal(np_(b.topk_idx), c["topk_idx"])
    check_layer_outputs(b, inp, c, g, shape.E)
    for e in range(shape.E):
        for n in ("dw_gate", "dw_up", "dw_down"):
            ops = g["wgrad_operands"].get(e, {}).get(n)
            allow = one_flip_allowance(ops) if ops else None
            check(getattr(b, n)[e], g[n][e], "mxfp8", f"{n}[{e}]", allowance=allow)
    if shape.I_shared:
        for n in ("ds_gate", "ds_up", "ds_down"):
            check(getattr(b, n), g[n], "bf16", n)


@pytest.mark.parametrize("I", [256, 512])
def test_mx_hot_expert_weight_gradients(I):
    """Three experts whose packed token range reaches the large-tile wgrad threshold
    (256 bytes; one exactly at it), the others short, over four minibatches: every
    output element by element."""
    shape, T_mb = Shape(T=1024, H=512, I=I, E=12, k=2, I_shared=256, zipf_s=2.0,
                        dtype="mxfp8"), 256
    say(f"mx hot-expert wgrads: {shape} T_mb={T_mb}")
    inp = make_inputs(shape, seed=0, device="cpu", with_dy=True)
    b = gpu_mx(shape, to_dev(inp), T_mb)
    c = moe_mx.layer_forward_mx(inp["x"], inp["logits"], shape.k, inp["w_gate"], inp["w_up"],
                                inp["w_down"], shared=shared_of(inp), T_mb=T_mb)
    g = moe_mx.layer_backward_mx(c, inp["dy"], keep_operands=True)
    np.testing.assert_array_equal(np_(b.topk_idx), c["topk_idx"])
    packed = [sum(-(-int(n) // 32) * 32 for n in np.bincount(
        c["topk_idx"][m * T_mb:(m + 1) * T_mb].ravel(), minlength=shape.E)[[e]])
        for e in range(shape.E) for m in range(shape.T // T_mb)]
    per_e = np.array(packed).reshape(shape.E, -1).sum(axis=1)
    assert (per_e >= 256).sum() == 3 and (per_e == 256).any(), per_e
    check_layer_outputs(b, inp, c, g, shape.E)
    for e in range(shape.E):
        for n in ("dw_gate", "dw_up", "dw_down"):
            ops = g["wgrad_operands"].get(e, {}).get(n)
            allow = one_flip_allowance(ops) if ops else None
            check(getattr(b, n)[e], g[n][e], "mxfp8", f"{n}[{e}]", allowance=allow)
    for n in ("ds_gate", "ds_up", "ds_down"):
        check(getattr(b, n), g[n], "bf16", n)


# Row counts around the 32-token blocks of the packed token axis, the 128-row tiles and
# the large-tile wgrad threshold (256 packed tokens), plus an expert without rows.
MX_EXACT_COUNTS = [0, 1, 31, 32, 33, 127, 128, 129, 255, 256, 257, 300]


@pytest.mark.parametrize("T_mb", [0, 512])
@pytest.mark.parametrize("HI", [(256, 256), (512, 512)])
def test_mx_layer_exact_row_counts(HI, T_mb):
    """Every output element by element.  Two rows of the 300-row expert hold E4M3
    codes of h that differ between the kernel's fp32 pre-activations and the oracle's
    fp64 ones (the pre-activations agree to 1.1e-5 and straddle a rounding midpoint),
    which moves those rows of y by up to 3.6 %: the allowance for such code choices
    covers them.  H = I = 256 runs the row-grouped MX GEMMs on the 128-row kernels,
    H = I = 512 on the 256-row kernels (K a multiple of 512)."""
    counts = np.array(MX_EXACT_COUNTS)
    H, I = HI
    shape = Shape(T=int(counts.sum()), H=H, I=I, E=len(counts), k=1, dtype="mxfp8")
    say(f"mx layer exact counts {MX_EXACT_COUNTS}: {shape} T_mb={T_mb}")
    inp = make_inputs(shape, seed=7, device="cpu", with_dy=True)
    # top-1 expert of token t fixed by a margin of 8 over N(0, 0.25) logits
    rng = np.random.default_rng(7)
    choice = rng.permutation(np.repeat(np.arange(shape.E), counts))
    L = 0.5 * rng.standard_normal((shape.T, shape.E)).astype(np.float32)
    L[np.arange(shape.T), choice] = 8.0
    inp["logits"] = torch.from_numpy(L)
    b = gpu_mx(shape, to_dev(inp), T_mb)
    c = moe_mx.layer_forward_mx(inp["x"], inp["logits"], shape.k, inp["w_gate"], inp["w_up"],
                                inp["w_down"], shared=None, T_mb=T_mb)
    g = moe_mx.layer_backward_mx(c, inp["dy"], keep_operands=True)
    np.testing.assert_array_equal(np_(b.topk_idx), c["topk_idx"])
    np.testing.assert_array_equal(np.bincount(c["topk_idx"].ravel(), minlength=shape.E), counts)
    check_layer_outputs(b, inp, c, g, shape.E)
    for e in range(shape.E):
        for n in ("dw_gate", "dw_up", "dw_down"):
            ops = g["wgrad_operands"].get(e, {}).get(n)
            allow = one_flip_allowance(ops) if ops else None
            check(getattr(b, n)[e], g[n][e], "mxfp8", f"{n}[{e}]", allowance=allow)


def test_mx_experts_without_rows_get_zero_gradients():
    shape, T_mb = SMALL_MX["sparse_experts"]
    say("mx: weight gradients of experts without rows are overwritten with zeros")
    from mixture_experts_layer_plan_amd import LayerBuffers, run_layer
    inp = to_dev(make_inputs(shape, seed=6, device="cpu", with_dy=True))
    b = LayerBuffers(shape.T, shape.H, shape.I, shape.E, shape.k, shape.I_shared, "mxfp8",
                     backward=True, T_minibatch=T_mb)
    for t in (b.dw_gate, b.dw_up, b.dw_down):
        t.fill_(1.0)
    run_layer(b, inp, backward=True)
    torch.cuda.synchronize()
    used = set(int(e) for e in np_(b.topk_idx).ravel())
    empty = [e for e in range(shape.E) if e not in used]
    assert empty and used, (empty, used)
    for e in empty:
        for t in (b.dw_gate, b.dw_up, b.dw_down):
            assert not t[e].any(), e
    for e in used:
        assert b.dw_gate[e].any() and b.dw_up[e].any() and b.dw_down[e].any(), e


def test_mx_outputs_bitwise_independent_of_minibatch_size():
    """y, dx, d_topk_w (row-local) and the weight gradients (token blocks over each
    expert's rows of the macro batch, one fixed K order) are bitwise the same for
    every minibatch size, ragged last minibatch included."""
    shape, _ = SMALL_MX["skew_ring"]
    say("mx minibatch-size invariance of every output")
    inp = to_dev(make_inputs(shape, seed=4, device="cpu", with_dy=True))
    outs = []
    for T_mb in (0, 256, 128, 96):
        b = gpu_mx(shape, inp, T_mb)
        outs.append(digest(b.y, b.dx, b.d_topk_w, b.dw_gate, b.dw_up, b.dw_down, b.ds_gate,
                           b.ds_up, b.ds_down))
    assert len(set(outs)) == 1, outs


@pytest.mark.parametrize("name", ["ring3_ragged", "skew_ring"])
def test_mx_replayed_activations_bitwise_equal_kept(name):
    """With MOE_REPLAY the forward keeps the last minibatch's pre-activations only and
    the backward replays the dispatch and up/gate GEMM of the others: every output
    is bitwise what the layer gives with all pre-activations kept."""
    from mixture_experts_layer_plan_amd import LayerBuffers, run_layer
    shape, T_mb = SMALL_MX[name]
    say(f"mx replay vs kept activations: {name}")
    inp = to_dev(make_inputs(shape, seed=8, device="cpu", with_dy=True))
    names = ("y", "dx", "d_topk_w", "d_logits", "dw_gate", "dw_up", "dw_down", "ds_gate",
             "ds_up", "ds_down")
    outs, saved = [], []
    for replay in (False, True):
        b = LayerBuffers(shape.T, shape.H, shape.I, shape.E, shape.k, shape.I_shared, "mxfp8",
                         backward=True, T_minibatch=T_mb, replay=replay)
        run_layer(b, inp, backward=True)
        torch.cuda.synchronize()
        outs.append(digest(*(getattr(b, n) for n in names)))
        saved.append(b.saved.numel())
    assert outs[0] == outs[1]
    n_mb = -(-shape.T // T_mb)
    assert saved[1] < saved[0] and n_mb > 1


def test_mx_bitwise_independent_of_persistent_grid():
    from mixture_experts_layer_plan_amd import binding
    shape, T_mb = Shape(T=1024, H=512, I=256, E=12, k=2, I_shared=256, zipf_s=2.0,
                        dtype="mxfp8"), 256
    say("mx determinism over persistent grid sizes")
    inp = to_dev(make_inputs(shape, seed=3, device="cpu", with_dy=True))
    outs = []
    try:
        for cus in (0, 8, 72):
            binding.moe_set_cu_budget(cus)
            b = gpu_mx(shape, inp, T_mb)
            outs.append(digest(b.y, b.dx, b.d_topk_w, b.dw_gate, b.dw_up, b.dw_down))
            del b
    finally:
        binding.moe_set_cu_budget(0)
    assert len(set(outs)) == 1, outs


def test_mx_full_size_weight_gradients_independent_of_minibatch_size():
    """At the MXFP8 workload's shape (T = 8192, H = 7168, I = 2048, E = 256, k = 8):
    every output is bitwise the same for minibatches of 2048, 1024 and one minibatch
    of all 8192 tokens, and with the activations of minibatches of 2048 replayed
    (compared on the device)."""
    from mixture_experts_layer_plan_amd import LayerBuffers, layer, run_layer
    shape = CONFIGS["kimi_mxfp8_ring"]
    say("mx full size: inputs on the device")
    inp = make_inputs(shape, seed=1, device="cuda", with_dy=True)
    ref = None
    names = ("y", "dx", "d_topk_w", "dw_gate", "dw_up", "dw_down", "ds_gate", "ds_up", "ds_down")
    wq = None
    for T_mb, replay in ((2048, False), (1024, False), (0, False), (2048, True)):
        say(f"mx full size: T_minibatch = {T_mb}, replay = {replay}")
        b = LayerBuffers(shape.T, shape.H, shape.I, shape.E, shape.k, shape.I_shared, "mxfp8",
                         backward=True, T_minibatch=T_mb, replay=replay)
        if wq is None:
            layer.quantize_weights(b, inp)
            wq = b.wq
        else:
            b.wq = wq
        run_layer(b, inp, backward=True, quantize=False)
        torch.cuda.synchronize()
        if ref is None:
            ref = {n: getattr(b, n) for n in names}
        else:
            for n in names:
                assert torch.equal(getattr(b, n), ref[n]), (T_mb, n)
        del b
        torch.cuda.empty_cache()


def test_mx_bitwise_repeatable():
    shape, T_mb = SMALL_MX["ring3_ragged"]
    say("mx repeatability")
    inp = to_dev(make_inputs(shape, seed=5, device="cpu", with_dy=True))
    d = [digest(*(getattr(gpu_mx(shape, inp, T_mb), n) for n in
                  ("y", "dx", "dw_gate", "dw_up", "dw_down", "d_topk_w"))) for _ in range(3)]
    assert d[0] == d[1] == d[2]


def _warm(qc, experts, kinds=("g_H", "u_H", "d_I", "d_H", "g_I", "u_I")):
    """Quantise the sampled experts' weights in threads (numpy releases the GIL in its
    array operations), each orientation once."""
    import concurrent.futures as cf
    import os
    jobs = [(k, e) for e in sorted(experts) for k in kinds]
    with cf.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 4)) as ex:
        list(ex.map(lambda j: qc.get(*j), jobs))


def test_mx_full_size_sampled():
    """The MXFP8 workload at full size (T = 8192 in minibatches of 2048, H = 7168,
    I = 2048, E = 256, k = 8, Zipf(1.2)): y, dx, d_topk_w and d_logits of six tokens
    (one from each minibatch and two more; chosen among the tokens whose experts are
    the most frequent ones, which keeps the oracle's weight quantisation bounded),
    element by element against the oracle's per-token MX definition; and column
    slices of the weight gradients of the expert with the most rows, a median one, one
    with a single row and one without rows."""
    from tolerance import mx_token_allowances
    name = "kimi_mxfp8_ring"
    shape = CONFIGS[name]
    say(f"{name}: inputs on the device")
    inp = make_inputs(shape, seed=0, device="cuda", with_dy=True)
    say(f"{name}: layer over {shape.T // shape.T_minibatch} minibatches")
    b = gpu_mx(shape, inp, shape.T_minibatch)
    L = np_(inp["logits"])
    idx, w = oracle.route(L, shape.k)
    np.testing.assert_array_equal(np_(b.topk_idx), idx)
    counts = np.bincount(idx.ravel(), minlength=shape.E)
    hot = set(np.argsort(-counts, kind="stable")[:16].tolist())
    overlap = lambda t: sum(int(e) in hot for e in idx[t])  # noqa: E731
    toks = []
    for m in range(shape.T // shape.T_minibatch):
        sl = range(m * shape.T_minibatch, (m + 1) * shape.T_minibatch)
        toks.append(max(sl, key=lambda t: (overlap(t), -t)))
    for t in sorted(range(shape.T), key=lambda t: (-overlap(t), -t)):
        if len(toks) == 6:
            break
        if t not in toks:
            toks.append(t)
    qc = moe_mx._QuantCache(inp["w_gate"], inp["w_up"], inp["w_down"])
    sh = shared_of(inp)
    experts = set(int(e) for t in toks for e in idx[t])
    say(f"{name}: oracle weights of {len(experts)} experts for tokens {toks}")
    _warm(qc, experts)
    y_g, dx_g, dg_g, dl_g = (np_(b.y.double()), np_(b.dx.double()), np_(b.d_topk_w),
                             np_(b.d_logits))
    for t in toks:
        say(f"{name}: token {t}")
        rows = []
        y_t, dx_t, dg_t = moe_mx.token_mx(inp["x"][t], idx[t], w[t], inp["dy"][t], qc, shared=sh,
                                          rows_out=rows)
        y_al, dx_al = mx_token_allowances(rows, qc)
        check(y_g[t], y_t, "mxfp8", f"y[{t}]", allowance=y_al)
        check(dx_g[t], dx_t, "mxfp8", f"dx[{t}]", allowance=dx_al)
        check(dg_g[t], dg_t, "mxfp8", f"d_topk_w[{t}]")
        dl_t = oracle.route_backward(idx[t:t + 1], w[t:t + 1], dg_t[None], shape.E)[0]
        check(dl_g[t], dl_t, "mxfp8", f"d_logits[{t}]")
    # weight-gradient slices of four experts
    pos = np.nonzero(counts)[0]
    chosen = {"most rows": int(np.argmax(counts)),
              "median": int(pos[np.argsort(counts[pos], kind="stable")[len(pos) // 2]]),
              "one row": int(pos[np.argmin(counts[pos])]),
              "no rows": int(np.nonzero(counts == 0)[0][0])}
    cols = [0, 777, shape.I - 1]
    for what, e in chosen.items():
        say(f"{name}: weight-gradient slices of expert {e} ({what}, {counts[e]} rows)")
        dWg, dWu, dWd, ops = moe_mx.expert_weight_grad_slices_mx(
            inp["x"], inp["dy"], idx, w, e, cols, inp["w_gate"][e], inp["w_up"][e],
            inp["w_down"][e], keep_operands=True)
        for n, ref, got in (("dw_gate", dWg, b.dw_gate[e][cols]), ("dw_up", dWu, b.dw_up[e][cols]),
                            ("dw_down", dWd, b.dw_down[e][:, cols])):
            allow = one_flip_allowance(ops[n]) if ops else None
            check(np_(got.double()), ref, "mxfp8", f"{n}[{e}] ({what})", allowance=allow)
    assert counts[chosen["one row"]] == 1 or counts[pos].min() > 1
