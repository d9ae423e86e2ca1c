"""Pins of the oracle's layer forward and backward: identity experts, per-token
direct evaluation, the dense special cases, finite differences and autograd."""
import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import oracle


def rand_layer(rng, T, H, I, E, k, shared=False, router=False, std=0.3):
    d = {
        "x": rng.standard_normal((T, H)),
        "w_gate": rng.standard_normal((E, I, H)) * std,
        "w_up": rng.standard_normal((E, I, H)) * std,
        "w_down": rng.standard_normal((E, H, I)) * std,
        "dy": rng.standard_normal((T, H)),
    }
    if router:
        d["w_router"] = rng.standard_normal((E, H)) * std
        d["logits"] = None
    else:
        d["w_router"] = None
        d["logits"] = rng.standard_normal((T, E))
    d["shared"] = None
    if shared:
        Is = I + 4
        d["shared"] = (rng.standard_normal((Is, H)) * std, rng.standard_normal((Is, H)) * std,
                       rng.standard_normal((H, Is)) * std)
    return d


def fwd(d, k):
    return oracle.layer_forward(d["x"], d["logits"], k, d["w_gate"], d["w_up"], d["w_down"],
                                shared=d["shared"], w_router=d["w_router"])


@pytest.mark.parametrize("k", [2, 4, 8])
def test_identity_experts_return_input(k):
    rng = np.random.default_rng(k)
    T, H, E = 37, 24, 11
    # bf16-representable inputs: every partial sum j*x/k is exact in float64
    x = torch.tensor(rng.standard_normal((T, H))).to(torch.bfloat16).double().numpy()
    idx = np.stack([rng.permutation(E)[:k] for _ in range(T)])
    p = oracle.build_plan(idx, E)
    X = oracle.dispatch(x, p["src_token"])
    y = oracle.combine(X, p["pos"], np.full((T, k), 1.0 / k))
    assert np.array_equal(y, x)


def test_scaled_identity_experts_pin_every_pair():
    rng = np.random.default_rng(7)
    T, H, E, k = 29, 8, 9, 3
    x = rng.standard_normal((T, H))
    idx, g = oracle.route(rng.standard_normal((T, E)), k)
    p = oracle.build_plan(idx, E)
    X = oracle.dispatch(x, p["src_token"])
    c = np.zeros(X.shape[0])
    for e in range(E):
        c[p["offsets"][e]:p["offsets"][e + 1]] = e + 1
    y = oracle.combine(c[:, None] * X, p["pos"], g)
    expect = x * (g * (idx + 1)).sum(1, keepdims=True)
    np.testing.assert_allclose(y, expect, rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("shared,router", [(False, False), (True, False), (False, True), (True, True)])
def test_planned_equals_per_token_direct(shared, router):
    rng = np.random.default_rng(11)
    T, H, I, E, k = 16, 12, 6, 5, 2
    d = rand_layer(rng, T, H, I, E, k, shared=shared, router=router)
    c = fwd(d, k)
    b = oracle.layer_backward(c, d["dy"])
    for t in range(T):
        yt = oracle.token_forward(d["x"][t], c["topk_idx"][t], c["topk_w"][t], d["w_gate"],
                                  d["w_up"], d["w_down"], shared=d["shared"])
        np.testing.assert_allclose(c["y"][t], yt, rtol=1e-12, atol=1e-12)
        dxt, dgt = oracle.token_backward(d["x"][t], c["topk_idx"][t], c["topk_w"][t], d["dy"][t],
                                         d["w_gate"], d["w_up"], d["w_down"], shared=d["shared"],
                                         w_router=d["w_router"])
        np.testing.assert_allclose(b["dx"][t], dxt, rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(b["dg"][t], dgt, rtol=1e-11, atol=1e-12)


def test_dg_identity_against_forward_outputs():
    """<dy_t, Y_r> (from the forward's Y) equals the fused <dy_t W_d, h_r>."""
    rng = np.random.default_rng(12)
    T, H, I, E, k = 20, 10, 6, 6, 3
    d = rand_layer(rng, T, H, I, E, k)
    c = fwd(d, k)
    b = oracle.layer_backward(c, d["dy"])
    for t in range(T):
        for j in range(k):
            r = c["plan"]["pos"][t, j]
            assert abs(b["dg"][t, j] - d["dy"][t] @ c["Y"][r]) <= 1e-12 * (1 + abs(b["dg"][t, j]))


def test_single_expert_is_dense_swiglu():
    rng = np.random.default_rng(13)
    T, H, I = 19, 16, 10
    d = rand_layer(rng, T, H, I, 1, 1)
    c = fwd(d, 1)
    x = torch.tensor(d["x"])
    ref = (F.silu(x @ torch.tensor(d["w_gate"][0]).T) * (x @ torch.tensor(d["w_up"][0]).T)) \
        @ torch.tensor(d["w_down"][0]).T
    np.testing.assert_allclose(c["y"], ref.numpy(), rtol=1e-12, atol=1e-13)
    assert np.all(c["topk_w"] == 1.0)


def test_k_equals_E_is_dense_softmax_mixture():
    rng = np.random.default_rng(14)
    T, H, I, E = 7, 8, 5, 4
    d = rand_layer(rng, T, H, I, E, E)
    c = fwd(d, E)
    p = scipy.special.softmax(d["logits"], axis=1)
    ref = np.zeros((T, H))
    x = torch.tensor(d["x"])
    for e in range(E):
        ye = (F.silu(x @ torch.tensor(d["w_gate"][e]).T) * (x @ torch.tensor(d["w_up"][e]).T)) \
            @ torch.tensor(d["w_down"][e]).T
        ref += p[:, e:e + 1] * ye.numpy()
    np.testing.assert_allclose(c["y"], ref, rtol=1e-12, atol=1e-13)


def torch_layer(params, idx, k, shared_keys, router):
    """The per-token definition written with torch ops, for autograd."""
    x = params["x"]
    L = x @ params["w_router"].T if router else params["logits"]
    sel = torch.gather(L, 1, idx)
    g = torch.softmax(sel, dim=1)
    T = x.shape[0]
    outs = []
    for t in range(T):
        yt = 0
        for j in range(k):
            e = int(idx[t, j])
            a = params["w_gate"][e] @ x[t]
            b = params["w_up"][e] @ x[t]
            yt = yt + g[t, j] * (params["w_down"][e] @ (F.silu(a) * b))
        if shared_keys:
            a = params["s_gate"] @ x[t]
            b = params["s_up"] @ x[t]
            yt = yt + params["s_down"] @ (F.silu(a) * b)
        outs.append(yt)
    return torch.stack(outs)


@pytest.mark.parametrize("shared,router", [(False, False), (True, True)])
def test_backward_matches_autograd(shared, router):
    rng = np.random.default_rng(21)
    T, H, I, E, k = 8, 16, 8, 4, 2
    d = rand_layer(rng, T, H, I, E, k, shared=shared, router=router)
    c = fwd(d, k)
    b = oracle.layer_backward(c, d["dy"])
    params = {n: torch.tensor(d[n], requires_grad=True) for n in ("x", "w_gate", "w_up", "w_down")}
    if router:
        params["w_router"] = torch.tensor(d["w_router"], requires_grad=True)
    else:
        params["logits"] = torch.tensor(d["logits"], requires_grad=True)
    if shared:
        for n, a in zip(("s_gate", "s_up", "s_down"), d["shared"]):
            params[n] = torch.tensor(a, requires_grad=True)
    y = torch_layer(params, torch.tensor(c["topk_idx"], dtype=torch.int64), k, shared, router)
    np.testing.assert_allclose(c["y"], y.detach().numpy(), rtol=1e-12, atol=1e-13)
    (y * torch.tensor(d["dy"])).sum().backward()
    pairs = [("dx", "x"), ("dw_gate", "w_gate"), ("dw_up", "w_up"), ("dw_down", "w_down")]
    pairs += [("dw_router", "w_router")] if router else [("dlogits", "logits")]
    if shared:
        pairs += [("ds_gate", "s_gate"), ("ds_up", "s_up"), ("ds_down", "s_down")]
    for ours, theirs in pairs:
        np.testing.assert_allclose(b[ours], params[theirs].grad.numpy(), rtol=1e-10, atol=1e-12,
                                   err_msg=ours)


def test_backward_finite_differences():
    rng = np.random.default_rng(22)
    T, H, I, E, k = 8, 16, 8, 4, 2
    d = rand_layer(rng, T, H, I, E, k, shared=True)
    c = fwd(d, k)
    b = oracle.layer_backward(c, d["dy"])
    eps = 1e-6

    def loss(dd):
        cc = fwd(dd, k)
        if not np.array_equal(cc["topk_idx"], c["topk_idx"]):
            return None
        return float((cc["y"] * d["dy"]).sum())

    checks = [("x", "dx", None), ("logits", "dlogits", None), ("w_gate", "dw_gate", None),
              ("w_up", "dw_up", None), ("w_down", "dw_down", None)]
    for name, gname, _ in checks:
        arr = d[name]
        flat_idx = rng.choice(arr.size, size=12, replace=False)
        for fi in flat_idx:
            ii = np.unravel_index(fi, arr.shape)
            dp = dict(d); dm = dict(d)
            ap = arr.copy(); ap[ii] += eps
            am = arr.copy(); am[ii] -= eps
            dp[name] = ap; dm[name] = am
            lp, lm = loss(dp), loss(dm)
            if lp is None or lm is None:
                continue
            num = (lp - lm) / (2 * eps)
            assert abs(num - b[gname][ii]) <= 1e-6 * max(1.0, abs(num)), (name, ii, num, b[gname][ii])
    # shared weights
    for si, gname in enumerate(("ds_gate", "ds_up", "ds_down")):
        arr = d["shared"][si]
        for fi in rng.choice(arr.size, size=8, replace=False):
            ii = np.unravel_index(fi, arr.shape)
            sp = list(d["shared"]); sm = list(d["shared"])
            a1 = arr.copy(); a1[ii] += eps; sp[si] = a1
            a2 = arr.copy(); a2[ii] -= eps; sm[si] = a2
            dp = dict(d, shared=tuple(sp)); dm = dict(d, shared=tuple(sm))
            num = (loss(dp) - loss(dm)) / (2 * eps)
            assert abs(num - b[gname][ii]) <= 1e-6 * max(1.0, abs(num))


def test_weight_grad_slices_match_full_backward():
    rng = np.random.default_rng(23)
    T, H, I, E, k = 30, 12, 10, 5, 2
    d = rand_layer(rng, T, H, I, E, k)
    c = fwd(d, k)
    b = oracle.layer_backward(c, d["dy"])
    p = c["plan"]
    cols = [1, 4, 9]
    for e in range(E):
        seg = slice(p["offsets"][e], p["offsets"][e + 1])
        tok, slot = p["src_token"][seg], p["src_slot"][seg]
        dg_, du_, dd_ = oracle.expert_weight_grad_slices(
            d["x"][tok], d["dy"][tok], c["topk_w"][tok, slot], d["w_gate"][e], d["w_up"][e],
            d["w_down"][e], cols)
        np.testing.assert_allclose(dg_, b["dw_gate"][e][cols], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(du_, b["dw_up"][e][cols], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(dd_, b["dw_down"][e][:, cols], rtol=1e-12, atol=1e-13)


def test_wave_heuristic_reproduces_pages_number():
    import json, os
    g = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "wave_heuristic.json")))
    assert oracle.min_minibatch_rows(g["n_sm"], 128, 256, g["I"]) == g["T_min"]
