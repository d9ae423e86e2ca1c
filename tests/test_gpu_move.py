"""GPU parity of the four row-movement operations (dispatch, combine,
reverse-combine, reverse-dispatch) through the exported building blocks."""
import numpy as np
import pytest
import torch

import oracle
from gpu_util import np_, say
from tolerance import check

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def B():
    from mixture_experts_layer_plan_amd import binding
    return binding


def setup(B, T, H, E, k, seed, dtype=torch.bfloat16):
    rng = np.random.default_rng(seed)
    L = rng.standard_normal((T, E)).astype(np.float32)
    idx, _ = oracle.route(L, k)
    s = B.shape(T, H, 128, E, k)
    plan = torch.empty(B.moe_plan_bytes(s), dtype=torch.uint8, device="cuda")
    B.moe_plan(s, torch.as_tensor(idx).cuda(), plan)
    x = torch.randn((T, H), generator=torch.Generator().manual_seed(seed)).to(dtype)
    return s, plan, idx, x


@pytest.mark.parametrize("T,H,E,k", [(1, 128, 4, 1), (300, 256, 8, 2), (1031, 7168, 64, 8)])
def test_dispatch_is_exact_gather(B, T, H, E, k):
    say(f"dispatch T={T} H={H} E={E} k={k}")
    s, plan, idx, x = setup(B, T, H, E, k, 1)
    X = torch.zeros((T * k, H), dtype=torch.bfloat16, device="cuda")
    B.moe_dispatch_bf16(s, plan, x.cuda(), X)
    dYu = torch.zeros_like(X)
    B.moe_reverse_combine_bf16(s, plan, x.cuda(), dYu)
    ref = oracle.build_plan(idx, E)
    expect = x[torch.as_tensor(ref["src_token"])]
    assert torch.equal(X.cpu(), expect)
    assert torch.equal(dYu.cpu(), expect)


@pytest.mark.parametrize("k", [2, 4, 8])
def test_identity_experts_return_input_bitwise(B, k):
    say(f"identity experts k={k}")
    T, H, E = 413, 512, 16
    s, plan, idx, x = setup(B, T, H, E, k, 2)
    X = torch.empty((T * k, H), dtype=torch.bfloat16, device="cuda")
    B.moe_dispatch_bf16(s, plan, x.cuda(), X)
    w = torch.full((T, k), 1.0 / k, dtype=torch.float32, device="cuda")
    y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    B.moe_combine_bf16(s, plan, X, w, None, y)
    assert torch.equal(y.cpu(), x)
    # f32 path as well
    xf = x.float()
    Xf = torch.empty((T * k, H), dtype=torch.float32, device="cuda")
    B.moe_dispatch_f32(s, plan, xf.cuda(), Xf)
    yf = torch.empty((T, H), dtype=torch.float32, device="cuda")
    B.moe_combine_f32(s, plan, Xf, w, None, yf)
    assert torch.equal(yf.cpu(), xf)


def test_scaled_identity_experts_pin_every_pair(B):
    say("scaled identity experts")
    T, H, E, k = 257, 256, 12, 3
    s, plan, idx, x = setup(B, T, H, E, k, 3)
    ref = oracle.build_plan(idx, E)
    X = torch.empty((T * k, H), dtype=torch.bfloat16, device="cuda")
    B.moe_dispatch_bf16(s, plan, x.cuda(), X)
    c = torch.zeros(T * k)
    for e in range(E):
        c[ref["offsets"][e]:ref["offsets"][e + 1]] = e + 1       # exact small integers
    Y = (X.float() * c.cuda()[:, None]).to(torch.bfloat16)      # Y_r = (e + 1) X_r, rounded to bf16
    g = np.random.default_rng(4).dirichlet(np.ones(k), size=T).astype(np.float32)
    y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    B.moe_combine_bf16(s, plan, Y, torch.as_tensor(g).cuda(), None, y)
    expect = oracle.combine(Y.cpu(), ref["pos"], g)
    check(y, expect, "bf16", "scaled identity combine")
    # the expert id of every pair is pinned: y = x * sum_j g_j c_{e_j} up to the Y rounding
    factor = (g.astype(np.float64) * (idx + 1)).sum(1, keepdims=True)
    check(y, np_(x.double()) * factor, "bf16", "scaled identity closed form")


@pytest.mark.parametrize("with_shared", [False, True])
def test_combine_and_reverse_dispatch_match_oracle(B, with_shared):
    say(f"combine / reverse-dispatch shared={with_shared}")
    T, H, E, k = 389, 384, 10, 4
    s, plan, idx, x = setup(B, T, H, E, k, 5)
    ref = oracle.build_plan(idx, E)
    gen = torch.Generator().manual_seed(6)
    Y = torch.randn((T * k, H), generator=gen).to(torch.bfloat16)
    sh = torch.randn((T, H), generator=gen).to(torch.bfloat16) if with_shared else None
    w = torch.rand((T, k), generator=gen)
    y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    B.moe_combine_bf16(s, plan, Y.cuda(), w.cuda(), sh.cuda() if sh is not None else None, y)
    check(y, oracle.combine(Y, ref["pos"], w, sh), "bf16", "combine")
    dx = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
    B.moe_reverse_dispatch_bf16(s, plan, Y.cuda(), sh.cuda() if sh is not None else None, dx)
    check(dx, oracle.combine(Y, ref["pos"], np.ones((T, k)), sh), "bf16", "reverse-dispatch")
    # fp32 combine against the oracle at fp32 tolerance
    yf = torch.empty((T, H), dtype=torch.float32, device="cuda")
    B.moe_combine_f32(s, plan, Y.float().cuda(), w.cuda(),
                      sh.float().cuda() if sh is not None else None, yf)
    check(yf, oracle.combine(Y.float(), ref["pos"], w, None if sh is None else sh.float()), "f32",
          "combine f32")
