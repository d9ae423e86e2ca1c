"""Pins of the MXFP8 layer oracle: row-local outputs do not depend on the minibatch
size, the result stays within MX rounding of the exact layer, and each operand is
blocked along its own contraction axis (operands whose rows or columns differ by
many binades survive only when blocked along the right axis)."""
import numpy as np
import pytest

import oracle
from oracle import moe_mx


def rand_layer(rng, T, H, I, E, std=0.3, shared=True):
    d = {"x": rng.standard_normal((T, H)), "logits": rng.standard_normal((T, E)),
         "w_gate": rng.standard_normal((E, I, H)) * std, "w_up": rng.standard_normal((E, I, H)) * std,
         "w_down": rng.standard_normal((E, H, I)) * std, "dy": rng.standard_normal((T, H))}
    d["shared"] = (rng.standard_normal((I, H)) * std, rng.standard_normal((I, H)) * std,
                   rng.standard_normal((H, I)) * std) if shared else None
    return d


def run_mx(d, k, T_mb):
    c = moe_mx.layer_forward_mx(d["x"], d["logits"], k, d["w_gate"], d["w_up"], d["w_down"],
                                shared=d["shared"], T_mb=T_mb)
    return c, moe_mx.layer_backward_mx(c, d["dy"])


def test_outputs_do_not_depend_on_minibatch_size():
    """Row-local outputs, and the weight gradients (whose token blocks run over each
    expert's rows of the whole macro batch), are the same for every minibatch size."""
    rng = np.random.default_rng(0)
    d = rand_layer(rng, 96, 64, 64, 6)
    ref_c, ref_g = run_mx(d, 2, 0)
    for T_mb in (32, 40, 7):
        c, g = run_mx(d, 2, T_mb)
        np.testing.assert_allclose(c["y"], ref_c["y"], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(g["dx"], ref_g["dx"], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(g["dg"], ref_g["dg"], rtol=1e-11, atol=1e-12)
        for n in ("dw_gate", "dw_up", "dw_down"):
            np.testing.assert_array_equal(g[n], ref_g[n])


def test_weight_gradient_blocks_span_minibatches():
    """An expert's first 32 rows form one block even when a minibatch boundary falls
    inside them: one token among the first 32 scaled by 2^12 flushes the small rows
    of its block (an effect of MX blocking the oracle keeps), and moving the boundary
    to T_mb = 10 changes nothing."""
    rng = np.random.default_rng(8)
    d = rand_layer(rng, 64, 64, 64, 1, shared=False)
    d["x"][20] *= 2.0 ** 12
    _, g0 = run_mx(d, 1, 0)
    _, g1 = run_mx(d, 1, 10)
    np.testing.assert_array_equal(g0["dw_gate"], g1["dw_gate"])
    # per-minibatch blocks (rows 0-9, 10-19, 20-29, ...) would keep row 5's small
    # values: the shared-block result differs from that blocking
    X = d["x"]
    blk = moe_mx.q_tokens(X[:32])
    per_mb = np.concatenate([moe_mx.q_tokens(X[i:i + 10]) for i in (0, 10, 20)])[:30]
    assert not np.array_equal(blk[:30], per_mb)


def rel(a, b):
    return np.linalg.norm(a - b) / np.linalg.norm(b)


def test_within_mx_rounding_of_the_exact_layer():
    rng = np.random.default_rng(1)
    d = rand_layer(rng, 80, 64, 96, 5)
    c, g = run_mx(d, 2, 32)
    ce = oracle.layer_forward(d["x"], d["logits"], 2, d["w_gate"], d["w_up"], d["w_down"],
                              shared=d["shared"])
    ge = oracle.layer_backward(ce, d["dy"])
    assert np.array_equal(c["topk_idx"], ce["topk_idx"])
    # E4M3 keeps 3 mantissa bits: a few 2^-5 relative errors per product chain
    for name, a, b in [("y", c["y"], ce["y"]), ("dx", g["dx"], ge["dx"]), ("dg", g["dg"], ge["dg"]),
                       ("dw_gate", g["dw_gate"], ge["dw_gate"]), ("dw_down", g["dw_down"], ge["dw_down"]),
                       ("ds_gate", g["ds_gate"], ge["ds_gate"])]:
        r = rel(a, b)
        assert r < 0.15, (name, r)
        if name != "ds_gate":                 # the shared expert is not quantised
            assert r > 1e-4, (name, r)
        else:
            assert r < 1e-12


def binade_scaled(rng, shape, axis):
    """Gaussian entries whose slices along `axis` differ by 2^+-10 from one to the next."""
    a = rng.standard_normal(shape)
    s = np.where(np.arange(shape[axis]) % 2 == 0, 2.0 ** 10, 2.0 ** -10)
    sh = [1] * len(shape)
    sh[axis] = shape[axis]
    return a * s.reshape(sh)


def test_forward_weights_are_blocked_along_H():
    """W_g rows alternate by 2^20: per-row blocks (along H) keep every row."""
    rng = np.random.default_rng(2)
    T, H, I, E = 40, 64, 64, 1
    d = rand_layer(rng, T, H, I, E, shared=False)
    d["w_gate"][0] = binade_scaled(rng, (I, H), 0)
    c, _ = run_mx(d, 1, 0)
    A_exact = d["x"] @ d["w_gate"][0].T
    A_mx = c["minibatches"][0]["A"]
    col_err = np.linalg.norm(A_mx - A_exact, axis=0) / np.linalg.norm(A_exact, axis=0)
    assert col_err.max() < 0.1


def test_tokens_are_blocked_along_H_in_the_forward():
    rng = np.random.default_rng(3)
    T, H, I, E = 40, 64, 64, 1
    d = rand_layer(rng, T, H, I, E, shared=False)
    d["x"] = binade_scaled(rng, (T, H), 0)                 # tokens differ by 2^20
    c, _ = run_mx(d, 1, 0)
    A_exact = d["x"] @ d["w_gate"][0].T
    A_mx = c["minibatches"][0]["A"]
    row_err = np.linalg.norm(A_mx - A_exact, axis=1) / np.linalg.norm(A_exact, axis=1)
    assert row_err.max() < 0.1


def test_dgrad_up_weights_are_blocked_along_I():
    """W_g columns alternate by 2^20: dX = dA W_g needs W_g blocked along I."""
    rng = np.random.default_rng(4)
    T, H, I, E = 40, 64, 64, 1
    d = rand_layer(rng, T, H, I, E, shared=False)
    d["w_gate"][0] = binade_scaled(rng, (I, H), 1)
    d["w_up"][0] = binade_scaled(rng, (I, H), 1)
    c, g = run_mx(d, 1, 0)
    ce = oracle.layer_forward(d["x"], d["logits"], 1, d["w_gate"], d["w_up"], d["w_down"])
    ge = oracle.layer_backward(ce, d["dy"])
    col_err = np.linalg.norm(g["dx"] - ge["dx"], axis=0) / np.linalg.norm(ge["dx"], axis=0)
    assert col_err.max() < 0.25


def test_weight_gradients_are_blocked_along_tokens():
    """Rows of x alternate by 2^20 across tokens; dW_g = Q_t(dA)^T Q_t(X) blocked along
    tokens would flush the small tokens' contributions in a shared block, so each
    block is checked to hold tokens of one binade: use 32 big then 32 small tokens."""
    rng = np.random.default_rng(5)
    T, H, I, E = 64, 64, 64, 1
    d = rand_layer(rng, T, H, I, E, shared=False)
    big = np.arange(T) < 32
    d["x"] = d["x"] * np.where(big, 1.0, 2.0 ** -12)[:, None]
    d["dy"] = d["dy"] * np.where(big, 2.0 ** -12, 1.0)[:, None]
    c, g = run_mx(d, 1, 0)
    ce = oracle.layer_forward(d["x"], d["logits"], 1, d["w_gate"], d["w_up"], d["w_down"])
    ge = oracle.layer_backward(ce, d["dy"])
    # both binades contribute comparably (x*dy ~ 2^-12 each); blocks of 32 tokens
    # from the segment start keep each binade in its own block
    assert rel(g["dw_gate"], ge["dw_gate"]) < 0.15


def test_q_tokens_blocks_start_at_first_row():
    a = np.ones((40, 4))
    a[35] = 2.0 ** 20                       # one huge row in the second block
    q = moe_mx.q_tokens(a)
    assert np.all(q[:32] == 1.0)            # first block untouched by the huge row
    assert np.all(q[32:35] == 0.0) and np.all(q[36:] == 0.0)
    assert np.all(q[35] == 2.0 ** 20)


def test_per_token_mx_equals_planned_rows():
    rng = np.random.default_rng(6)
    d = rand_layer(rng, 48, 64, 64, 5)
    c, g = run_mx(d, 2, 16)
    qc = c["qcache"]
    for t in (0, 17, 47):
        y_t, dx_t, dg_t = moe_mx.token_mx(d["x"][t], c["topk_idx"][t], c["topk_w"][t], d["dy"][t],
                                          qc, shared=d["shared"])
        np.testing.assert_allclose(y_t, c["y"][t], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(dx_t, g["dx"][t], rtol=1e-11, atol=1e-12)
        np.testing.assert_allclose(dg_t, g["dg"][t], rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------------------------
# One pin per remaining quantisation point.  Each builds an operand whose slices
# differ by 2^20 across the axis that must NOT be blocked, checks the MX layer per
# slice against the exact layer, and, with the point moved to the other axis (a
# mistake planted in the oracle for the test), checks that the same comparison
# fails: the pin would catch a shared wrong axis in the oracle and the kernels.

def _swap(monkeypatch, point):
    """Put quantisation point `point` on the other axis."""
    if point is None:
        return
    if point in moe_mx.WEIGHT_AXIS:
        which, axis = moe_mx.WEIGHT_AXIS[point]
        monkeypatch.setitem(moe_mx.WEIGHT_AXIS, point, (which, "cols" if axis == "rows" else "rows"))
    else:
        monkeypatch.setitem(moe_mx.ACT_AXIS, point, "tokens")


def _exact(d, k=1):
    ce = oracle.layer_forward(d["x"], d["logits"], k, d["w_gate"], d["w_up"], d["w_down"])
    return ce, oracle.layer_backward(ce, d["dy"])


def _worst(a, ref, axis):
    """Largest relative error over the slices along `axis` (norms over the other axis)."""
    return np.max(np.linalg.norm(a - ref, axis=axis) / np.linalg.norm(ref, axis=axis))


def _small_layer(seed):
    rng = np.random.default_rng(seed)
    return rng, rand_layer(rng, 40, 64, 64, 1, shared=False)


@pytest.mark.parametrize("swap", [None, "d_I"])
def test_down_weights_are_blocked_along_I_in_the_forward(monkeypatch, swap):
    """W_d rows alternate by 2^20: Y = Q_I(h) Q_I(W_d)^T keeps every column of y only
    with W_d blocked along I (per row of W_d)."""
    _swap(monkeypatch, swap)
    rng, d = _small_layer(10)
    d["w_down"][0] = binade_scaled(rng, d["w_down"][0].shape, 0)
    c, _ = run_mx(d, 1, 0)
    ce, _ = _exact(d)
    worst = _worst(c["y"], ce["y"], 0)
    assert (worst < 0.3) if swap is None else (worst > 0.6), worst


@pytest.mark.parametrize("swap", [None, "d_H"])
def test_down_weights_are_blocked_along_H_in_dgrad_down(monkeypatch, swap):
    """W_d columns alternate by 2^20: dh' = Q_H(dy) Q_H(W_d) keeps every column of dh'
    (seen through the rows of dW_g = Q_t(dA)^T Q_t(X), dA ~ dh') only with W_d blocked
    along H (per column of W_d)."""
    _swap(monkeypatch, swap)
    rng, d = _small_layer(11)
    d["w_down"][0] = binade_scaled(rng, d["w_down"][0].shape, 1)
    _, g = run_mx(d, 1, 0)
    _, ge = _exact(d)
    worst = _worst(g["dw_gate"][0], ge["dw_gate"][0], 1)
    assert (worst < 0.3) if swap is None else (worst > 0.6), worst


@pytest.mark.parametrize("swap", [None, "h"])
def test_h_is_blocked_along_I(monkeypatch, swap):
    """Tokens alternate by 2^20 (so rows of h by about 2^40): Y = Q_I(h) W_d^T keeps
    every row of y only with h blocked along I (per row)."""
    _swap(monkeypatch, swap)
    rng, d = _small_layer(12)
    d["x"] = binade_scaled(rng, d["x"].shape, 0)
    c, _ = run_mx(d, 1, 0)
    ce, _ = _exact(d)
    worst = _worst(c["y"], ce["y"], 1)
    assert (worst < 0.3) if swap is None else (worst > 0.6), worst


@pytest.mark.parametrize("swap", [None, "dy", "dA", "dB"])
def test_dy_and_dgrad_up_activations_are_blocked_along_their_rows(monkeypatch, swap):
    """Rows of dy alternate by 2^20, and so do the rows of dh', dA and dB:
    dh' = Q_H(dy) Q_H(W_d) and dX = Q_I(dA) Q_I(W_g) + Q_I(dB) Q_I(W_u) keep every row
    of dx only with dy blocked along H and dA, dB each blocked along I (per row)."""
    _swap(monkeypatch, swap)
    rng, d = _small_layer(13)
    d["dy"] = binade_scaled(rng, d["dy"].shape, 0)
    _, g = run_mx(d, 1, 0)
    _, ge = _exact(d)
    worst = _worst(g["dx"], ge["dx"], 1)
    assert (worst < 0.3) if swap is None else (worst > 0.6), worst


@pytest.mark.parametrize("swap", [None, "g_H", "x"])
def test_forward_blocking_pins_fail_when_swapped(monkeypatch, swap):
    """The earlier forward pins (W_g along H; x along H) with their point swapped."""
    _swap(monkeypatch, swap)
    rng = np.random.default_rng(2)
    d = rand_layer(rng, 40, 64, 64, 1, shared=False)
    if swap == "x":
        d["x"] = binade_scaled(rng, (40, 64), 0)
    else:
        d["w_gate"][0] = binade_scaled(rng, (64, 64), 0)
    c, _ = run_mx(d, 1, 0)
    A_exact = d["x"] @ d["w_gate"][0].T
    A_mx = c["minibatches"][0]["A"]
    worst = _worst(A_mx, A_exact, 1 if swap == "x" else 0)
    assert (worst < 0.3) if swap is None else (worst > 0.6), worst


@pytest.mark.parametrize("swap", ["g_I", "u_I"])
def test_dgrad_up_weight_pin_fails_when_swapped(monkeypatch, swap):
    """test_dgrad_up_weights_are_blocked_along_I with one weight on the other axis."""
    _swap(monkeypatch, swap)
    rng = np.random.default_rng(4)
    d = rand_layer(rng, 40, 64, 64, 1, shared=False)
    d["w_gate"][0] = binade_scaled(rng, (64, 64), 1)
    d["w_up"][0] = binade_scaled(rng, (64, 64), 1)
    _, g = run_mx(d, 1, 0)
    _, ge = _exact(d)
    assert _worst(g["dx"], ge["dx"], 0) > 0.5


@pytest.mark.parametrize("T_mb", [0, 24])
def test_expert_weight_grad_slices_mx_equal_the_full_backward(T_mb):
    rng = np.random.default_rng(9)
    d = rand_layer(rng, 72, 64, 96, 5, shared=False)
    c, g = run_mx(d, 2, T_mb)
    cols = [0, 17, 95]
    for e in range(5):
        dWg, dWu, dWd = moe_mx.expert_weight_grad_slices_mx(
            d["x"], d["dy"], c["topk_idx"], c["topk_w"], e, cols, d["w_gate"][e], d["w_up"][e],
            d["w_down"][e])
        np.testing.assert_allclose(dWg, g["dw_gate"][e][cols], rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(dWu, g["dw_up"][e][cols], rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(dWd, g["dw_down"][e][:, cols], rtol=1e-11, atol=1e-13)


def test_token_rows_out_match_the_planned_rows():
    rng = np.random.default_rng(10)
    d = rand_layer(rng, 40, 64, 64, 4, shared=False)
    c, g = run_mx(d, 2, 0)
    g2 = moe_mx.layer_backward_mx(c, d["dy"], keep_operands=True)
    plan = c["minibatches"][0]["plan"]
    t = 7
    rows = []
    moe_mx.token_mx(d["x"][t], c["topk_idx"][t], c["topk_w"][t], d["dy"][t], c["qcache"],
                    rows_out=rows)
    for j, row in enumerate(rows):
        r = plan["pos"][t, j]
        assert row["e"] == c["topk_idx"][t, j]
        np.testing.assert_allclose(row["h"], c["minibatches"][0]["h"][r], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(row["dA"], g2["row_values"][0]["dA"][r], rtol=1e-12, atol=1e-14)
