"""Float tolerances of the parity tests.

bf16 path: normwise ||got - ref||_F / ||ref||_F <= 1e-2 and per element
|got_i - ref_i| <= 3e-2 * max(|ref_i|, rms(ref)).  fp32 path: 1e-5 and 1e-4 in the
same forms.  MXFP8 path: 5e-2 in both forms, against the oracle fed the same
dequantised MX operands.  The rms floor keeps near-zero elements from demanding
a relative accuracy that no rounded intermediate can give.

MXFP8 weight gradients also get a per-element allowance for one flipped code.
The kernel quantises fp32 operands, the oracle fp64 ones; a value within fp32
rounding of an E4M3 rounding midpoint lands on the neighbouring code on one side
(OCP MX v1.0: three mantissa bits, so neighbouring codes differ by at most 2^-3 of
the value).  A flip in a_t moves element (i, j) of sum_t a_t^T b_t by at most
2^-3 |a_ti| |b_tj|; the allowance covers one such term per element:
2^-3 max_t |a_ti| |b_tj| over the oracle's quantised operands.  The normwise
bound is unchanged.
"""
import numpy as np

TOL = {"bf16": (1e-2, 3e-2), "f32": (1e-5, 1e-4), "mxfp8": (5e-2, 5e-2)}


def f64(a):
    if hasattr(a, "detach"):
        import torch
        return a.detach().to("cpu", torch.float64).numpy()
    return np.asarray(a, dtype=np.float64)


def one_flip_allowance(pairs, chunk=16):
    """2^-3 max_t |a_ti| |b_tj| over all (a, b) in pairs (see above)."""
    out = None
    for a, b in pairs:
        a, b = np.abs(a), np.abs(b)
        for t0 in range(0, a.shape[0], chunk):
            m = np.max(a[t0:t0 + chunk, :, None] * b[t0:t0 + chunk, None, :], axis=0)
            out = m if out is None else np.maximum(out, m)
    return 0.125 * out


def check(got, ref, kind="bf16", what="", allowance=None):
    g, r = f64(got), f64(ref)
    assert g.shape == r.shape, f"{what}: shape {g.shape} vs {r.shape}"
    norm_tol, elem_tol = TOL[kind]
    nr = np.linalg.norm(r)
    d = g - r
    if nr == 0:
        assert np.all(g == 0), f"{what}: expected zeros"
        return
    rel = np.linalg.norm(d) / nr
    assert rel <= norm_tol, f"{what}: normwise rel err {rel:.3e} > {norm_tol}"
    rms = nr / np.sqrt(r.size)
    bound = elem_tol * np.maximum(np.abs(r), rms)
    if allowance is not None:
        bound = bound + allowance
    bad = np.abs(d) > bound
    assert not bad.any(), (f"{what}: {bad.sum()} of {r.size} elements out of tolerance; worst "
                           f"{np.max(np.abs(d) / bound):.2f}x the bound")
    return rel


def check_norm(got, ref, kind="bf16", what=""):
    """The normwise bound alone (see test_mx_hot_expert_weight_gradients)."""
    g, r = f64(got), f64(ref)
    assert g.shape == r.shape, f"{what}: shape {g.shape} vs {r.shape}"
    nr = np.linalg.norm(r)
    rel = np.linalg.norm(g - r) / nr if nr else np.linalg.norm(g)
    assert rel <= TOL[kind][0], f"{what}: normwise rel err {rel:.3e} > {TOL[kind][0]}"
    return rel
