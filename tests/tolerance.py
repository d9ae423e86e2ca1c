"""Float tolerances of the parity tests.

bf16 path: normwise ||got - ref||_F / ||ref||_F <= 1e-2 and per element
|got_i - ref_i| <= 3e-2 * max(|ref_i|, rms(ref)).  fp32 path: 1e-5 and 1e-4 in the
same forms.  MXFP8 path: 5e-2 in both forms, against the oracle fed the same
dequantised MX operands.  The rms floor keeps near-zero elements from demanding
a relative accuracy that no rounded intermediate can give.
"""
import numpy as np

TOL = {"bf16": (1e-2, 3e-2), "f32": (1e-5, 1e-4), "mxfp8": (5e-2, 5e-2)}


def f64(a):
    if hasattr(a, "detach"):
        import torch
        return a.detach().to("cpu", torch.float64).numpy()
    return np.asarray(a, dtype=np.float64)


def check(got, ref, kind="bf16", what=""):
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
    bad = np.abs(d) > bound
    assert not bad.any(), (f"{what}: {bad.sum()} of {r.size} elements out of tolerance; worst "
                           f"{np.max(np.abs(d) / bound):.2f}x the bound")
    return rel
