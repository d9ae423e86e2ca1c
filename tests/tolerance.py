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

MXFP8 y and dx get an allowance for the E4M3 codes of h and of dZ = (dA | dB)
that the kernel may choose differently from the oracle.  These intermediates are
quantised from values the kernel computes in fp32 and the oracle in fp64, so where
a value lies near a rounding midpoint (or a block maximum near a power of two,
which moves the block's scale) the two pick neighbouring codes.  The allowance
bounds that effect from the arithmetic rather than from an observed failure:
  * error of a K-term fp32 dot product of exactly representable products (the MX
    operands' products are exact in fp32): |err| <= gamma_K sum_k |a_k b_k| with
    gamma_K = K u / (1 - K u), u = 2^-24 (the standard worst-case bound);
  * first-order propagation through the SwiGLU forward and backward formulas, plus
    16 u of the result for the elementwise roundings and expf;
  * for each element, the largest move of its dequantised value over every input
    within that error (both block scales the block maximum allows, codes at both
    ends of the interval; rounding is monotone, so the ends give the extremes);
  * propagated to y and dx through |weights|: y_t gets sum_j |g_tj| sum_i
    spread(h)_ri |W_d[e][:, i]| and dx_t sum_j sum_i spread(dA)_ri |W_g[e][i, :]| +
    spread(dB)_ri |W_u[e][i, :]| (all quantised weights, as the GEMMs use them).
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


U32 = 2.0 ** -24


def gamma(n):
    """Worst-case relative error factor of an n-term fp32 sum."""
    return n * U32 / (1.0 - n * U32)


def mx_value_spread(v, err, axis=-1):
    """Largest |dequant(Q(v')) - dequant(Q(v))| over all v' with |v' - v| <= err
    elementwise, Q the OCP MX quantiser of the oracle in blocks of 32 along axis."""
    from oracle.mx import e4m3_decode, e4m3_encode, mx_roundtrip
    v = np.asarray(v, dtype=np.float64)
    err = np.broadcast_to(np.asarray(err, dtype=np.float64), v.shape)
    ref = mx_roundtrip(v, axis)
    vb, eb, rb = (np.moveaxis(a, axis, -1) for a in (v, err, ref))
    shp = vb.shape
    blk = shp[:-1] + (shp[-1] // 32, 32)
    vb, eb, rb = vb.reshape(blk), eb.reshape(blk), rb.reshape(blk)

    def scale_exp(amax):
        _, ex = np.frexp(np.where(amax > 0, amax, 1.0))
        return np.clip(np.where(amax > 0, ex - 1 - 8, -127), -127, 127)

    x_lo = scale_exp(np.max(np.maximum(np.abs(vb) - eb, 0.0), axis=-1))
    x_hi = scale_exp(np.max(np.abs(vb) + eb, axis=-1))
    spread = np.zeros_like(vb)
    for d in range(min(int(np.max(x_hi - x_lo)), 3) + 1):
        X = np.exp2(np.minimum(x_lo + d, x_hi).astype(np.float64))[..., None]
        for w in (vb - eb, vb + eb):
            val = e4m3_decode(e4m3_encode(np.clip(w / X, -448.0, 448.0))) * X
            spread = np.maximum(spread, np.abs(val - rb))
    # a block whose scale may differ by more than 3 binades (values within err of
    # zero): every element may move by its whole magnitude
    wide = (x_hi - x_lo > 3)[..., None]
    spread = np.where(wide, np.maximum(spread, np.abs(vb) + eb + np.abs(rb)), spread)
    return np.moveaxis(spread.reshape(shp), -1, axis)


def _silu(a):
    return a / (1.0 + np.exp(-a))


def _dsilu(a):
    s = 1.0 / (1.0 + np.exp(-a))
    return s * (1.0 + a * (1.0 - s))


def _d2silu(a):
    s = 1.0 / (1.0 + np.exp(-a))
    return s * (1.0 - s) * (2.0 + a * (1.0 - 2.0 * s))


def mx_row_spreads(Xq, A, B, h, Wg_q, Wu_q, dyq=None, Wd_H_q=None, dhp=None, g=None):
    """Value spreads of the quantised h (and dA, dB when the backward operands are
    given) of rows of one expert: Xq [n, H] the quantised token rows, A, B, h the
    oracle's fp64 values, Wg_q, Wu_q [I, H] the quantised forward weights; for the
    backward dyq [n, H], Wd_H_q [H, I], dhp [n, I] and the gates g [n]."""
    H = Xq.shape[1]
    aX = np.abs(Xq)
    eA = gamma(H) * (aX @ np.abs(Wg_q).T)
    eB = gamma(H) * (aX @ np.abs(Wu_q).T)
    eh = np.abs(_dsilu(A) * B) * eA + np.abs(_silu(A)) * eB + 16 * U32 * np.abs(h)
    out = {"h": mx_value_spread(h, eh, -1)}
    if dyq is not None:
        edhp = gamma(H) * (np.abs(dyq) @ np.abs(Wd_H_q))
        gg = np.abs(g)[:, None]
        ds, sl = _dsilu(A), _silu(A)
        dA = g[:, None] * dhp * B * ds
        dB = g[:, None] * dhp * sl
        sig = 1.0 / (1.0 + np.exp(-A))
        eA_ = gg * (np.abs(B * ds) * edhp + np.abs(dhp * ds) * eB
                    + np.abs(dhp * B * _d2silu(A)) * eA) \
            + 16 * U32 * gg * np.abs(dhp * B) * sig * (1.0 + np.abs(A) * (1.0 - sig))
        eB_ = gg * (np.abs(sl) * edhp + np.abs(dhp * ds) * eA) + 16 * U32 * np.abs(dB)
        out["dA"] = mx_value_spread(dA, eA_, -1)
        out["dB"] = mx_value_spread(dB, eB_, -1)
    return out


def mx_layer_allowances(inp_x, inp_dy, c, g, E):
    """Allowances of the MX layer's y and dx for the code choices of h and dZ (see
    the module docstring), from the oracle's forward cache ``c`` and backward ``g``
    (``keep_operands=True``)."""
    from oracle import moe_mx
    xf, dyf = f64(inp_x), f64(inp_dy)
    qc = c["qcache"]
    w = c["topk_w"]
    y_al = np.zeros_like(xf)
    dx_al = np.zeros_like(xf)
    for m, mb in enumerate(c["minibatches"]):
        sl, plan = mb["slice"], mb["plan"]
        rv = g["row_values"][m]
        xq = moe_mx.q_act("x", xf[sl])
        dyq = moe_mx.q_act("dy", dyf[sl])
        for e in range(E):
            r0, r1 = int(plan["offsets"][e]), int(plan["offsets"][e + 1])
            if r1 == r0:
                continue
            st = plan["src_token"][r0:r1]
            gr = w[sl][st, plan["src_slot"][r0:r1]]
            sp = mx_row_spreads(xq[st], mb["A"][r0:r1], mb["B"][r0:r1], mb["h"][r0:r1],
                                qc.get("g_H", e), qc.get("u_H", e), dyq[st], qc.get("d_H", e),
                                rv["dhp"][r0:r1], gr)
            ya = (np.abs(gr)[:, None] * sp["h"]) @ np.abs(qc.get("d_I", e)).T
            xa = sp["dA"] @ np.abs(qc.get("g_I", e)) + sp["dB"] @ np.abs(qc.get("u_I", e))
            np.add.at(y_al, sl.start + st, ya)
            np.add.at(dx_al, sl.start + st, xa)
    return y_al, dx_al


def mx_token_allowances(rows, qc):
    """The y and dx allowances of one token from its rows (``token_mx(...,
    rows_out=rows)``) and the oracle's quantised weights ``qc``."""
    y_al = dx_al = 0.0
    for row in rows:
        e = row["e"]
        one = lambda k: np.asarray(row[k])[None]  # noqa: E731
        sp = mx_row_spreads(one("xq"), one("A"), one("B"), one("h"), qc.get("g_H", e),
                            qc.get("u_H", e), one("dyq"), qc.get("d_H", e), one("dhp"),
                            np.array([row["g"]]))
        y_al = y_al + abs(row["g"]) * (sp["h"] @ np.abs(qc.get("d_I", e)).T)[0]
        dx_al = dx_al + (sp["dA"] @ np.abs(qc.get("g_I", e)) + sp["dB"] @ np.abs(qc.get("u_I", e)))[0]
    return y_al, dx_al


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
