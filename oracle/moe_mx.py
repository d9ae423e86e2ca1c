"""MXFP8 variant of the layer oracle.  TEST INFRASTRUCTURE ONLY (see the package
docstring).

MoK trains in MXFP8, with the conversion inside the kernel and the shared expert
kept in BF16 (sebask.de, "Mixture-of-Kittens: Cursors Open-Source-Ansatz für
effizientes MoE-Training auf NVL72", § Determinismus und MXFP8-Unterstützung;
stamatios.com, "Cursor abre código de megakernel MoE para GPUs NVL72", § Outras
características).  The pages do not say which operands are quantised or along
which axis; the reading taken here: every operand of the six expert GEMMs is
replaced by dequant(Q(.)) along that GEMM's contraction axis (blocks of 32, OCP
rule in ``oracle.mx``), and everything else is the fp64 definition of
``oracle.moe``:

  forward   A = Q_H(X) Q_H(W_g)^T, B = Q_H(X) Q_H(W_u)^T, h = silu(A) B,
            Y = Q_I(h) Q_I(W_d)^T                        (Q_H: along H, per row)
  backward  dh' = Q_H(dYu) Q_H(W_d) (W_d blocked along H), dg = <dh', h>,
            dA, dB as in the bf16 definition,
            dX = Q_2I(dA|dB) [Q_I(W_g); Q_I(W_u)]      (weights blocked along I)
            dW_d[e] = Q_t(dYu)^T Q_t(g h), dW_g[e] = Q_t(dA)^T Q_t(X),
            dW_u[e] = Q_t(dB)^T Q_t(X)
where Q_t blocks along the tokens of expert e: its rows of the whole macro batch
(every minibatch, in token order), 32 rows at a time from its first row, the
last block zero-padded.

Tokens are processed in consecutive minibatches of T_mb (the ring-buffer macro
batch, stamatios.com § Ring token buffers); each minibatch has its own plan.
The weight-gradient blocks span minibatches so that the gradients do not depend
on T_mb: the pages state that the fixed order makes results independent of the
batch size (sebask.de, § Determinismus und MXFP8-Unterstützung).  The shared
expert is the exact bf16-input definition.
"""
from __future__ import annotations

import numpy as np

from .moe import _f64, build_plan, combine, dense_swiglu, dsilu, route, route_backward, silu
from .mx import mx_roundtrip


def q_rows(a) -> np.ndarray:
    """dequant(Q(a)) in blocks of 32 along the last axis."""
    return mx_roundtrip(_f64(a), axis=-1)


def q_cols(a) -> np.ndarray:
    """dequant(Q(a)) in blocks of 32 along axis 0 (the length must be a multiple of 32)."""
    return mx_roundtrip(_f64(a), axis=0)


def q_tokens(a) -> np.ndarray:
    """dequant(Q(a)) in blocks of 32 rows from the first row, last block zero-padded."""
    a = _f64(a)
    n = a.shape[0]
    pad = (-n) % 32
    if pad:
        a = np.concatenate([a, np.zeros((pad,) + a.shape[1:])])
    return mx_roundtrip(a, axis=0)[:n]


# Axis of the 32-element blocks at each quantisation point: every operand is
# blocked along the contraction axis of its own GEMM (module docstring).  The tables
# name each point so that a test can put one point on the wrong axis and show that
# a pin fails.  Activations: "x", "h", "dy", "dA", "dB" are blocked along the row
# (q_rows); the wgrad operands along the tokens of an expert's segment (q_tokens).
ACT_AXIS = {"x": "rows", "h": "rows", "dy": "rows", "dA": "rows", "dB": "rows",
            "wgrad": "tokens"}
# Weights: (which weight, axis).  W_g, W_u [I, H] and W_d [H, I] per expert; "rows"
# blocks along the last axis, "cols" along the first.
WEIGHT_AXIS = {
    "g_H": ("gate", "rows"),   # GEMM1: K = H
    "u_H": ("up", "rows"),
    "d_I": ("down", "rows"),   # GEMM2: K = I
    "d_H": ("down", "cols"),   # dgrad-down: K = H
    "g_I": ("gate", "cols"),   # dgrad-up: K = I
    "u_I": ("up", "cols"),
}


def _q_axis(axis: str, a) -> np.ndarray:
    return {"rows": q_rows, "cols": q_cols, "tokens": q_tokens}[axis](a)


def q_act(point: str, a) -> np.ndarray:
    """dequant(Q(a)) of the activation operand at quantisation point ``point``."""
    return _q_axis(ACT_AXIS[point], a)


class _QuantCache:
    """Per-expert quantised weights, each orientation computed once."""

    def __init__(self, w_gate, w_up, w_down):
        self.w = {"gate": w_gate, "up": w_up, "down": w_down}
        self.c = {}

    def get(self, kind, e):
        key = (kind, int(e))
        if key not in self.c:
            which, axis = WEIGHT_AXIS[kind]
            self.c[key] = _q_axis(axis, self.w[which][e])
        return self.c[key]


def minibatch_slices(T: int, T_mb: int):
    T_mb = T_mb or T
    return [slice(s, min(T, s + T_mb)) for s in range(0, T, T_mb)]


def layer_forward_mx(x, logits, k, w_gate, w_up, w_down, shared=None, T_mb=0,
                     qcache: _QuantCache | None = None) -> dict:
    """Forward of the MXFP8 layer over consecutive minibatches of T_mb tokens."""
    xf = _f64(x)
    L = _f64(logits)
    T, H = xf.shape
    E = L.shape[1]
    idx, g = route(L, k)
    qc = qcache or _QuantCache(w_gate, w_up, w_down)
    y = np.zeros((T, H))
    mbs = []
    for sl in minibatch_slices(T, T_mb):
        plan = build_plan(idx[sl], E)
        xq = q_act("x", xf[sl])
        n_rows = int(plan["offsets"][E])
        X = xq[plan["src_token"][:n_rows]]
        Y = np.zeros((n_rows, H))
        A = B = h = None
        for e in range(E):
            r0, r1 = int(plan["offsets"][e]), int(plan["offsets"][e + 1])
            if r1 == r0:
                continue
            Ae = X[r0:r1] @ qc.get("g_H", e).T
            Be = X[r0:r1] @ qc.get("u_H", e).T
            he = silu(Ae) * Be
            if A is None:
                I = Ae.shape[1]
                A, B, h = np.zeros((n_rows, I)), np.zeros((n_rows, I)), np.zeros((n_rows, I))
            A[r0:r1], B[r0:r1], h[r0:r1] = Ae, Be, he
            Y[r0:r1] = q_act("h", he) @ qc.get("d_I", e).T
        shared_out = dense_swiglu(xf[sl], *shared)[3] if shared is not None else None
        y[sl] = combine(Y, plan["pos"], g[sl], shared_out)
        mbs.append({"slice": sl, "plan": plan, "A": A, "B": B, "h": h, "Y": Y})
    return {"y": y, "topk_idx": idx, "topk_w": g, "minibatches": mbs, "x": xf, "E": E, "k": k,
            "shared": shared, "qcache": qc, "w": (w_gate, w_up, w_down)}


def layer_backward_mx(cache: dict, dy, keep_operands: bool = False) -> dict:
    """Backward of ``layer_forward_mx`` (selection held fixed).  With
    ``keep_operands`` the result also holds the quantised operands of the three
    weight-gradient products, ``wgrad_operands[e][name]`` = [(a, b)] with
    dW[e] = a^T b (names dw_down: (dYu, g h), dw_gate: (dA, X),
    dw_up: (dB, X)), from which a test bounds what one quantisation step of a
    single product term can move an element, and ``row_values[m]`` = the
    unquantised dh', dA and dB of minibatch m's rows (in plan order)."""
    dyf = _f64(dy)
    xf = cache["x"]
    T, H = xf.shape
    E, k = cache["E"], cache["k"]
    g = cache["topk_w"]
    qc = cache["qcache"]
    w_gate, w_up, w_down = cache["w"]
    dWg = [None] * E
    dWu = [None] * E
    dWd = [None] * E
    dx = np.zeros((T, H))
    dg = np.zeros((T, k))
    operands = {}
    row_values = []
    wrows = {}
    for mb in cache["minibatches"]:
        sl, plan = mb["slice"], mb["plan"]
        n_rows = int(plan["offsets"][E])
        st = plan["src_token"][:n_rows]
        ss = plan["src_slot"][:n_rows]
        dyq = q_act("dy", dyf[sl])
        dY_rows = dyf[sl][st]
        X_rows = xf[sl][st]
        g_rows = g[sl][st, ss]
        dX = np.zeros((n_rows, H))
        dg_rows = np.zeros(n_rows)
        if keep_operands:
            I = mb["h"].shape[1] if mb["h"] is not None else 0
            rv = {"dhp": np.zeros((n_rows, I)), "dA": np.zeros((n_rows, I)),
                  "dB": np.zeros((n_rows, I))}
            row_values.append(rv)
        for e in range(E):
            r0, r1 = int(plan["offsets"][e]), int(plan["offsets"][e + 1])
            if r1 == r0:
                continue
            A, B, h = mb["A"][r0:r1], mb["B"][r0:r1], mb["h"][r0:r1]
            dhp = dyq[st[r0:r1]] @ qc.get("d_H", e)
            dg_rows[r0:r1] = np.sum(dhp * h, axis=1)
            gr = g_rows[r0:r1][:, None]
            dh = gr * dhp
            dA = dh * B * dsilu(A)
            dB = dh * silu(A)
            if keep_operands:
                rv["dhp"][r0:r1], rv["dA"][r0:r1], rv["dB"][r0:r1] = dhp, dA, dB
            dX[r0:r1] = q_act("dA", dA) @ qc.get("g_I", e) + q_act("dB", dB) @ qc.get("u_I", e)
            # this minibatch's rows of the weight-gradient operands, in token order
            rows_e = wrows.setdefault(e, {"dYu": [], "gh": [], "dA": [], "dB": [], "X": []})
            for name, v in (("dYu", dY_rows[r0:r1]), ("gh", gr * h), ("dA", dA), ("dB", dB),
                            ("X", X_rows[r0:r1])):
                rows_e[name].append(v)
        P = plan["pos"]
        Tm = P.shape[0]
        for t in range(Tm):
            for j in range(k):
                if P[t, j] >= 0:
                    dx[sl.start + t] += dX[P[t, j]]
                    dg[sl.start + t, j] = dg_rows[P[t, j]]
    # weight gradients: each expert's rows of all minibatches, quantised along those
    # tokens in blocks of 32 from the first
    for e, rows_e in wrows.items():
        q = {name: q_act("wgrad", np.concatenate(v)) for name, v in rows_e.items()}
        ops = ((q["dYu"], q["gh"]), (q["dA"], q["X"]), (q["dB"], q["X"]))
        for store, name, (a, b) in zip((dWd, dWg, dWu), ("dw_down", "dw_gate", "dw_up"), ops):
            store[e] = a.T @ b
            if keep_operands:
                operands.setdefault(e, {})[name] = [(a, b)]
    for e in range(E):
        if dWg[e] is None:
            dWg[e] = np.zeros(tuple(w_gate[e].shape))
            dWu[e] = np.zeros(tuple(w_up[e].shape))
            dWd[e] = np.zeros(tuple(w_down[e].shape))
    out = {"dg": dg, "dw_gate": np.stack(dWg), "dw_up": np.stack(dWu), "dw_down": np.stack(dWd)}
    if keep_operands:
        out["wgrad_operands"] = operands
        out["row_values"] = row_values
    if cache["shared"] is not None:
        Sg, Su, Sd = (_f64(a) for a in cache["shared"])
        As, Bs = xf @ Sg.T, xf @ Su.T
        hs = silu(As) * Bs
        dhs = dyf @ Sd
        dAs = dhs * Bs * dsilu(As)
        dBs = dhs * silu(As)
        out["ds_down"] = dyf.T @ hs
        out["ds_gate"] = dAs.T @ xf
        out["ds_up"] = dBs.T @ xf
        dx += dAs @ Sg + dBs @ Su
    out["dx"] = dx
    out["dlogits"] = route_backward(cache["topk_idx"], g, dg, E)
    return out


def token_mx(x_t, idx_t, w_t, dy_t, qc: _QuantCache, shared=None, backward=True, rows_out=None):
    """One token straight from the MX definition (no plan, no minibatch): returns
    (y_t, dx_t, dg_t); dx_t and dg_t are None without ``backward``.  The
    row-local quantisations (x and dy along H, h along I, dA and dB along I) do not
    depend on the minibatch, so these equal the planned results row for row.  With a
    list ``rows_out``, each of the token's k rows appends its unquantised values
    (dict: e, g, A, B, h and, with ``backward``, dhp, dA, dB) and the quantised token
    rows xq, dyq."""
    v = q_act("x", _f64(x_t)[None])[0]
    g = _f64(w_t)
    y = np.zeros_like(v)
    dx = np.zeros_like(v) if backward else None
    dg = np.zeros(len(idx_t)) if backward else None
    d = q_act("dy", _f64(dy_t)[None])[0] if backward else None
    for j, e in enumerate(np.asarray(idx_t).astype(int)):
        A = qc.get("g_H", e) @ v
        B = qc.get("u_H", e) @ v
        h = silu(A) * B
        y += g[j] * (qc.get("d_I", e) @ q_act("h", h[None])[0])
        row = {"e": int(e), "g": g[j], "A": A, "B": B, "h": h, "xq": v, "dyq": d}
        if backward:
            dhp = qc.get("d_H", e).T @ d
            dg[j] = float(dhp @ h)
            dh = g[j] * dhp
            dA = dh * B * dsilu(A)
            dB = dh * silu(A)
            dx += (qc.get("g_I", e).T @ q_act("dA", dA[None])[0]
                   + qc.get("u_I", e).T @ q_act("dB", dB[None])[0])
            row.update(dhp=dhp, dA=dA, dB=dB)
        if rows_out is not None:
            rows_out.append(row)
    if shared is not None:
        Sg, Su, Sd = (_f64(a) for a in shared)
        xf = _f64(x_t)
        A = Sg @ xf
        B = Su @ xf
        y += Sd @ (silu(A) * B)
        if backward:
            dh = Sd.T @ _f64(dy_t)
            dx += Sg.T @ (dh * B * dsilu(A)) + Su.T @ (dh * silu(A))
    return y, dx, dg


def _weight_rows(kind, W, rows):
    """Rows ``rows`` of quantisation point ``kind`` of weight W (blocks along each row
    need only those rows)."""
    W = _f64(W)
    return q_rows(W[rows]) if WEIGHT_AXIS[kind][1] == "rows" else q_cols(W)[rows]


def _weight_cols(kind, W, cols):
    """Columns ``cols`` of quantisation point ``kind`` of weight W (blocks along each
    column need only those columns)."""
    W = _f64(W)
    return q_cols(W[:, cols]) if WEIGHT_AXIS[kind][1] == "cols" else q_rows(W)[:, cols]


def expert_weight_grad_slices_mx(x, dy, topk_idx, topk_w, e, cols, w_gate_e, w_up_e, w_down_e,
                                 keep_operands=False):
    """Slices of one expert's MX weight gradients straight from the definition:
    (dW_g[cols, :], dW_u[cols, :], dW_d[:, cols]) for the intermediate indices
    ``cols``.  The expert's rows are its pairs (t, j) with topk_idx[t, j] = e in
    ascending t (its rows of every minibatch, in order); the token-axis operands are
    blocked along those rows from the first (module docstring).  Everything used is
    column- or row-local: the rows ``cols`` of W_g, W_u quantised along H, the columns
    ``cols`` of W_d quantised along H, x and dy rows quantised along H.  Cost is
    linear in the expert's rows.  With ``keep_operands`` also returns the quantised
    (a, b) pairs of the three products (dW = a^T b) for the one-flip allowance."""
    xf, dyf = _f64(x), _f64(dy)
    idx = np.asarray(topk_idx)
    g_all = _f64(topk_w)
    ts, js = np.nonzero(idx == e)            # row-major: ascending t, then j
    order = np.lexsort((js, ts))
    ts, js = ts[order], js[order]
    H = xf.shape[1]
    cols = np.asarray(cols)
    if len(ts) == 0:
        z = np.zeros((len(cols), H))
        return (z, z.copy(), np.zeros((H, len(cols)))) + (({},) if keep_operands else ())
    Xq = q_act("x", xf[ts])                  # along H, per row
    Dq = q_act("dy", dyf[ts])
    g = g_all[ts, js][:, None]
    Wg_c = _weight_rows("g_H", w_gate_e, cols)   # [c, H]
    Wu_c = _weight_rows("u_H", w_up_e, cols)
    Wd_c = _weight_cols("d_H", w_down_e, cols)   # [H, c]
    A = Xq @ Wg_c.T
    B = Xq @ Wu_c.T
    h = silu(A) * B
    dhp = Dq @ Wd_c
    dh = g * dhp
    dA = dh * B * dsilu(A)
    dB = dh * silu(A)
    Xt = q_act("wgrad", xf[ts])
    ops = ((q_act("wgrad", dA), Xt), (q_act("wgrad", dB), Xt),
           (q_act("wgrad", dyf[ts]), q_act("wgrad", g * h)))
    dWg, dWu = ops[0][0].T @ ops[0][1], ops[1][0].T @ ops[1][1]
    dWd = ops[2][0].T @ ops[2][1]
    if keep_operands:
        return dWg, dWu, dWd, {"dw_gate": [ops[0]], "dw_up": [ops[1]], "dw_down": [ops[2]]}
    return dWg, dWu, dWd
