"""fp64 oracle of the MoE layer: router, plan, dispatch, SwiGLU experts, combine and
the mirrored backward.  TEST INFRASTRUCTURE ONLY (see the package docstring).

Citations name the page and its section:
  [SEB §…]  sebask.de, "Mixture-of-Kittens: Cursors Open-Source-Ansatz für effizientes
            MoE-Training auf NVL72", section named after §.
  [STA §…]  stamatios.com, "Cursor abre código de megakernel MoE para GPUs NVL72",
            section named after §.
  [IHAL ¶…] ihal.it article on the Apache-2.0 release of MoK, paragraph named after ¶.

What the layer computes (plain definition, reached exactly up to summation order):
  y_t = sum_j g_{t,j} * FFN_{e_{t,j}}(x_t)  [+ S(x_t) with a shared expert],
  FFN_e(v) = (silu(v W_g[e]^T) * (v W_u[e]^T)) W_d[e]^T.
A router sends each token to a selection of experts, each a small feed-forward net
with up, gate and down projections [SEB intro]; the experts are SwiGLU
[STA §Outras características; IHAL ¶precision/SwiGLU]; a shared expert may sit beside
them [STA §Outras características].  The plan, dispatch and combine reorder rows
without changing this value: the pull schedule's order follows from the routing
[SEB §Das Scheduling] and needs no sort [STA §Escolha da direção de comunicação].

Readings taken where the pages are silent:
  * score function: softmax; gates renormalised over the selected k;
  * selection on raw logits, order (logit desc, expert id asc), ties to the lower id;
  * rows of an expert in ascending flat pair index t*k+j (= ascending token);
  * the gate multiplies the expert output in the combine; backward uses dh = g*dh';
  * SwiGLU is silu(gate) * up with separate W_g, W_u [E,I,H] and W_d [E,H,I];
  * the router-weight gradient is dg_{t,j} = <dy_t, Y_{t,j}> = <dy_t W_d[e], h>.
"""
from __future__ import annotations

import numpy as np


def _f64(a) -> np.ndarray:
    """Exact float64 copy of a numpy array or torch tensor (bf16/fp32 widen exactly)."""
    if hasattr(a, "detach"):  # torch.Tensor
        import torch
        return a.detach().to("cpu", torch.float64).numpy()
    return np.asarray(a, dtype=np.float64)


def _i64(a) -> np.ndarray:
    if hasattr(a, "detach"):
        return a.detach().to("cpu").numpy().astype(np.int64)
    return np.asarray(a).astype(np.int64)


def sigmoid(a):
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-a))


def silu(a):
    """silu(a) = a * sigmoid(a)."""
    return a * sigmoid(a)


def dsilu(a):
    """d/da silu(a) = s (1 + a (1 - s)), s = sigmoid(a)."""
    s = sigmoid(a)
    return s * (1.0 + a * (1.0 - s))


# --------------------------------------------------------------------------- router
def router_logits(x, w_router) -> np.ndarray:
    """Router scores of the tiny fp32 workload: L = x W_r^T [SEB intro: the router
    distributes tokens to a selection of experts]."""
    return _f64(x) @ _f64(w_router).T


def route(logits, k: int):
    """Top-k selection and gates [SEB intro].

    Experts are ordered by (logit descending, expert id ascending) and the first k
    are taken; the gates are the softmax of the k selected logits, which equals the
    softmax over all experts renormalised over the selection.
    Returns (topk_idx int32 [T,k], topk_w float64 [T,k]).
    """
    L = _f64(logits)
    T, E = L.shape
    ids = np.arange(E)
    idx = np.empty((T, k), dtype=np.int32)
    w = np.empty((T, k), dtype=np.float64)
    for t in range(T):
        order = np.lexsort((ids, -L[t]))     # last key is primary: -logit ascending
        sel = order[:k]
        idx[t] = sel
        z = np.exp(L[t, sel] - L[t, sel[0]])
        w[t] = z / z.sum()
    return idx, w


def route_backward(topk_idx, topk_w, d_topk_w, E: int) -> np.ndarray:
    """Gradient of the logits from the gradient of the k gates.

    With g_j = exp(L_{e_j}) / sum_{i in sel} exp(L_{e_i}):
    dL_{e_j} = g_j (dg_j - sum_i g_i dg_i); unselected experts get 0.
    The router-weight gradient dg is the one fused into the SwiGLU backward
    [STA §Outras características].
    """
    idx = _i64(topk_idx)
    g = _f64(topk_w)
    dg = _f64(d_topk_w)
    T, k = idx.shape
    dL = np.zeros((T, E), dtype=np.float64)
    for t in range(T):
        s = float(np.dot(g[t], dg[t]))
        for j in range(k):
            dL[t, idx[t, j]] = g[t, j] * (dg[t, j] - s)
    return dL


# ----------------------------------------------------------------------------- plan
def build_plan(topk_idx, E: int) -> dict:
    """Sort-free schedule table [SEB §Das Scheduling; STA §Escolha da direção].

    A counting sort of the T*k (token, slot) pairs by expert: per-expert counts,
    exclusive prefix offsets, and the pull list (src_token, src_slot) in which the
    rows of expert e are its pairs in ascending flat index p = t*k + j.  ``pos`` is
    the inverse map (pair -> row), used by the combine and reverse-dispatch.
    Pairs whose expert id lies outside [0, E) are left out and set ``err``; their
    ``pos`` is -1 and the unused tail of src_token/src_slot is -1.
    """
    idx = _i64(topk_idx)
    T, k = idx.shape
    flat = idx.reshape(-1)
    R = flat.size
    counts = np.zeros(E, dtype=np.int64)
    err = False
    for p in range(R):                       # histogram
        e = flat[p]
        if 0 <= e < E:
            counts[e] += 1
        else:
            err = True
    offsets = np.zeros(E + 1, dtype=np.int64)
    for e in range(E):                       # exclusive prefix sum
        offsets[e + 1] = offsets[e] + counts[e]
    cursor = offsets[:-1].copy()
    src_token = np.full(R, -1, dtype=np.int64)
    src_slot = np.full(R, -1, dtype=np.int64)
    pos = np.full(R, -1, dtype=np.int64)
    for p in range(R):                       # stable scatter in pair order
        e = flat[p]
        if not (0 <= e < E):
            continue
        r = cursor[e]
        cursor[e] += 1
        src_token[r] = p // k
        src_slot[r] = p % k
        pos[p] = r
    return {"counts": counts, "offsets": offsets, "src_token": src_token,
            "src_slot": src_slot, "pos": pos.reshape(T, k), "err": err,
            "T": T, "k": k, "E": E}


def tile_list(counts, offsets, bm: int) -> np.ndarray:
    """Row tiles of the grouped GEMMs: for each expert in id order, one (expert,
    first row) entry per bm rows of its segment.  Returns int64 [n_tiles, 2]."""
    out = []
    for e in range(len(counts)):
        for m in range(-(-int(counts[e]) // bm)):
            out.append((e, int(offsets[e]) + m * bm))
    return np.array(out, dtype=np.int64).reshape(-1, 2)


# ------------------------------------------------------------------------ movement
def dispatch(x, src_token) -> np.ndarray:
    """Pull gather: row r of the expert-ordered matrix is token src_token[r]
    [SEB §Push oder Pull: dispatch pulls; STA §Escolha da direção]."""
    X = _f64(x)
    st = _i64(src_token)
    st = st[st >= 0]
    return X[st]


def combine(Y, pos, topk_w, shared_out=None) -> np.ndarray:
    """Weighted sum back in token order: y_t = sum_j g_{t,j} Y[pos[t,j]]
    [SEB §Push oder Pull: combine keeps the token order; STA §Outras características:
    fixed operation order]."""
    Y = _f64(Y)
    P = _i64(pos)
    g = _f64(topk_w)
    T, k = P.shape
    y = np.zeros((T, Y.shape[1]), dtype=np.float64)
    for t in range(T):
        for j in range(k):
            if P[t, j] >= 0:
                y[t] += g[t, j] * Y[P[t, j]]
    if shared_out is not None:
        y += _f64(shared_out)
    return y


# ------------------------------------------------------------------------- experts
def expert_ffn(X_e, Wg_e, Wu_e, Wd_e):
    """SwiGLU expert on its rows: A = X W_g^T, B = X W_u^T, h = silu(A) * B,
    Y = h W_d^T [SEB intro: up/gate/down; STA §Outras características: SwiGLU]."""
    X_e = _f64(X_e)
    A = X_e @ _f64(Wg_e).T
    B = X_e @ _f64(Wu_e).T
    h = silu(A) * B
    Y = h @ _f64(Wd_e).T
    return A, B, h, Y


def dense_swiglu(x, s_gate, s_up, s_down):
    """Always-on shared expert: the same SwiGLU on every token with weight 1
    [STA §Outras características: shared expert kept in BF16 under MXFP8]."""
    return expert_ffn(x, s_gate, s_up, s_down)


def layer_forward(x, logits, k, w_gate, w_up, w_down, shared=None, w_router=None) -> dict:
    """Planned forward: route, plan, dispatch, experts one by one, combine.

    ``w_gate[e]`` etc. may be any per-expert indexable (numpy, torch, or a lazy
    loader) so that large expert stacks can be streamed one expert at a time.
    ``shared`` is None or (s_gate, s_up, s_down).  ``w_router`` given means the
    logits are computed as x W_r^T (``logits`` is then ignored).
    Returns a dict with y and everything the backward needs.
    """
    xf = _f64(x)
    T, H = xf.shape
    if w_router is not None:
        L = router_logits(xf, w_router)
    else:
        L = _f64(logits)
    E = L.shape[1]
    idx, g = route(L, k)
    plan = build_plan(idx, E)
    X = dispatch(xf, plan["src_token"])
    n_rows = X.shape[0]
    I = None
    A = B = h = None
    Y = np.zeros((n_rows, H), dtype=np.float64)
    off = plan["offsets"]
    for e in range(E):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 == r0:
            continue
        Ae, Be, he, Ye = expert_ffn(X[r0:r1], w_gate[e], w_up[e], w_down[e])
        if A is None:
            I = Ae.shape[1]
            A = np.zeros((n_rows, I)); B = np.zeros((n_rows, I)); h = np.zeros((n_rows, I))
        A[r0:r1], B[r0:r1], h[r0:r1], Y[r0:r1] = Ae, Be, he, Ye
    shared_out = None
    shared_cache = None
    if shared is not None:
        As, Bs, hs, ys = dense_swiglu(xf, *shared)
        shared_out = ys
        shared_cache = (As, Bs, hs)
    y = combine(Y, plan["pos"], g, shared_out)
    return {"y": y, "logits": L, "topk_idx": idx, "topk_w": g, "plan": plan, "X": X,
            "A": A, "B": B, "h": h, "Y": Y, "shared_out": shared_out,
            "shared_cache": shared_cache, "x": xf, "E": E, "k": k,
            "w": (w_gate, w_up, w_down), "shared": shared, "w_router": w_router}


def layer_backward(cache: dict, dy) -> dict:
    """Backward of ``layer_forward`` with the top-k selection held fixed
    [SEB §Push oder Pull: the four operations; STA §Escolha da direção: one table
    for all four; STA §Outras características: router-weight gradient fused into the
    SwiGLU backward].

    Steps: reverse-combine dYu = dy[src_token]; per expert dh' = dYu W_d[e];
    dg_r = <dh'_r, h_r>; dh = g dh'; dA = dh B silu'(A); dB = dh silu(A);
    dW_d[e] = sum_r g_r dYu_r (x) h_r; dW_g[e] = dA^T X_e; dW_u[e] = dB^T X_e;
    dX = dA W_g[e] + dB W_u[e]; reverse-dispatch dx_t = sum_j dX[pos[t,j]];
    shared expert backward; router backward from dg; with a router GEMM also
    dW_r = dL^T x and dx += dL W_r.
    """
    dyf = _f64(dy)
    plan = cache["plan"]
    st, ss, off = plan["src_token"], plan["src_slot"], plan["offsets"]
    E, k = cache["E"], cache["k"]
    xf = cache["x"]
    T, H = xf.shape
    w_gate, w_up, w_down = cache["w"]
    g = cache["topk_w"]
    X = cache["X"]
    n_rows = X.shape[0]
    dYu = dyf[st[:n_rows]]
    g_rows = g[st[:n_rows], ss[:n_rows]]
    dX = np.zeros((n_rows, H))
    dg_rows = np.zeros(n_rows)
    dWg, dWu, dWd = [], [], []
    for e in range(E):
        r0, r1 = int(off[e]), int(off[e + 1])
        if r1 == r0:                         # no rows: zero gradients, weights not read
            dWg.append(np.zeros(tuple(w_gate[e].shape))); dWu.append(np.zeros(tuple(w_up[e].shape)))
            dWd.append(np.zeros(tuple(w_down[e].shape)))
            continue
        Wg_e, Wu_e, Wd_e = _f64(w_gate[e]), _f64(w_up[e]), _f64(w_down[e])
        A, B, h = cache["A"][r0:r1], cache["B"][r0:r1], cache["h"][r0:r1]
        dhp = dYu[r0:r1] @ Wd_e
        dg_rows[r0:r1] = np.sum(dhp * h, axis=1)
        gr = g_rows[r0:r1][:, None]
        dh = gr * dhp
        dA = dh * B * dsilu(A)
        dB = dh * silu(A)
        dWd.append((gr * dYu[r0:r1]).T @ h)
        dWg.append(dA.T @ X[r0:r1])
        dWu.append(dB.T @ X[r0:r1])
        dX[r0:r1] = dA @ Wg_e + dB @ Wu_e
    P = plan["pos"]
    dx = np.zeros((T, H))
    dg = np.zeros((T, k))
    for t in range(T):
        for j in range(k):
            if P[t, j] >= 0:
                dx[t] += dX[P[t, j]]
                dg[t, j] = dg_rows[P[t, j]]
    out = {"dx_experts": dx.copy(), "dX": dX, "dg": dg,
           "dw_gate": np.stack(dWg), "dw_up": np.stack(dWu), "dw_down": np.stack(dWd)}
    if cache["shared"] is not None:
        Sg, Su, Sd = (_f64(a) for a in cache["shared"])
        As, Bs, hs = cache["shared_cache"]
        dhs = dyf @ Sd
        dAs = dhs * Bs * dsilu(As)
        dBs = dhs * silu(As)
        out["ds_down"] = dyf.T @ hs
        out["ds_gate"] = dAs.T @ xf
        out["ds_up"] = dBs.T @ xf
        dxs = dAs @ Sg + dBs @ Su
        out["dx_shared"] = dxs
        dx += dxs
    dL = route_backward(cache["topk_idx"], g, dg, E)
    out["dlogits"] = dL
    if cache["w_router"] is not None:
        Wr = _f64(cache["w_router"])
        out["dw_router"] = dL.T @ xf
        dx += dL @ Wr
    out["dx"] = dx
    return out


# ------------------------------------------------------ per-token direct definition
def token_forward(x_t, idx_t, w_t, w_gate, w_up, w_down, shared=None) -> np.ndarray:
    """y_t straight from the definition, one token at a time (no plan, no grouping)."""
    v = _f64(x_t)
    y = np.zeros_like(v)
    for j, e in enumerate(_i64(idx_t)):
        y += float(w_t[j]) * expert_ffn(v[None, :], w_gate[e], w_up[e], w_down[e])[3][0]
    if shared is not None:
        y += dense_swiglu(v[None, :], *shared)[3][0]
    return y


def token_backward(x_t, idx_t, w_t, dy_t, w_gate, w_up, w_down, shared=None, w_router=None):
    """(dx_t, dg_t) for one token straight from the definition.

    dg_{t,j} = <dy_t, FFN_{e_j}(x_t)> is taken directly (not through h), and dx_t
    is the chain rule through each selected expert (and the router if given).
    """
    v = _f64(x_t)
    d = _f64(dy_t)
    g = _f64(w_t)
    idx = _i64(idx_t)
    dx = np.zeros_like(v)
    dg = np.zeros(len(idx))
    for j, e in enumerate(idx):
        Wg_e, Wu_e, Wd_e = _f64(w_gate[e]), _f64(w_up[e]), _f64(w_down[e])
        A = Wg_e @ v
        B = Wu_e @ v
        Yj = Wd_e @ (silu(A) * B)
        dg[j] = float(d @ Yj)
        dh = g[j] * (Wd_e.T @ d)
        dx += Wg_e.T @ (dh * B * dsilu(A)) + Wu_e.T @ (dh * silu(A))
    if shared is not None:
        Sg, Su, Sd = (_f64(a) for a in shared)
        A = Sg @ v
        B = Su @ v
        dh = Sd.T @ d
        dx += Sg.T @ (dh * B * dsilu(A)) + Su.T @ (dh * silu(A))
    if w_router is not None:
        Wr = _f64(w_router)
        s = float(g @ dg)
        for j, e in enumerate(idx):
            dx += g[j] * (dg[j] - s) * Wr[e]
    return dx, dg


def expert_weight_grad_slices(rows_x, rows_dy, rows_g, Wg_e, Wu_e, Wd_e, cols):
    """Slices of one expert's weight gradients from the definition.

    ``rows_x``/``rows_dy``/``rows_g`` hold, for every pair routed to the expert, the
    token's x, dy and gate.  Returns (dW_g[cols, :], dW_u[cols, :], dW_d[:, cols])
    where dW_g = sum_r dA_r (x) x_r, dW_u = sum_r dB_r (x) x_r and
    dW_d = sum_r g_r dy_r (x) h_r, restricted to the intermediate indices ``cols``.
    Cost is linear in the rows, so large experts can be sampled.
    """
    X = _f64(rows_x)
    D = _f64(rows_dy)
    g = _f64(rows_g)[:, None]
    Wg_c = _f64(Wg_e)[cols]          # [c, H]
    Wu_c = _f64(Wu_e)[cols]
    Wd_c = _f64(Wd_e)[:, cols]       # [H, c]
    A = X @ Wg_c.T
    B = X @ Wu_c.T
    h = silu(A) * B
    dh = g * (D @ Wd_c)
    dA = dh * B * dsilu(A)
    dB = dh * silu(A)
    return dA.T @ X, dB.T @ X, (g * D).T @ h


# ------------------------------------------------------------- minibatch heuristic
def min_minibatch_rows(n_cu: int, tile_m: int, tile_n: int, I: int) -> float:
    """Smallest row count that gives the up/gate grouped GEMM (output width 2I) at
    least two full waves of tiles over n_cu compute units
    [STA §Granularidade do overlap: minibatch of at least two full SM waves per
    grouped GEMM].  Rows T are cut into T/tile_m row tiles and 2I into 2I/tile_n
    column tiles; two waves need (T/tile_m)(2I/tile_n) >= 2 n_cu.
    """
    return 2.0 * n_cu * tile_m * tile_n / (2.0 * I)


def ceil_div(a: int, b: int) -> int:
    return -(-a // b)

