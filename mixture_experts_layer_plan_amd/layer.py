"""Device buffers for one layer shape and the call sequence of one training step.

``LayerBuffers`` allocates (through torch, on the current device) every output,
the plan, the saved activations and the workspaces that the C-ABI asks for.
``run_layer`` enqueues route -> plan -> [MX weight quantisation ->] forward [-> backward ->
router backward]
on the current stream.  Both only move pointers; the arithmetic is in libmoe.so.
"""
from __future__ import annotations

import torch

from . import binding as B


class LayerBuffers:
    def __init__(self, T, H, I, E, k, I_shared=0, dtype="bf16", backward=True,
                 router_gemm=False, device="cuda", T_minibatch=0, replay=False,
                 fused_forward=False):
        if dtype not in ("bf16", "f32", "mxfp8"):
            raise ValueError(f"unsupported dtype {dtype}")
        if router_gemm and dtype != "f32":
            # the router GEMM calls take fp32 x and accumulate into an fp32 dx
            raise ValueError("router_gemm needs dtype 'f32'")
        self.dtype = dtype
        self.dt = B.DTYPES[dtype]
        flags = (B.MOE_REPLAY if replay else 0) | (B.MOE_FUSED_FORWARD if fused_forward else 0)
        self.s = B.shape(T, H, I, E, k, I_shared, T_minibatch, flags)
        tdt = torch.float32 if dtype == "f32" else torch.bfloat16
        dev = torch.device(device)
        u8 = dict(dtype=torch.uint8, device=dev)
        self.tdt = tdt
        self.topk_idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        self.topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
        self.plan = torch.empty(B.moe_plan_bytes(self.s), **u8)
        self.saved = torch.empty(B.moe_saved_bytes(self.s, self.dt), **u8)
        self.ws_fwd = torch.empty(B.moe_workspace_bytes(self.s, self.dt, False), **u8)
        self.wq = torch.empty(B.moe_mx_weights_bytes(self.s), **u8) if dtype == "mxfp8" else None
        self.y = torch.empty((T, H), dtype=tdt, device=dev)
        self.logits = torch.empty((T, E), dtype=torch.float32, device=dev) if router_gemm else None
        self.backward = backward
        if backward:
            self.ws_bwd = torch.empty(B.moe_workspace_bytes(self.s, self.dt, True), **u8)
            self.dx = torch.empty((T, H), dtype=tdt, device=dev)
            self.dw_gate = torch.empty((E, I, H), dtype=tdt, device=dev)
            self.dw_up = torch.empty((E, I, H), dtype=tdt, device=dev)
            self.dw_down = torch.empty((E, H, I), dtype=tdt, device=dev)
            if I_shared:
                self.ds_gate = torch.empty((I_shared, H), dtype=tdt, device=dev)
                self.ds_up = torch.empty((I_shared, H), dtype=tdt, device=dev)
                self.ds_down = torch.empty((H, I_shared), dtype=tdt, device=dev)
            else:
                self.ds_gate = self.ds_up = self.ds_down = None
            self.d_topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
            self.d_logits = torch.empty((T, E), dtype=torch.float32, device=dev)
            self.dw_router = torch.empty((E, H), dtype=torch.float32, device=dev) if router_gemm else None

    def plan_views(self) -> dict:
        return B.plan_views(self.s, self.plan)


def quantize_weights(b: LayerBuffers, inp: dict, stream=None):
    """MXFP8 weights in the six orientations the MX GEMMs read (once per weight update)."""
    B.moe_quantize_weights_mxfp8(b.s, inp["w_gate"], inp["w_up"], inp["w_down"], b.wq, stream)


def run_forward(b: LayerBuffers, inp: dict, stream=None, quantize=True):
    """route -> plan -> forward; for MXFP8 also the weight quantisation unless
    ``quantize`` is False (weights already quantised into ``b.wq``)."""
    s = b.s
    if "w_router" in inp:
        if b.logits is None:
            raise ValueError("inputs carry w_router but the buffers have no router GEMM")
        B.moe_router_logits_f32(s, inp["x"], inp["w_router"], b.logits, stream)
        logits = b.logits
    else:
        logits = inp["logits"]
    B.moe_route(s, logits, b.topk_idx, b.topk_w, stream)
    B.moe_plan(s, b.topk_idx, b.plan, stream)
    if b.dtype == "mxfp8":
        if quantize:
            quantize_weights(b, inp, stream)
        B.moe_forward_mxfp8(s, b.plan, inp["x"], b.topk_w, b.wq, inp.get("s_gate"),
                            inp.get("s_up"), inp.get("s_down"), b.y, b.saved, b.ws_fwd, stream)
        return
    fwd = B.moe_forward_bf16 if b.dtype == "bf16" else B.moe_forward_f32
    fwd(s, b.plan, inp["x"], b.topk_w, inp["w_gate"], inp["w_up"], inp["w_down"],
        inp.get("s_gate"), inp.get("s_up"), inp.get("s_down"), b.y, b.saved, b.ws_fwd, stream)


def run_backward(b: LayerBuffers, inp: dict, stream=None):
    s = b.s
    if b.dtype == "mxfp8":
        B.moe_backward_mxfp8(s, b.plan, inp["x"], b.topk_w, b.wq, inp.get("s_gate"),
                             inp.get("s_up"), inp.get("s_down"), b.saved, inp["dy"], b.dx,
                             b.dw_gate, b.dw_up, b.dw_down, b.ds_gate, b.ds_up, b.ds_down,
                             b.d_topk_w, b.ws_bwd, stream)
    else:
        bwd = B.moe_backward_bf16 if b.dtype == "bf16" else B.moe_backward_f32
        bwd(s, b.plan, inp["x"], b.topk_w, inp["w_gate"], inp["w_up"], inp["w_down"],
            inp.get("s_gate"), inp.get("s_up"), inp.get("s_down"), b.saved, inp["dy"], b.dx,
            b.dw_gate, b.dw_up, b.dw_down, b.ds_gate, b.ds_up, b.ds_down, b.d_topk_w, b.ws_bwd,
            stream)
    B.moe_route_backward(s, b.topk_idx, b.topk_w, b.d_topk_w, b.d_logits, stream)
    if "w_router" in inp:
        B.moe_router_backward_f32(s, inp["x"], inp["w_router"], b.d_logits, b.dw_router, b.dx,
                                  stream)


def run_layer(b: LayerBuffers, inp: dict, backward: bool = True, stream=None, quantize=True):
    run_forward(b, inp, stream, quantize)
    if backward:
        run_backward(b, inp, stream)
