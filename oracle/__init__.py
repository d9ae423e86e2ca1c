"""Plain, slow, obviously-correct CPU oracle of the deterministic MoE layer.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call anything in this package.
The product path (``include/moe.h`` + ``mixture_experts_layer_plan_amd``) never
imports it, links it or falls back to it, and this package imports nothing from
the product path: the two share no code.

Everything here is numpy float64 on the exact input values (bf16 and fp32 inputs
convert to float64 without rounding).  No intermediate is rounded to bf16.  Each
function cites the passage of the pages it follows; where the pages leave a step
open the reading taken is stated at the function.

Pins (``tests/test_oracle_*.py``, run with ``-m "not gpu"``) tie every function to
something other than itself: brute force over all k-subsets for top-k, exhaustive
enumeration of routings and a library stable sort for the plan, identity and
scaled-identity experts for dispatch/combine, per-token direct evaluation and the
E=1 dense-SwiGLU special case for the layer, central finite differences and
torch.autograd for the backward, hand examples and torch's float8_e4m3fn cast for
the MX quantiser.
"""
from .moe import (  # noqa: F401
    route, router_logits, build_plan, tile_list, dispatch, combine, expert_ffn,
    dense_swiglu, layer_forward, layer_backward, route_backward,
    token_forward, token_backward, expert_weight_grad_slices, silu, dsilu,
    min_minibatch_rows,
)
from .mx import (  # noqa: F401
    e4m3_encode, e4m3_decode, mx_quantize, mx_dequantize, mx_roundtrip,
)
