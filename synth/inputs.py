"""Workload shapes and seeded generators.

The shapes mirror the workloads the MoK pages measure on: Kimi-2.5-sized experts
(H=7168, I=2048) and a few thousand tokens per GPU (stamatios.com, "Cursor abre código
de megakernel MoE para GPUs NVL72", § Granularidade do overlap and § Resultados),
plus a tiny fp32 case and a mid-sized bf16 case.  Expert count and top-k for the
large shapes (E=256, k=8) are workload choices, not statements of the pages.

Value recipe (all draws are float32 from ``torch.randn`` then cast):
  x ~ N(0,1); expert and shared weights ~ N(0, 0.02); dy ~ N(0,1);
  router weight (tiny config) ~ N(0, 0.02);
  router logits (other configs) = N(0,1) noise + b_e, where b_e = -s * ln(rank_e) and
  rank_e = 1 + (a seeded random permutation of the experts), i.e. the log of a
  Zipf(s) pmf up to a constant; s = 0 gives plain N(0,1) logits.
bf16 tensors are rounded from the float32 draw with round-to-nearest-even.
"""
from __future__ import annotations

import dataclasses
import math

import torch

# tensor ids for the per-tensor generators
TID_X, TID_NOISE, TID_PERM, TID_DY, TID_WR = 1, 2, 3, 4, 5
TID_SG, TID_SU, TID_SD = 6, 7, 8
TID_WG, TID_WU, TID_WD = 11, 12, 13


@dataclasses.dataclass(frozen=True)
class Shape:
    T: int
    H: int
    I: int
    E: int
    k: int
    I_shared: int = 0
    T_minibatch: int = 0
    dtype: str = "bf16"          # "f32", "bf16" or "mxfp8"
    router: str = "logits"       # "logits": logits are an input; "gemm": logits = x W_r^T
    zipf_s: float = 0.0
    backward: bool = True
    replay: bool = False         # MXFP8: keep the last minibatch's activations only
    fused_forward: bool = False  # bf16: up/gate and down GEMMs in one launch

    @property
    def R(self) -> int:
        return self.T * self.k


CONFIGS: dict[str, Shape] = {
    # tiny fp32 layer, forward+backward, router GEMM included
    "tiny_f32": Shape(T=256, H=256, I=128, E=8, k=2, dtype="f32", router="gemm"),
    # bf16 forward, near-uniform load
    "mid_bf16_fwd": Shape(T=4096, H=2048, I=1024, E=64, k=6, backward=False),
    # bf16 forward at the pages' expert shape, Zipf(1.1) skew
    "kimi_bf16_fwd": Shape(T=2048, H=7168, I=2048, E=256, k=8, zipf_s=1.1, backward=False),
    # bf16 forward+backward with a shared expert, Zipf(1.2) skew
    "kimi_bf16_fwdbwd": Shape(T=4096, H=7168, I=2048, E=256, k=8, I_shared=2048, zipf_s=1.2),
    # the same with the forward's two expert GEMMs in one persistent launch
    "kimi_bf16_fwdbwd_fused": Shape(T=4096, H=7168, I=2048, E=256, k=8, I_shared=2048,
                                    zipf_s=1.2, fused_forward=True),
    # MXFP8 forward+backward over 4 minibatches of 2048 tokens through a ring buffer
    "kimi_mxfp8_ring": Shape(T=8192, H=7168, I=2048, E=256, k=8, I_shared=2048,
                             T_minibatch=2048, dtype="mxfp8", zipf_s=1.2),
    # the same with the activations of all but the last minibatch replayed in the
    # backward instead of kept
    "kimi_mxfp8_ring_replay": Shape(T=8192, H=7168, I=2048, E=256, k=8, I_shared=2048,
                                    T_minibatch=2048, dtype="mxfp8", zipf_s=1.2, replay=True),
    # one GPU's share of an expert-parallel layer: 4 local experts, every token on all
    # four (k = E), so each expert gets exactly 4096 rows; bf16 forward+backward
    "ep_share_bf16": Shape(T=4096, H=7168, I=2048, E=4, k=4),
}


def shape_of(name_or_shape, **overrides) -> Shape:
    s = CONFIGS[name_or_shape] if isinstance(name_or_shape, str) else name_or_shape
    return dataclasses.replace(s, **overrides) if overrides else s


def _gen(device, seed: int, tid: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed * 1_000_003 + tid)
    return g


def _randn(shape, device, seed, tid, std=1.0, dtype=torch.float32):
    t = torch.randn(shape, generator=_gen(device, seed, tid), device=device, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def zipf_bias(E: int, s: float, seed: int, device="cpu") -> torch.Tensor:
    """Per-expert additive logit bias b_e = -s ln(rank_e); rank is a seeded permutation."""
    if s == 0.0:
        return torch.zeros(E, dtype=torch.float32, device=device)
    perm = torch.randperm(E, generator=_gen("cpu", seed, TID_PERM))
    rank = (perm + 1).to(torch.float64)
    return (-s * torch.log(rank)).to(torch.float32).to(device)


def _expert_weights(E, rows, cols, device, seed, tid, dtype):
    """[E, rows, cols] N(0, 0.02) drawn one expert at a time (bounded fp32 temporaries)."""
    out = torch.empty((E, rows, cols), dtype=dtype, device=device)
    g = _gen(device, seed, tid)
    for e in range(E):
        t = torch.randn((rows, cols), generator=g, device=device, dtype=torch.float32)
        out[e].copy_(t.mul_(0.02))
    return out


def make_inputs(shape: Shape, seed: int = 0, device="cpu", with_dy: bool | None = None) -> dict:
    """All layer inputs of ``shape`` as torch tensors on ``device``.

    Keys: x, logits (router="logits") or w_router (router="gemm"), w_gate [E,I,H],
    w_up [E,I,H], w_down [E,H,I], s_gate/s_up [Is,H], s_down [H,Is] (I_shared > 0),
    dy [T,H] (backward).  Activations and weights are bf16 except for dtype "f32".
    The MXFP8 workload takes the same bf16 tensors; quantisation is part of the layer.
    """
    wdt = torch.float32 if shape.dtype == "f32" else torch.bfloat16
    T, H, I, E = shape.T, shape.H, shape.I, shape.E
    d = {}
    d["x"] = _randn((T, H), device, seed, TID_X, dtype=wdt)
    if shape.router == "gemm":
        d["w_router"] = _randn((E, H), device, seed, TID_WR, std=0.02, dtype=wdt)
    else:
        noise = _randn((T, E), device, seed, TID_NOISE)
        d["logits"] = (noise + zipf_bias(E, shape.zipf_s, seed, device)[None, :]).contiguous()
    d["w_gate"] = _expert_weights(E, I, H, device, seed, TID_WG, wdt)
    d["w_up"] = _expert_weights(E, I, H, device, seed, TID_WU, wdt)
    d["w_down"] = _expert_weights(E, H, I, device, seed, TID_WD, wdt)
    if shape.I_shared:
        Is = shape.I_shared
        d["s_gate"] = _randn((Is, H), device, seed, TID_SG, std=0.02, dtype=wdt)
        d["s_up"] = _randn((Is, H), device, seed, TID_SU, std=0.02, dtype=wdt)
        d["s_down"] = _randn((H, Is), device, seed, TID_SD, std=0.02, dtype=wdt)
    if with_dy if with_dy is not None else shape.backward:
        d["dy"] = _randn((T, H), device, seed, TID_DY, dtype=wdt)
    return d


def minibatches(shape: Shape) -> int:
    tm = shape.T_minibatch or shape.T
    return math.ceil(shape.T / tm)
