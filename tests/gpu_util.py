"""Shared helpers of the GPU parity tests (inputs on the host, copies to the device)."""
import hashlib
import sys

import numpy as np
import torch


def say(*a):
    """Print and flush before a GPU step so a failing run names its case."""
    print(*a, flush=True)
    sys.stdout.flush()


def dev(t):
    return t.to("cuda") if t is not None else None


def to_dev(inp: dict) -> dict:
    return {k: dev(v) for k, v in inp.items()}


def np_(t):
    return t.detach().cpu().numpy()


def digest(*tensors) -> str:
    h = hashlib.sha256()
    for t in tensors:
        if t is None:
            continue
        h.update(t.detach().contiguous().view(torch.uint8).cpu().numpy().tobytes())
    return h.hexdigest()


def shared_of(inp):
    return (inp["s_gate"], inp["s_up"], inp["s_down"]) if "s_gate" in inp else None
