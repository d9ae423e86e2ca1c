"""MI355X-native deterministic MoE layer: a C-ABI library of gfx950 HIP kernels
(include/moe.h) and a thin ctypes binding with the same entry-point names."""
from . import binding  # noqa: F401
from .binding import *  # noqa: F401,F403
from .layer import LayerBuffers, run_layer  # noqa: F401
