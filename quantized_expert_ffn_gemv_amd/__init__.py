"""MI355X-native quantized routed-expert MoE layer: HIP kernels behind a C ABI
(include/moe.h, libmoe.so) and a thin ctypes binding (moe.py)."""
from . import moe  # noqa: F401
from .moe import (  # noqa: F401
    DeviceLayer,
    make_workspace,
    moe_forward_decode,
    moe_forward_prefill,
    moe_residual_add,
    moe_rmsnorm,
    moe_route,
    moe_workspace_bytes,
)
