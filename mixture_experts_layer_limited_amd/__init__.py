"""MI355X (gfx950) mixture-of-experts layer: Python binding of libmoe_gfx950.

The computation lives in the HIP kernels of csrc/ behind the C ABI declared in
include/moe.h; this package only marshals arguments (_abi) and sequences the
calls of one layer (layer.MoELayer).
"""
from ._abi import *  # noqa: F401,F403
from ._abi import MoEError, lib, make_cfg, moe_cfg  # noqa: F401
from .layer import LayerShape, MoELayer  # noqa: F401
