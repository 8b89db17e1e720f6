"""MX-quantised sparse MoE expert block for AMD Instinct MI355X (gfx950).

The block runs in the HIP library libmxmoe.so (C ABI in include/mxmoe.h); `binding` is its thin
ctypes wrapper with the same entry-point names, `weights` prepares expert weights with the
library's own quantise and prepack kernels, and `build` compiles the library."""
from . import binding  # noqa: F401
from .binding import (  # noqa: F401
    Shape, Options, MxMoeError, lib, mxmoe_status_string, mxmoe_route, mxmoe_align,
    mxmoe_align_capacity, mxmoe_align_workspace_bytes, mxmoe_quantize, mxmoe_prepacked_bytes,
    mxmoe_prepack, mxmoe_workspace_bytes, mxmoe_workspace_view, mxmoe_forward,
)
