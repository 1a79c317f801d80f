"""MI355X (gfx950) MoE expert layer: HIP kernels behind a C ABI (libmoe.so,
include/moe.h) and a thin ctypes binding with the same entry-point names."""
from . import lib  # noqa: F401
from .lib import (  # noqa: F401
    EXPORTS, MoeAux, MoeDesc, MoeError, MoeWeights, desc_from_config, load_library, moe_combine,
    moe_grouped_ffn, moe_layer, moe_pack_weights, moe_packed_bytes, moe_permute, moe_route_topk,
    moe_status_str, moe_workspace_bytes,
)
