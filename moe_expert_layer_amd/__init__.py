"""MI355X (gfx950) MoE expert layer: HIP kernels behind a C ABI, with a thin ctypes binding.

The layer runs route -> permute -> FC1 + (OAI-)SwiGLU + 1x128 requant -> FC2 -> combine
on one GPU's share of the experts.  ``binding`` holds the entry points (same names as
the C ABI); ``synth`` makes seeded synthetic inputs; ``build`` compiles the library.
"""
from .binding import (  # noqa: F401
    MoeError, MoeLayerDesc, alloc_workspace, desc_from_workload, lib, make_desc, moe_grouped_fc1_swiglu,
    moe_grouped_fc2_combine, moe_layer, moe_route_permute, moe_workspace_size,
)
