"""One sparse MoE layer on MI355X (gfx950): router GEMV, exact top-k with
softmax gates, 4-bit/bf16/fp32 SwiGLU expert GEMVs, grouped multi-token path
and weighted combine, all as HIP kernels behind the C ABI of include/moe.h.

The Python side only marshals arguments (``binding.Layer``).
"""
from .binding import (  # noqa: F401
    EXPORTS, LIB_PATH, MOE_BF16, MOE_F32, MOE_LAYER_FORCE_EXACT_REFINE, MOE_LAYER_SCREEN_OFF, MOE_LAYER_SCREEN_ON,
    MOE_LAYER_WINDOW_SCREEN_OFF, MOE_Q4B32,
    MOE_ROUTE_GIVEN, MOE_ROUTE_INTERNAL, MOE_ROUTER_EH, MOE_ROUTER_HE, Decoder, Layer, LayerDesc,
    MoeError, load_library,
)
