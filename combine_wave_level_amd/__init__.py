"""MI355X-native (gfx950) share of a fine-grained expert-parallel MoE layer.

The compute path is the HIP library ``libmoe.so`` (C ABI: include/moe.h);
``combine_wave_level_amd.moe`` is its thin Python binding.
"""
from . import moe  # noqa: F401
from .moe import (  # noqa: F401
    MOE_ACT_RELU2, MOE_ACT_SWIGLU, MOE_BF16, MOE_F32, MOE_FLAG_SERIAL, MoEError, Problem, backward, combine,
    dispatch, ffn_waved, ffn_waved_fp8, forward, pack_weights, pack_weights_bwd, problem, quantize_fp8, route,
    wgrad, workspace, workspace_size,
)
