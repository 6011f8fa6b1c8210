"""float64 CPU oracle of the MoE layer share (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP
library and never imports it.
"""
from .moe_oracle import (  # noqa: F401
    decode_bf16,
    router_logits,
    route,
    dispatch,
    expert_ffn,
    combine,
    forward,
    forward_tokens,
    wgrad,
    backward,
    backward_tokens,
    e4m3_decode,
    e4m3_encode,
    quantize_fp8_per_token,
)
