"""CPU oracle of the MoE token-routing path (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP path.
"""
from .moe_oracle import (  # noqa: F401
    SENT,
    bf16_bits_to_f32,
    combine,
    combine_epilogue,
    create_indices,
    dispatch,
    dispatch_mxfp4,
    f32_to_bf16_rne,
    mask_routing_padding,
    mxfp4_dequantize,
    mxfp4_quantize,
)
