"""Plain float64 CPU oracle for the Wan DiT attention sublayer.

TEST INFRASTRUCTURE ONLY. Nothing in the product path may import, call or link
this package: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it. It shares no code, tables or
constants with the HIP library and imports nothing from it.

Everything here is written from the pages' statement of the method (see the
docstring of each function for the passage it follows) in the simplest form
that can be checked by eye: float64 NumPy, library matmul/exp/sin/cos as steps,
no blocking, fusion or reordering.
"""

from .wan_oracle import (  # noqa: F401
    bf16_bits_to_f64,
    f64_to_bf16_bits,
    bf16_round,
    layer_norm,
    adaln_modulate_gate,
    rms_norm,
    rope3d_pair_split,
    rope3d_token_positions,
    rope3d_angles,
    rope3d_rotate,
    qk_norm_rope3d,
    attention,
    self_attention,
    cross_attention,
    chunk_causal_visible,
    chunk_causal_attention,
    linear,
    e4m3_bits_to_f64,
    f64_to_e4m3_bits,
    quantize_int8_blocks,
    quantize_v_mxfp8,
    attention_8bit,
)
