"""wanattn: the attention sublayer of a Wan2.1/2.2 DiT block on MI355X (gfx950).

The compute lives in the HIP library ``libwanattn.so`` (C ABI declared in
``include/wanattn.h``); this package is its thin torch binding plus the
synthetic-workload definitions. Importing it does not load the library; the
first call does, and fails loudly if it has not been built.
"""

from ._lib import (  # noqa: F401
    WAN_NORM,
    WAN_NORM_PER_HEAD,
    WAN_ROPE,
    WanError,
    lib,
)
from .ops import (  # noqa: F401
    adaln_modulate_gate,
    chunk_causal_attn_fwd,
    cross_attn_fwd,
    linear_fwd,
    qk_norm_rope3d,
    quantize_qkv_8bit,
    self_attn_fwd,
    self_attn_fwd_8bit,
)

__version__ = "0.1.0"
