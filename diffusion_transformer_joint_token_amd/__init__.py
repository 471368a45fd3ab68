"""Joint text+image DiT attention step for MI355X (gfx950).

Four entry points, each a thin binding of the C ABI in include/dit_attn.h:
``build_token_metadata`` -> ``qknorm_rope`` -> ``forward`` / ``forward_cached``.
Importing the package loads the in-tree ``libdit_attn.so`` and fails if it is
missing; there is no other implementation behind these names.
"""
from .api import (LN2, LOG2E, DitAttnError, TokenMeta, build_token_metadata,  # noqa: F401
                  dit_attn_build_token_metadata, dit_attn_forward, dit_attn_forward_cached, dit_attn_qknorm_rope,
                  forward, forward_cached, prescaled_q_factor, qknorm_rope)
from ._lib import LIB_PATH  # noqa: F401
