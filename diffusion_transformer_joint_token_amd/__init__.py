"""Joint text+image DiT attention step for MI355X (gfx950).

Thin bindings of the C ABI in include/dit_attn.h:
``build_token_metadata`` -> ``qknorm_rope`` -> ``forward`` / ``forward_cached``,
with ``build_key_valid`` and the ``key_valid`` argument of the two attention
calls for padded text tokens, and ``cfg_norm_rescale`` for the guidance step
that combines a denoising step's two predictions.  Importing the package loads the in-tree
``libdit_attn.so`` and fails if it is missing; there is no other
implementation behind these names.
"""
from .api import (LN2, LOG2E, DitAttnError, KeyValid, TokenMeta, build_key_valid,  # noqa: F401
                  build_token_metadata, cfg_norm_rescale, dit_attn_build_key_valid, dit_attn_cfg_norm_rescale, dit_attn_build_token_metadata, dit_attn_forward,
                  dit_attn_forward_cached, dit_attn_forward_cached_padded, dit_attn_forward_cached_qnorm,
                  dit_attn_forward_padded,
                  dit_attn_qknorm_rope, dit_attn_qknorm_rope_ex, dit_attn_time_aware_rope_factors, forward,
                  forward_cached, forward_cached_qnorm, prescaled_q_factor, qknorm_rope, time_aware_rope_factors)
from ._lib import LIB_PATH  # noqa: F401
