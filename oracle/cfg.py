"""Classifier-free guidance with norm rescaling (oracle, float64).

Test infrastructure: see the package docstring.

Source: NucleusMoE-Image pipeline article, section 4.3: with a guidance scale
above 1 the pipeline runs a conditional and an unconditional forward, mixes
them as uncond + scale * (cond - uncond), and then rescales each token's
mixed prediction to the norm of its conditional prediction (norms over the
last axis, the token's channels), so that a large guidance scale does not
inflate the update step.

Reading where the page is silent: a token whose mixed prediction is exactly
zero has no direction to rescale; its output is zero.
"""
from __future__ import annotations

import numpy as np


def norm_rescaled_cfg(cond, uncond, guidance_scale: float) -> np.ndarray:
    """cond, uncond: [..., C] predictions; returns the rescaled guided
    prediction of the same shape."""
    cond = np.asarray(cond, dtype=np.float64)
    uncond = np.asarray(uncond, dtype=np.float64)
    comb = uncond + float(guidance_scale) * (cond - uncond)
    cond_norm = np.sqrt(np.sum(cond * cond, axis=-1, keepdims=True))
    comb_norm = np.sqrt(np.sum(comb * comb, axis=-1, keepdims=True))
    scale = np.divide(cond_norm, comb_norm, out=np.zeros_like(comb_norm), where=comb_norm > 0)
    return comb * scale
