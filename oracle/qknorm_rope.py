"""Per-head RMSNorm of Q/K and multi-axis rotary embedding (oracle, float64).

Test infrastructure: see the package docstring.

Sources:
  * NucleusMoE-Image pipeline article, section 6.3: the attention processor
    applies an optional RMSNorm to Q and K (qk_norm = rms_norm), then the
    rotary embedding built over the (frame, height, width) axes with
    axes_dims_rope (16, 56, 56); the height/width axes use a centred layout;
  * QwenImage21Transformer2DModel API page, constructor: axes_dims_rope are the
    rotary dims of the frame, height and width axes; eps 1e-6;
  * Lumina-Next DiT article, configuration table: norm_eps 1e-5, qk_norm, and
    the 2D RoPE needs head_dim divisible by 4 (each of the two axes takes
    head_dim / 2 channels, rotated in pairs); section 4: the rotary table is
    complex-valued (a (384, 384, 4) table for head_dim 8, i.e. one complex
    factor per channel pair).

Readings where the pages are silent: the norm is (mean over the head's D
channels of x^2 + eps)^(-1/2) times a per-channel weight shared by all heads;
the rotary base is 10000 on every axis; channel pairs are adjacent (2j, 2j+1)
-- the complex-multiplication form the complex table implies; each axis has
its own frequency ladder theta^(-2j/d_a) over its d_a channels; axes occupy
the head's channels in the order the axes are listed.
"""
from __future__ import annotations

from typing import Sequence

import numpy as np


def rms_norm(x: np.ndarray, weight: np.ndarray, eps: float) -> np.ndarray:
    """y = x / sqrt(mean(x^2) + eps) * weight over the last axis (one head)."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(weight, dtype=np.float64)


def rope(x: np.ndarray, pos: np.ndarray, axes: Sequence[int], theta: float = 10000.0) -> np.ndarray:
    """Rotate channel pairs of x ([..., S, H, D]) by per-token, per-axis phases.

    pos is [S, n] integer positions (n >= len(axes)); axis a owns channels
    [o_a, o_a + d_a) with o_a the sum of the earlier axes' dims; inside it,
    pair j = (o_a + 2j, o_a + 2j + 1) turns by pos[s, a] * theta^(-2j/d_a).
    """
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    if sum(axes) != D or any(d % 2 for d in axes):
        raise ValueError("rotary axes must be even and sum to head_dim")
    y = x.copy()
    pos = np.asarray(pos, dtype=np.float64)
    offset = 0
    for a, d_a in enumerate(axes):
        for j in range(d_a // 2):
            omega = theta ** (-2.0 * j / d_a)
            phase = pos[:, a] * omega                    # [S]
            c = np.cos(phase)[:, None]                   # broadcast over heads
            s = np.sin(phase)[:, None]
            i0, i1 = offset + 2 * j, offset + 2 * j + 1
            x0, x1 = x[..., i0], x[..., i1]
            y[..., i0] = x0 * c - x1 * s
            y[..., i1] = x0 * s + x1 * c
        offset += d_a
    return y


def qknorm_rope(x: np.ndarray, weight: np.ndarray, eps: float, pos: np.ndarray,
                axes: Sequence[int], theta: float = 10000.0) -> np.ndarray:
    """RMSNorm first, then the rotation (the order of the attention processor)."""
    return rope(rms_norm(x, weight, eps), pos, axes, theta)
