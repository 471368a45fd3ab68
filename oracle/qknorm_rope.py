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
    factor per channel pair);
  * Lumina-Next DiT article, section 3: with qk_norm on, the self-attention
    normalises Q and K with a LayerNorm across heads; section 4: the pipeline
    rebuilds the 2D rotary table at every denoising step from a linear factor
    and an NTK factor, one of them set to scaling_factor and the other to 1
    depending on whether the (reversed, 0 = noise) timestep has passed
    scaling_watershed.

Readings where the pages are silent: the norm is (mean over the head's D
channels of x^2 + eps)^(-1/2) times a per-channel weight shared by all heads;
the rotary base is 10000 on every axis; channel pairs are adjacent (2j, 2j+1)
-- the complex-multiplication form the complex table implies; each axis has
its own frequency ladder theta^(-2j/d_a) over its d_a channels; axes occupy
the head's channels in the order the axes are listed.  LayerNorm across heads
normalises each token's Q (or K) over all heads' channels together (mean
removed, biased variance, eps inside the square root) with a per-channel
weight and bias over those heads x head_dim channels.  The rotary factors
follow their usual definitions, which the article names but does not print:
the linear factor divides the positions (position interpolation), the NTK
factor multiplies the rotary base.  The switch's comparison is lost from the
page's text; the reading is that steps before the watershed (t below it) take
the linear factor.
"""
from __future__ import annotations

from typing import Sequence

import numpy as np


def rms_norm(x: np.ndarray, weight: np.ndarray, eps: float) -> np.ndarray:
    """y = x / sqrt(mean(x^2) + eps) * weight over the last axis (one head)."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(weight, dtype=np.float64)


def layer_norm_across_heads(x: np.ndarray, weight=None, bias=None, eps: float = 1e-5) -> np.ndarray:
    """x [..., H, D]: per token, y = (x - mean) / sqrt(var + eps) * weight + bias
    with mean and (biased) variance over all H * D channels; weight and bias
    are [H * D] (None: 1 and 0)."""
    x = np.asarray(x, dtype=np.float64)
    shape = x.shape
    flat = x.reshape(shape[:-2] + (shape[-2] * shape[-1],))
    mean = flat.mean(axis=-1, keepdims=True)
    cen = flat - mean
    var = (cen * cen).mean(axis=-1, keepdims=True)
    y = cen / np.sqrt(var + eps)
    if weight is not None:
        y = y * np.asarray(weight, dtype=np.float64)
    if bias is not None:
        y = y + np.asarray(bias, dtype=np.float64)
    return y.reshape(shape)


def time_aware_rope_factors(t: float, watershed: float, scaling_factor: float):
    """(linear_factor, ntk_factor) of the denoising step at reversed timestep t
    (0 = noise, 1 = image): before the watershed the linear factor carries the
    scaling, from it on the NTK factor does."""
    if t < watershed:
        return float(scaling_factor), 1.0
    return 1.0, float(scaling_factor)


def rope(x: np.ndarray, pos: np.ndarray, axes: Sequence[int], theta: float = 10000.0,
         linear_factor: float = 1.0, ntk_factor: float = 1.0) -> np.ndarray:
    """Rotate channel pairs of x ([..., S, H, D]) by per-token, per-axis phases.

    pos is [S, n] positions (n >= len(axes)); axis a owns channels
    [o_a, o_a + d_a) with o_a the sum of the earlier axes' dims; inside it,
    pair j = (o_a + 2j, o_a + 2j + 1) turns by
    (pos[s, a] / linear_factor) * (theta * ntk_factor)^(-2j/d_a).
    """
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    if sum(axes) != D or any(d % 2 for d in axes):
        raise ValueError("rotary axes must be even and sum to head_dim")
    y = x.copy()
    pos = np.asarray(pos, dtype=np.float64) / float(linear_factor)
    base = float(theta) * float(ntk_factor)
    offset = 0
    for a, d_a in enumerate(axes):
        for j in range(d_a // 2):
            omega = base ** (-2.0 * j / d_a)
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
                axes: Sequence[int], theta: float = 10000.0, norm: str = "rms_per_head", bias=None,
                linear_factor: float = 1.0, ntk_factor: float = 1.0) -> np.ndarray:
    """The norm first, then the rotation (the order of the attention processor).
    norm: "rms_per_head" (weight [D]) or "layer_across_heads" (weight, bias
    [H * D])."""
    if norm == "rms_per_head":
        y = rms_norm(x, weight, eps)
    elif norm == "layer_across_heads":
        y = layer_norm_across_heads(x, weight, bias, eps)
    else:
        raise ValueError("unknown norm")
    return rope(y, pos, axes, theta, linear_factor, ntk_factor)
