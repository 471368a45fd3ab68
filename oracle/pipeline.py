"""The whole attention step on one workload, composed from the oracle parts.

Test infrastructure: see the package docstring.

Order of the step (NucleusMoE-Image pipeline article, section 6.3;
QwenImage21Transformer2DModel API page): token metadata from image_pad_mask and
img_shapes, then RMSNorm + rotary embedding of Q and K (V untouched), then
masked attention.  In the cached-prefix case (kv_cache_mode "cached") the
prefix keys arrive already normalised and rotated and the prefix values raw;
only the new tokens are normalised, rotated and queried, against the cached
keys followed by their own.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

from . import attention as att
from . import metadata as meta
from . import qknorm_rope as qr


def token_metadata(image_pad_mask, img_shapes, pos_mode: str) -> Dict[str, np.ndarray]:
    return meta.build_token_metadata(image_pad_mask, img_shapes, pos_mode)


def step(vals: Dict[str, np.ndarray], md: Dict[str, np.ndarray], *, axes: Sequence[int], eps: float,
         mask_mode: str, prefix_len: int = 0, theta: float = 10000.0,
         rows: Optional[Sequence[int]] = None, scale: Optional[float] = None) -> Dict[str, np.ndarray]:
    """vals: float64 arrays q, k, v (new tokens, BSHD), wq, wk [D], and for a
    cached prefix k_cache, v_cache.  md: the oracle's token metadata over the
    logical sequence.  Returns q_prime, k_prime (new tokens), o and lse for the
    requested query rows (rows index the new tokens)."""
    P = prefix_len
    pos_new = md["pos_ids"][P:]
    q_prime = qr.qknorm_rope(vals["q"], vals["wq"], eps, pos_new, axes, theta)
    k_prime = qr.qknorm_rope(vals["k"], vals["wk"], eps, pos_new, axes, theta)
    if P > 0:
        k_all = np.concatenate([vals["k_cache"], k_prime], axis=1)
        v_all = np.concatenate([vals["v_cache"], vals["v"]], axis=1)
    else:
        k_all, v_all = k_prime, vals["v"]
    o, lse = att.attention(q_prime, k_all, v_all, md["image_ids"], mask_mode, scale=scale,
                           q_offset=P, rows=rows)
    return {"q_prime": q_prime, "k_prime": k_prime, "o": o, "lse": lse}
