"""The whole attention step on one workload, composed from the oracle parts.

Test infrastructure: see the package docstring.

Order of the step (NucleusMoE-Image pipeline article, section 6.3;
QwenImage21Transformer2DModel API page): token metadata from image_pad_mask and
img_shapes, then RMSNorm + rotary embedding of Q and K (V untouched), then
masked attention.

The two cache modes of the QwenImage21Transformer2DModel API page (``forward``'s
``kv_cache_mode``):

* "extract": the first denoising step runs over the whole joint sequence and
  keeps the keys and values of the timestep-independent prefix (the text and
  condition tokens before the target block, which the ``causal_condition``
  note makes independent of the target): the cache is rows [0, P) of that
  step's normalised and rotated K' and of its raw V.
* "cached": later steps run only the target tokens, logical positions
  [P, P + S_new): their Q and K are normalised and rotated at those positions
  and attend to the cached keys followed by their own.

``step`` computes either: with ``prefix_len = 0`` the full step, with
``prefix_len = P`` the cached step (then ``vals`` holds the new tokens' q, k,
v and the cache as k_cache, v_cache).
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence

import numpy as np

from . import attention as att
from . import qknorm_rope as qr


def step(vals: Dict[str, np.ndarray], md: Dict[str, np.ndarray], *, axes: Sequence[int], eps: float,
         mask_mode: str, prefix_len: int = 0, theta: float = 10000.0,
         rows: Optional[Sequence[int]] = None, scale: Optional[float] = None,
         key_valid: Optional[np.ndarray] = None) -> Dict[str, np.ndarray]:
    """vals: float64 arrays q, k, v (the step's query tokens, BSHD), wq, wk [D],
    and for a cached prefix k_cache (post norm and rotation) and v_cache (raw).
    md: the oracle's token metadata over the logical sequence (prefix + new).
    key_valid: optional per-sample key flags [B, P + S_new].  Returns q_prime
    and k_prime (the new tokens), and o and lse for the requested query rows
    (rows index the new tokens; all of them by default)."""
    P = prefix_len
    # The new tokens sit at logical positions P .. P + S_new - 1.
    pos_new = md["pos_ids"][P:]
    q_prime = qr.qknorm_rope(vals["q"], vals["wq"], eps, pos_new, axes, theta)
    k_prime = qr.qknorm_rope(vals["k"], vals["wk"], eps, pos_new, axes, theta)
    if P > 0:
        k_all = np.concatenate([vals["k_cache"], k_prime], axis=1)
        v_all = np.concatenate([vals["v_cache"], vals["v"]], axis=1)
    else:
        k_all, v_all = k_prime, vals["v"]
    o, lse = att.attention(q_prime, k_all, v_all, md["image_ids"], mask_mode, scale=scale, q_offset=P, rows=rows,
                           key_valid=key_valid)
    return {"q_prime": q_prime, "k_prime": k_prime, "o": o, "lse": lse}


def extract_cache(full: Dict[str, np.ndarray], v: np.ndarray, prefix_len: int) -> Dict[str, np.ndarray]:
    """The "extract" mode's cache from a full step's result: rows [0, P) of its
    K' and of the raw V it attended to."""
    P = prefix_len
    return {"k_cache": full["k_prime"][:, :P], "v_cache": np.asarray(v)[:, :P]}
