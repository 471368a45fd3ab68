"""Masked softmax attention over the joint sequence (oracle, float64).

Test infrastructure: see the package docstring.

Sources:
  * QwenImage21Transformer2DModel API page, block-causal attention: a query
    attends a key when q_idx >= kv_idx or both lie in the same image block, so
    the joint sequence is causal while each image block stays bidirectional;
    the default processor runs one attention call per prefix segment, the flex
    processor one call with a block mask, and both give the same result;
  * same page, causal_condition and forward(kv_cache, kv_cache_mode): text and
    condition-image tokens do not depend on the timestep, so their keys and
    values are extracted once and reused ("cached") by later steps, in which
    only the target tokens are processed;
  * NucleusMoE-Image pipeline article, section 6.3: grouped-query attention by
    repeating each KV head for its group of query heads (repeat_interleave), so
    query head h reads KV head h // (H / H_kv).

  * same page, forward(encoder_hidden_states_mask): a per-sample boolean over
    the text tokens marks the valid ones; padded text positions are excluded
    from attention, i.e. as keys (``key_valid``, one flag per batch sample and
    logical key position).

Readings: the softmax scale is 1/sqrt(head_dim); "same image block" needs an
image id >= 0 on both sides (text ids are -1 and never match); in the full
mode every key is allowed.  lse is the natural-log log-sum-exp of the scaled
logits over the allowed keys.  Padding removes keys only (a padded text
position still has a query row, computed like any other); a row left with
no allowed key has output 0 and lse -inf.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import numpy as np


def allowed_matrix(q_index: np.ndarray, k_index: np.ndarray, image_ids: np.ndarray,
                   mask_mode: str) -> np.ndarray:
    """Boolean [len(q_index), len(k_index)]: may query q attend key k.
    Indices are positions in the logical joint sequence."""
    q_index = np.asarray(q_index)
    k_index = np.asarray(k_index)
    if mask_mode == "full":
        return np.ones((q_index.size, k_index.size), dtype=bool)
    if mask_mode != "block_causal":
        raise ValueError("unknown mask mode")
    ids = np.asarray(image_ids)
    qi = ids[q_index][:, None]
    ki = ids[k_index][None, :]
    causal = k_index[None, :] <= q_index[:, None]
    same_block = (qi >= 0) & (qi == ki)
    return causal | same_block


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, image_ids: np.ndarray, mask_mode: str,
              scale: Optional[float] = None, q_offset: int = 0, rows: Optional[Sequence[int]] = None,
              chunk: int = 2048, key_valid: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """O = softmax(scale * Q K^T + M) V per (batch, head), GQA by head groups.

    q: [B, Sq, H, D]; k, v: [B, Sk, Hk, D] (keys cover the logical positions
    0..Sk-1).  Query row i sits at logical position q_offset + i (q_offset is
    the cached-prefix length).  rows: which query rows to compute (default all).
    key_valid: optional bool [B, Sk]; False keys are excluded for that sample.
    Returns (o [B, len(rows), H, D], lse [B, H, len(rows)]).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Sq, H, D = q.shape
    Sk, Hk = k.shape[1], k.shape[2]
    if H % Hk:
        raise ValueError("heads must be a multiple of kv_heads")
    group = H // Hk
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    rows = np.arange(Sq) if rows is None else np.asarray(rows)
    out = np.zeros((B, rows.size, H, v.shape[3]))
    lse = np.zeros((B, H, rows.size))
    k_index = np.arange(Sk)
    for c0 in range(0, rows.size, chunk):
        r = rows[c0:c0 + chunk]
        allow_all = allowed_matrix(r + q_offset, k_index, image_ids, mask_mode)
        for b in range(B):
            allow = allow_all if key_valid is None else allow_all & np.asarray(key_valid[b], dtype=bool)[None, :]
            live = allow.any(axis=1)  # rows with at least one allowed key
            for h in range(H):
                g = h // group
                logits = scale * (q[b, r, h, :] @ k[b, :, g, :].T)
                logits = np.where(allow, logits, -np.inf)
                m = np.where(live, logits.max(axis=1), 0.0)[:, None]
                p = np.exp(logits - m)
                denom = p.sum(axis=1, keepdims=True)
                safe = np.where(live[:, None], denom, 1.0)
                out[b, c0:c0 + r.size, h, :] = np.where(live[:, None], (p @ v[b, :, g, :]) / safe, 0.0)
                lse[b, h, c0:c0 + r.size] = np.where(live, (m + np.log(safe))[:, 0], -np.inf)
    return out, lse


def segments(image_ids: np.ndarray) -> list:
    """Split the sequence into maximal text runs and single image blocks:
    [(start, end, is_image)]."""
    ids = list(np.asarray(image_ids))
    segs = []
    start = 0
    for s in range(1, len(ids) + 1):
        if s == len(ids) or ids[s] != ids[start]:
            segs.append((start, s, ids[start] >= 0))
            start = s
    return segs


def attention_multipass(q: np.ndarray, k: np.ndarray, v: np.ndarray, image_ids: np.ndarray,
                        scale: Optional[float] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Block-causal attention as one pass per prefix segment: the queries of
    segment [a, c) attend keys [0, c); keys before a are all visible, keys
    inside the segment causally for a text run and all of them for an image
    block.  Written without the per-pair predicate, as a second, independent
    construction of the mask."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, S, H, D = q.shape
    group = H // k.shape[2]
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = np.zeros_like(q)
    lse = np.zeros((B, H, S))
    for (a, c, is_image) in segments(image_ids):
        n = c - a
        inner = np.ones((n, n), dtype=bool) if is_image else np.tril(np.ones((n, n), dtype=bool))
        allow = np.concatenate([np.ones((n, a), dtype=bool), inner], axis=1)  # [n, c]
        for b in range(B):
            for h in range(H):
                g = h // group
                logits = scale * (q[b, a:c, h, :] @ k[b, :c, g, :].T)
                logits = np.where(allow, logits, -np.inf)
                m = logits.max(axis=1, keepdims=True)
                p = np.exp(logits - m)
                denom = p.sum(axis=1, keepdims=True)
                out[b, a:c, h, :] = (p @ v[b, :c, g, :]) / denom
                lse[b, h, a:c] = (m + np.log(denom))[:, 0]
    return out, lse


def attention_bruteforce(q, k, v, image_ids, mask_mode: str, scale: Optional[float] = None,
                         q_offset: int = 0, key_valid=None):
    """Quadruple Python loops with math.exp; tiny inputs only.  Returns nested
    lists o[b][i][h][d] and lse[b][h][i]."""
    B, Sq, H, D = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Sk, Hk = len(k[0]), len(k[0][0])
    group = H // Hk
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    o = [[[[0.0] * D for _ in range(H)] for _ in range(Sq)] for _ in range(B)]
    lse = [[[0.0] * Sq for _ in range(H)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            g = h // group
            for i in range(Sq):
                qi = q_offset + i
                logits = []
                for j in range(Sk):
                    if mask_mode == "full":
                        ok = True
                    else:
                        same = image_ids[qi] >= 0 and image_ids[qi] == image_ids[j]
                        ok = j <= qi or same
                    if key_valid is not None and not key_valid[b][j]:
                        ok = False
                    if ok:
                        dot = 0.0
                        for d in range(D):
                            dot += float(q[b][i][h][d]) * float(k[b][j][g][d])
                        logits.append((j, scale * dot))
                if not logits:  # every allowed key is padding
                    lse[b][h][i] = -math.inf
                    continue
                m = max(val for _, val in logits)
                weights = [(j, math.exp(val - m)) for j, val in logits]
                total = sum(wt for _, wt in weights)
                for d in range(D):
                    acc = 0.0
                    for j, wt in weights:
                        acc += wt * float(v[b][j][g][d])
                    o[b][i][h][d] = acc / total
                lse[b][h][i] = m + math.log(total)
    return o, lse
