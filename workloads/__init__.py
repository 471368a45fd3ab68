"""Seeded synthetic workloads for the joint text+image DiT attention step.

This module is the one piece shared by the CPU oracle and the HIP path: it
holds the five workload descriptions and the seeded random inputs drawn for
them.  It contains none of the method's arithmetic (no normalisation, no
rotary phases, no masking, no softmax); it only lays out which tokens are text
and which are image, draws N(0, 1) numbers and rounds them to bf16.

Shapes follow the pages' 1024^2-class workloads:
  * 1024 px / VAE factor 8 / patch 2 gives a 64x64 latent token grid and the
    text stream defaults to 1024 tokens (NucleusMoE-Image pipeline article,
    section 1 and section 6);
  * Lumina-Next: hidden 2304 over 32 heads gives head_dim 72, GQA through
    num_kv_heads, eps 1e-5 (Lumina-Next DiT article, configuration table);
  * Qwen-Image 2.1: 32 heads x 128, rotary axes (16, 56, 56), eps 1e-6, text
    followed by the target image, condition images in the text stream
    (QwenImage21Transformer2DModel API page, constructor and class notes).

No public dataset or benchmark is involved; every tensor is synthetic.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Sequence, Tuple

import numpy as np

__all__ = ["Workload", "WORKLOADS", "VARIANTS", "CfgWorkload", "CFG_WORKLOADS", "draw_cfg", "get", "sequence_inputs", "draw", "bf16_round_bits",
           "bf16_bits_to_f64", "small_workload", "n_text_tokens", "text_mask"]


@dataclass(frozen=True)
class Workload:
    """One synthetic attention-step configuration.

    layout: the whole logical joint sequence in order, as segments
      ("T", n) for n text tokens or ("I", f, h, w) for one image block of
      f*h*w latent tokens.  The last image block is the target image.
    prefix_len: for the cached-prefix case, the number of leading tokens whose
      K/V come from the cache; queries exist only for the remaining tokens.
    """
    name: str
    batch: int
    heads: int
    kv_heads: int
    head_dim: int
    layout: Tuple[tuple, ...]
    axes: Tuple[int, ...]
    pos_mode: str            # "centered_fhw" | "grid_hw"
    mask_mode: str           # "full" | "block_causal"
    eps: float
    dtype: str               # "bf16" | "f32"
    unit_weights: bool
    seed: int
    prefix_len: int = 0
    rope_theta: float = 10000.0
    description: str = ""
    qk_norm: str = "rms_per_head"  # or "layer_across_heads" (weights and biases over heads x head_dim)
    rope_linear: float = 1.0        # rotary linear factor (positions divided by it)
    rope_ntk: float = 1.0           # rotary NTK factor (base multiplied by it)

    @property
    def seq_len(self) -> int:
        """Logical joint-sequence length (prefix included)."""
        return sum(seg[1] if seg[0] == "T" else seg[1] * seg[2] * seg[3] for seg in self.layout)

    @property
    def n_new(self) -> int:
        """Number of query tokens (sequence minus cached prefix)."""
        return self.seq_len - self.prefix_len


WORKLOADS: Dict[str, Workload] = {w.name: w for w in [
    Workload("tiny_f32_block_causal", 1, 2, 2, 32, (("T", 16), ("I", 1, 4, 4)), (4, 14, 14),
             "centered_fhw", "block_causal", 1e-6, "f32", True, 0,
             description="fp32, 2 heads x 32, text 16 then one 1x4x4 image block"),
    Workload("lumina_next_full_gqa", 2, 32, 8, 72, (("I", 1, 64, 64),), (36, 36),
             "grid_hw", "full", 1e-5, "bf16", False, 1,
             description="CFG pair, 32 q / 8 kv heads x 72, 2D RoPE 36/36 over 64x64"),
    Workload("qwen_image21_t1024_i64x64", 2, 32, 32, 128, (("T", 1024), ("I", 1, 64, 64)), (16, 56, 56),
             "centered_fhw", "block_causal", 1e-6, "bf16", False, 2,
             description="1024 text + one 1x64x64 target block (5120 tokens)"),
    Workload("cond_images_t256_2x32x32_t256_i64x64", 1, 32, 32, 128,
             (("T", 256), ("I", 1, 32, 32), ("I", 1, 32, 32), ("T", 256), ("I", 1, 64, 64)), (16, 56, 56),
             "centered_fhw", "block_causal", 1e-6, "bf16", False, 3,
             description="two adjacent condition blocks, 6656 tokens"),
    Workload("cached_prefix_decode_i128x128", 1, 32, 32, 128,
             (("T", 1024), ("I", 1, 64, 64), ("I", 1, 128, 128)), (16, 56, 56),
             "centered_fhw", "block_causal", 1e-6, "bf16", False, 4, prefix_len=5120,
             description="cached K/V prefix of 5120 tokens, 16384 target queries vs 21504 keys"),
]}

# The order in which the five configurations are usually listed.
ORDER: List[str] = list(WORKLOADS)

# Variants beyond the five configurations.
#   NucleusMoE image-query attention (NucleusMoE-Image article, section 6 for
#   16 heads x 128 and axes (16, 56, 56); section 6.3 for image queries only,
#   over the image keys and the cached text keys, every pair allowed).  The
#   text is the cached prefix (its K/V do not change across steps) and the
#   64x64 image tokens are the queries; a CFG pair.  The article gives no KV
#   head count: 16, no grouping.
VARIANTS: Dict[str, Workload] = {w.name: w for w in [
    Workload("nucleus_image_query_t1024_i64x64", 2, 16, 16, 128, (("T", 1024), ("I", 1, 64, 64)), (16, 56, 56),
             "centered_fhw", "full", 1e-6, "bf16", False, 5, prefix_len=1024,
             description="4096 image queries over 1024 cached text + 4096 image keys, full mask"),
    # Lumina-Next at twice the trained resolution (Lumina-Next DiT article,
    # section 3: qk_norm as a LayerNorm across heads; section 4: time-aware
    # rotary scaling for resolution extrapolation): 2048 px -> a 128x128 token
    # grid, scaling factor 2, a step past the watershed (NTK factor 2).
    Workload("lumina_next_2k_lnheads_ntk2", 2, 32, 8, 72, (("I", 1, 128, 128),), (36, 36),
             "grid_hw", "full", 1e-5, "bf16", False, 6,
             description="CFG pair, 32 q / 8 kv heads x 72, 128x128 grid, LayerNorm across heads, NTK factor 2",
             qk_norm="layer_across_heads", rope_ntk=2.0),
]}


@dataclass(frozen=True)
class CfgWorkload:
    """The guidance step of a denoising step: the conditional and unconditional
    predictions of `batch` images of `tokens` tokens with `channels` channels
    each (NucleusMoE-Image pipeline article, section 4.3; section 1 and the
    transformer configuration of section 6 for 1024 px -> 64x64 tokens of
    64 packed latent channels; guidance_scale 4.0 is the pipeline default)."""
    name: str
    batch: int
    tokens: int
    channels: int
    guidance: float
    dtype: str
    seed: int
    description: str = ""

    @property
    def rows(self) -> int:
        return self.batch * self.tokens


CFG_WORKLOADS: Dict[str, CfgWorkload] = {w.name: w for w in [
    CfgWorkload("nucleus_cfg_b32_1024px", 32, 4096, 64, 4.0, "bf16", 7,
                description="32 images at 1024 px: 131072 tokens x 64 channels, guidance 4.0"),
]}


def draw_cfg(rows: int, channels: int, seed: int, dtype: str = "bf16"):
    """Seeded (cond, uncond) predictions [rows, channels] as (bits, vals)
    dicts like `draw`: rng = default_rng(seed); float32 base, d1, d2 standard
    normals drawn in that order; cond = base + 0.3 d1, uncond = base + 0.3 d2
    (two predictions of one step agree on most of their content); each
    rounded once to the dtype."""
    rng = np.random.default_rng(seed)
    base = rng.standard_normal((rows, channels), dtype=np.float32)
    d1 = rng.standard_normal((rows, channels), dtype=np.float32)
    d2 = rng.standard_normal((rows, channels), dtype=np.float32)
    bits, vals = {}, {}
    for name, x in (("cond", base + np.float32(0.3) * d1), ("uncond", base + np.float32(0.3) * d2)):
        if dtype == "bf16":
            b = bf16_round_bits(x)
            bits[name], vals[name] = b, bf16_bits_to_f64(b)
        else:
            bits[name] = np.ascontiguousarray(x, dtype=np.float32)
            vals[name] = bits[name].astype(np.float64)
    return bits, vals


def get(name_or_index) -> Workload:
    if isinstance(name_or_index, int):
        return WORKLOADS[ORDER[name_or_index]]
    if name_or_index in VARIANTS:
        return VARIANTS[name_or_index]
    return WORKLOADS[name_or_index]


def small_workload(name: str, batch: int, heads: int, kv_heads: int, head_dim: int, layout,
                   axes, pos_mode="centered_fhw", mask_mode="block_causal", eps=1e-6,
                   dtype="bf16", unit_weights=False, seed=0, prefix_len=0, qk_norm="rms_per_head",
                   rope_linear=1.0, rope_ntk=1.0) -> Workload:
    """A reduced workload of the same structure, for tests that must finish fast."""
    return Workload(name, batch, heads, kv_heads, head_dim, tuple(tuple(s) for s in layout), tuple(axes),
                    pos_mode, mask_mode, eps, dtype, unit_weights, seed, prefix_len, qk_norm=qk_norm,
                    rope_linear=rope_linear, rope_ntk=rope_ntk)


def sequence_inputs(w: Workload) -> Tuple[np.ndarray, List[Tuple[int, int, int]]]:
    """The two inputs the token-metadata step takes: image_pad_mask (uint8 [S],
    1 on image tokens) and img_shapes (list of (frames, height, width) per image
    block in order of appearance; the target image comes last)."""
    mask: List[int] = []
    shapes: List[Tuple[int, int, int]] = []
    for seg in w.layout:
        if seg[0] == "T":
            mask += [0] * seg[1]
        else:
            f, h, wd = seg[1:]
            mask += [1] * (f * h * wd)
            shapes.append((f, h, wd))
    return np.asarray(mask, dtype=np.uint8), shapes


def n_text_tokens(w: Workload) -> int:
    return sum(seg[1] for seg in w.layout if seg[0] == "T")


def text_mask(w: Workload, seed: int, kind: str = "right", min_valid: int = 1) -> np.ndarray:
    """Seeded per-sample text masks, uint8 [batch, text tokens], 1 = valid.

    "right": a tokenizer's padding -- sample b keeps its first L_b text tokens,
      L_b uniform in [min_valid, n_text] (default_rng(seed).integers);
    "random": every entry an independent fair coin (patterns no tokenizer
      makes, for the masking logic itself);
    "none": all valid."""
    n = n_text_tokens(w)
    out = np.ones((w.batch, n), dtype=np.uint8)
    rng = np.random.default_rng(seed)
    if kind == "right":
        for b in range(w.batch):
            L = int(rng.integers(min(min_valid, n), n + 1))
            out[b, L:] = 0
    elif kind == "random":
        out = rng.integers(0, 2, size=(w.batch, n)).astype(np.uint8)
    elif kind != "none":
        raise ValueError(kind)
    return out


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even) and
    return the raw 16-bit patterns as uint16.  Inputs are finite normals."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    """Exact float64 values of bfloat16 bit patterns."""
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


@dataclass
class Drawn:
    """Inputs of one workload.  For each tensor name, `bits` holds what the GPU
    receives (uint16 bf16 patterns, or float32 for an fp32 workload) and `vals`
    the exact same numbers as float64 for the oracle."""
    workload: Workload
    bits: Dict[str, np.ndarray] = field(default_factory=dict)
    vals: Dict[str, np.ndarray] = field(default_factory=dict)


def _store(d: Drawn, name: str, x32: np.ndarray) -> None:
    if d.workload.dtype == "bf16":
        b = bf16_round_bits(x32)
        d.bits[name] = b
        d.vals[name] = bf16_bits_to_f64(b)
    else:
        d.bits[name] = np.ascontiguousarray(x32, dtype=np.float32)
        d.vals[name] = d.bits[name].astype(np.float64)


def draw(w: Workload, parts: Sequence[str] = ("q", "k", "v", "wq", "wk", "bq", "bk", "k_cache", "v_cache")) -> Drawn:
    """Seeded inputs in BSHD layout: rng = default_rng(seed); float32 standard
    normals drawn in the fixed order q, k, v (the query tokens: all tokens, or
    the tokens after the cached prefix), then the norm weights w_q, w_k
    (1 + 0.02 N(0,1), unless unit; [head_dim], or [heads x head_dim] for a
    LayerNorm across heads, which then also draws biases b_q, b_k as
    0.02 N(0,1)), then the cached prefix K (already normed and rotated) and
    raw V.  Each is rounded once to the workload dtype.  Drawing always
    follows the full order so a subset of `parts` yields identical values."""
    rng = np.random.default_rng(w.seed)
    B, S, H, Hk, D, P = w.batch, w.n_new, w.heads, w.kv_heads, w.head_dim, w.prefix_len
    d = Drawn(w)
    shapes = {"q": (B, S, H, D), "k": (B, S, Hk, D), "v": (B, S, Hk, D)}
    for name in ("q", "k", "v"):
        x = rng.standard_normal(shapes[name], dtype=np.float32)
        if name in parts:
            _store(d, name, x)
    across = w.qk_norm == "layer_across_heads"
    for name in ("wq", "wk"):
        n_ch = ((H if name == "wq" else Hk) * D) if across else D
        if w.unit_weights:
            x = np.ones((n_ch,), np.float32)
        else:
            x = (1.0 + 0.02 * rng.standard_normal((n_ch,), dtype=np.float32)).astype(np.float32)
        if name in parts:
            _store(d, name, x)
    if across:  # LayerNorm biases, 0.02 N(0, 1)
        for name in ("bq", "bk"):
            n_ch = (H if name == "bq" else Hk) * D
            x = (0.02 * rng.standard_normal((n_ch,), dtype=np.float32)).astype(np.float32)
            if name in parts:
                _store(d, name, x)
    if P > 0:
        for name in ("k_cache", "v_cache"):
            x = rng.standard_normal((B, P, Hk, D), dtype=np.float32)
            if name in parts:
                _store(d, name, x)
    return d
