"""Token metadata of the joint text+image sequence (oracle, pure Python loops).

Test infrastructure: see the package docstring.

Source: QwenImage21Transformer2DModel API page, ``build_token_metadata``.
The function takes ``image_pad_mask`` (True on image-token positions) and
``img_shapes`` (frames, height, width) per image, condition images first and
the target image last.  It returns ``image_ids`` (text = -1, a distinct id per
image block) and ``target_token_mask``.  The page stresses that block
boundaries come from the token counts in ``img_shapes`` and not from runs of
True in the mask: two condition images with no text between them form one run
of True but stay two blocks.

Readings where the pages are silent (each is listed in the design notes):
  * a count mismatch between the mask and img_shapes is an error, and so is a
    block whose tokens are not contiguous in the sequence (the page places
    condition tokens in reserved slots of the text stream, one run per image);
  * ``kv_limit[s]`` (not on the pages; a derived quantity) is the exclusive
    bound of the keys query s may see under the block-causal rule;
  * rotary positions: "centered_fhw" gives image token (f, h, w) of block b
    the position (frame_offset_b + f, h - H/2, w - W/2) (the centred
    height/width layout of scale_rope, NucleusMoE-Image article section 6.3)
    and text token number t (counting text tokens in sequence order) the
    position max_vid_index + t on every axis, with max_vid_index one past the
    largest image coordinate (text phases continue after the images, same
    section); "grid_hw" gives image tokens (h, w) from 0 (the Lumina-Next
    patch embedder crops its 2D table to the token grid, Lumina-Next DiT
    article section 1) and has no text tokens.
"""
from __future__ import annotations

from typing import Dict, List, Sequence, Tuple

import numpy as np

TEXT_ID = -1


class MetadataError(ValueError):
    """Invalid layout: the pages' contract cannot be met."""


def build_token_metadata(image_pad_mask: Sequence[int], img_shapes: Sequence[Tuple[int, int, int]],
                         pos_mode: str = "centered_fhw") -> Dict[str, np.ndarray]:
    mask = [bool(m) for m in image_pad_mask]
    seq_len = len(mask)
    shapes = [tuple(int(v) for v in s) for s in img_shapes]
    for (f, h, w) in shapes:
        if f <= 0 or h <= 0 or w <= 0:
            raise MetadataError("image block with an empty extent")
        if pos_mode == "centered_fhw" and (h % 2 or w % 2):
            raise MetadataError("centred positions need even height and width")
        if pos_mode == "grid_hw" and f != 1:
            raise MetadataError("2D positions take single-frame images")
    counts = [f * h * w for (f, h, w) in shapes]
    if sum(1 for m in mask if m) != sum(counts):
        raise MetadataError("image_pad_mask marks a different number of tokens than img_shapes")

    # Assign the r-th image token (in sequence order) to the block whose running
    # token count covers r.
    image_ids = [TEXT_ID] * seq_len
    block, used = 0, 0
    for s in range(seq_len):
        if not mask[s]:
            continue
        if used == counts[block]:
            block, used = block + 1, 0
        image_ids[s] = block
        used += 1

    # Each block must occupy one contiguous run of positions.
    first: List[int] = [-1] * len(shapes)
    last: List[int] = [-1] * len(shapes)
    for s, b in enumerate(image_ids):
        if b >= 0:
            if first[b] < 0:
                first[b] = s
            last[b] = s
    for b in range(len(shapes)):
        if last[b] - first[b] + 1 != counts[b]:
            raise MetadataError("an image block's tokens are not contiguous")

    n_img = len(shapes)
    target = [1 if (b >= 0 and b == n_img - 1) else 0 for b in image_ids]

    kv_limit = [0] * seq_len
    for s, b in enumerate(image_ids):
        kv_limit[s] = s + 1 if b < 0 else last[b] + 1

    pos = [[0, 0, 0] for _ in range(seq_len)]
    if pos_mode == "centered_fhw":
        frame_offset = 0
        max_coord = -1
        for b, (f, h, w) in enumerate(shapes):
            for local in range(counts[b]):
                fi = local // (h * w)
                hi = (local // w) % h
                wi = local % w
                p = [frame_offset + fi, hi - h // 2, wi - w // 2]
                pos[first[b] + local] = p
                max_coord = max(max_coord, *p)
            frame_offset += f
        max_vid_index = max_coord + 1 if n_img > 0 else 0
        t = 0
        for s in range(seq_len):
            if image_ids[s] < 0:
                pos[s] = [max_vid_index + t] * 3
                t += 1
    elif pos_mode == "grid_hw":
        if any(b < 0 for b in image_ids):
            raise MetadataError("2D positions are defined for image tokens only")
        for b, (f, h, w) in enumerate(shapes):
            for local in range(counts[b]):
                pos[first[b] + local] = [local // w, local % w, 0]
    else:
        raise MetadataError("unknown position mode")

    return {
        "image_ids": np.asarray(image_ids, dtype=np.int32),
        "target_mask": np.asarray(target, dtype=np.uint8),
        "pos_ids": np.asarray(pos, dtype=np.int32).reshape(seq_len, 3),
        "kv_limit": np.asarray(kv_limit, dtype=np.int32),
    }
