"""Text key padding over the joint sequence (oracle).

Test infrastructure: see the package docstring.

Source: QwenImage21Transformer2DModel API page, forward's
encoder_hidden_states_mask -- a (batch, text_sequence_length) boolean that
marks the valid text tokens; padded positions are kept out of attention.

Reading: the j-th text token of the joint sequence (in sequence order, the
tokens where image_pad_mask is 0) is the j-th position of the text mask;
image tokens are always valid.  A text mask whose length differs from the
number of text tokens is a data error.
"""
from __future__ import annotations

import numpy as np


class KeyPaddingError(ValueError):
    pass


def joint_key_valid(image_pad_mask, text_valid) -> np.ndarray:
    """bool [B, S]: may key s be attended for sample b."""
    mask = [int(x) for x in np.asarray(image_pad_mask).reshape(-1)]
    tv = np.asarray(text_valid, dtype=bool)
    if tv.ndim != 2:
        raise KeyPaddingError("text mask must be [batch, text tokens]")
    n_text = sum(1 for x in mask if x == 0)
    if tv.shape[1] != n_text:
        raise KeyPaddingError("text mask has %d positions for %d text tokens" % (tv.shape[1], n_text))
    out = np.ones((tv.shape[0], len(mask)), dtype=bool)
    for b in range(tv.shape[0]):
        j = 0
        for s, is_image in enumerate(mask):
            if not is_image:
                out[b, s] = bool(tv[b, j])
                j += 1
    return out
