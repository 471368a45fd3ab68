"""Plant plausible mistakes in the oracle (on the CPU) and check that at least
one pin catches each: evidence that the pins constrain the oracle."""
import numpy as np
import pytest

import oracle.attention as att
import oracle.cfg as ocfg
import oracle.key_padding as kp
import oracle.metadata as meta
import oracle.pipeline as opipe
import oracle.qknorm_rope as qr
from tests import oracle_pins as pins


def _fails(pin_list):
    for pin in pin_list:
        try:
            pin()
        except AssertionError:
            return True
    return False


def _allowed_strict_causal(q_index, k_index, image_ids, mask_mode):
    m = att.allowed_matrix.__wrapped__(q_index, k_index, image_ids, mask_mode)
    return m & ~(np.asarray(k_index)[None, :] == np.asarray(q_index)[:, None]) | (
        (np.asarray(image_ids)[np.asarray(q_index)][:, None] >= 0) & m)


def _allowed_text_matches_text(q_index, k_index, image_ids, mask_mode):
    if mask_mode == "full":
        return np.ones((len(q_index), len(k_index)), bool)
    ids = np.asarray(image_ids)
    causal = np.asarray(k_index)[None, :] <= np.asarray(q_index)[:, None]
    return causal | (ids[q_index][:, None] == ids[k_index][None, :])


def _rms_sum(x, weight, eps):
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps) * weight


def _rms_eps_outside(x, weight, eps):
    x = np.asarray(x, dtype=np.float64)
    return x / (np.sqrt(np.mean(x * x, axis=-1, keepdims=True)) + eps) * weight


def _rope_rotate_half(x, pos, axes, theta=10000.0, linear_factor=1.0, ntk_factor=1.0):
    x = np.asarray(x, dtype=np.float64)
    y = x.copy()
    pos = np.asarray(pos, dtype=np.float64) / linear_factor
    theta = theta * ntk_factor
    off = 0
    for a, d_a in enumerate(axes):
        half = d_a // 2
        for j in range(half):
            ph = pos[:, a] * theta ** (-2.0 * j / d_a)
            c, s = np.cos(ph)[:, None], np.sin(ph)[:, None]
            x0, x1 = x[..., off + j], x[..., off + j + half]
            y[..., off + j] = x0 * c - x1 * s
            y[..., off + j + half] = x0 * s + x1 * c
        off += d_a
    return y


def _rope_shared_ladder(x, pos, axes, theta=10000.0, linear_factor=1.0, ntk_factor=1.0):
    """Mistake: one frequency ladder over the whole head instead of per axis."""
    x = np.asarray(x, dtype=np.float64)
    y = x.copy()
    D = x.shape[-1]
    pos = np.asarray(pos, dtype=np.float64) / linear_factor
    theta = theta * ntk_factor
    off = 0
    for a, d_a in enumerate(axes):
        for j in range(d_a // 2):
            ph = pos[:, a] * theta ** (-2.0 * (off // 2 + j) / D)
            c, s = np.cos(ph)[:, None], np.sin(ph)[:, None]
            x0, x1 = x[..., off + 2 * j], x[..., off + 2 * j + 1]
            y[..., off + 2 * j] = x0 * c - x1 * s
            y[..., off + 2 * j + 1] = x0 * s + x1 * c
        off += d_a
    return y


def _rope_sign_flip(x, pos, axes, theta=10000.0, linear_factor=1.0, ntk_factor=1.0):
    return qr_rope_orig(x, -np.asarray(pos), axes, theta, linear_factor, ntk_factor)


def _rope_ntk_as_interpolation(x, pos, axes, theta=10000.0, linear_factor=1.0, ntk_factor=1.0):
    # Mistake: the NTK factor divides the positions like the linear one.
    return qr_rope_orig(x, pos, axes, theta, linear_factor * ntk_factor, 1.0)


def _rope_linear_multiplies(x, pos, axes, theta=10000.0, linear_factor=1.0, ntk_factor=1.0):
    # Mistake: the linear factor multiplies the positions.
    return qr_rope_orig(x, pos, axes, theta, 1.0 / linear_factor, ntk_factor)


def _ln_per_head(x, weight=None, bias=None, eps=1e-5):
    # Mistake: each head normalised on its own.
    x = np.asarray(x, dtype=np.float64)
    cen = x - x.mean(axis=-1, keepdims=True)
    y = cen / np.sqrt((cen * cen).mean(axis=-1, keepdims=True) + eps)
    y = y.reshape(x.shape[:-2] + (-1,))
    if weight is not None:
        y = y * weight
    if bias is not None:
        y = y + bias
    return y.reshape(x.shape)


def _ln_no_centering(x, weight=None, bias=None, eps=1e-5):
    # Mistake: RMS over the heads' channels (mean not removed).
    x = np.asarray(x, dtype=np.float64)
    flat = x.reshape(x.shape[:-2] + (-1,))
    y = flat / np.sqrt((flat * flat).mean(axis=-1, keepdims=True) + eps)
    if weight is not None:
        y = y * weight
    if bias is not None:
        y = y + bias
    return y.reshape(x.shape)


def _time_aware_swapped(t, watershed, scaling_factor):
    # Mistake: the branches swapped.
    return (1.0, float(scaling_factor)) if t < watershed else (float(scaling_factor), 1.0)


def _cfg_no_rescale(cond, uncond, guidance_scale):
    # Mistake: plain CFG, the norm rescaling left out.
    cond = np.asarray(cond, dtype=np.float64)
    uncond = np.asarray(uncond, dtype=np.float64)
    return uncond + guidance_scale * (cond - uncond)


def _rescaled(comb, ref):
    return comb * (np.linalg.norm(ref, axis=-1, keepdims=True) / np.linalg.norm(comb, axis=-1, keepdims=True))


def _cfg_rescale_to_uncond(cond, uncond, guidance_scale):
    # Mistake: rescaled to the unconditional prediction's norm.
    cond = np.asarray(cond, dtype=np.float64)
    uncond = np.asarray(uncond, dtype=np.float64)
    return _rescaled(uncond + guidance_scale * (cond - uncond), uncond)


def _cfg_swapped_mix(cond, uncond, guidance_scale):
    # Mistake: mixed as cond + scale * (uncond - cond).
    cond = np.asarray(cond, dtype=np.float64)
    uncond = np.asarray(uncond, dtype=np.float64)
    return _rescaled(cond + guidance_scale * (uncond - cond), cond)


cfg_orig = ocfg.norm_rescaled_cfg
qr_rope_orig = qr.rope
att_attention_orig = att.attention


def _attention_gqa_modulo(q, k, v, image_ids, mask_mode, scale=None, q_offset=0, rows=None, chunk=2048,
                          key_valid=None):
    # Mistake: query head h reads KV head h % H_kv instead of h // G.
    H, Hk = q.shape[2], k.shape[2]
    perm = [h % Hk for h in range(H)]
    ke = np.asarray(k)[:, :, perm]
    ve = np.asarray(v)[:, :, perm]
    return att_attention_orig(q, ke, ve, image_ids, mask_mode, scale, q_offset, rows, chunk, key_valid)


def _attention_no_scale(q, k, v, image_ids, mask_mode, scale=None, q_offset=0, rows=None, chunk=2048,
                        key_valid=None):
    return att_attention_orig(q, k, v, image_ids, mask_mode, 1.0, q_offset, rows, chunk, key_valid)


def _attention_padding_masks_queries(q, k, v, image_ids, mask_mode, scale=None, q_offset=0, rows=None,
                                     chunk=2048, key_valid=None):
    # Mistake: padding removes the padded positions' query rows instead of their keys.
    o, lse = att_attention_orig(q, k, v, image_ids, mask_mode, scale, q_offset, rows, chunk)
    if key_valid is not None:
        r = np.arange(np.asarray(q).shape[1]) if rows is None else np.asarray(rows)
        dead = ~np.asarray(key_valid, bool)[:, r + q_offset]
        o = np.where(dead[:, :, None, None], 0.0, o)
    return o, lse


kp_orig = kp.joint_key_valid


def _key_valid_by_position(image_pad_mask, text_valid):
    # Mistake: the text flag is indexed by sequence position instead of text ordinal.
    mask = np.asarray(image_pad_mask).reshape(-1)
    tv = np.asarray(text_valid, bool)
    out = np.ones((tv.shape[0], mask.size), bool)
    for s in range(mask.size):
        if mask[s] == 0:
            out[:, s] = tv[:, min(s, tv.shape[1] - 1)]
    return out


def _metadata_merge_runs(image_pad_mask, img_shapes, pos_mode="centered_fhw"):
    """Mistake: blocks taken from contiguous runs of True (merges adjacent images)."""
    md = meta_build_orig(image_pad_mask, img_shapes, pos_mode)
    ids = md["image_ids"].copy()
    run, prev = -1, False
    for s, m in enumerate(image_pad_mask):
        if m and not prev:
            run += 1
        ids[s] = run if m else -1
        prev = bool(m)
    md["image_ids"] = ids
    return md


meta_build_orig = meta.build_token_metadata


def _metadata_kv_limit_off_by_one(image_pad_mask, img_shapes, pos_mode="centered_fhw"):
    md = meta_build_orig(image_pad_mask, img_shapes, pos_mode)
    md["kv_limit"] = md["kv_limit"] - (md["image_ids"] >= 0)
    return md


def _metadata_uncentred(image_pad_mask, img_shapes, pos_mode="centered_fhw"):
    md = meta_build_orig(image_pad_mask, img_shapes, pos_mode)
    if pos_mode == "centered_fhw":
        pos = md["pos_ids"].copy()
        off = 0
        for s, b in enumerate(md["image_ids"]):
            if b >= 0:
                f, h, w = img_shapes[b]
                pos[s, 1] += h // 2
                pos[s, 2] += w // 2
        md["pos_ids"] = pos
    return md


pipe_step_orig = opipe.step


def _pipeline_positions_from_start(vals, md, **kw):
    # Mistake: the new tokens take the rotary positions of the first S_new
    # tokens of the sequence instead of their own, [P, P + S_new).
    P, S_new = kw.get("prefix_len", 0), np.asarray(vals["q"]).shape[1]
    md2 = dict(md)
    pos = np.array(md["pos_ids"], copy=True)
    pos[P:P + S_new] = md["pos_ids"][:S_new]
    md2["pos_ids"] = pos
    return pipe_step_orig(vals, md2, **kw)


def _pipeline_cached_rows_without_offset(vals, md, **kw):
    # Mistake: the cached step's attention called without the prefix offset,
    # so its query rows take the key bounds of the sequence's first tokens.
    out = pipe_step_orig(vals, md, **kw)
    if kw.get("prefix_len", 0) == 0:
        return out
    k_all = np.concatenate([vals["k_cache"], out["k_prime"]], axis=1)
    v_all = np.concatenate([vals["v_cache"], vals["v"]], axis=1)
    o, lse = att.attention(out["q_prime"], k_all, v_all, md["image_ids"], kw["mask_mode"], rows=kw.get("rows"),
                           key_valid=kw.get("key_valid"))
    out.update(o=o, lse=lse)
    return out

def _wrap_allowed(fn):
    orig = att.allowed_matrix

    def wrapped(*a, **k):
        return fn(*a, **k)
    wrapped.__wrapped__ = orig
    return wrapped


MUTATIONS = [
    ("block_causal_drops_diagonal", att, "allowed_matrix",
     lambda q, k, ids, mode: (att.allowed_matrix.__wrapped__(q, k, ids, mode)
                              & ~(np.asarray(k)[None, :] == np.asarray(q)[:, None])) if mode != "full"
     else np.ones((len(q), len(k)), bool)),
    ("text_ids_count_as_one_block", att, "allowed_matrix", _allowed_text_matches_text),
    ("rmsnorm_sum_not_mean", qr, "rms_norm", _rms_sum),
    ("rmsnorm_eps_outside_sqrt", qr, "rms_norm", _rms_eps_outside),
    ("rope_rotate_half_pairs", qr, "rope", _rope_rotate_half),
    ("rope_shared_frequency_ladder", qr, "rope", _rope_shared_ladder),
    ("rope_negated_phase", qr, "rope", _rope_sign_flip),
    ("gqa_modulo_head_map", att, "attention", _attention_gqa_modulo),
    ("softmax_scale_missing", att, "attention", _attention_no_scale),
    ("metadata_merges_adjacent_images", meta, "build_token_metadata", _metadata_merge_runs),
    ("metadata_kv_limit_off_by_one", meta, "build_token_metadata", _metadata_kv_limit_off_by_one),
    ("metadata_positions_uncentred", meta, "build_token_metadata", _metadata_uncentred),
    ("padding_masks_queries_not_keys", att, "attention", _attention_padding_masks_queries),
    ("padding_flag_by_position", kp, "joint_key_valid", _key_valid_by_position),
    ("rope_ntk_as_interpolation", qr, "rope", _rope_ntk_as_interpolation),
    ("rope_linear_multiplies_positions", qr, "rope", _rope_linear_multiplies),
    ("layernorm_per_head", qr, "layer_norm_across_heads", _ln_per_head),
    ("layernorm_without_centering", qr, "layer_norm_across_heads", _ln_no_centering),
    ("time_aware_branches_swapped", qr, "time_aware_rope_factors", _time_aware_swapped),
    ("cfg_without_rescale", ocfg, "norm_rescaled_cfg", _cfg_no_rescale),
    ("cfg_rescaled_to_uncond_norm", ocfg, "norm_rescaled_cfg", _cfg_rescale_to_uncond),
    ("cfg_mix_direction_swapped", ocfg, "norm_rescaled_cfg", _cfg_swapped_mix),
    ("pipeline_positions_from_sequence_start", opipe, "step", _pipeline_positions_from_start),
    ("pipeline_cached_rows_without_offset", opipe, "step", _pipeline_cached_rows_without_offset),
]


@pytest.mark.parametrize("name,module,attr,fn", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutation_is_caught(monkeypatch, name, module, attr, fn):
    if attr == "allowed_matrix":
        fn = _wrap_allowed(fn)
    monkeypatch.setattr(module, attr, fn)
    assert _fails(pins.ALL_PINS), "no pin caught the planted mistake %s" % name
