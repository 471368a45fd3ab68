"""Pins of the fp64 oracle against facts fixed by the pages or by mathematics.

Each pin is a plain function that raises AssertionError when the oracle
disagrees.  ``test_oracle_*.py`` run them; ``test_oracle_mutations.py`` plants
plausible mistakes in the oracle and checks that some pin catches each one.
None of these re-types the oracle's own formula: they use hand-derived
fixtures, closed forms, invariants, library routines (torch SDPA in float64 on
the CPU, torch.repeat_interleave) and brute force.
"""
from __future__ import annotations

import math

import numpy as np
import torch

import oracle.attention as att
import oracle.cfg as ocfg
import oracle.key_padding as kp
import oracle.metadata as meta
import oracle.pipeline as pipe
import oracle.qknorm_rope as qr
from tests import goldens
from workloads import Workload, sequence_inputs, small_workload


# --------------------------------------------------------------------------- helpers
def _layout_inputs(layout):
    w = small_workload("fixture", 1, 1, 1, 8, layout, (8,))
    return sequence_inputs(w)


def _sdpa(q, k, v, is_causal=False):
    """torch SDPA in float64 on the CPU; inputs BSHD numpy, output BSHD numpy."""
    tq = torch.from_numpy(np.ascontiguousarray(q.transpose(0, 2, 1, 3)))
    tk = torch.from_numpy(np.ascontiguousarray(k.transpose(0, 2, 1, 3)))
    tv = torch.from_numpy(np.ascontiguousarray(v.transpose(0, 2, 1, 3)))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=is_causal)
    return o.numpy().transpose(0, 2, 1, 3)


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# --------------------------------------------------------------------------- metadata
def pin_metadata_goldens():
    """Hand-derived fixtures (tests/golden/metadata_*.txt), each citing its rule."""
    for name in goldens.metadata_fixtures():
        g = goldens.load(name)
        mask, shapes = _layout_inputs(g["layout"])
        md = meta.build_token_metadata(mask, shapes, g["pos_mode"])
        for key in ("image_ids", "target_mask", "kv_limit", "pos_ids"):
            assert np.array_equal(md[key].astype(np.int64), g[key]), (name, key, md[key], g[key])


def random_layout(rng, max_tokens=60):
    segs = []
    n = 0
    while n < max_tokens:
        if rng.random() < 0.5:
            t = int(rng.integers(1, 6))
            segs.append(("T", t))
            n += t
        else:
            f, h, w = int(rng.integers(1, 3)), 2 * int(rng.integers(1, 3)), 2 * int(rng.integers(1, 3))
            segs.append(("I", f, h, w))
            n += f * h * w
    return tuple(segs)


def pin_kv_limit_is_predicate_prefix(trials=40):
    """For every query, the set of keys the literal block-causal predicate allows
    (brute force over all pairs, straight from the page's rule) is exactly the
    prefix [0, kv_limit[q]); kv_limit never decreases along the sequence."""
    rng = np.random.default_rng(11)
    for _ in range(trials):
        layout = random_layout(rng)
        mask, shapes = _layout_inputs(layout)
        md = meta.build_token_metadata(mask, shapes)
        ids = md["image_ids"]
        S = len(ids)
        for qi in range(S):
            allowed = [kj for kj in range(S) if kj <= qi or (ids[qi] >= 0 and ids[qi] == ids[kj])]
            assert allowed == list(range(md["kv_limit"][qi])), (layout, qi)
        assert np.all(np.diff(md["kv_limit"]) >= 0)


def pin_metadata_errors():
    """Readings for inputs the pages leave undefined raise errors."""
    def expect_error(mask, shapes, mode="centered_fhw"):
        try:
            meta.build_token_metadata(mask, shapes, mode)
        except meta.MetadataError:
            return
        raise AssertionError("no error for %r %r" % (mask, shapes))
    expect_error([1, 1, 1], [(1, 2, 2)])                 # count mismatch
    expect_error([1, 1, 0, 1, 1], [(1, 2, 2)])           # block split by text
    expect_error([1] * 6, [(1, 3, 2)])                   # odd height, centred
    expect_error([0, 1, 1], [(1, 1, 2)], "grid_hw")      # text in 2D mode
    expect_error([1] * 8, [(2, 2, 2)], "grid_hw")        # multi-frame in 2D mode


# --------------------------------------------------------------------------- rmsnorm
def pin_rmsnorm_closed_forms():
    # x = (3, 4), eps = 0: mean square 12.5, so y = x * sqrt(2) / 5.
    y = qr.rms_norm(np.array([3.0, 4.0]), np.ones(2), 0.0)
    assert np.allclose(y, [3 * math.sqrt(2) / 5, 4 * math.sqrt(2) / 5], rtol=0, atol=1e-15)
    # With unit weights mean(y^2) = m / (m + eps), m = mean(x^2); use a large eps
    # so that any other placement of eps shows.
    x = _rand((3, 5, 4, 16), 1)
    for eps in (0.0, 0.5, 3.0):
        y = qr.rms_norm(x, np.ones(16), eps)
        m = np.mean(x * x, axis=-1)
        assert np.allclose(np.mean(y * y, axis=-1), m / (m + eps), rtol=1e-12, atol=0)
    # The weight multiplies channel by channel.
    wv = 1.0 + 0.1 * _rand((16,), 2)
    assert np.allclose(qr.rms_norm(x, wv, 1e-6), qr.rms_norm(x, np.ones(16), 1e-6) * wv, rtol=1e-13)
    # Each head is normalised on its own: changing head 0 leaves head 1.
    x2 = x.copy()
    x2[:, :, 0, :] *= 7.0
    assert np.array_equal(qr.rms_norm(x2, wv, 1e-6)[:, :, 1:], qr.rms_norm(x, wv, 1e-6)[:, :, 1:])


# --------------------------------------------------------------------------- rope
def pin_rope_rotation():
    axes = (16, 56, 56)
    rng = np.random.default_rng(3)
    x = rng.standard_normal((2, 7, 3, 128))
    pos = rng.integers(-40, 1100, size=(7, 3))
    y = qr.rope(x, pos, axes)
    # A rotation keeps every channel pair's length, hence each head's norm.
    pairs_x = np.hypot(x[..., 0::2], x[..., 1::2])
    pairs_y = np.hypot(y[..., 0::2], y[..., 1::2])
    assert np.allclose(pairs_x, pairs_y, rtol=1e-12)
    # Position 0 is the identity.
    assert np.allclose(qr.rope(x, np.zeros((7, 3), int), axes), x, rtol=0, atol=0)


def pin_rope_pairing_and_ladder():
    """Adjacent pairs (2j, 2j+1); the first pair of each axis turns by exactly the
    position in radians; closed-form ladder points theta^(-2j/d):
    d = 16, j = 2 -> 0.1 and j = 4 -> 0.01; d = 4 (Lumina mini 4+4), j = 1 -> 0.01."""
    def turn(axes, axis, pair, p):
        D = sum(axes)
        off = sum(axes[:axis])
        x = np.zeros((1, 1, 1, D))
        x[..., off + 2 * pair] = 1.0
        pos = np.zeros((1, 3), int)
        pos[0, axis] = p
        y = qr.rope(x, pos, axes)[0, 0, 0]
        nz = np.flatnonzero(np.abs(y) > 1e-300)
        assert set(nz) <= {off + 2 * pair, off + 2 * pair + 1}, (axes, axis, pair, nz)
        return y[off + 2 * pair], y[off + 2 * pair + 1]
    for axes in ((16, 56, 56), (36, 36), (4, 4), (8, 4, 4)):
        for a in range(len(axes)):
            c, s = turn(axes, a, 0, 5)
            assert abs(c - math.cos(5)) < 1e-15 and abs(s - math.sin(5)) < 1e-15
    for (axes, a, j, omega) in (((16, 56, 56), 0, 2, 0.1), ((16, 56, 56), 0, 4, 0.01), ((4, 4), 1, 1, 0.01)):
        p = 300
        c, s = turn(axes, a, j, p)
        assert abs(c - math.cos(p * omega)) < 1e-12 and abs(s - math.sin(p * omega)) < 1e-12, (axes, j)
    # A position on one axis moves only that axis's channels.
    x = _rand((1, 1, 1, 128), 4)
    pos = np.array([[0, 9, 0]])
    y = qr.rope(x, pos, (16, 56, 56))
    assert np.array_equal(y[..., :16], x[..., :16]) and np.array_equal(y[..., 72:], x[..., 72:])
    assert not np.allclose(y[..., 16:72], x[..., 16:72])


def pin_rope_relative():
    """q.k after rotation depends on the positions only through their difference."""
    axes = (16, 56, 56)
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 1, 1, 128))
    k = rng.standard_normal((1, 1, 1, 128))
    for _ in range(20):
        pq = rng.integers(-64, 1100, size=(1, 3))
        pk = rng.integers(-64, 1100, size=(1, 3))
        shift = rng.integers(-500, 500, size=(1, 3))
        d0 = np.sum(qr.rope(q, pq, axes) * qr.rope(k, pk, axes))
        d1 = np.sum(qr.rope(q, pq + shift, axes) * qr.rope(k, pk + shift, axes))
        assert abs(d0 - d1) < 1e-9 * (1 + abs(d0))


# --------------------------------------------------------------------------- Lumina-Next variants
def pin_layernorm_across_heads():
    """LayerNorm over all heads' channels of a token (Lumina-Next DiT article,
    section 3): = torch.nn.functional.layer_norm (float64) on the flattened
    heads x head_dim channels with the same weight and bias; closed forms of
    the output's mean and variance; invariant to a shift of the token; the
    heads' relative scale survives (a per-head norm would erase it)."""
    x = _rand((2, 5, 4, 18), 31) * 3.0 + 0.7
    H, D = 4, 18
    w = 1.0 + 0.1 * _rand((H * D,), 32)
    b = 0.05 * _rand((H * D,), 33)
    for eps in (1e-5, 0.5):
        y = qr.layer_norm_across_heads(x, w, b, eps)
        ref = torch.nn.functional.layer_norm(torch.from_numpy(x.reshape(2, 5, H * D)), (H * D,),
                                             torch.from_numpy(w), torch.from_numpy(b), eps)
        assert np.allclose(y.reshape(2, 5, H * D), ref.numpy(), rtol=1e-12, atol=1e-13)
    # unit affine: mean 0 and variance v / (v + eps) over the token's channels
    eps = 0.5
    y = qr.layer_norm_across_heads(x, None, None, eps).reshape(2, 5, H * D)
    v = x.reshape(2, 5, H * D).var(axis=-1)
    assert np.allclose(y.mean(axis=-1), 0.0, atol=1e-13)
    assert np.allclose(y.var(axis=-1), v / (v + eps), rtol=1e-12)
    # a constant added to every channel of a token changes nothing
    assert np.allclose(qr.layer_norm_across_heads(x + 5.0, w, b, 1e-5), qr.layer_norm_across_heads(x, w, b, 1e-5),
                       rtol=1e-9, atol=1e-10)
    # head 0 ten times larger than head 1 stays ten times larger (eps = 0, zero-mean heads)
    z = _rand((1, 1, 2, 8), 34)
    z -= z.mean(axis=-1, keepdims=True)
    z[0, 0, 1] = z[0, 0, 0] / 10.0
    yz = qr.layer_norm_across_heads(z, None, None, 0.0)
    assert abs(np.linalg.norm(yz[0, 0, 0]) / np.linalg.norm(yz[0, 0, 1]) - 10.0) < 1e-12


def pin_scaled_rope():
    """Rotary factors (Lumina-Next DiT article, section 4): with the linear
    factor L a position L * p turns pair 0 of every axis by exactly p rad, as a
    position p does unscaled; the NTK factor N leaves pair 0 (frequency 1)
    alone and moves the ladder to (theta * N)^(-2j/d): theta 100, N 4, d 4,
    j 1 -> 1/20, so position 20 turns that pair by exactly 1 rad.  Rotations
    stay rotations and factors 1 change nothing."""
    x = _rand((1, 3, 2, 8), 35)
    pos = np.array([[0, 7, 0], [0, 0, 11], [0, 5, 9]])
    axes = (4, 4)
    pos2 = pos[:, 1:]
    for L in (2.0, 3.0):
        assert np.allclose(qr.rope(x, L * pos2, axes, linear_factor=L), qr.rope(x, pos2, axes), rtol=1e-13,
                           atol=1e-14)
    e = np.zeros((1, 1, 1, 8))
    e[..., 2] = 1.0  # axis 0, pair 1
    y = qr.rope(e, np.array([[20, 0]]), axes, theta=100.0, ntk_factor=4.0)[0, 0, 0]
    assert abs(y[2] - math.cos(1.0)) < 1e-14 and abs(y[3] - math.sin(1.0)) < 1e-14
    e0 = np.zeros((1, 1, 1, 8))
    e0[..., 4] = 1.0  # axis 1, pair 0
    y0 = qr.rope(e0, np.array([[0, 3]]), axes, ntk_factor=7.0)[0, 0, 0]
    assert abs(y0[4] - math.cos(3.0)) < 1e-15 and abs(y0[5] - math.sin(3.0)) < 1e-15
    y = qr.rope(x, pos2, axes, linear_factor=1.7, ntk_factor=3.1)
    assert np.allclose(np.hypot(y[..., 0::2], y[..., 1::2]), np.hypot(x[..., 0::2], x[..., 1::2]), rtol=1e-12)
    assert np.array_equal(qr.rope(x, pos2, axes, linear_factor=1.0, ntk_factor=1.0), qr.rope(x, pos2, axes))


def pin_time_aware_factors():
    """Lumina-Next DiT article, section 4: one factor carries scaling_factor,
    the other is 1, switched at scaling_watershed (reading: steps before the
    watershed take the linear factor)."""
    assert qr.time_aware_rope_factors(0.1, 0.3, 2.0) == (2.0, 1.0)
    assert qr.time_aware_rope_factors(0.3, 0.3, 2.0) == (1.0, 2.0)
    assert qr.time_aware_rope_factors(0.9, 0.3, 2.0) == (1.0, 2.0)
    assert qr.time_aware_rope_factors(0.5, 0.3, 1.0) == (1.0, 1.0)


# --------------------------------------------------------------------------- norm-rescaled CFG
def pin_cfg_norm_rescale():
    """NucleusMoE-Image article, section 4.3: every token's output has the
    conditional prediction's norm and the mixed prediction's direction; scale 1
    returns the conditional prediction, scale 0 the unconditional one rescaled;
    a hand-worked token; a zero mixed prediction gives zero (reading)."""
    rng = np.random.default_rng(41)
    cond = rng.standard_normal((2, 9, 64))
    unc = rng.standard_normal((2, 9, 64))
    for g in (0.0, 1.0, 2.5, 7.0, -1.5):
        out = ocfg.norm_rescaled_cfg(cond, unc, g)
        comb = unc + g * (cond - unc)
        assert np.allclose(np.linalg.norm(out, axis=-1), np.linalg.norm(cond, axis=-1), rtol=1e-13)
        cos = np.sum(out * comb, axis=-1) / (np.linalg.norm(out, axis=-1) * np.linalg.norm(comb, axis=-1))
        assert np.allclose(cos, 1.0, rtol=0, atol=1e-13)
    assert np.allclose(ocfg.norm_rescaled_cfg(cond, unc, 1.0), cond, rtol=1e-13, atol=1e-14)
    g0 = ocfg.norm_rescaled_cfg(cond, unc, 0.0)
    assert np.allclose(g0, unc * (np.linalg.norm(cond, axis=-1) / np.linalg.norm(unc, axis=-1))[..., None],
                       rtol=1e-13)
    # cond (3, 4) (norm 5), uncond (1, 0), scale 2: mixed = (1, 0) + 2 * (2, 4) = (5, 8),
    # norm sqrt(89); output = (5, 8) * 5 / sqrt(89).
    out = ocfg.norm_rescaled_cfg([3.0, 4.0], [1.0, 0.0], 2.0)
    assert np.allclose(out, np.array([5.0, 8.0]) * 5.0 / math.sqrt(89.0), rtol=0, atol=1e-15)
    # homogeneous of degree 1 in (cond, uncond)
    assert np.allclose(ocfg.norm_rescaled_cfg(3.0 * cond, 3.0 * unc, 4.0), 3.0 * ocfg.norm_rescaled_cfg(cond, unc, 4.0),
                       rtol=1e-12)
    z = ocfg.norm_rescaled_cfg(np.ones((1, 4)), np.ones((1, 4)) * 2.0, 2.0)  # mixed = 2 - 2 = 0 exactly
    assert np.array_equal(z, np.zeros((1, 4)))


# --------------------------------------------------------------------------- attention
def pin_full_is_sdpa():
    """One image block and no text: the full mask and the block-causal mask both
    equal plain bidirectional attention (torch SDPA, float64, CPU)."""
    rng = np.random.default_rng(6)
    q, k, v = (rng.standard_normal((2, 24, 4, 16)) for _ in range(3))
    ids = np.zeros(24, int)
    ref = _sdpa(q, k, v)
    for mode in ("full", "block_causal"):
        o, _ = att.attention(q, k, v, ids, mode)
        assert np.allclose(o, ref, rtol=1e-10, atol=1e-12), mode


def pin_text_only_is_causal():
    """No image block: block-causal equals plain causal attention."""
    rng = np.random.default_rng(7)
    q, k, v = (rng.standard_normal((2, 20, 3, 8)) for _ in range(3))
    ids = -np.ones(20, int)
    o, _ = att.attention(q, k, v, ids, "block_causal")
    assert np.allclose(o, _sdpa(q, k, v, is_causal=True), rtol=1e-10, atol=1e-12)
    o2, _ = att.attention_multipass(q, k, v, ids)
    assert np.allclose(o2, o, rtol=1e-10, atol=1e-12)


def pin_gqa_is_repeat_interleave():
    """GQA equals multi-head attention over K/V heads expanded by
    repeat_interleave (each KV head serves a contiguous group of query heads)."""
    rng = np.random.default_rng(8)
    q = rng.standard_normal((1, 12, 6, 8))
    k, v = (rng.standard_normal((1, 12, 2, 8)) for _ in range(2))
    ids = np.zeros(12, int)
    o, _ = att.attention(q, k, v, ids, "full")
    ke = torch.repeat_interleave(torch.from_numpy(k), 3, dim=2).numpy()
    ve = torch.repeat_interleave(torch.from_numpy(v), 3, dim=2).numpy()
    assert np.allclose(o, _sdpa(q, ke, ve), rtol=1e-10, atol=1e-12)


def pin_singlepass_equals_multipass(trials=12):
    """The one-pass masked result equals the per-prefix-segment multi-pass result
    (the page states both processors give the same output)."""
    rng = np.random.default_rng(9)
    layouts = [(("T", 16), ("I", 1, 4, 4)),
               (("T", 8), ("I", 1, 4, 4), ("I", 1, 2, 4), ("T", 6), ("I", 1, 4, 4)),
               (("I", 1, 2, 2), ("I", 1, 2, 2))]
    layouts += [random_layout(rng, 50) for _ in range(trials)]
    for layout in layouts:
        mask, shapes = _layout_inputs(layout)
        ids = meta.build_token_metadata(mask, shapes)["image_ids"]
        S = len(ids)
        q = rng.standard_normal((1, S, 4, 8))
        k, v = (rng.standard_normal((1, S, 2, 8)) for _ in range(2))
        o1, l1 = att.attention(q, k, v, ids, "block_causal")
        o2, l2 = att.attention_multipass(q, k, v, ids)
        assert np.allclose(o1, o2, rtol=1e-10, atol=1e-12), layout
        assert np.allclose(l1, l2, rtol=1e-10, atol=1e-12), layout


def pin_adjacent_blocks_stay_separate():
    """Rows of the first of two adjacent condition blocks do not see the second
    block's keys; the second block sees the first (it comes earlier)."""
    mask, shapes = _layout_inputs((("T", 3), ("I", 1, 2, 2), ("I", 1, 2, 2), ("I", 1, 2, 2)))
    ids = meta.build_token_metadata(mask, shapes)["image_ids"]
    rng = np.random.default_rng(10)
    S = len(ids)
    q, k, v = (rng.standard_normal((1, S, 2, 8)) for _ in range(3))
    o, _ = att.attention(q, k, v, ids, "block_causal")
    k2, v2 = k.copy(), v.copy()
    k2[:, 7:11] += 1.0
    v2[:, 7:11] += 1.0                      # perturb block 1 (positions 7..10)
    o2, _ = att.attention(q, k2, v2, ids, "block_causal")
    assert np.array_equal(o[:, :7], o2[:, :7])           # text and block 0 unaffected
    assert not np.allclose(o[:, 7:], o2[:, 7:])


def pin_cached_equals_full():
    """Cached-prefix decode: the target rows computed from cached prefix K/V equal
    the same rows of the full forward; the prefix rows do not depend on the
    target's K/V."""
    layout = (("T", 6), ("I", 1, 2, 2), ("I", 1, 2, 4))
    mask, shapes = _layout_inputs(layout)
    ids = meta.build_token_metadata(mask, shapes)["image_ids"]
    S, P = len(ids), 10
    rng = np.random.default_rng(12)
    q = rng.standard_normal((2, S, 4, 8))
    k, v = (rng.standard_normal((2, S, 2, 8)) for _ in range(2))
    full, full_lse = att.attention(q, k, v, ids, "block_causal")
    cached, cached_lse = att.attention(q[:, P:], k, v, ids, "block_causal", q_offset=P)
    assert np.allclose(cached, full[:, P:], rtol=1e-12, atol=1e-14)
    assert np.allclose(cached_lse, full_lse[:, :, P:], rtol=1e-12, atol=1e-14)
    k2, v2 = k.copy(), v.copy()
    k2[:, P:] = rng.standard_normal(k2[:, P:].shape)
    v2[:, P:] = rng.standard_normal(v2[:, P:].shape)
    full2, _ = att.attention(q, k2, v2, ids, "block_causal")
    assert np.array_equal(full2[:, :P], full[:, :P])


def _nested(a):
    return a.tolist()


def pin_bruteforce_tiny():
    """The vectorised oracle equals explicit loops on the pages' tiny shapes:
    the tiny fp32 layout (2 heads x 32, text 16 + 1x4x4), the Lumina mini test
    (3 heads over 1 KV head, head_dim 8, 2D rope 4+4 on a 4x4 grid) and the
    NucleusMoE dummy test's axes (8, 4, 4) (head_dim 16)."""
    rng = np.random.default_rng(13)
    cases = [((("T", 16), ("I", 1, 4, 4)), 2, 2, 32, (4, 14, 14), "centered_fhw", "block_causal"),
             ((("I", 1, 4, 4),), 3, 1, 8, (4, 4), "grid_hw", "full"),
             ((("T", 5), ("I", 1, 2, 4), ("T", 2), ("I", 1, 2, 2)), 2, 1, 16, (8, 4, 4), "centered_fhw",
              "block_causal")]
    for layout, H, Hk, D, axes, pos_mode, mode in cases:
        mask, shapes = _layout_inputs(layout)
        md = meta.build_token_metadata(mask, shapes, pos_mode)
        S = len(mask)
        q = qr.qknorm_rope(rng.standard_normal((1, S, H, D)), np.ones(D), 1e-6, md["pos_ids"], axes)
        k = qr.qknorm_rope(rng.standard_normal((1, S, Hk, D)), np.ones(D), 1e-6, md["pos_ids"], axes)
        v = rng.standard_normal((1, S, Hk, D))
        o, lse = att.attention(q, k, v, md["image_ids"], mode)
        ob, lb = att.attention_bruteforce(_nested(q), _nested(k), _nested(v), list(md["image_ids"]), mode)
        assert np.allclose(o, np.asarray(ob), rtol=1e-11, atol=1e-13), layout
        assert np.allclose(lse, np.asarray(lb), rtol=1e-11, atol=1e-13), layout


def pin_lse_definition():
    """lse is log sum_k exp(logit_k) over allowed keys: with V = identity-like
    one-hot values the output row is exp(logit - lse) per key (torch.logsumexp
    cross-check on a tiny block-causal case)."""
    mask, shapes = _layout_inputs((("T", 3), ("I", 1, 2, 2)))
    ids = meta.build_token_metadata(mask, shapes)["image_ids"]
    S, D = 7, 8
    rng = np.random.default_rng(14)
    q, k = (rng.standard_normal((1, S, 1, D)) for _ in range(2))
    v = np.zeros((1, S, 1, S))
    v[0, :, 0, :] = np.eye(S)
    o, lse = att.attention(q, k, v, ids, "block_causal")
    logits = torch.from_numpy(q[0, :, 0] @ k[0, :, 0].T / math.sqrt(D))
    allowed = torch.tensor([[j <= i or (ids[i] >= 0 and ids[i] == ids[j]) for j in range(S)] for i in range(S)])
    ref_lse = torch.logsumexp(logits.masked_fill(~allowed, -math.inf), dim=1).numpy()
    assert np.allclose(lse[0, 0], ref_lse, rtol=1e-12, atol=1e-13)
    probs = torch.softmax(logits.masked_fill(~allowed, -math.inf), dim=1).numpy()
    assert np.allclose(o[0, :, 0, :], probs, rtol=1e-12, atol=1e-14)


# --------------------------------------------------------------------------- key padding
def pin_key_padding_fixtures():
    """Hand-derived: the j-th text token of the joint sequence takes the j-th
    flag of the per-sample text mask, image tokens are always valid
    (QwenImage21Transformer2DModel API page, forward's
    encoder_hidden_states_mask); a mask of the wrong length is a data error."""
    # sequence: text, text, image, image, text, image
    got = kp.joint_key_valid([0, 0, 1, 1, 0, 1], [[1, 0, 1], [0, 1, 1]])
    assert got.tolist() == [[True, False, True, True, True, True],
                            [False, True, True, True, True, True]]
    # text after the images (condition-image layouts put text between blocks)
    got = kp.joint_key_valid([1, 1, 0, 0], [[0, 1]])
    assert got.tolist() == [[True, True, False, True]]
    try:
        kp.joint_key_valid([0, 1, 0], [[1, 1, 1]])
    except kp.KeyPaddingError:
        pass
    else:
        raise AssertionError("a text mask of the wrong length must be rejected")


def _sdpa_masked(q, k, v, allowed):
    """torch SDPA, float64, CPU, boolean attn_mask (True = attend); BSHD."""
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x.transpose(0, 2, 1, 3))) for x in (q, k, v))
    o = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=torch.from_numpy(allowed))
    return o.numpy().transpose(0, 2, 1, 3)


def pin_key_padding_is_masked_sdpa():
    """Block-causal attention with per-sample padded text keys equals torch SDPA
    given the literal predicate AND the key flags; with every key valid it
    equals attention without padding."""
    mask, shapes = _layout_inputs((("T", 9), ("I", 1, 2, 4), ("T", 4), ("I", 1, 2, 2)))
    ids = meta.build_token_metadata(mask, shapes)["image_ids"]
    S = len(mask)
    rng = np.random.default_rng(21)
    q, k, v = (rng.standard_normal((2, S, 2, 8)) for _ in range(3))
    n_text = int((np.asarray(mask) == 0).sum())
    tv = rng.random((2, n_text)) < 0.6
    tv[:, 0] = True  # keep one valid key for every row (rows without any are pinned below)
    valid = kp.joint_key_valid(mask, tv)
    o, _ = att.attention(q, k, v, ids, "block_causal", key_valid=valid)
    pred = np.array([[j <= i or (ids[i] >= 0 and ids[i] == ids[j]) for j in range(S)] for i in range(S)])
    for b in range(2):
        ref = _sdpa_masked(q[b:b + 1], k[b:b + 1], v[b:b + 1], pred & valid[b][None, :])
        assert np.allclose(o[b:b + 1], ref, rtol=1e-10, atol=1e-12), b
    o_all, lse_all = att.attention(q, k, v, ids, "block_causal", key_valid=np.ones((2, S), bool))
    o_ref, lse_ref = att.attention(q, k, v, ids, "block_causal")
    assert np.array_equal(o_all, o_ref) and np.array_equal(lse_all, lse_ref)


def pin_key_padding_is_compaction():
    """Under the full mask, padded keys behave as if they were removed: equal to
    torch SDPA over K and V with those rows deleted."""
    rng = np.random.default_rng(22)
    S = 20
    q, k, v = (rng.standard_normal((1, S, 3, 16)) for _ in range(3))
    valid = np.ones((1, S), bool)
    valid[0, [2, 3, 11, 19]] = False
    o, _ = att.attention(q, k, v, np.zeros(S, int), "full", key_valid=valid)
    keep = valid[0]
    ref = _sdpa(q, k[:, keep], v[:, keep])
    assert np.allclose(o, ref, rtol=1e-10, atol=1e-12)


def pin_key_padding_bruteforce_and_empty_rows():
    """Vectorised == loops with padding; a row whose allowed keys are all padded
    (leading padded text under the block-causal rule) has output 0 and lse -inf."""
    mask, shapes = _layout_inputs((("T", 4), ("I", 1, 2, 2)))
    ids = meta.build_token_metadata(mask, shapes)["image_ids"]
    S = len(mask)
    rng = np.random.default_rng(23)
    q, k, v = (rng.standard_normal((2, S, 2, 4)) for _ in range(3))
    valid = kp.joint_key_valid(mask, [[0, 0, 1, 1], [1, 0, 0, 1]])
    o, lse = att.attention(q, k, v, ids, "block_causal", key_valid=valid)
    ob, lb = att.attention_bruteforce(_nested(q), _nested(k), _nested(v), list(ids), "block_causal",
                                      key_valid=valid.tolist())
    assert np.allclose(o, np.asarray(ob), rtol=1e-11, atol=1e-13)
    assert np.allclose(lse, np.asarray(lb), rtol=1e-11, atol=1e-13)
    # sample 0: rows 0 and 1 see only keys 0..1, both padded
    assert np.all(o[0, :2] == 0.0) and np.all(np.isneginf(lse[0, :, :2]))
    assert np.all(np.isfinite(lse[0, :, 2:])) and np.all(np.isfinite(lse[1]))


# --------------------------------------------------------------------------- the composed step
def pin_pipeline_step():
    """The composed step (oracle.pipeline).
    1. Text only, no cache: O equals causal torch SDPA (float64, CPU) over the
       normed and rotated Q and K at the metadata's positions, and the query
       rows asked for equal the same rows of the whole output.
    2. The "extract" then "cached" flow (QwenImage21Transformer2DModel API
       page, forward's kv_cache modes; the causal_condition note): on a
       layout [text, condition image, text, target image] the full step's
       target rows equal a cached step over the target tokens alone whose
       cache is rows [0, P) of the full step's K' and raw V, for O, lse and
       the target tokens' K'; with padded text keys too."""
    rng = np.random.default_rng(31)
    axes = (4, 6, 6)
    D = sum(axes)
    mask, shapes = _layout_inputs((("T", 11),))
    md = meta.build_token_metadata(mask, shapes)
    S = len(mask)
    vals = {"q": rng.standard_normal((2, S, 4, D)), "k": rng.standard_normal((2, S, 2, D)),
            "v": rng.standard_normal((2, S, 2, D)), "wq": 1 + 0.1 * rng.standard_normal(D),
            "wk": 1 + 0.1 * rng.standard_normal(D)}
    out = pipe.step(vals, md, axes=axes, eps=1e-6, mask_mode="block_causal")
    qp = qr.qknorm_rope(vals["q"], vals["wq"], 1e-6, md["pos_ids"], axes)
    kp_ = qr.qknorm_rope(vals["k"], vals["wk"], 1e-6, md["pos_ids"], axes)
    ke = torch.repeat_interleave(torch.from_numpy(kp_), 2, dim=2).numpy()
    ve = torch.repeat_interleave(torch.from_numpy(vals["v"]), 2, dim=2).numpy()
    assert np.allclose(out["o"], _sdpa(qp, ke, ve, is_causal=True), rtol=1e-10, atol=1e-12)
    sub = pipe.step(vals, md, axes=axes, eps=1e-6, mask_mode="block_causal", rows=[0, 5, 10])
    assert np.allclose(sub["o"], out["o"][:, [0, 5, 10]], rtol=1e-12, atol=1e-14)

    layout = (("T", 5), ("I", 1, 2, 2), ("T", 3), ("I", 1, 2, 4))
    mask, shapes = _layout_inputs(layout)
    md = meta.build_token_metadata(mask, shapes)
    S, P = len(mask), 12
    vals = {"q": rng.standard_normal((2, S, 4, D)), "k": rng.standard_normal((2, S, 2, D)),
            "v": rng.standard_normal((2, S, 2, D)), "wq": 1 + 0.1 * rng.standard_normal(D),
            "wk": 1 + 0.1 * rng.standard_normal(D)}
    tv = np.array([[1, 1, 0, 1, 1, 0, 1, 1], [1, 0, 1, 1, 1, 1, 1, 0]], bool)
    for key_valid in (None, kp.joint_key_valid(mask, tv)):
        full = pipe.step(vals, md, axes=axes, eps=1e-6, mask_mode="block_causal", key_valid=key_valid)
        new = {n: vals[n][:, P:] for n in ("q", "k", "v")}
        new.update(wq=vals["wq"], wk=vals["wk"], **pipe.extract_cache(full, vals["v"], P))
        cached = pipe.step(new, md, axes=axes, eps=1e-6, mask_mode="block_causal", prefix_len=P,
                           key_valid=key_valid)
        assert np.allclose(cached["o"], full["o"][:, P:], rtol=1e-12, atol=1e-14)
        assert np.allclose(cached["lse"], full["lse"][:, :, P:], rtol=1e-12, atol=1e-14)
        assert np.allclose(cached["k_prime"], full["k_prime"][:, P:], rtol=1e-12, atol=1e-14)


ALL_PINS = [pin_metadata_goldens, pin_kv_limit_is_predicate_prefix, pin_metadata_errors,
            pin_rmsnorm_closed_forms, pin_rope_rotation, pin_rope_pairing_and_ladder, pin_rope_relative,
            pin_full_is_sdpa, pin_text_only_is_causal, pin_gqa_is_repeat_interleave,
            pin_singlepass_equals_multipass, pin_adjacent_blocks_stay_separate, pin_cached_equals_full,
            pin_bruteforce_tiny, pin_lse_definition, pin_key_padding_fixtures, pin_key_padding_is_masked_sdpa,
            pin_key_padding_is_compaction, pin_key_padding_bruteforce_and_empty_rows, pin_layernorm_across_heads,
            pin_scaled_rope, pin_time_aware_factors, pin_cfg_norm_rescale, pin_pipeline_step]
