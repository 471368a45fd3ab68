"""GPU parity of text key padding: the key-validity builder and the padded
attention entry points through the C ABI against the fp64 oracle.

Text masks come from the seeded generator in ``workloads`` ("right": a
tokenizer's right padding with a per-sample valid length; "random": an
independent coin per text token; plus hand-made masks that empty whole query
rows).  The oracle's ``key_padding.joint_key_valid`` maps them onto the joint
sequence; nothing expected comes from the GPU.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle.attention as oatt
import oracle.key_padding as okp
import oracle.metadata as ometa
import oracle.qknorm_rope as oqr
import workloads as wl
from tests.gpu_helpers import (assert_all_written, assert_literal_mean, assert_parity, nan_outputs, oracle_rows,
                               sample_rows, to_device, to_host)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dit():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu-marked tests need an MI355X")
    import diffusion_transformer_joint_token_amd as d
    return d


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def pack_bits(valid: np.ndarray) -> np.ndarray:
    """bool [B, S] -> uint64 [B, ceil(S/64)], bit j of word t = key 64 t + j."""
    B, S = valid.shape
    W = (S + 63) // 64
    padded = np.zeros((B, W * 64), dtype=np.uint64)
    padded[:, :S] = valid
    shifts = np.arange(64, dtype=np.uint64)
    return (padded.reshape(B, W, 64) << shifts).sum(axis=2, dtype=np.uint64)


def _gpu_bits(kv) -> np.ndarray:
    return kv.bits.cpu().numpy().view(np.uint64)


def _build(dit, mask: np.ndarray, tv: np.ndarray):
    kv = dit.build_key_valid(torch.from_numpy(mask).cuda(), torch.from_numpy(tv).cuda())
    kv.check()
    return kv


# --------------------------------------------------------------------------- builder
def _builder_cases():
    rng = np.random.default_rng(40)
    cases = []
    for name, w in wl.WORKLOADS.items():
        for kind in ("right", "random"):
            cases.append((w.layout, 3, kind, 7 + len(cases)))
    cases.append(((("T", 1),), 2, "random", 1))
    cases.append(((("I", 1, 4, 4), ("T", 63), ("I", 1, 2, 2), ("T", 65)), 2, "random", 2))
    cases.append(((("T", 64),), 1, "none", 3))
    for i in range(8):  # longer layouts: several 8192-token passes of the scan
        segs, n = [], 0
        while n < 20000:
            if rng.random() < 0.5:
                t = int(rng.integers(1, 900))
                segs.append(("T", t))
            else:
                hh, ww = 2 * int(rng.integers(1, 40)), 2 * int(rng.integers(1, 40))
                segs.append(("I", 1, hh, ww))
                t = hh * ww
            n += t
        cases.append((tuple(segs), 2, "random" if i % 2 else "right", 100 + i))
    return cases


def test_key_valid_bit_exact(dit):
    for layout, B, kind, seed in _builder_cases():
        w = wl.small_workload("kv", B, 1, 1, 8, layout, (8,))
        mask, _ = wl.sequence_inputs(w)
        tv = wl.text_mask(w, seed, kind)
        _say("key_valid S=%d B=%d %s" % (w.seq_len, B, kind))
        kv = _build(dit, mask, tv)
        torch.cuda.synchronize()
        ref = pack_bits(okp.joint_key_valid(mask, tv))
        got = _gpu_bits(kv)
        assert got.shape == ref.shape
        assert np.array_equal(got, ref), (layout[:4], kind)


def test_key_valid_strided_rows_and_status(dit):
    w = wl.small_workload("kv", 3, 1, 1, 8, (("T", 70), ("I", 1, 8, 8), ("T", 30)), (8,))
    mask, _ = wl.sequence_inputs(w)
    tv = wl.text_mask(w, 5, "random")
    # text mask rows inside a wider buffer, bits rows with spare words
    wide = torch.zeros(3, 128, dtype=torch.uint8, device="cuda")
    wide[:, :100] = torch.from_numpy(tv).cuda()
    out = dit.KeyValid(torch.full((3, 7), -1, dtype=torch.int64, device="cuda"),
                       torch.full((1,), -1, dtype=torch.int32, device="cuda"))
    dit.build_key_valid(torch.from_numpy(mask).cuda(), wide[:, :100], out=out)
    out.check()
    got = out.bits.cpu().numpy().view(np.uint64)
    ref = pack_bits(okp.joint_key_valid(mask, tv))
    assert np.array_equal(got[:, :3], ref)
    assert np.all(got[:, 3:] == np.uint64(0xFFFFFFFFFFFFFFFF))  # words past ceil(S/64) untouched
    # a text mask of the wrong length is a device data error
    for n in (99, 101):
        kv = dit.build_key_valid(torch.from_numpy(mask).cuda(), torch.ones(3, n, dtype=torch.uint8, device="cuda"))
        torch.cuda.synchronize()
        assert int(kv.status.item()) == 5
    # no text tokens at all: every key valid, n_text = 0
    mask2, _ = wl.sequence_inputs(wl.small_workload("kv", 2, 1, 1, 8, (("I", 1, 10, 10),), (8,)))
    kv = _build(dit, mask2, np.zeros((2, 0), dtype=np.uint8))
    ref = pack_bits(np.ones((2, 100), dtype=bool))
    assert np.array_equal(_gpu_bits(kv), ref)


# --------------------------------------------------------------------------- attention, every row
PAD_CASES = [
    # (B, H, Hk, D, layout, mask_mode, dtype, prefix, text mask)
    (2, 4, 2, 128, (("T", 100), ("I", 1, 6, 10), ("T", 37), ("I", 1, 4, 8)), "block_causal", "bf16", 0, "right"),
    (2, 4, 2, 128, (("T", 100), ("I", 1, 6, 10), ("T", 37), ("I", 1, 4, 8)), "full", "bf16", 0, "random"),
    (3, 6, 3, 72, (("T", 150), ("I", 1, 14, 22)), "full", "bf16", 0, "random"),
    (2, 4, 4, 80, (("T", 130), ("I", 1, 10, 12)), "block_causal", "bf16", 64, "right"),
    (2, 2, 1, 16, (("T", 5), ("I", 1, 2, 4), ("T", 70), ("I", 1, 8, 8)), "block_causal", "bf16", 0, "random"),
    (2, 4, 4, 64, (("T", 256), ("I", 1, 8, 8), ("T", 30), ("I", 1, 10, 16)), "block_causal", "bf16", 0, "lead"),
    (2, 4, 2, 128, (("T", 130), ("I", 1, 4, 8), ("I", 1, 10, 20)), "block_causal", "bf16", 162, "random"),
    (2, 2, 2, 128, (("T", 64), ("I", 1, 8, 8), ("I", 1, 16, 16)), "block_causal", "bf16", 128, "right"),
    (2, 2, 2, 32, (("T", 16), ("I", 1, 4, 4)), "block_causal", "f32", 0, "lead"),
    (2, 2, 2, 96, (("T", 40), ("I", 1, 6, 6), ("T", 9)), "block_causal", "f32", 17, "random"),
    (2, 3, 1, 128, (("T", 200),), "full", "bf16", 0, "empty"),
    (2, 3, 1, 64, (("T", 200),), "block_causal", "f32", 0, "empty"),
]


def _text_mask(w, kind, seed):
    if kind in ("right", "random"):
        return wl.text_mask(w, seed, kind)
    n = wl.n_text_tokens(w)
    tv = wl.text_mask(w, seed, "random")
    if kind == "lead":     # the first text tokens padded: early causal rows see no valid key
        tv[:, :7] = 0
        tv[1, :] = 0       # sample 1: every text token padded
    elif kind == "empty":  # sample 0 all padded (every row empty), sample 1 random
        tv[0, :] = 0
    assert tv.shape[1] == n
    return tv


def _case_id(c):
    return "B%dH%d_%dD%d_%s_%s_P%d_%s" % (c[0], c[1], c[2], c[3], c[5], c[6], c[7], c[8])


def _check_lse(gpu_lse: np.ndarray, ref: np.ndarray, dtype: str, what="lse"):
    dead = np.isneginf(ref)
    assert np.array_equal(np.isneginf(gpu_lse), dead), "%s: -inf rows differ" % what
    assert_parity(np.where(dead, 0.0, gpu_lse), np.where(dead, 0.0, ref), "f32", what,
                  atol=1e-2 if dtype == "bf16" else 1e-5)


@pytest.mark.parametrize("prescaled", [False, True], ids=["plain", "prescaled"])
@pytest.mark.parametrize("case", PAD_CASES, ids=_case_id)
def test_padded_attention_all_rows(dit, case, prescaled):
    B, H, Hk, D, layout, mode, dtype, P, kind = case
    w = wl.small_workload("p", B, H, Hk, D, layout, (D,), dtype=dtype, seed=3 * D + P, prefix_len=P)
    _say("padded attention %s %s" % (_case_id(case), "prescaled" if prescaled else "plain"))
    d = wl.draw(w)
    mask, shapes = wl.sequence_inputs(w)
    md = ometa.build_token_metadata(mask, shapes)
    m = dit.build_token_metadata(torch.from_numpy(mask).cuda(), shapes)
    m.check()
    tv = _text_mask(w, kind, D + P)
    valid = okp.joint_key_valid(mask, tv)
    kv = _build(dit, mask, tv)
    q_vals, q_bits, scale = d.vals["q"], d.bits["q"], None
    if prescaled:
        c = dit.prescaled_q_factor(D)
        if dtype == "bf16":
            q_bits = wl.bf16_round_bits((d.vals["q"] * c).astype(np.float32))
            q_vals = wl.bf16_bits_to_f64(q_bits) / c
        else:
            q_bits = (d.vals["q"] * c).astype(np.float32)
            q_vals = q_bits.astype(np.float64) / c
        scale = dit.LN2
    q = to_device(q_bits, dtype)
    k, v = (to_device(d.bits[n], dtype) for n in ("k", "v"))
    if P:
        kc, vc = to_device(d.bits["k_cache"], dtype), to_device(d.bits["v_cache"], dtype)
        o, lse = dit.forward_cached(q, kc, vc, k, v, mode, m, softmax_scale=scale, return_lse=True, key_valid=kv)
        k_all = np.concatenate([d.vals["k_cache"], d.vals["k"]], axis=1)
        v_all = np.concatenate([d.vals["v_cache"], d.vals["v"]], axis=1)
    else:
        o, lse = dit.forward(q, k, v, mode, m, softmax_scale=scale, return_lse=True, key_valid=kv)
        k_all, v_all = d.vals["k"], d.vals["v"]
    torch.cuda.synchronize()
    ro, rl = oatt.attention(q_vals, k_all, v_all, md["image_ids"], mode, q_offset=P, key_valid=valid)
    assert_parity(to_host(o), ro, dtype, "O")
    _check_lse(lse.cpu().double().numpy(), rl, dtype)
    if kind in ("lead", "empty"):
        assert np.isneginf(rl).any()  # the case does exercise rows with no valid key


@pytest.mark.parametrize("mode", ["block_causal", "full"])
def test_runs_of_empty_tiles(dit, mode):
    """Padded runs that empty whole 64-key tiles (the kernel never visits
    those tiles): a run at key 0, runs of odd and even tile counts, a run
    reaching the end of a text segment; sample 1 unpadded in the same launch."""
    layout = (("T", 400), ("I", 1, 8, 16), ("T", 300), ("I", 1, 10, 12))
    w = wl.small_workload("r", 2, 4, 2, 128, layout, (128,), seed=31, mask_mode=mode)
    d = wl.draw(w)
    mask, shapes = wl.sequence_inputs(w)
    md = ometa.build_token_metadata(mask, shapes)
    m = dit.build_token_metadata(torch.from_numpy(mask).cuda(), shapes)
    tv = np.ones((2, 700), dtype=np.uint8)
    for a, b in ((0, 150), (200, 330), (390, 520), (600, 700)):  # text ordinals
        tv[0, a:b] = 0
    valid = okp.joint_key_valid(mask, tv)
    kv = _build(dit, mask, tv)
    q, k, v = (to_device(d.bits[n], "bf16") for n in ("q", "k", "v"))
    o, lse = dit.forward(q, k, v, mode, m, return_lse=True, key_valid=kv)
    o1, lse1 = dit.forward(q[1:], k[1:], v[1:], mode, m, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oatt.attention(d.vals["q"], d.vals["k"], d.vals["v"], md["image_ids"], mode, key_valid=valid)
    assert_parity(to_host(o), ro, "bf16", "O")
    _check_lse(lse.cpu().double().numpy(), rl, "bf16")
    # the all-valid sample matches the unpadded kernel bit for bit
    assert torch.equal(o[1:], o1) and torch.equal(lse[1:], lse1)


def test_all_valid_bits_match_unpadded_bitwise(dit):
    """Every bit set: the padded kernels give the unpadded results bit for bit
    (bf16 and f32, plain and cached)."""
    for dtype, D, P in (("bf16", 128, 0), ("bf16", 72, 0), ("f32", 64, 0), ("bf16", 128, 130), ("bf16", 64, 192)):
        layout = (("T", 200), ("I", 1, 8, 8), ("I", 1, 12, 16))
        w = wl.small_workload("a", 2, 4, 2, D, layout, (D,), dtype=dtype, seed=D + P, prefix_len=P)
        d = wl.draw(w)
        mask, shapes = wl.sequence_inputs(w)
        m = dit.build_token_metadata(torch.from_numpy(mask).cuda(), shapes)
        ones = torch.full((2, (w.seq_len + 63) // 64), -1, dtype=torch.int64, device="cuda")
        q, k, v = (to_device(d.bits[n], dtype) for n in ("q", "k", "v"))
        for mode in ("block_causal", "full"):
            if P:
                kc, vc = to_device(d.bits["k_cache"], dtype), to_device(d.bits["v_cache"], dtype)
                a, la = dit.forward_cached(q, kc, vc, k, v, mode, m, return_lse=True)
                b, lb = dit.forward_cached(q, kc, vc, k, v, mode, m, return_lse=True, key_valid=ones)
            else:
                a, la = dit.forward(q, k, v, mode, m, return_lse=True)
                b, lb = dit.forward(q, k, v, mode, m, return_lse=True, key_valid=ones)
            torch.cuda.synchronize()
            assert torch.equal(a, b) and torch.equal(la, lb), (dtype, D, P, mode)


def test_padding_equals_dropping_the_keys(dit):
    """Image queries against a right-padded text prefix (cached entry point,
    full mask) equal the same queries against the prefix cut to its valid
    tokens; both within the bar of the oracle's padded attention."""
    L, n_text = 77, 128
    layout = (("T", n_text), ("I", 1, 8, 16))
    w = wl.small_workload("d", 1, 4, 4, 128, layout, (128,), seed=11, prefix_len=n_text, mask_mode="full")
    d = wl.draw(w)
    mask, shapes = wl.sequence_inputs(w)
    tv = np.zeros((1, n_text), dtype=np.uint8)
    tv[0, :L] = 1
    kv = _build(dit, mask, tv)
    q, k, v = (to_device(d.bits[n], "bf16") for n in ("q", "k", "v"))
    kc, vc = to_device(d.bits["k_cache"], "bf16"), to_device(d.bits["v_cache"], "bf16")
    o_pad = dit.forward_cached(q, kc, vc, k, v, "full", key_valid=kv)
    o_drop = dit.forward_cached(q, kc[:, :L].contiguous(), vc[:, :L].contiguous(), k, v, "full")
    torch.cuda.synchronize()
    ids = ometa.build_token_metadata(mask, shapes)["image_ids"]
    k_all = np.concatenate([d.vals["k_cache"], d.vals["k"]], axis=1)
    v_all = np.concatenate([d.vals["v_cache"], d.vals["v"]], axis=1)
    ref, _ = oatt.attention(d.vals["q"], k_all, v_all, ids, "full", q_offset=n_text,
                            key_valid=okp.joint_key_valid(mask, tv))
    assert_parity(to_host(o_pad), ref, "bf16", "O padded")
    assert_parity(to_host(o_drop), ref, "bf16", "O dropped")


# --------------------------------------------------------------------------- full-size workloads
PAD_WORKLOADS = ["qwen_image21_t1024_i64x64", "cond_images_t256_2x32x32_t256_i64x64",
                 "cached_prefix_decode_i128x128"]


@pytest.mark.parametrize("name", PAD_WORKLOADS)
def test_padded_pipeline_workloads(dit, name):
    """metadata + key validity -> norm+rope (prescaled Q) -> padded attention at
    full size, right-padded text (a per-sample valid length); sampled rows."""
    w = wl.WORKLOADS[name]
    _say("padded pipeline %s" % name)
    d = wl.draw(w)
    mask, shapes = wl.sequence_inputs(w)
    md = ometa.build_token_metadata(mask, shapes, w.pos_mode)
    m = dit.build_token_metadata(torch.from_numpy(mask).cuda(), shapes, w.pos_mode)
    m.check()
    tv = wl.text_mask(w, 2024, "right", min_valid=1)
    valid = okp.joint_key_valid(mask, tv)
    kv = _build(dit, mask, tv)
    P = w.prefix_len
    q, k, v = (to_device(d.bits[n], w.dtype) for n in ("q", "k", "v"))
    wq, wk = to_device(d.bits["wq"], w.dtype), to_device(d.bits["wk"], w.dtype)
    qp, kp = dit.qknorm_rope(q, k, m.pos_ids[P:], w.axes, w.eps, wq, wk,
                             q_scale=dit.prescaled_q_factor(w.head_dim))
    o, lse = nan_outputs(q)
    if P:
        kc, vc = to_device(d.bits["k_cache"], w.dtype), to_device(d.bits["v_cache"], w.dtype)
        dit.forward_cached(qp, kc, vc, kp, v, w.mask_mode, m, softmax_scale=dit.LN2, key_valid=kv, out=o,
                           lse_out=lse)
    else:
        dit.forward(qp, kp, v, w.mask_mode, m, softmax_scale=dit.LN2, key_valid=kv, out=o, lse_out=lse)
    torch.cuda.synchronize()
    # a right-padded prefix of at least one valid text token leaves every row a key
    assert_all_written(o, lse, name)
    rows = sample_rows(w)
    pos = md["pos_ids"][P:]
    rq = oqr.qknorm_rope(d.vals["q"][:, rows], d.vals["wq"], w.eps, pos[rows], w.axes)
    rk = oqr.qknorm_rope(d.vals["k"], d.vals["wk"], w.eps, pos, w.axes)
    k_all = np.concatenate([d.vals["k_cache"], rk], axis=1) if P else rk
    v_all = np.concatenate([d.vals["v_cache"], d.vals["v"]], axis=1) if P else d.vals["v"]
    ro, rl = oracle_rows(oatt.attention, rq, k_all, v_all, md["image_ids"], w.mask_mode, P, rows, key_valid=valid)
    idx = torch.from_numpy(rows).cuda()
    stats = assert_parity(to_host(o[:, idx]), ro, w.dtype, "O")
    assert_literal_mean(to_host(o[:, idx]), ro, "O")
    _check_lse(lse[:, :, idx].cpu().double().numpy(), rl, w.dtype)
    _say("  %s valid text %s rows=%d max=%.3g mean=%.3g" % (name, tv.sum(axis=1).tolist(), rows.size,
                                                            stats["max"], stats["mean"]))


# --------------------------------------------------------------------------- image-query joint attention
@pytest.mark.parametrize("kind", ["right", "random"])
@pytest.mark.parametrize("heads", [(4, 1), (4, 4)], ids=["gqa4", "mha"])
def test_image_query_attention_key_order(dit, kind, heads):
    """NucleusMoE-style attention: image queries over the image keys and the
    text keys, every pair allowed, padded text keys left out.  The GPU takes
    the text as the cached prefix (keys [text; image]); the oracle gets the
    keys in the article's order [image; text].  Under the full mask the key
    order is not part of the result."""
    H, Hk = heads
    n_text = 150
    layout = (("T", n_text), ("I", 1, 10, 12))
    w = wl.small_workload("n", 2, H, Hk, 128, layout, (16, 56, 56), seed=H + Hk, prefix_len=n_text,
                          mask_mode="full")
    d = wl.draw(w)
    mask, shapes = wl.sequence_inputs(w)
    tv = wl.text_mask(w, 17, kind)
    kv = _build(dit, mask, tv)
    q, k, v = (to_device(d.bits[n], "bf16") for n in ("q", "k", "v"))
    kc, vc = to_device(d.bits["k_cache"], "bf16"), to_device(d.bits["v_cache"], "bf16")
    o, lse = dit.forward_cached(q, kc, vc, k, v, "full", return_lse=True, key_valid=kv)
    torch.cuda.synchronize()
    n_img = w.n_new
    k_img_txt = np.concatenate([d.vals["k"], d.vals["k_cache"]], axis=1)
    v_img_txt = np.concatenate([d.vals["v"], d.vals["v_cache"]], axis=1)
    valid = np.concatenate([np.ones((2, n_img), bool), tv.astype(bool)], axis=1)
    ro, rl = oatt.attention(d.vals["q"], k_img_txt, v_img_txt, np.zeros(n_img + n_text, np.int32), "full",
                            key_valid=valid)
    assert_parity(to_host(o), ro, "bf16", "O")
    _check_lse(lse.cpu().double().numpy(), rl, "bf16")


def test_image_query_workload_sampled(dit):
    """The NucleusMoE image-query variant at full size (B 2, 16 heads x 128,
    1024 cached text keys of which a right-padded prefix is valid, 4096 image
    queries): metadata + key validity -> norm+rope (prescaled Q) -> padded
    cached attention, sampled rows against the oracle."""
    w = wl.get("nucleus_image_query_t1024_i64x64")
    _say("image-query variant %s" % w.name)
    d = wl.draw(w)
    mask, shapes = wl.sequence_inputs(w)
    md = ometa.build_token_metadata(mask, shapes, w.pos_mode)
    m = dit.build_token_metadata(torch.from_numpy(mask).cuda(), shapes, w.pos_mode)
    m.check()
    tv = wl.text_mask(w, 2024, "right")
    valid = okp.joint_key_valid(mask, tv)
    kv = _build(dit, mask, tv)
    P = w.prefix_len
    q, k, v = (to_device(d.bits[n], w.dtype) for n in ("q", "k", "v"))
    wq, wk = to_device(d.bits["wq"], w.dtype), to_device(d.bits["wk"], w.dtype)
    kc, vc = to_device(d.bits["k_cache"], w.dtype), to_device(d.bits["v_cache"], w.dtype)
    qp, kp = dit.qknorm_rope(q, k, m.pos_ids[P:], w.axes, w.eps, wq, wk,
                             q_scale=dit.prescaled_q_factor(w.head_dim))
    o, lse = nan_outputs(q)
    dit.forward_cached(qp, kc, vc, kp, v, "full", m, softmax_scale=dit.LN2, key_valid=kv, out=o, lse_out=lse)
    torch.cuda.synchronize()
    assert_all_written(o, lse, w.name)
    rows = sample_rows(w)
    pos = md["pos_ids"][P:]
    rq = oqr.qknorm_rope(d.vals["q"][:, rows], d.vals["wq"], w.eps, pos[rows], w.axes)
    rk = oqr.qknorm_rope(d.vals["k"], d.vals["wk"], w.eps, pos, w.axes)
    k_all = np.concatenate([d.vals["k_cache"], rk], axis=1)
    v_all = np.concatenate([d.vals["v_cache"], d.vals["v"]], axis=1)
    ro, rl = oatt.attention(rq, k_all, v_all, md["image_ids"], "full", q_offset=P, key_valid=valid)
    idx = torch.from_numpy(rows).cuda()
    stats = assert_parity(to_host(o[:, idx]), ro, w.dtype, "O")
    assert_literal_mean(to_host(o[:, idx]), ro, "O")
    _check_lse(lse[:, :, idx].cpu().double().numpy(), rl, w.dtype)
    _say("  valid text %s rows=%d max=%.3g mean=%.3g" % (tv.sum(axis=1).tolist(), rows.size, stats["max"],
                                                        stats["mean"]))


def test_metadata_and_key_valid_at_maximum_sizes(dit):
    """A ~250k-token joint sequence (multi-frame blocks, hundreds of 1024-token
    chunks, the checker's scan over the whole mask) and exactly MAX_IMAGES
    (64) image blocks: token metadata and key-validity bits bit-exact against
    the oracle.  One block more is refused on the host."""
    from diffusion_transformer_joint_token_amd import _lib
    big = (("T", 3000), ("I", 4, 160, 160), ("T", 777), ("I", 1, 256, 256), ("T", 5), ("I", 2, 200, 200))
    many = tuple(seg for _ in range(_lib.MAX_IMAGES) for seg in (("T", 3), ("I", 1, 2, 2)))
    for layout, tag in ((big, "250k tokens"), (many, "64 image blocks")):
        w = wl.small_workload("max", 2, 1, 1, 8, layout, (8,))
        mask, shapes = wl.sequence_inputs(w)
        _say("maximum sizes: %s (S=%d, %d blocks)" % (tag, w.seq_len, len(shapes)))
        ref = ometa.build_token_metadata(mask, shapes, "centered_fhw")
        m = dit.build_token_metadata(torch.from_numpy(mask).cuda(), shapes, "centered_fhw")
        m.check()
        for key in ("image_ids", "target_mask", "pos_ids", "kv_limit"):
            got = getattr(m, key).cpu().numpy()
            assert np.array_equal(got, ref[key].astype(got.dtype)), (tag, key)
        tv = wl.text_mask(w, 21, "random")
        kv = _build(dit, mask, tv)
        torch.cuda.synchronize()
        assert np.array_equal(_gpu_bits(kv), pack_bits(okp.joint_key_valid(mask, tv))), tag
    over = many + (("T", 3), ("I", 1, 2, 2))
    w = wl.small_workload("over", 1, 1, 1, 8, over, (8,))
    mask, shapes = wl.sequence_inputs(w)
    assert len(shapes) == _lib.MAX_IMAGES + 1
    with pytest.raises(dit.DitAttnError) as err:
        dit.build_token_metadata(torch.from_numpy(mask).cuda(), shapes, "centered_fhw")
    assert err.value.status == _lib.ERR_SHAPE
