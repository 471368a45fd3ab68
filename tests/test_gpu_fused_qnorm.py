"""GPU parity of attention on raw Q (dit_attn_forward_cached_qnorm): the
kernel applies Q's per-head RMSNorm, its rotary embedding and the softmax
scale as it loads Q, with K normed by dit_attn_qknorm_rope_ex in its K-only
form.  Checked through the C ABI against the fp64 oracle (every element on
small cases with several query and key tiles and ragged tails, with and
without rotary factors; sampled rows at full size), and the fused output
against the two-kernel path.  Inputs come from the seeded generator in
``workloads``; nothing expected comes from the GPU.
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
                               rne_bf16, sample_rows, to_device, to_host)

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


def _check_lse(gpu_lse: np.ndarray, ref: np.ndarray, what="lse"):
    dead = np.isneginf(ref)
    assert np.array_equal(np.isneginf(gpu_lse), dead), "%s: -inf rows differ" % what
    assert_parity(np.where(dead, 0.0, gpu_lse), np.where(dead, 0.0, ref), "f32", what, atol=1e-2)


def _fused(dit, w, d, m, kv=None, unit=False):
    """K-only norm, then attention on raw Q into NaN-filled O and lse
    buffers; returns (o, lse, k')."""
    P = w.prefix_len
    q, k, v = (to_device(d.bits[n], w.dtype) for n in ("q", "k", "v"))
    wq = None if unit else to_device(d.bits["wq"], w.dtype)
    wk = None if unit else to_device(d.bits["wk"], w.dtype)
    rk = dict(rope_linear_factor=w.rope_linear, rope_ntk_factor=w.rope_ntk)
    qo, kp = dit.dit_attn_qknorm_rope_ex(None, k, m.pos_ids[P:], w.axes, w.eps, k_weight=wk, **rk)
    assert qo is None
    kc = to_device(d.bits["k_cache"], w.dtype) if P else None
    vc = to_device(d.bits["v_cache"], w.dtype) if P else None
    o, lse = nan_outputs(q)
    dit.forward_cached_qnorm(q, kc, vc, kp, v, m.pos_ids[P:], w.axes, w.eps, q_weight=wq, mask_mode=w.mask_mode,
                             meta=m, key_valid=kv, out=o, lse_out=lse, **rk)
    torch.cuda.synchronize()
    return o, lse, kp


FUSED_CASES = [
    # (B, H, Hk, D, layout, axes, mask_mode, prefix, unit weights, text mask[, linear, ntk])
    (2, 4, 2, 128, (("T", 100), ("I", 1, 6, 10), ("T", 37), ("I", 1, 4, 8)), (16, 56, 56), "block_causal", 0,
     False, None),
    (2, 4, 2, 128, (("T", 100), ("I", 1, 6, 10), ("T", 37), ("I", 1, 4, 8)), (32, 48, 48), "full", 0, True, None),
    (1, 6, 3, 72, (("I", 1, 14, 22),), (24, 24, 24), "full", 0, False, None),
    (2, 4, 2, 80, (("T", 90), ("I", 1, 10, 12)), (16, 32, 32), "block_causal", 45, False, "random"),
    (2, 2, 1, 16, (("T", 5), ("I", 1, 2, 4), ("T", 70), ("I", 1, 8, 8)), (4, 6, 6), "block_causal", 0, False, None),
    (1, 4, 4, 64, (("T", 256), ("I", 1, 8, 8), ("I", 1, 8, 8), ("T", 30), ("I", 1, 10, 16)), (16, 24, 24),
     "block_causal", 0, False, None),
    (1, 4, 2, 128, (("T", 130), ("I", 1, 4, 8), ("I", 1, 10, 20)), (16, 56, 56), "block_causal", 162, False, None),
    (1, 2, 2, 128, (("T", 64), ("I", 1, 8, 8), ("I", 1, 16, 16)), (16, 56, 56), "block_causal", 128, True, None),
    (2, 3, 3, 96, (("T", 40), ("I", 1, 6, 6), ("T", 9)), (32, 32, 32), "block_causal", 17, False, None),
    (2, 4, 2, 128, (("T", 100), ("I", 1, 6, 10), ("T", 37), ("I", 1, 4, 8)), (16, 56, 56), "block_causal", 0,
     False, "random"),
    (2, 4, 2, 128, (("T", 130), ("I", 1, 4, 8), ("I", 1, 10, 20)), (16, 56, 56), "full", 130, False, "right"),
    (2, 2, 2, 32, (("T", 70), ("I", 1, 6, 6)), (8, 12, 12), "block_causal", 64, False, "random"),
    (1, 1, 1, 128, (("T", 1),), (16, 56, 56), "block_causal", 0, False, None),
    (1, 2, 1, 8, (("I", 1, 4, 6),), (4, 2, 2), "full", 0, False, None),
    # head dim 72 on the 80-channel instance with a 64-aligned cached prefix and padded text (GQA 4:1)
    (2, 4, 1, 72, (("T", 64), ("I", 1, 8, 12), ("T", 20)), (24, 24, 24), "block_causal", 64, False, "right"),
    # time-aware rotary scaling (the Lumina-Next factors) with the per-head RMSNorm
    (2, 4, 2, 72, (("I", 1, 12, 18),), (24, 24, 24), "full", 0, False, None, 2.0, 1.0),
    (1, 4, 4, 128, (("T", 70), ("I", 1, 8, 12)), (16, 56, 56), "block_causal", 64, False, None, 1.0, 3.0),
]


def _case_id(c):
    S = sum(s[1] if s[0] == "T" else s[1] * s[2] * s[3] for s in c[4])
    return "B%dH%d_%dD%d_%s_S%dP%d%s%s%s" % (c[0], c[1], c[2], c[3], c[6], S, c[7], "_unit" if c[8] else "",
                                           "_" + c[9] if c[9] else "",
                                           "_lin%g_ntk%g" % c[10:12] if len(c) > 10 else "")


@pytest.mark.parametrize("case", FUSED_CASES, ids=_case_id)
def test_fused_qnorm_attention_all_rows(dit, case):
    """Every element of O and the lse, and of K' from the K-only norm, against
    the oracle.  Q' comes from the oracle in fp64 from
    the raw Q, so the kernel's Q norm, rotation and scale are all checked.
    The attention's inputs in this data flow are bf16: Q' times the folded
    scale c = log2(e)/sqrt(D), rounded once, and K' as the norm kernel stores
    it.  The reference O and lse take the oracle's Q' and K' through those
    same two roundings.  (Rows with one to three valid keys, which random
    text padding makes, move by up to ~1e-2 under these roundings alone, as
    they do in the two-kernel path.)  Without padding every output is also
    held to the bar against the unrounded oracle's Q' and K'."""
    B, H, Hk, D, layout, axes, mode, P, unit, kind = case[:10]
    lin, ntk = case[10:12] if len(case) > 10 else (1.0, 1.0)
    w = wl.small_workload("f", B, H, Hk, D, layout, axes, mask_mode=mode, seed=5 * D + P, prefix_len=P,
                          unit_weights=unit, rope_linear=lin, rope_ntk=ntk)
    _say("fused qnorm attention %s" % _case_id(case))
    d = wl.draw(w)
    mask, shapes = wl.sequence_inputs(w)
    md = ometa.build_token_metadata(mask, shapes)
    m = dit.build_token_metadata(torch.from_numpy(mask).cuda(), shapes)
    m.check()
    kv, valid = None, None
    if kind is not None:
        tv = wl.text_mask(w, D + P, kind)
        valid = okp.joint_key_valid(mask, tv)
        kv = dit.build_key_valid(torch.from_numpy(mask).cuda(), torch.from_numpy(tv).cuda())
        kv.check()
    o, lse, kp = _fused(dit, w, d, m, kv, unit)
    pos = md["pos_ids"][P:]
    okw = dict(linear_factor=lin, ntk_factor=ntk)
    rq = oqr.qknorm_rope(d.vals["q"], d.vals["wq"], w.eps, pos, axes, **okw)
    rk = oqr.qknorm_rope(d.vals["k"], d.vals["wk"], w.eps, pos, axes, **okw)
    assert_parity(to_host(kp), rk, "bf16", "k'")
    c = dit.prescaled_q_factor(D)
    rq_in, rk_in = rne_bf16(rq * c) / c, rne_bf16(rk)
    k_all = np.concatenate([d.vals["k_cache"], rk_in], axis=1) if P else rk_in
    v_all = np.concatenate([d.vals["v_cache"], d.vals["v"]], axis=1) if P else d.vals["v"]
    ro, rl = oatt.attention(rq_in, k_all, v_all, md["image_ids"], mode, q_offset=P, key_valid=valid)
    assert_all_written(o, lse, "fused", lse_may_be_neg_inf=kind is not None)
    assert_parity(to_host(o), ro, "bf16", "O")
    _check_lse(lse.cpu().double().numpy(), rl)
    if kind is None:
        k_all = np.concatenate([d.vals["k_cache"], rk], axis=1) if P else rk
        ro_u, rl_u = oatt.attention(rq, k_all, v_all, md["image_ids"], mode, q_offset=P)
        assert_parity(to_host(o), ro_u, "bf16", "O (unrounded Q', K')")
        _check_lse(lse.cpu().double().numpy(), rl_u, "lse (unrounded Q', K')")


def test_fused_matches_two_kernel_path(dit):
    """Fused and unfused (norm kernel with the folded scale, then attention
    with scale ln 2) compute the same rounded Q' up to the summation order of
    the sum of squares: both within the oracle bar, and almost every output
    element bit-identical."""
    w = wl.small_workload("f", 2, 8, 4, 128, (("T", 300), ("I", 1, 16, 24), ("T", 20), ("I", 1, 12, 20)),
                          (16, 56, 56), seed=77)
    d = wl.draw(w)
    mask, shapes = wl.sequence_inputs(w)
    m = dit.build_token_metadata(torch.from_numpy(mask).cuda(), shapes)
    m.check()
    o_f, lse_f, kp_f = _fused(dit, w, d, m)
    q, k, v = (to_device(d.bits[n], w.dtype) for n in ("q", "k", "v"))
    wq, wk = to_device(d.bits["wq"], w.dtype), to_device(d.bits["wk"], w.dtype)
    qp, kp = dit.qknorm_rope(q, k, m.pos_ids, w.axes, w.eps, wq, wk, q_scale=dit.prescaled_q_factor(128))
    o_u, lse_u = dit.forward(qp, kp, v, w.mask_mode, m, softmax_scale=dit.LN2, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(kp_f, kp)
    same = float((o_f == o_u).float().mean())
    _say("  fused vs two-kernel: %.4f of O bit-identical, max |dO| %.3g" % (
        same, float((o_f.float() - o_u.float()).abs().max())))
    assert same >= 0.95
    assert_parity(to_host(o_f), to_host(o_u), "bf16", "O fused vs unfused")
    assert_parity(lse_f.cpu().double().numpy(), lse_u.cpu().double().numpy(), "f32", "lse", atol=1e-3)


def test_k_only_norm_every_kernel(dit):
    """K-only form of dit_attn_qknorm_rope_ex on each norm kernel (per-head,
    flat, LayerNorm across heads), with the rotary factors: K' against the
    oracle; with the RMSNorm also bit-identical to K' of the call with Q (each
    head's sum of squares has the same order either way; the LayerNorm's block
    reduction is laid out over all the token's items, so only parity holds)."""
    cases = [
        (2, 32, 8, 128, (16, 56, 56), "rms_per_head", 1.0, 1.0),      # per-head kernel
        (3, 2, 1, 48, (16, 16, 16), "rms_per_head", 1.0, 1.0),        # flat kernel (6 chunks per head)
        (2, 32, 8, 72, (24, 24, 24), "rms_per_head", 1.0, 2.0),       # flat, 7 tokens per work-group
        (1, 6, 3, 72, (24, 24, 24), "rms_per_head", 1.0, 1.0),        # flat, 3 tokens per work-group
        (2, 4, 2, 72, (24, 24, 24), "layer_across_heads", 2.0, 1.0),
        (1, 4, 4, 64, (16, 24, 24), "rms_per_head", 1.0, 3.0),
    ]
    for B, H, Hk, D, axes, norm, lin, ntk in cases:
        w = wl.small_workload("t", B, H, Hk, D, (("T", 33), ("I", 1, 6, 8), ("I", 1, 10, 12)), axes, seed=D,
                              qk_norm=norm, rope_linear=lin, rope_ntk=ntk)
        _say("k only %s D%d H%d/%d lin %g ntk %g" % (norm, D, H, Hk, lin, ntk))
        d = wl.draw(w)
        mask, shapes = wl.sequence_inputs(w)
        md = ometa.build_token_metadata(mask, shapes)
        m = dit.build_token_metadata(torch.from_numpy(mask).cuda(), shapes)
        q, k = to_device(d.bits["q"], "bf16"), to_device(d.bits["k"], "bf16")
        wq, wk = to_device(d.bits["wq"], "bf16"), to_device(d.bits["wk"], "bf16")
        kw = dict(norm=norm, k_weight=wk, rope_linear_factor=lin, rope_ntk_factor=ntk)
        if norm == "layer_across_heads":
            kw["k_bias"] = to_device(d.bits["bk"], "bf16")
        qkw = dict(q_weight=wq, q_bias=to_device(d.bits["bq"], "bf16") if norm == "layer_across_heads" else None)
        _, kp = dit.dit_attn_qknorm_rope_ex(q, k, m.pos_ids, axes, w.eps, **kw, **qkw)
        none, kp2 = dit.dit_attn_qknorm_rope_ex(None, k, m.pos_ids, axes, w.eps, **kw)
        torch.cuda.synchronize()
        assert none is None
        okw = dict(norm=norm, linear_factor=lin, ntk_factor=ntk)
        rk = oqr.qknorm_rope(d.vals["k"], d.vals["wk"], w.eps, md["pos_ids"], axes,
                             bias=d.vals["bk"] if norm == "layer_across_heads" else None, **okw)
        assert_parity(to_host(kp2), rk, "bf16", "k' (K only)")
        if norm == "rms_per_head":
            assert torch.equal(kp2, kp)
        else:
            assert_parity(to_host(kp), rk, "bf16", "k' (with Q)")


FULL = [n for n in list(wl.WORKLOADS) + list(wl.VARIANTS)
        if wl.get(n).dtype == "bf16" and wl.get(n).qk_norm == "rms_per_head"]


@pytest.mark.parametrize("name", FULL)
def test_fused_workloads_sampled(dit, name):
    """The fused step at full size, in the launch configuration the benchmark
    times: every element of O and lse written, and sampled query rows (at
    least one in every 128-row query tile) against the unrounded oracle."""
    w = wl.get(name)
    _say("fused workload %s" % name)
    d = wl.draw(w)
    mask, shapes = wl.sequence_inputs(w)
    md = ometa.build_token_metadata(mask, shapes, w.pos_mode)
    m = dit.build_token_metadata(torch.from_numpy(mask).cuda(), shapes, w.pos_mode)
    m.check()
    o, lse, _ = _fused(dit, w, d, m)
    assert_all_written(o, lse, name)
    P = w.prefix_len
    rows = sample_rows(w)
    pos = md["pos_ids"][P:]
    qp = oqr.qknorm_rope(d.vals["q"][:, rows], d.vals["wq"], w.eps, pos[rows], w.axes)
    kp = oqr.qknorm_rope(d.vals["k"], d.vals["wk"], w.eps, pos, w.axes)
    k_all = np.concatenate([d.vals["k_cache"], kp], axis=1) if P else kp
    v_all = np.concatenate([d.vals["v_cache"], d.vals["v"]], axis=1) if P else d.vals["v"]
    ro, rl = oracle_rows(oatt.attention, qp, k_all, v_all, md["image_ids"], w.mask_mode, P, rows)
    idx = torch.from_numpy(rows).cuda()
    stats = assert_parity(to_host(o[:, idx]), ro, "bf16", "O")
    lit = assert_literal_mean(to_host(o[:, idx]), ro, "O")
    assert_parity(lse[:, :, idx].cpu().double().numpy(), rl, "f32", "lse", atol=1e-2)
    _say("  %s rows=%d max=%.3g mean=%.3g (unrounded %.3g)" % (name, rows.size, stats["max"], stats["mean"], lit))


def test_fused_padded_workload_sampled(dit):
    """The headline workload with right-padded text, fused: sampled rows."""
    w = wl.get("qwen_image21_t1024_i64x64")
    d = wl.draw(w)
    mask, shapes = wl.sequence_inputs(w)
    md = ometa.build_token_metadata(mask, shapes, w.pos_mode)
    m = dit.build_token_metadata(torch.from_numpy(mask).cuda(), shapes, w.pos_mode)
    tv = wl.text_mask(w, 12, "right")
    valid = okp.joint_key_valid(mask, tv)
    kv = dit.build_key_valid(torch.from_numpy(mask).cuda(), torch.from_numpy(tv).cuda())
    kv.check()
    o, lse, _ = _fused(dit, w, d, m, kv)
    assert_all_written(o, lse, "padded headline", lse_may_be_neg_inf=True)
    rows = sample_rows(w, seed=3)
    pos = md["pos_ids"]
    qp = oqr.qknorm_rope(d.vals["q"][:, rows], d.vals["wq"], w.eps, pos[rows], w.axes)
    kp = oqr.qknorm_rope(d.vals["k"], d.vals["wk"], w.eps, pos, w.axes)
    ro, rl = oracle_rows(oatt.attention, qp, kp, d.vals["v"], md["image_ids"], w.mask_mode, 0, rows,
                         key_valid=valid)
    idx = torch.from_numpy(rows).cuda()
    assert_parity(to_host(o[:, idx]), ro, "bf16", "O")
    assert_literal_mean(to_host(o[:, idx]), ro, "O")
    _check_lse(lse[:, :, idx].cpu().double().numpy(), rl)


def test_fused_strided_views_and_in_place_k(dit):
    """Q, K and V as views of one projection buffer (heads interleaved, a
    spare head between them), K normed in place, O written into a wider
    buffer: bit-identical to the same call on contiguous copies, and the
    spare head and the columns around O untouched."""
    B, H, Hk, D = 2, 4, 2, 128
    w = wl.small_workload("v", B, H, Hk, D, (("T", 77), ("I", 1, 8, 12), ("I", 1, 6, 10)), (16, 56, 56), seed=9)
    d = wl.draw(w)
    mask, shapes = wl.sequence_inputs(w)
    m = dit.build_token_metadata(torch.from_numpy(mask).cuda(), shapes)
    m.check()
    q, k, v = (to_device(d.bits[n], "bf16") for n in ("q", "k", "v"))
    wq, wk = to_device(d.bits["wq"], "bf16"), to_device(d.bits["wk"], "bf16")
    S = w.n_new
    qkv = torch.full((B, S, H + 2 * Hk + 1, D), 7.0, dtype=torch.bfloat16, device="cuda")
    qkv[:, :, :H] = q
    qkv[:, :, H:H + Hk] = k
    qkv[:, :, H + Hk + 1:] = v  # spare head H + Hk stays 7
    qv, kv, vv = qkv[:, :, :H], qkv[:, :, H:H + Hk], qkv[:, :, H + Hk + 1:]
    wide = torch.full((B, S, H + 1, D), -3.0, dtype=torch.bfloat16, device="cuda")
    ov = wide[:, :, 1:]
    dit.dit_attn_qknorm_rope_ex(None, kv, m.pos_ids, w.axes, w.eps, k_weight=wk, k_out=kv)
    dit.forward_cached_qnorm(qv, None, None, kv, vv, m.pos_ids, w.axes, w.eps, q_weight=wq, mask_mode=w.mask_mode,
                             meta=m, out=ov)
    _, kp = dit.dit_attn_qknorm_rope_ex(None, k, m.pos_ids, w.axes, w.eps, k_weight=wk)
    o = dit.forward_cached_qnorm(q, None, None, kp, v, m.pos_ids, w.axes, w.eps, q_weight=wq, mask_mode=w.mask_mode,
                                 meta=m)
    torch.cuda.synchronize()
    assert torch.equal(kv, kp)
    assert torch.equal(ov, o)
    assert torch.all(qkv[:, :, H + Hk] == 7.0) and torch.all(wide[:, :, 0] == -3.0)
    assert torch.equal(qv, q) and torch.equal(vv, v)
