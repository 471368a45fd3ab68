"""GPU parity of the Lumina-Next forms of the norm + rotary step: LayerNorm
across heads and the time-aware rotary factors (dit_attn_qknorm_rope_ex)
through the C ABI against the fp64 oracle; then the 2K extrapolation variant
workload end to end (sampled rows).  Inputs come from the seeded generator in
``workloads``; nothing expected comes from the GPU.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle.attention as oatt
import oracle.metadata as ometa
import oracle.qknorm_rope as oqr
import workloads as wl
from tests.gpu_helpers import (assert_all_written, assert_literal_mean, assert_parity, nan_outputs, sample_rows,
                               to_device, to_host)

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


def _meta(dit, w):
    mask, shapes = wl.sequence_inputs(w)
    m = dit.build_token_metadata(torch.from_numpy(mask).cuda(), shapes, w.pos_mode)
    m.check()
    return m, ometa.build_token_metadata(mask, shapes, w.pos_mode)


NORM_CASES = [
    # (B, H, Hk, D, axes, layout, pos_mode, dtype, unit weights, bias, linear, ntk)
    (2, 32, 8, 72, (36, 36), (("I", 1, 6, 10),), "grid_hw", "bf16", False, True, 1.0, 2.0),
    (1, 4, 2, 16, (8, 4, 4), (("T", 5), ("I", 1, 4, 8)), "centered_fhw", "bf16", False, True, 2.0, 1.0),
    (2, 6, 6, 128, (16, 56, 56), (("T", 20), ("I", 2, 4, 4)), "centered_fhw", "bf16", False, False, 1.0, 3.0),
    (1, 2, 1, 8, (4, 4), (("I", 1, 5, 6),), "grid_hw", "bf16", True, False, 3.0, 1.0),
    (2, 4, 4, 64, (32, 32), (("I", 1, 4, 9),), "grid_hw", "f32", False, True, 1.0, 2.0),
    (1, 3, 1, 32, (16, 16), (("I", 1, 8, 7),), "grid_hw", "f32", False, True, 2.0, 1.0),
    (1, 32, 32, 128, (16, 56, 56), (("T", 7), ("I", 1, 2, 4)), "centered_fhw", "bf16", False, True, 1.0, 1.0),
]


def _case_id(c):
    return "B%dH%d_%dD%d_%s_lin%g_ntk%g%s" % (c[0], c[1], c[2], c[3], c[7], c[10], c[11], "_bias" if c[9] else "")


@pytest.mark.parametrize("case", NORM_CASES, ids=_case_id)
def test_layernorm_across_heads_scaled_rope(dit, case):
    """Every element of Q' and K' (LayerNorm across heads with weight and bias,
    then scaled rotary), the Q scale, and in place on views of one fused
    buffer.  (32 + 32) heads x 16 chunks is the largest item count (1024 per
    token, 4 items per thread)."""
    B, H, Hk, D, axes, layout, mode, dtype, unit, bias, lin, ntk = case
    w = wl.small_workload("l", B, H, Hk, D, layout, axes, pos_mode=mode, dtype=dtype, unit_weights=unit,
                          seed=D + H, qk_norm="layer_across_heads", rope_linear=lin, rope_ntk=ntk, eps=1e-5)
    _say("layernorm across heads %s" % _case_id(case))
    d = wl.draw(w)
    m, md = _meta(dit, w)
    q, k = to_device(d.bits["q"], dtype), to_device(d.bits["k"], dtype)
    wq, wk = to_device(d.bits["wq"], dtype), to_device(d.bits["wk"], dtype)
    bq = to_device(d.bits["bq"], dtype) if bias else None
    bk = to_device(d.bits["bk"], dtype) if bias else None
    kw = dict(norm="layer_across_heads", q_bias=bq, k_bias=bk, rope_linear_factor=lin, rope_ntk_factor=ntk)
    qo, ko = dit.qknorm_rope(q, k, m.pos_ids, axes, w.eps, wq, wk, **kw)
    torch.cuda.synchronize()
    okw = dict(norm="layer_across_heads", linear_factor=lin, ntk_factor=ntk)
    rq = oqr.qknorm_rope(d.vals["q"], d.vals["wq"], w.eps, md["pos_ids"], axes, bias=d.vals["bq"] if bias else None,
                         **okw)
    rk = oqr.qknorm_rope(d.vals["k"], d.vals["wk"], w.eps, md["pos_ids"], axes, bias=d.vals["bk"] if bias else None,
                         **okw)
    assert_parity(to_host(qo), rq, dtype, "q'")
    assert_parity(to_host(ko), rk, dtype, "k'")
    qs, ks = dit.qknorm_rope(q, k, m.pos_ids, axes, w.eps, wq, wk, q_scale=0.3, **kw)
    torch.cuda.synchronize()
    assert_parity(to_host(qs), 0.3 * rq, dtype, "q' x 0.3")
    assert torch.equal(ks, ko)
    fused = torch.zeros(B, q.shape[1], H + 2 * Hk + 1, D, dtype=q.dtype, device="cuda")
    fused[:, :, :H] = q
    fused[:, :, H:H + Hk] = k
    qv, kv = fused[:, :, :H], fused[:, :, H:H + Hk]
    dit.qknorm_rope(qv, kv, m.pos_ids, axes, w.eps, wq, wk, inplace=True, **kw)
    torch.cuda.synchronize()
    assert torch.equal(qv, qo) and torch.equal(kv, ko)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_rms_with_scaled_rope_and_ex_identity(dit, dtype):
    """Per-head RMSNorm with both rotary factors against the oracle; with
    factors 1 the extended entry point equals the plain one bit for bit."""
    w = wl.small_workload("r", 2, 4, 2, 64, (("T", 30), ("I", 1, 6, 8)), (16, 24, 24), dtype=dtype, seed=11)
    d = wl.draw(w)
    m, md = _meta(dit, w)
    q, k = to_device(d.bits["q"], dtype), to_device(d.bits["k"], dtype)
    wq, wk = to_device(d.bits["wq"], dtype), to_device(d.bits["wk"], dtype)
    for lin, ntk in ((2.0, 1.0), (1.0, 2.5), (1.5, 3.0)):
        qo, ko = dit.qknorm_rope(q, k, m.pos_ids, w.axes, w.eps, wq, wk, rope_linear_factor=lin, rope_ntk_factor=ntk)
        torch.cuda.synchronize()
        rq = oqr.qknorm_rope(d.vals["q"], d.vals["wq"], w.eps, md["pos_ids"], w.axes, linear_factor=lin,
                             ntk_factor=ntk)
        rk = oqr.qknorm_rope(d.vals["k"], d.vals["wk"], w.eps, md["pos_ids"], w.axes, linear_factor=lin,
                             ntk_factor=ntk)
        assert_parity(to_host(qo), rq, dtype, "q' lin %g ntk %g" % (lin, ntk))
        assert_parity(to_host(ko), rk, dtype, "k' lin %g ntk %g" % (lin, ntk))
    a = dit.qknorm_rope(q, k, m.pos_ids, w.axes, w.eps, wq, wk, q_scale=0.7)
    b = dit.dit_attn_qknorm_rope_ex(q, k, m.pos_ids, w.axes, w.eps, q_weight=wq, k_weight=wk, q_scale=0.7)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_lumina_2k_variant_pipeline(dit):
    """The Lumina-Next 2K variant (B 2, 32 q / 8 kv heads x 72, 128x128 grid,
    LayerNorm across heads, NTK factor 2, full mask) through metadata ->
    norm+rope (prescaled Q) -> attention; sampled tokens of Q'/K' and sampled
    attention rows against the oracle."""
    w = wl.get("lumina_next_2k_lnheads_ntk2")
    _say("lumina 2k variant")
    d = wl.draw(w)
    m, md = _meta(dit, w)
    q, k, v = (to_device(d.bits[n], w.dtype) for n in ("q", "k", "v"))
    wq, wk, bq, bk = (to_device(d.bits[n], w.dtype) for n in ("wq", "wk", "bq", "bk"))
    kw = dict(norm=w.qk_norm, q_bias=bq, k_bias=bk, rope_linear_factor=w.rope_linear, rope_ntk_factor=w.rope_ntk)
    qp0, kp = dit.qknorm_rope(q, k, m.pos_ids, w.axes, w.eps, wq, wk, **kw)
    qp, _ = dit.qknorm_rope(q, k, m.pos_ids, w.axes, w.eps, wq, wk, q_scale=dit.prescaled_q_factor(w.head_dim), **kw)
    o, lse = nan_outputs(q)
    dit.forward(qp, kp, v, w.mask_mode, m, softmax_scale=dit.LN2, out=o, lse_out=lse)
    torch.cuda.synchronize()
    assert_all_written(o, lse, w.name)
    okw = dict(norm=w.qk_norm, linear_factor=w.rope_linear, ntk_factor=w.rope_ntk)
    rows = sample_rows(w, 40)
    idx = torch.from_numpy(rows).cuda()
    pos = md["pos_ids"]
    rq = oqr.qknorm_rope(d.vals["q"][:, rows], d.vals["wq"], w.eps, pos[rows], w.axes, bias=d.vals["bq"], **okw)
    rk = oqr.qknorm_rope(d.vals["k"], d.vals["wk"], w.eps, pos, w.axes, bias=d.vals["bk"], **okw)
    assert_parity(to_host(qp0[:, idx]), rq, w.dtype, "q'")
    assert_parity(to_host(kp[:, idx]), rk[:, rows], w.dtype, "k'")
    ro, rl = oatt.attention(rq, rk, d.vals["v"], md["image_ids"], w.mask_mode)
    stats = assert_parity(to_host(o[:, idx]), ro, w.dtype, "O")
    assert_literal_mean(to_host(o[:, idx]), ro, "O")
    assert_parity(lse[:, :, idx].cpu().double().numpy(), rl, "f32", "lse", atol=1e-2)
    _say("  rows=%d max=%.3g mean=%.3g" % (rows.size, stats["max"], stats["mean"]))
