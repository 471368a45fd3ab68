"""GPU parity of the "extract" then "cached" flow of a denoising loop
(QwenImage21Transformer2DModel API page, forward's kv_cache / kv_cache_mode,
and the causal_condition note that makes the text and condition keys
independent of the target).

Step 1 runs the whole joint sequence: the norm kernel writes K' of every
token, and rows [0, P) of that very buffer -- P = every token before the
target block -- are the cache, read in place with the raw V rows [0, P).
Later steps run only the target block: K' of its tokens at their own
positions [P, P + S_new), then the cached attention on its raw Q (Q's norm
and rotation inside the attention kernel, the benchmark's form).  The cached
step is checked against the oracle's own extract-then-cached flow
(oracle.pipeline) on sampled rows, at least one in every 128-row query tile
of the target, and against the full step's target rows on the device.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle.metadata as ometa
import oracle.pipeline as opipe
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


@pytest.mark.parametrize("name", ["qwen_image21_t1024_i64x64", "cond_images_t256_2x32x32_t256_i64x64"])
def test_extract_then_cached_step(dit, name):
    w = wl.get(name)
    last = w.layout[-1]
    assert last[0] == "I" and w.prefix_len == 0
    S = w.seq_len
    P = S - last[1] * last[2] * last[3]
    _say("extract then cached %s (prefix %d, target %d)" % (name, P, S - P))
    d = wl.draw(w, parts=("q", "k", "v", "wq", "wk"))
    mask, shapes = wl.sequence_inputs(w)
    md = ometa.build_token_metadata(mask, shapes, w.pos_mode)
    m = dit.build_token_metadata(torch.from_numpy(mask).cuda(), shapes, w.pos_mode)
    m.check()
    q, k, v = (to_device(d.bits[n], w.dtype) for n in ("q", "k", "v"))
    wq, wk = to_device(d.bits["wq"], w.dtype), to_device(d.bits["wk"], w.dtype)

    # Step 1 ("extract"): the whole sequence.  K' of every token goes to kp_full.
    _, kp_full = dit.dit_attn_qknorm_rope_ex(None, k, m.pos_ids, w.axes, w.eps, k_weight=wk)
    o_full, lse_full = nan_outputs(q)
    dit.forward_cached_qnorm(q, None, None, kp_full, v, m.pos_ids, w.axes, w.eps, q_weight=wq,
                             mask_mode=w.mask_mode, meta=m, out=o_full, lse_out=lse_full)

    # Step 2 ("cached"): the target block against the cache, which is rows
    # [0, P) of step 1's K' buffer and of V, read in place (strided views).
    q_new, k_new, v_new = q[:, P:], k[:, P:], v[:, P:]
    k_cache, v_cache = kp_full[:, :P], v[:, :P]
    _, kp_new = dit.dit_attn_qknorm_rope_ex(None, k_new, m.pos_ids[P:], w.axes, w.eps, k_weight=wk)
    o_new, lse_new = nan_outputs(q_new)
    dit.forward_cached_qnorm(q_new, k_cache, v_cache, kp_new, v_new, m.pos_ids[P:], w.axes, w.eps, q_weight=wq,
                             mask_mode=w.mask_mode, meta=m, out=o_new, lse_out=lse_new)
    torch.cuda.synchronize()
    assert_all_written(o_new, lse_new, "cached step")
    assert_all_written(o_full, lse_full, "full step")
    # K' of the target tokens is the same whichever step computes it, and each
    # row's result depends only on its own keys and the fixed key tiling.
    assert torch.equal(kp_new, kp_full[:, P:])
    assert torch.equal(o_new, o_full[:, P:])
    assert torch.equal(lse_new, lse_full[:, :, P:])

    # The oracle's flow: a full step whose K' rows [0, P) and raw V rows
    # [0, P) become the cache, then the cached step of the target block.
    tgt = wl.small_workload("t", w.batch, w.heads, w.kv_heads, w.head_dim, w.layout, w.axes, prefix_len=P)
    rows = sample_rows(tgt)
    kw = dict(axes=w.axes, eps=w.eps, mask_mode=w.mask_mode, theta=w.rope_theta)
    full = opipe.step(d.vals, md, rows=[0], **kw)
    new = {n: d.vals[n][:, P:] for n in ("q", "k", "v")}
    new.update(wq=d.vals["wq"], wk=d.vals["wk"], **opipe.extract_cache(full, d.vals["v"], P))
    ref = opipe.step(new, md, prefix_len=P, rows=rows, **kw)
    idx = torch.from_numpy(rows).cuda()
    stats = assert_parity(to_host(o_new[:, idx]), ref["o"], "bf16", "O (cached step)")
    lit = assert_literal_mean(to_host(o_new[:, idx]), ref["o"], "O (cached step)")
    assert_parity(lse_new[:, :, idx].cpu().double().numpy(), ref["lse"], "f32", "lse (cached step)", atol=1e-2)
    assert_parity(to_host(kp_new[:, idx]), ref["k_prime"][:, rows], "bf16", "K' of the target tokens")
    _say("  %s rows=%d max=%.3g mean=%.3g (unrounded %.3g)" % (name, rows.size, stats["max"], stats["mean"], lit))
