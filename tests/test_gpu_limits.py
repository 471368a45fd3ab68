"""GPU parity at the address limit of the attention kernels: keys are addressed
with 32-bit byte offsets inside one (batch, kv-head) slice, and the host
accepts a slice only while its span (keys x row stride) stays below 2^31
bytes.  These tests place K and V as strided views into ~2.1 GB buffers whose
row stride puts the last key row just under that limit -- with a ragged key
count, so the last tile's rows past the end sit beyond 2^31 and must read as
zeros -- and compare with the same keys stored contiguously (bit-identical:
only the addressing differs) and with the oracle on sampled rows.  One row
stride more is refused on the host before anything is launched.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle.attention as oatt
import oracle.metadata as ometa
import workloads as wl
from diffusion_transformer_joint_token_amd import _lib
from tests.gpu_helpers import QUERY_TILE, assert_parity, nan_outputs, to_device, to_host

pytestmark = pytest.mark.gpu

D = 128
S_KEYS = 4000                     # not a multiple of the 64-key tile
STRIDE = 268432                   # elements per key row: 4000 * 268432 * 2 B = 2,147,456,000 < 2^31 - 1
assert S_KEYS * STRIDE * 2 < 2 ** 31 - 1 <= S_KEYS * (STRIDE + 8) * 2
assert (STRIDE * 2) % 16 == 0


@pytest.fixture(scope="module")
def dit():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu-marked tests need an MI355X")
    import diffusion_transformer_joint_token_amd as d
    return d


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _strided(src: torch.Tensor, stride: int) -> torch.Tensor:
    """src [1, S, 1, D] copied into rows `stride` elements apart of a buffer of
    S * STRIDE elements (the view's last element always lies inside it)."""
    S = src.shape[1]
    buf = torch.empty(S * STRIDE, dtype=src.dtype, device=src.device)
    view = buf.as_strided((1, S, 1, D), (S * STRIDE, stride, D, 1))
    view.copy_(src)
    return view


def _rows(n: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    rows = {0, 1, n - 1}
    for t0 in range(0, n, QUERY_TILE):
        rows.add(int(rng.integers(t0, min(t0 + QUERY_TILE, n))))
    return np.array(sorted(rows))


@pytest.mark.parametrize("cached", [False, True], ids=["keys", "cache"])
def test_key_offsets_just_below_2_31(dit, cached):
    """Full mask, 4 query heads on one KV head.  keys: the 4000 keys are the
    new tokens (4000 queries); cache: they are the cached prefix, read in place,
    and 130 new tokens (queries) follow contiguously."""
    S_new = 130 if cached else S_KEYS
    P = S_KEYS if cached else 0
    layout = (("I", 1, 40, 100), ("T", 130)) if cached else (("I", 1, 40, 100),)
    w = wl.small_workload("limit", 1, 4, 1, D, layout, (D,), dtype="bf16", seed=31, prefix_len=P)
    assert w.n_new == S_new
    _say("key offsets near 2^31: %s (P %d, new %d, row stride %d B)" % ("cache" if cached else "keys", P, S_new,
                                                                       2 * STRIDE))
    d = wl.draw(w)
    mask, shapes = wl.sequence_inputs(w)
    md = ometa.build_token_metadata(mask, shapes)
    q, k, v = (to_device(d.bits[n], "bf16") for n in ("q", "k", "v"))
    o_ref, lse_ref = nan_outputs(q)
    o, lse = nan_outputs(q)
    if cached:
        kc, vc = to_device(d.bits["k_cache"], "bf16"), to_device(d.bits["v_cache"], "bf16")
        kc_far, vc_far = _strided(kc, STRIDE), _strided(vc, STRIDE)
        dit.forward_cached(q, kc, vc, k, v, "full", None, out=o_ref, lse_out=lse_ref)
        dit.forward_cached(q, kc_far, vc_far, k, v, "full", None, out=o, lse_out=lse)
        k_all = np.concatenate([d.vals["k_cache"], d.vals["k"]], axis=1)
        v_all = np.concatenate([d.vals["v_cache"], d.vals["v"]], axis=1)
        k_bad = kc_far.as_strided(kc_far.shape, (S_KEYS * STRIDE, STRIDE + 8, D, 1))
        with pytest.raises(dit.DitAttnError) as err:
            dit.forward_cached(q, k_bad, vc_far, k, v, "full", None)
    else:
        k_far, v_far = _strided(k, STRIDE), _strided(v, STRIDE)
        dit.forward(q, k, v, "full", None, out=o_ref, lse_out=lse_ref)
        dit.forward(q, k_far, v_far, "full", None, out=o, lse_out=lse)
        k_all, v_all = d.vals["k"], d.vals["v"]
        k_bad = k_far.as_strided(k_far.shape, (S_KEYS * STRIDE, STRIDE + 8, D, 1))
        with pytest.raises(dit.DitAttnError) as err:
            dit.forward(q, k_bad, v_far, "full", None)
    torch.cuda.synchronize()
    assert err.value.status == _lib.ERR_UNSUPPORTED
    assert torch.isfinite(o).all() and torch.isfinite(lse).all()
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)
    rows = _rows(S_new, 7)
    ro, rl = oatt.attention(d.vals["q"], k_all, v_all, md["image_ids"], "full", q_offset=P, rows=rows)
    idx = torch.from_numpy(rows).cuda()
    stats = assert_parity(to_host(o[:, idx]), ro, "bf16", "O")
    assert_parity(lse[:, :, idx].cpu().double().numpy(), rl, "f32", "lse", atol=1e-2)
    _say("  rows %d max %.3g mean %.3g" % (rows.size, stats["max"], stats["mean"]))
    del o, o_ref
    torch.cuda.empty_cache()
