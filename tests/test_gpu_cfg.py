"""GPU parity of the norm-rescaled classifier-free guidance kernel through the
C ABI against the fp64 oracle (every element), on seeded inputs from
``workloads.draw_cfg``: row widths that map to every lane layout of the
kernel, ragged row counts, strided and in-place rows, several guidance scales,
rows whose mix is exactly zero, and the benchmark workload at full size.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

import oracle.cfg as ocfg
import workloads as wl
from tests.gpu_helpers import assert_parity, to_device, to_host

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dit():
    if not torch.cuda.is_available():
        pytest.fail("no GPU visible: the gpu-marked tests need an MI355X")
    import diffusion_transformer_joint_token_amd as d
    return d


CASES = [
    # (rows, channels, dtype): lanes per row = chunks rounded up to a power of two (<= 64),
    # 1, 2, 4 or 8 chunks per lane beyond that
    (1, 8, "bf16"), (37, 16, "bf16"), (4097, 64, "bf16"), (300, 72, "bf16"), (129, 128, "bf16"),
    (65, 1032, "bf16"), (9, 4096, "bf16"), (33, 4, "f32"), (500, 64, "f32"), (77, 100, "f32"),
    (5, 2048, "f32"),
    # large, with a ragged tail
    (131149, 64, "bf16"), (65600, 64, "f32"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "R%dC%d_%s" % c)
def test_cfg_rows(dit, case):
    rows, C, dtype = case
    print("cfg %s" % (case,), flush=True)
    bits, vals = wl.draw_cfg(rows, C, rows + C, dtype)
    cond, unc = to_device(bits["cond"], dtype), to_device(bits["uncond"], dtype)
    for g in (4.0, 1.0, 0.0, -2.0, 7.5):
        out = dit.cfg_norm_rescale(cond, unc, g)
        torch.cuda.synchronize()
        assert_parity(to_host(out), ocfg.norm_rescaled_cfg(vals["cond"], vals["uncond"], g), dtype,
                      "cfg R%d C%d g %g" % (rows, C, g))


def test_cfg_strided_in_place_and_zero_rows(dit):
    rows, C = 300, 64
    bits, vals = wl.draw_cfg(rows, C, 3)
    cond, unc = to_device(bits["cond"], "bf16"), to_device(bits["uncond"], "bf16")
    # rows whose mix is exactly zero: at scale 2, uncond = 2 cond gives mix 0
    cond[5] = 0.25
    unc[5] = 0.5
    cond[17] = 0.0
    unc[17] = 0.0
    c64 = vals["cond"].copy()
    u64 = vals["uncond"].copy()
    c64[5], u64[5], c64[17], u64[17] = 0.25, 0.5, 0.0, 0.0
    ref = ocfg.norm_rescaled_cfg(c64, u64, 2.0)
    out = dit.cfg_norm_rescale(cond, unc, 2.0)
    torch.cuda.synchronize()
    assert torch.all(out[5] == 0) and torch.all(out[17] == 0)
    assert_parity(to_host(out), ref, "bf16", "zero rows")
    # rows inside wider buffers (row strides 80 and 72 channels), output strided too
    wc = torch.zeros(rows, 80, dtype=torch.bfloat16, device="cuda")
    wu = torch.zeros(rows, 72, dtype=torch.bfloat16, device="cuda")
    wo = torch.full((rows, 88), 3.0, dtype=torch.bfloat16, device="cuda")
    wc[:, :C] = cond
    wu[:, :C] = unc
    dit.cfg_norm_rescale(wc[:, :C], wu[:, :C], 2.0, out=wo[:, :C])
    torch.cuda.synchronize()
    assert torch.equal(wo[:, :C], out) and torch.all(wo[:, C:] == 3.0)
    # in place over the conditional prediction, and over the unconditional one
    c2, u2 = cond.clone(), unc.clone()
    dit.cfg_norm_rescale(c2, unc, 2.0, out=c2)
    dit.cfg_norm_rescale(cond, u2, 2.0, out=u2)
    torch.cuda.synchronize()
    assert torch.equal(c2, out) and torch.equal(u2, out)
    # [batch, tokens, channels] tensors are rows of the last axis
    out3 = dit.cfg_norm_rescale(cond.view(3, 100, C), unc.view(3, 100, C), 2.0)
    torch.cuda.synchronize()
    assert torch.equal(out3.view(rows, C), out)


def test_cfg_workload_full(dit):
    """The benchmark's workload (32 images at 1024 px, 131072 x 64, guidance
    4.0), every element."""
    w = wl.CFG_WORKLOADS["nucleus_cfg_b32_1024px"]
    bits, vals = wl.draw_cfg(w.rows, w.channels, w.seed, w.dtype)
    cond, unc = to_device(bits["cond"], w.dtype), to_device(bits["uncond"], w.dtype)
    out = dit.cfg_norm_rescale(cond.view(w.batch, w.tokens, w.channels), unc.view(w.batch, w.tokens, w.channels),
                               w.guidance)
    torch.cuda.synchronize()
    stats = assert_parity(to_host(out).reshape(w.rows, w.channels),
                          ocfg.norm_rescaled_cfg(vals["cond"], vals["uncond"], w.guidance), w.dtype, w.name)
    print("  %s max %.3g mean %.3g" % (w.name, stats["max"], stats["mean"]), flush=True)
    sys.stdout.flush()
