"""Device upload of seeded inputs and the parity criteria of the GPU tests.

Tolerances (bf16 results, from the stated bar of max-abs 1e-2 / mean-abs 1e-3
against the fp64 oracle, widened only by the output format's own resolution):
  * every element: |gpu - oracle| <= max(1e-2, ulp_bf16(oracle)) -- a bf16 value
    of magnitude >= 2 cannot be stored closer than half an ulp (>= 7.8e-3) and a
    correctly computed fp32 result may round to either neighbour;
  * mean over elements of |gpu - bf16(oracle)| <= 1e-3, with bf16() the
    round-to-nearest-even image of the oracle in the output format.
fp32 results: every element within 1e-5 of the oracle.
"""
from __future__ import annotations

import numpy as np
import torch

from workloads import bf16_bits_to_f64, bf16_round_bits

ATOL_BF16 = 1e-2
MEAN_BF16 = 1e-3
ATOL_F32 = 1e-5


def to_device(bits: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.float32)).to(device)


def to_host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return bf16_bits_to_f64(t.contiguous().view(torch.int16).numpy().view(np.uint16))
    return t.double().numpy()


def bf16_ulp(x: np.ndarray) -> np.ndarray:
    ax = np.maximum(np.abs(x), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(ax)) - 7)


def rne_bf16(x: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f64(bf16_round_bits(np.asarray(x, dtype=np.float64).astype(np.float32)))


def assert_parity(gpu: np.ndarray, ora: np.ndarray, dtype: str, what: str, atol=None) -> dict:
    gpu = np.asarray(gpu, dtype=np.float64)
    ora = np.asarray(ora, dtype=np.float64)
    assert gpu.shape == ora.shape, (what, gpu.shape, ora.shape)
    assert np.all(np.isfinite(gpu)), "%s: non-finite GPU values" % what
    err = np.abs(gpu - ora)
    if dtype == "bf16":
        bound = np.maximum(ATOL_BF16 if atol is None else atol, bf16_ulp(ora))
        worst = np.unravel_index(np.argmax(err - bound), err.shape)
        assert np.all(err <= bound), "%s: max err %.3g at %s (gpu %.6g oracle %.6g bound %.3g)" % (
            what, err[worst], worst, gpu[worst], ora[worst], bound[worst])
        mean = float(np.mean(np.abs(gpu - rne_bf16(ora))))
        assert mean <= MEAN_BF16, "%s: mean err %.3g" % (what, mean)
    else:
        tol = ATOL_F32 if atol is None else atol
        worst = np.unravel_index(np.argmax(err), err.shape)
        assert err[worst] <= tol, "%s: max err %.3g at %s (gpu %.9g oracle %.9g)" % (
            what, err[worst], worst, gpu[worst], ora[worst])
        mean = float(np.mean(err))
    return {"max": float(err.max()), "mean": mean}
