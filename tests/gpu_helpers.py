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
QUERY_TILE = 128  # query rows per work-group of the bf16 attention launch


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


def assert_literal_mean(gpu: np.ndarray, ora: np.ndarray, what: str) -> float:
    """The stated mean-abs bar taken literally: mean |gpu - oracle| <= 1e-3
    against the unrounded oracle.  Used at full size, where O is far below 1
    in magnitude and the output format's own rounding is far below the bar."""
    mean = float(np.mean(np.abs(np.asarray(gpu, np.float64) - np.asarray(ora, np.float64))))
    assert mean <= MEAN_BF16, "%s: mean |gpu - oracle| %.3g > %.3g" % (what, mean, MEAN_BF16)
    return mean


def sample_rows(w, n_random=24, seed=0):
    """Query rows (indices into the query tokens) for full-size checks: the
    first and last rows, rows around every segment boundary, one row drawn in
    every 128-row query tile -- so every work-group of the launch (one per
    batch, head and query tile; the oracle computes all batches and heads of a
    row) is compared -- and n_random more random rows."""
    S = w.n_new
    rows = {0, 1, 2, 3, S - 1, S - 2, S - 3}
    start = 0
    for seg in w.layout:
        n = seg[1] if seg[0] == "T" else seg[1] * seg[2] * seg[3]
        for r in (start - 1, start, start + 1, start + n - 1):
            q = r - w.prefix_len
            if 0 <= q < S:
                rows.add(q)
        start += n
    rng = np.random.default_rng(seed)
    for t0 in range(0, S, QUERY_TILE):
        rows.add(int(rng.integers(t0, min(S, t0 + QUERY_TILE))))
    rows.update(int(x) for x in rng.integers(0, S, size=n_random))
    out = np.array(sorted(rows))
    assert set(out // QUERY_TILE) == set(range((S + QUERY_TILE - 1) // QUERY_TILE))
    return out


def nan_outputs(q: torch.Tensor):
    """O and lse buffers for a call on queries q ([B, S, H, D]) filled with NaN,
    so that any element the launch fails to write shows up."""
    B, S, H, _ = q.shape
    o = torch.full(q.shape, float("nan"), dtype=q.dtype, device=q.device)
    lse = torch.full((B, H, S), float("nan"), dtype=torch.float32, device=q.device)
    return o, lse


def assert_all_written(o: torch.Tensor, lse: torch.Tensor, what: str, lse_may_be_neg_inf: bool = False):
    """Every element of a NaN-prefilled O and lse was written with a finite
    value (lse may be -inf on rows with no valid key, when padding allows it)."""
    bad_o = int((~torch.isfinite(o)).sum())
    assert bad_o == 0, "%s: %d elements of O not written or not finite" % (what, bad_o)
    ok = torch.isfinite(lse)
    if lse_may_be_neg_inf:
        ok = ok | torch.isneginf(lse)
    bad_l = int((~ok).sum())
    assert bad_l == 0, "%s: %d lse entries not written or not finite" % (what, bad_l)


def oracle_rows(attention, qp_rows, k_all, v_all, image_ids, mask_mode, P, rows, key_valid=None):
    """The oracle's O and lse for the given query rows, computed one row at a
    time (row r of the query tokens is logical position P + r)."""
    B, _, H, D = np.asarray(qp_rows).shape
    ro = np.zeros((B, rows.size, H, D))
    rl = np.zeros((B, H, rows.size))
    for j, r in enumerate(rows):
        oj, lj = attention(qp_rows[:, j:j + 1], k_all, v_all, image_ids, mask_mode, q_offset=P + int(r),
                           key_valid=key_valid)
        ro[:, j] = oj[:, 0]
        rl[:, :, j] = lj[:, :, 0]
    return ro, rl
