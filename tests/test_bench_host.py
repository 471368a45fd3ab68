"""Host-side logic of bench.py (CPU only, no GPU call): the useful-pair count
behind `value`, the text-mask mapping used for padded runs, the rule that
keeps a stale HBM-traffic record out of the line, the refusal of more than
one GPU, and the counter summarisation arithmetic on synthetic counter
files.  Reference values come from the oracle's literal mask predicate and
key flags, or are written out by hand."""
from __future__ import annotations

import csv
import json
import os

import numpy as np
import pytest

import bench
import oracle.attention as oatt
import oracle.key_padding as okp
import oracle.metadata as ometa
import workloads as wl


def _brute_pairs(w, valid=None):
    mask, shapes = wl.sequence_inputs(w)
    md = ometa.build_token_metadata(mask, shapes, w.pos_mode)
    q_index = np.arange(w.prefix_len, w.seq_len)
    allow = oatt.allowed_matrix(q_index, np.arange(w.seq_len), md["image_ids"], w.mask_mode)
    if valid is None:
        return int(allow.sum()) * w.batch, md
    return int(sum((allow & valid[b][None, :]).sum() for b in range(w.batch))), md


LAYOUTS = [
    ((("T", 16), ("I", 1, 4, 4)), 0, "block_causal"),
    ((("T", 30), ("I", 1, 4, 6), ("I", 1, 2, 4), ("T", 9), ("I", 1, 6, 6)), 0, "block_causal"),
    ((("T", 30), ("I", 1, 4, 6), ("I", 1, 2, 4), ("T", 9), ("I", 1, 6, 6)), 47, "block_causal"),
    ((("I", 1, 8, 8),), 0, "full"),
    ((("T", 20), ("I", 1, 6, 6)), 20, "full"),
]


@pytest.mark.parametrize("layout,P,mode", LAYOUTS)
def test_useful_pairs_match_the_literal_mask(layout, P, mode):
    """value's numerator: allowed (q, k) pairs from kv_limit (and, with text
    padding, the valid keys) equal a count of the oracle's literal
    block-causal predicate."""
    w = wl.small_workload("b", 2, 1, 1, 8, layout, (8,), mask_mode=mode, prefix_len=P)
    ref, md = _brute_pairs(w)
    assert bench.useful_pairs(md["kv_limit"], w) == ref
    if wl.n_text_tokens(w):
        mask, _ = wl.sequence_inputs(w)
        tv = wl.text_mask(w, 5, "random")
        valid = okp.joint_key_valid(mask, tv)
        ref_v, _ = _brute_pairs(w, valid)
        assert bench.useful_pairs(md["kv_limit"], w, bench.text_valid_keys(mask, tv)) == ref_v


def test_headline_pair_count_closed_form():
    """1024 causal text rows then 4096 image rows over all 5120 keys, per head
    and batch entry: 1024 * 1025 / 2 + 4096 * 5120."""
    w = wl.get("qwen_image21_t1024_i64x64")
    mask, shapes = wl.sequence_inputs(w)
    md = ometa.build_token_metadata(mask, shapes, w.pos_mode)
    assert bench.useful_pairs(md["kv_limit"], w) == (1024 * 1025 // 2 + 4096 * 5120) * w.batch


def test_text_valid_keys_is_the_oracle_key_flags():
    w = wl.small_workload("b", 3, 1, 1, 8, (("I", 1, 2, 4), ("T", 13), ("I", 1, 4, 4), ("T", 5)), (8,))
    mask, _ = wl.sequence_inputs(w)
    for kind in ("right", "random", "none"):
        tv = wl.text_mask(w, 11, kind)
        assert np.array_equal(bench.text_valid_keys(mask, tv), okp.joint_key_valid(mask, tv))


def test_traffic_record_only_for_the_same_source_and_workload(tmp_path):
    src = tmp_path / "kernel.hip"
    src.write_text("// kernel source\n")
    rec = {"kernel_source_sha256": bench.source_sha(str(src)), "workload": "wl_a", "hbm_bytes_per_launch": 123.0}
    path = tmp_path / "traffic.json"
    path.write_text(json.dumps(rec))
    w_a = wl.small_workload("wl_a", 1, 1, 1, 8, (("T", 4),), (8,))
    w_b = wl.small_workload("wl_b", 1, 1, 1, 8, (("T", 4),), (8,))
    assert bench.measured_traffic(w_a, str(path), str(src)) == 123.0
    assert bench.measured_traffic(w_b, str(path), str(src)) is None        # other workload
    src.write_text("// kernel source, edited\n")
    assert bench.measured_traffic(w_a, str(path), str(src)) is None        # kernel changed since
    assert bench.measured_traffic(w_a, str(tmp_path / "missing.json"), str(src)) is None


def test_more_than_one_gpu_is_refused(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def _write_counters(d, rows):
    os.makedirs(d, exist_ok=True)
    with open(os.path.join(d, "run_counter_collection.csv"), "w", newline="") as fh:
        wr = csv.DictWriter(fh, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        wr.writeheader()
        for r in rows:
            wr.writerow(dict(zip(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"], r)))


def test_counter_summary_scales_by_the_copy_calibration(tmp_path, monkeypatch):
    """Per-dispatch means of counters summed over their instances, scaled by
    (copied bytes) / (what the counter read for the copy)."""
    root = str(tmp_path)
    # two attention dispatches, each counter split over two instances
    _write_counters(os.path.join(root, "fetch"), [
        (1, "attn_fwd_bf16_kernel<...>", "FETCH_SIZE", 100.0), (1, "attn_fwd_bf16_kernel<...>", "FETCH_SIZE", 50.0),
        (2, "attn_fwd_bf16_kernel<...>", "FETCH_SIZE", 70.0), (2, "attn_fwd_bf16_kernel<...>", "FETCH_SIZE", 80.0),
        (3, "qknorm_rope_kernel<...>", "FETCH_SIZE", 40.0), (4, "token_meta_kernel", "FETCH_SIZE", 2.0)])
    _write_counters(os.path.join(root, "write"), [
        (1, "attn_fwd_bf16_kernel<...>", "WRITE_SIZE", 30.0), (2, "attn_fwd_bf16_kernel<...>", "WRITE_SIZE", 34.0),
        (3, "qknorm_rope_kernel<...>", "WRITE_SIZE", 40.0), (4, "token_meta_kernel", "WRITE_SIZE", 1.0)])
    _write_counters(os.path.join(root, "copy_fetch"), [(9, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 128.0)])
    _write_counters(os.path.join(root, "copy_write"), [(9, "__amd_rocclr_copyBuffer", "WRITE_SIZE", 256.0)])
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    assert bench.summarize_counters(root, 1, "wl") == 0          # 1 MiB copied = 1024 KiB
    rec = json.loads(out.read_text())
    fs, ws = 1024 / 128, 1024 / 256                               # fetch scale 8, write scale 4
    assert rec["fetch_scale"] == pytest.approx(fs) and rec["write_scale"] == pytest.approx(ws)
    att = rec["kernels"]["attention"]
    assert att["fetch_bytes"] == pytest.approx(150.0 * 1024 * fs)  # mean of 150 and 150 KiB per dispatch
    assert att["write_bytes"] == pytest.approx(32.0 * 1024 * ws)
    assert rec["hbm_bytes_per_launch"] == pytest.approx(att["fetch_bytes"] + att["write_bytes"])
    assert rec["kernels"]["qknorm_rope"]["hbm_bytes"] == pytest.approx(40.0 * 1024 * (fs + ws))


def test_clock_ramp_runs_whole_batches_until_the_time_is_up():
    """The clock ramp runs untimed calls in batches of ten, synchronising after
    each batch, until its wall-clock floor has passed; it reports the calls."""
    class _Cuda:
        syncs = 0

        @classmethod
        def synchronize(cls):
            cls.syncs += 1

    class _Torch:
        cuda = _Cuda

    calls = []
    n = bench.ramp_clocks(_Torch, lambda: calls.append(1), 0.02)
    assert n == len(calls) and n >= 10 and n % 10 == 0
    assert _Cuda.syncs == n // 10
    _Cuda.syncs = 0
    assert bench.ramp_clocks(_Torch, lambda: None, 0.0) == 0 and _Cuda.syncs == 0


def test_clock_reading_never_raises():
    """The bench's clock record is a dict of MHz lists, or an error entry where
    no device (or no amdsmi) is there, as on a CPU-only host; it never raises."""
    import bench
    got = bench.read_clocks()
    assert isinstance(got, dict)
    assert "error" in got or ("sclk_mhz" in got and "mclk_mhz" in got)


@pytest.mark.parametrize("head_dim,padded,fused,want", [
    (128, False, True, "attn_fwd_bf16_kernel<128,4,qnorm>"),
    (72, False, True, "attn_fwd_bf16_kernel<80,4,qnorm>"),
    (72, True, False, "attn_fwd_bf16_kernel<80,4,padded>"),
    (96, False, False, "attn_fwd_bf16_kernel<96,4>"),
    (40, False, False, "attn_fwd_bf16_kernel<64,4>"),
])
def test_kernel_label_names_the_launched_instance(head_dim, padded, fused, want):
    """The label in the line names the template instance the launcher picks
    for the head dim (65..80 runs as the 80-channel instance)."""
    assert bench.kernel_label(head_dim, padded, fused) == want


@pytest.mark.parametrize("head_dim,want", [(128, 1.0), (64, 1.0), (72, (80 + 96) / 144.0), (96, 1.0), (40, 128 / 80.0)])
def test_padded_work_factor(head_dim, want):
    """MFMA work per useful FLOP from head-dim padding: QK^T over the kernel
    instance's channels, PV in 32-channel blocks."""
    assert bench.padded_work_factor(head_dim) == pytest.approx(want)
