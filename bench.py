#!/usr/bin/env python3
"""Benchmark of the joint text+image DiT attention step on one MI355X.

A step is one pass of the whole path on one batch of synthetic inputs that
are already resident in HBM: token metadata -> QK-RMSNorm + rotary -> masked
attention (the cached-prefix workload runs the cached attention entry point
instead of the plain one).  For bf16 with the per-head RMSNorm, Q's norm,
rotary embedding and softmax scale run inside the attention kernel as it
loads Q (dit_attn_forward_cached_qnorm) and the norm kernel handles K alone;
--unfused-q times the two-kernel form (the norm kernel writes Q' to HBM and
the attention reads it back).  Default workload: batch 2, 32 heads x 128,
1024 text tokens followed by one 1x64x64 target image block (5120 tokens),
block-causal mask, bf16.

Prints ONE JSON line on stdout.  ``value`` is the useful attention FLOP rate
of the whole step: 4 * head_dim * (allowed (q, k) pairs) * heads * batch per
step (QK^T and PV only, masked pairs not counted) divided by the measured step
time.  ``roofline`` covers the dominant kernel (attention), timed with HIP
events on its own stream; ``cpu_baseline`` is the fp64 oracle on the host
cores for a bounded sample of query rows of the same workload.
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import workloads as wl  # noqa: E402

METRIC = "attention fwd useful TFLOP/s + % bf16 MFMA peak (4096 img + 1024 text, 32×128)"
PEAK_BF16_TFLOPS = 2516.6      # 256 CU x 4096 FLOP/clk x 2.4 GHz, dense bf16 MFMA
PEAK_SCLK_GHZ = 2.4            # the shader clock the published MFMA peak is quoted at
PEAK_HBM_GBS = 8000.0
DEFAULT_WORKLOAD = "qwen_image21_t1024_i64x64"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_hbm_traffic.json")
ATTN_SOURCE = os.path.join(ROOT, "diffusion_transformer_joint_token_amd", "csrc", "attn_fwd.hip")
CFG_TRAFFIC_FILE = os.path.join(ROOT, "profiles", "cfg_norm_rescale_hbm_traffic.json")
CFG_SOURCE = os.path.join(ROOT, "diffusion_transformer_joint_token_amd", "csrc", "cfg.hip")


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def useful_pairs(kv_limit: np.ndarray, w: wl.Workload, valid_keys=None) -> int:
    """Allowed (q, k) pairs summed over the batch, per head, for the workload's
    query rows; with valid_keys (bool [B, S]) padded keys are not counted."""
    lim = (np.full(w.n_new, w.seq_len, dtype=np.int64) if w.mask_mode == "full"
           else kv_limit[w.prefix_len:].astype(np.int64))
    if valid_keys is None:
        return int(lim.sum()) * w.batch
    below = np.concatenate([np.zeros((w.batch, 1), np.int64), np.cumsum(valid_keys, axis=1)], axis=1)
    return int(below[:, lim].sum())


def text_valid_keys(mask: np.ndarray, tv: np.ndarray) -> np.ndarray:
    """bool [B, S] for the FLOP count: image tokens, and text tokens whose
    entry (by text ordinal) in the sample's text mask is set."""
    text = mask == 0
    ordinal = np.cumsum(text) - 1
    out = np.ones((tv.shape[0], mask.size), dtype=bool)
    out[:, text] = tv[:, ordinal[text]] != 0
    return out


def cpu_model() -> str:
    """The host CPU's model name (Linux /proc/cpuinfo), or "" if unknown."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


_SMI = {}


def read_clocks() -> dict:
    """Current shader clock of each XCD and memory clock of GPU 0, in MHz, and
    the socket power in W, read in-process through the amdsmi library (the
    data `amd-smi metric` shows), or {"error": ...}."""
    try:
        import amdsmi
        if "handle" not in _SMI:
            amdsmi.amdsmi_init()
            _SMI["handle"] = amdsmi.amdsmi_get_processor_handles()[0]
        m = amdsmi.amdsmi_get_gpu_metrics_info(_SMI["handle"])
    except Exception as e:  # noqa: BLE001  (no amdsmi, no device, no permission)
        return {"error": "%s: %s" % (type(e).__name__, e)}

    def mhz(v):
        vals = v if isinstance(v, (list, tuple)) else [v]
        return [int(x) for x in vals if isinstance(x, (int, float)) and 0 < x < 65535]
    out = {"sclk_mhz": mhz(m.get("current_gfxclks", [])), "mclk_mhz": mhz(m.get("current_uclk", []))}
    p = m.get("current_socket_power")
    if isinstance(p, (int, float)) and 0 < p < 65535:
        out["socket_power_w"] = p
    return out


def clocks_under_load(torch, run, seconds: float = 1.5) -> dict:
    """Run `run()` back to back for `seconds` while another thread reads the
    clocks once, half-way through: the clocks the timed steps ran at."""
    import threading
    box = {}

    def probe():
        time.sleep(seconds / 2)
        box.update(read_clocks())
    th = threading.Thread(target=probe)
    t0 = time.perf_counter()
    th.start()
    while time.perf_counter() - t0 < seconds:
        for _ in range(10):
            run()
        torch.cuda.synchronize()
    th.join()
    return box


def source_sha(path: str) -> str:
    with open(path, "rb") as fh:
        return hashlib.sha256(fh.read()).hexdigest()


def kernel_label(head_dim: int, padded: bool, fused: bool) -> str:
    """Template instance of the bf16 attention kernel that a head dim runs:
    the head dim rounded up to 32 channels, except 65..80 (Lumina-Next's 72),
    which takes five 16-channel QK^T steps as an 80-channel instance."""
    dp = 80 if 64 < head_dim <= 80 else (head_dim + 31) // 32 * 32
    return "attn_fwd_bf16_kernel<%d,4%s%s>" % (dp, ",padded" if padded else "", ",qnorm" if fused else "")


def padded_work_factor(head_dim: int) -> float:
    """MFMA work the bf16 kernel issues per useful FLOP from head-dim padding:
    QK^T contracts over the instance's channel count (80 for 65..80, else the
    head dim rounded up to 32) and PV produces 32-channel blocks, so
    (qk + pv) / (2 * head_dim).  1.0 for head dims that are multiples of 32."""
    qk = 80 if 64 < head_dim <= 80 else (head_dim + 31) // 32 * 32
    pv = (head_dim + 31) // 32 * 32
    return (qk + pv) / (2.0 * head_dim)


def measured_traffic(w, path: str = TRAFFIC_FILE, source: str = ATTN_SOURCE):
    """HBM bytes per launch from the committed rocprofv3 counter runs, or None
    when they were taken on another kernel source or workload."""
    try:
        with open(path) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_sha256") != source_sha(source) or rec.get("workload") != w.name:
        return None
    return rec.get("hbm_bytes_per_launch")


class Step:
    """Device buffers and the launch sequence of one step."""

    def __init__(self, w: wl.Workload, device, text_padding: str = "none", fuse_q: bool = True):
        import torch
        import diffusion_transformer_joint_token_amd as dit
        self.torch, self.dit, self.w = torch, dit, w
        # Q's norm inside the attention kernel: bf16, per-head RMSNorm only.
        self.fused = fuse_q and w.dtype == "bf16" and w.qk_norm == "rms_per_head"
        d = wl.draw(w)
        self.drawn = d

        def dev(name):
            bits = np.ascontiguousarray(d.bits[name])
            if w.dtype == "bf16":
                return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(device)
            return torch.from_numpy(bits).to(device)
        self.q, self.k, self.v = dev("q"), dev("k"), dev("v")
        self.wq, self.wk = dev("wq"), dev("wk")
        across = w.qk_norm == "layer_across_heads"
        self.bq, self.bk = (dev("bq"), dev("bk")) if across else (None, None)
        # Norm and rotary options of the workload, as qknorm_rope keywords.
        self.norm_kw = dict(norm=w.qk_norm, q_bias=self.bq, k_bias=self.bk, rope_linear_factor=w.rope_linear,
                            rope_ntk_factor=w.rope_ntk)
        self.kc = dev("k_cache") if w.prefix_len else None
        self.vc = dev("v_cache") if w.prefix_len else None
        mask, self.shapes = wl.sequence_inputs(w)
        self.mask = torch.from_numpy(mask).to(device)
        self.meta = dit.TokenMeta.empty(w.seq_len, device)
        # Padded text: a seeded per-sample text mask; its key-validity bits are
        # rebuilt with the metadata every step and passed to the attention.
        self.tv, self.kv, self.tv_dev = None, None, None
        if text_padding != "none":
            self.tv = wl.text_mask(w, 2024, text_padding)
            self.tv_dev = torch.from_numpy(self.tv).to(device)
            self.kv = dit.KeyValid(torch.empty(w.batch, (w.seq_len + 63) // 64, dtype=torch.int64, device=device),
                                   torch.empty(1, dtype=torch.int32, device=device))
        self.qp = None if self.fused else torch.empty_like(self.q)
        self.kp = torch.empty_like(self.k)
        self.o = torch.empty_like(self.q)
        self.stream = torch.cuda.current_stream()

    def metadata(self):
        self.dit.build_token_metadata(self.mask, self.shapes, self.w.pos_mode, out=self.meta)
        if self.kv is not None:
            self.dit.build_key_valid(self.mask, self.tv_dev, out=self.kv)

    def norm_launch(self, q, k, pos_ids, qp, kp):
        """The norm kernel on (q, k).  Fused: K only.  Otherwise Q' and K',
        with the softmax scale and log2(e) folded into Q' (one rounding), so
        the attention exponentiates its MFMA output directly."""
        w = self.w
        if self.fused:
            self.dit.dit_attn_qknorm_rope_ex(None, k, pos_ids, w.axes, w.eps, k_weight=self.wk, k_out=kp,
                                             rope_theta=w.rope_theta, **self.norm_kw)
        else:
            self.dit.qknorm_rope(q, k, pos_ids, w.axes, w.eps, self.wq, self.wk, q_out=qp, k_out=kp,
                                 q_scale=self.dit.prescaled_q_factor(w.head_dim), **self.norm_kw)

    def attention_launch(self, q, qp, k_cache, v_cache, kp, v, out, pos_ids):
        w = self.w
        if self.fused:
            self.dit.forward_cached_qnorm(q, k_cache, v_cache, kp, v, pos_ids, w.axes, w.eps, q_weight=self.wq,
                                          rope_theta=w.rope_theta, rope_linear_factor=w.rope_linear,
                                          rope_ntk_factor=w.rope_ntk, mask_mode=w.mask_mode, meta=self.meta,
                                          out=out, key_valid=self.kv)
        elif k_cache is not None:
            self.dit.forward_cached(qp, k_cache, v_cache, kp, v, w.mask_mode, self.meta,
                                    softmax_scale=self.dit.LN2, out=out, key_valid=self.kv)
        else:
            self.dit.forward(qp, kp, v, w.mask_mode, self.meta, softmax_scale=self.dit.LN2, out=out,
                             key_valid=self.kv)

    def norm_rope(self):
        self.norm_launch(self.q, self.k, self.meta.pos_ids[self.w.prefix_len:], self.qp, self.kp)

    def attention(self):
        if self.fused:
            self.attention_launch(self.q, None, self.kc, self.vc, self.kp, self.v, self.o,
                                  self.meta.pos_ids[self.w.prefix_len:])
        elif self.w.prefix_len:
            self.dit.forward_cached(self.qp, self.kc, self.vc, self.kp, self.v, self.w.mask_mode, self.meta,
                                    softmax_scale=self.dit.LN2, out=self.o, key_valid=self.kv)
        else:
            self.dit.forward(self.qp, self.kp, self.v, self.w.mask_mode, self.meta, softmax_scale=self.dit.LN2,
                             out=self.o, key_valid=self.kv)

    def run(self):
        self.metadata()
        self.norm_rope()
        self.attention()


def ramp_clocks(torch, run, min_s: float) -> int:
    """Run `run()` in batches of ten until at least `min_s` seconds of wall
    time have passed with the GPU busy, and return how many calls that took.
    A few milliseconds of work after start-up, or after the GPU has idled
    while the host did other work, leave the shader clock below where it
    settles: a timed pass right after ten headline steps came out 2-7 %
    slower than the passes after it."""
    n, t0 = 0, time.perf_counter()
    while time.perf_counter() - t0 < min_s:
        for _ in range(10):
            run()
        n += 10
        torch.cuda.synchronize()
    return n


def time_gpu(step: Step, steps: int, warmup: int, ramp_s: float = 0.3):
    """The step time comes from `steps` back-to-back steps bracketed by one
    pair of HIP events on the launch stream (and the host wall clock), with a
    synchronisation on both sides; a second pass of `steps` steps with events
    between the kernels gives the per-kernel breakdown (those events are not
    inside the step time).  Before it: `warmup` steps, then whole steps until
    `ramp_s` seconds have passed (the clock ramp)."""
    torch = step.torch
    for _ in range(warmup):
        step.run()
    step.meta.check()
    ramp_steps = ramp_clocks(torch, step.run, ramp_s)
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    t_start.record(step.stream)
    for _ in range(steps):
        step.run()
    t_end.record(step.stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = t_start.elapsed_time(t_end) / steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True),
           torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for e in ev:
        e[0].record(step.stream)
        step.metadata()
        e[1].record(step.stream)
        step.norm_rope()
        e[2].record(step.stream)
        step.attention()
        e[3].record(step.stream)
    torch.cuda.synchronize()
    meta_ms = float(np.mean([a.elapsed_time(b) for a, b, _, _ in ev]))
    norm_ms = float(np.mean([b.elapsed_time(c) for _, b, c, _ in ev]))
    attn_ms = [c.elapsed_time(d) for _, _, c, d in ev]
    return {"wall_ms_per_step": 1e3 * wall / steps, "step_ms": step_ms, "ramp_steps": ramp_steps,
            "step_ms_with_kernel_events": ev[0][0].elapsed_time(ev[-1][3]) / steps, "meta_ms": meta_ms,
            "norm_ms": norm_ms, "attn_ms_mean": float(np.mean(attn_ms)), "attn_ms_min": float(np.min(attn_ms)),
            "attn_ms_median": float(np.median(attn_ms))}


def time_norm_cold(step: Step, reps: int = 30, copies: int = 3, ramp_s: float = 0.3):
    """K2 alone, rotating `copies` separate input copies so that the Q/K read
    by one launch were not touched by the launches just before it (the
    headline workload's Q+K, 168 MB, or its K alone with K', would
    otherwise partly stay in the 256 MB Infinity Cache)."""
    torch, w = step.torch, step.w
    P = w.prefix_len
    qs = [step.q] + [step.q.clone() for _ in range(copies - 1)]
    ks = [step.k] + [step.k.clone() for _ in range(copies - 1)]

    def launch(i):
        step.norm_launch(qs[i % copies], ks[i % copies], step.meta.pos_ids[P:], step.qp, step.kp)
    for i in range(copies):
        launch(i)
    ramp_clocks(torch, lambda: launch(0), ramp_s)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(ev):
        a.record(step.stream)
        launch(i)
        b.record(step.stream)
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in ev]
    del qs, ks
    return {"ms_mean": float(np.mean(ms)), "ms_median": float(np.median(ms)), "ms_min": float(np.min(ms))}


def multistep(step: Step, n_steps: int, reps: int, warmup: int, full_ms: float, ramp_s: float = 0.3):
    """Step 1 runs the whole joint sequence; its norm kernel writes K' of every
    token, so rows [0, P) of that buffer are the cache (P = every token before
    the target block: text and condition images, which do not change with the
    timestep).  Steps 2..N re-run only the target block: norm+rope of its
    tokens and the cached-prefix attention against the step-1 cache.  Returns
    the timings, the amortised speedup over N full steps and whether the
    cached rows equal the full-step rows bit for bit."""
    torch, dit, w = step.torch, step.dit, step.w
    last = w.layout[-1]
    if last[0] != "I":
        raise SystemExit("--multistep needs a sequence that ends with the target image block")
    P = w.seq_len - last[1] * last[2] * last[3]
    if P == 0 or w.prefix_len:
        raise SystemExit("--multistep needs a workload with tokens before the target block and no cache of its own")
    q_new, k_new, v_new = step.q[:, P:], step.k[:, P:], step.v[:, P:]
    k_cache, v_cache = step.kp[:, :P], step.v[:, :P]
    qp_new = None if step.fused else torch.empty_like(q_new, memory_format=torch.contiguous_format)
    kp_new = torch.empty_like(k_new, memory_format=torch.contiguous_format)
    o_new = torch.empty_like(q_new, memory_format=torch.contiguous_format)
    def cached():
        step.norm_launch(q_new, k_new, step.meta.pos_ids[P:], qp_new, kp_new)
        step.attention_launch(q_new, qp_new, k_cache, v_cache, kp_new, v_new, o_new, step.meta.pos_ids[P:])
    step.run()
    for _ in range(warmup):
        cached()
    torch.cuda.synchronize()
    same = bool(torch.equal(o_new, step.o[:, P:]))
    ramp_clocks(torch, cached, ramp_s)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0.record(step.stream)
    for _ in range(reps):
        cached()
    t1.record(step.stream)
    torch.cuda.synchronize()
    cached_ms = t0.elapsed_time(t1) / reps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps)]
    for e in ev:
        e[0].record(step.stream)
        step.norm_launch(q_new, k_new, step.meta.pos_ids[P:], qp_new, kp_new)
        e[1].record(step.stream)
        step.attention_launch(q_new, qp_new, k_cache, v_cache, kp_new, v_new, o_new, step.meta.pos_ids[P:])
        e[2].record(step.stream)
    torch.cuda.synchronize()
    amort = (full_ms + (n_steps - 1) * cached_ms) / n_steps
    return {"steps": n_steps, "prefix_tokens": P, "target_tokens": w.seq_len - P, "full_step_ms": full_ms,
            "cached_step_ms": cached_ms, "amortised_ms_per_step": amort, "speedup_vs_full_steps": full_ms / amort,
            "cached_norm_ms": float(np.mean([a.elapsed_time(b) for a, b, _ in ev])),
            "cached_attention_ms": float(np.mean([b.elapsed_time(c) for _, b, c in ev])),
            "cached_rows_equal_full_rows": same}


OTHER_CONFIGS = ("lumina_next_full_gqa", "cond_images_t256_2x32x32_t256_i64x64", "cached_prefix_decode_i128x128")


def measure_config(name: str, steps: int, warmup: int, ramp_s: float) -> dict:
    """Step and attention-kernel times of one more bf16 workload, measured the
    way the headline is (time_gpu), for the line's `configs` object."""
    import torch
    w = wl.get(name)
    step = Step(w, "cuda")
    step.run()
    torch.cuda.synchronize()
    step.meta.check()
    pairs = useful_pairs(step.meta.kv_limit.cpu().numpy(), w)
    flops = 4.0 * w.head_dim * pairs * w.heads
    t = time_gpu(step, steps, warmup, ramp_s)
    attn = flops / (t["attn_ms_mean"] * 1e-3) / 1e12
    elem = 2 if w.dtype == "bf16" else 4
    normed = w.kv_heads if step.fused else w.heads + w.kv_heads
    norm_bytes = 2 * w.batch * w.n_new * normed * w.head_dim * elem
    out = {"workload": name, "batch": w.batch, "heads": w.heads, "kv_heads": w.kv_heads, "head_dim": w.head_dim,
           "seq_len": w.seq_len, "queries": w.n_new, "mask": w.mask_mode, "flops_per_step": flops,
           "step_ms": t["step_ms"], "step_tflops": flops / (t["step_ms"] * 1e-3) / 1e12,
           "attention_ms_mean": t["attn_ms_mean"], "attention_ms_min": t["attn_ms_min"],
           "attention_tflops": attn, "attention_frac_bf16_peak": attn / PEAK_BF16_TFLOPS,
           "attention_mfma_work_frac": attn * padded_work_factor(w.head_dim) / PEAK_BF16_TFLOPS,
           "qknorm_rope_ms": t["norm_ms"], "qknorm_rope_frac_hbm": norm_bytes / (t["norm_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
           "token_metadata_ms": t["meta_ms"],
           "kernel": kernel_label(w.head_dim, False, step.fused)}
    del step
    torch.cuda.empty_cache()
    return out


def library_gemm_reference(torch, n: int = 8192, seconds: float = 1.5) -> dict:
    """The vendor library's bf16 GEMM (torch.matmul, hipBLASLt) on n x n x n
    contiguous operands, timed back to back on the same card after a clock
    ramp: the MFMA rate that dense library code reaches under the card's power
    limit, beside the published peak (context for the roofline fraction)."""
    x = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    y = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    z = torch.empty(n, n, device="cuda", dtype=torch.bfloat16)
    run = lambda: torch.matmul(x, y, out=z)  # noqa: E731
    ramp_clocks(torch, run, 0.4)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 50
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    clocks = clocks_under_load(torch, run, seconds)
    tflops = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
    del x, y, z
    torch.cuda.empty_cache()
    return {"op": "torch.matmul bf16 %dx%dx%d (hipBLASLt)" % (n, n, n), "ms": ms, "tflops": tflops,
            "frac_bf16_peak": tflops / PEAK_BF16_TFLOPS, "clocks_under_load": clocks}


def cpu_single_thread() -> dict:
    """The oracle on one host thread for the tiny fp32 workload (every query
    row) and the Lumina mini shape of the Lumina-Next article's standalone
    test (3 query heads over 1 KV head, head_dim 8, 2D rotary 4 + 4 on a 4x4
    grid, full mask): seconds and fp64 useful GFLOP/s."""
    import oracle.attention as oatt
    import oracle.metadata as ometa
    import oracle.qknorm_rope as oqr
    try:
        from threadpoolctl import threadpool_limits
    except Exception:  # noqa: BLE001
        threadpool_limits = None
    cases = [wl.get("tiny_f32_block_causal"),
             wl.small_workload("lumina_mini", 1, 3, 1, 8, (("I", 1, 4, 4),), (4, 4), pos_mode="grid_hw",
                               mask_mode="full", dtype="f32", seed=0)]
    out = {}
    import contextlib
    ctx = threadpool_limits(1) if threadpool_limits else contextlib.nullcontext()
    with ctx:
        for w in cases:
            d = wl.draw(w)
            mask, shapes = wl.sequence_inputs(w)
            reps, t0 = 0, time.perf_counter()
            while time.perf_counter() - t0 < 0.5:
                md = ometa.build_token_metadata(mask, shapes, w.pos_mode)
                qp = oqr.qknorm_rope(d.vals["q"], d.vals["wq"], w.eps, md["pos_ids"], w.axes)
                kp = oqr.qknorm_rope(d.vals["k"], d.vals["wk"], w.eps, md["pos_ids"], w.axes)
                oatt.attention(qp, kp, d.vals["v"], md["image_ids"], w.mask_mode)
                reps += 1
            el = (time.perf_counter() - t0) / reps
            lim = (np.full(w.n_new, w.seq_len) if w.mask_mode == "full"
                   else ometa.build_token_metadata(mask, shapes, w.pos_mode)["kv_limit"])
            flops = 4.0 * w.head_dim * int(np.sum(lim)) * w.batch * w.heads
            out[w.name] = {"seconds_per_step": el, "gflops": flops / el / 1e9, "threads": 1,
                           "step": "metadata + norm/rope of Q and K + attention, all rows"}
    return out


def cpu_baseline(w: wl.Workload, drawn: wl.Drawn, budget_s: float = 12.0, text_valid=None):
    """The fp64 oracle (as it stands) on the host: norm + rope of the sampled
    query rows, then their attention rows; rows drawn at random from the
    workload until the time budget is used.  Scaled to the useful FLOP rate
    (with a text mask: padded keys left out and not counted)."""
    import oracle.attention as oatt
    import oracle.key_padding as okp
    import oracle.metadata as ometa
    import oracle.qknorm_rope as oqr
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = len(os.sched_getaffinity(0))
    mask, shapes = wl.sequence_inputs(w)
    md = ometa.build_token_metadata(mask, shapes, w.pos_mode)
    P = w.prefix_len
    pos = md["pos_ids"][P:]
    t0 = time.perf_counter()
    nkw = dict(norm=w.qk_norm, linear_factor=w.rope_linear, ntk_factor=w.rope_ntk)
    kp = oqr.qknorm_rope(drawn.vals["k"], drawn.vals["wk"], w.eps, pos, w.axes, bias=drawn.vals.get("bk"), **nkw)
    k_all = np.concatenate([drawn.vals["k_cache"], kp], axis=1) if P else kp
    v_all = np.concatenate([drawn.vals["v_cache"], drawn.vals["v"]], axis=1) if P else drawn.vals["v"]
    valid = okp.joint_key_valid(mask, text_valid) if text_valid is not None else None
    below = (np.concatenate([np.zeros((w.batch, 1), np.int64), np.cumsum(valid, axis=1)], axis=1)
             if valid is not None else None)
    rng = np.random.default_rng(0)
    rows_done, pairs = 0, 0
    chunk = 64
    while time.perf_counter() - t0 < budget_s:
        rows = np.sort(rng.choice(w.n_new, size=chunk, replace=False))
        qp = oqr.qknorm_rope(drawn.vals["q"][:, rows], drawn.vals["wq"], w.eps, pos[rows], w.axes,
                             bias=drawn.vals.get("bq"), **nkw)
        for j, r in enumerate(rows):
            oatt.attention(qp[:, j:j + 1], k_all, v_all, md["image_ids"], w.mask_mode, q_offset=P + int(r),
                           key_valid=valid)
        rows_done += rows.size
        lim = md["kv_limit"][P + rows] if w.mask_mode == "block_causal" else np.full(rows.size, w.seq_len)
        pairs += int(lim.sum()) * w.batch if below is None else int(below[:, lim].sum())
    elapsed = time.perf_counter() - t0
    flops = 4.0 * w.head_dim * pairs * w.heads
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": "%d random query rows (all %d heads x batch %d) of %s, each row's attention computed on "
                      "its own (one oracle call per row), incl. K norm+rope of every token; %.1f s wall; BLAS "
                      "threads %d" % (rows_done, w.heads, w.batch, w.name, elapsed, threads),
            "seconds": elapsed}


def bench_cfg(name: str, steps: int, warmup: int, cpu_budget: float, no_cpu: bool,
              ramp_s: float = 0.3) -> dict:
    """The norm-rescaled guidance step on its own: `steps` back-to-back
    launches rotating over enough (cond, uncond, out) copies that one launch's
    data were not touched by the launches just before it (more than the 256 MB
    Infinity Cache).  One pair of HIP events on the launch stream brackets all
    of them (a pair per launch would add about 2 us to a 12 us kernel); the
    per-launch pairs of a second pass give the median and minimum."""
    import torch
    import diffusion_transformer_joint_token_amd as dit
    w = wl.CFG_WORKLOADS[name]
    bits, vals = wl.draw_cfg(w.rows, w.channels, w.seed, w.dtype)

    def dev(x):
        if w.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
        return torch.from_numpy(np.ascontiguousarray(x)).cuda()
    elem = 2 if w.dtype == "bf16" else 4
    per_call = 3 * w.rows * w.channels * elem           # read cond + uncond, write out
    copies = max(2, -(-(512 << 20) // per_call))        # > 2x the Infinity Cache in flight
    conds = [dev(bits["cond"]) for _ in range(copies)]
    uncs = [dev(bits["uncond"]) for _ in range(copies)]
    outs = [torch.empty_like(conds[0]) for _ in range(copies)]
    stream = torch.cuda.current_stream()
    for i in range(warmup):
        dit.cfg_norm_rescale(conds[i % copies], uncs[i % copies], w.guidance, out=outs[i % copies])
    ramp_steps = ramp_clocks(torch, lambda: dit.cfg_norm_rescale(conds[0], uncs[0], w.guidance, out=outs[0]),
                             ramp_s)
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for i in range(steps):
        dit.cfg_norm_rescale(conds[i % copies], uncs[i % copies], w.guidance, out=outs[i % copies])
    t1.record(stream)
    torch.cuda.synchronize()
    ms_mean = t0.elapsed_time(t1) / steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i, (a, b) in enumerate(ev):
        a.record(stream)
        dit.cfg_norm_rescale(conds[i % copies], uncs[i % copies], w.guidance, out=outs[i % copies])
        b.record(stream)
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in ev]
    gbs = per_call / (ms_mean * 1e-3) / 1e9
    line = {
        "metric": "norm-rescaled CFG GB/s (HBM bytes moved per second)", "value": gbs, "unit": "GB/s",
        "n_gpus": 1, "steps": steps, "warmup": warmup, "ms_per_step": ms_mean, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "rows": w.rows, "channels": w.channels, "guidance": w.guidance,
                   "step": "uncond + s (cond - uncond), rescaled per token to ||cond||"},
        "per_launch_events": {"ms_median": float(np.median(ms)), "ms_min": float(np.min(ms))},
        "rotated_copies": copies,
        "clock_ramp": {"seconds": ramp_s, "launches": ramp_steps},
        "roofline": {"bound": "hbm", "achieved": gbs, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": gbs / PEAK_HBM_GBS, "traffic": measured_traffic(w, CFG_TRAFFIC_FILE, CFG_SOURCE),
                     "kernel": "cfg_norm_rescale_kernel",
                     "bytes_per_launch": per_call, "launch_ms_mean": ms_mean},
        "cpu_baseline": None,
    }
    if not no_cpu:
        import oracle.cfg as ocfg
        try:
            from threadpoolctl import threadpool_info
            threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        except Exception:  # noqa: BLE001
            threads = len(os.sched_getaffinity(0))
        rng = np.random.default_rng(0)
        t0, done = time.perf_counter(), 0
        while time.perf_counter() - t0 < cpu_budget:
            r0 = int(rng.integers(0, w.rows - 4096))
            ocfg.norm_rescaled_cfg(vals["cond"][r0:r0 + 4096], vals["uncond"][r0:r0 + 4096], w.guidance)
            done += 4096
        el = time.perf_counter() - t0
        line["cpu_baseline"] = {"value": 3 * done * w.channels * elem / el / 1e9, "unit": "GB/s",
                                "cores": int(threads), "kind": "oracle",
                                "sample": "%d rows (blocks of 4096) of %s, %.1f s" % (done, w.name, el)}
    return line


def _counter_rows(path: str):
    import csv
    import glob
    rows = []
    for f in sorted(glob.glob(os.path.join(path, "**", "*counter_collection.csv"), recursive=True)):
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    if not rows:
        raise SystemExit("no rocprofv3 counter_collection.csv under %s" % path)
    return rows


def _per_dispatch(rows, kernel_substr: str, counter: str) -> float:
    """Mean over dispatches of one kernel of a counter summed over its instances."""
    per = {}
    for r in rows:
        if kernel_substr in r["Kernel_Name"] and r["Counter_Name"] == counter:
            per[r["Dispatch_Id"]] = per.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit("counter %s not found for kernel %s" % (counter, kernel_substr))
    return sum(per.values()) / len(per)


def summarize_cfg_counters(root: str, copy_mib: int, workload: str) -> int:
    """CPU only: FETCH_SIZE / WRITE_SIZE of the guidance kernel (runs fetch/
    and write/ under root) scaled by the copy calibration runs (copy_fetch/,
    copy_write/), written as the traffic record bench.py --cfg reads."""
    fetch = _per_dispatch(_counter_rows(os.path.join(root, "fetch")), "cfg_norm_rescale", "FETCH_SIZE")
    write = _per_dispatch(_counter_rows(os.path.join(root, "write")), "cfg_norm_rescale", "WRITE_SIZE")
    cf = _per_dispatch(_counter_rows(os.path.join(root, "copy_fetch")), "copyBuffer", "FETCH_SIZE")
    cw = _per_dispatch(_counter_rows(os.path.join(root, "copy_write")), "copyBuffer", "WRITE_SIZE")
    copy_kib = copy_mib * 1024.0
    fs, ws = copy_kib / cf, copy_kib / cw
    rec = {"kernel": "cfg_norm_rescale_kernel", "workload": workload, "kernel_source_sha256": source_sha(CFG_SOURCE),
           "copy_bytes": copy_mib << 20, "copy_fetch_kib": cf, "copy_write_kib": cw, "fetch_scale": fs,
           "write_scale": ws, "fetch_bytes": fetch * fs * 1024.0, "write_bytes": write * ws * 1024.0}
    rec["hbm_bytes_per_launch"] = rec["fetch_bytes"] + rec["write_bytes"]
    print(json.dumps(rec, indent=1, sort_keys=True))
    return 0


def summarize_counters(root: str, copy_mib: int, workload: str) -> int:
    """Turn rocprofv3 --pmc runs into the HBM-traffic record bench.py reports.

    Expects sub-directories of ``root``: fetch/ and write/ (FETCH_SIZE and
    WRITE_SIZE over a bench.py run), copy_fetch/ and copy_write/ (the same
    counters over ``bench.py --copy-calibration copy_mib``) and optionally
    sq/ (SQ_* counters).  Each counter is scaled by (known copy bytes) /
    (counter reading for the copy kernel)."""
    copy_bytes = copy_mib << 20
    cf = _per_dispatch(_counter_rows(os.path.join(root, "copy_fetch")), "copyBuffer", "FETCH_SIZE")
    cw = _per_dispatch(_counter_rows(os.path.join(root, "copy_write")), "copyBuffer", "WRITE_SIZE")
    fetch_scale, write_scale = copy_bytes / (cf * 1024.0), copy_bytes / (cw * 1024.0)
    fr, wr = _counter_rows(os.path.join(root, "fetch")), _counter_rows(os.path.join(root, "write"))
    rec = {"workload": workload, "kernel": "attn_fwd_bf16_kernel", "kernel_source_sha256": source_sha(ATTN_SOURCE),
           "copy_bytes": copy_bytes, "copy_fetch_kib": cf, "copy_write_kib": cw, "fetch_scale": fetch_scale,
           "write_scale": write_scale, "kernels": {}}
    for name, key in (("attention", "attn_fwd_bf16"), ("qknorm_rope", "qknorm_rope"), ("token_metadata", "token_meta")):
        f = _per_dispatch(fr, key, "FETCH_SIZE") * 1024.0 * fetch_scale
        wb = _per_dispatch(wr, key, "WRITE_SIZE") * 1024.0 * write_scale
        rec["kernels"][name] = {"fetch_bytes": f, "write_bytes": wb, "hbm_bytes": f + wb}
    rec["hbm_bytes_per_launch"] = rec["kernels"]["attention"]["hbm_bytes"]
    sq_dir = os.path.join(root, "sq")
    if os.path.isdir(sq_dir):
        sq = _counter_rows(sq_dir)
        names = sorted({r["Counter_Name"] for r in sq})
        rec["attention_sq"] = {n: _per_dispatch(sq, "attn_fwd_bf16", n) for n in names}
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(rec, fh, indent=1, sort_keys=True)
    print(json.dumps(rec, indent=1, sort_keys=True))
    return 0


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--clock-ramp-s", type=float, default=0.3, metavar="S",
                    help="after the warm-up steps, keep running untimed steps until S seconds have passed, so "
                         "that the timed steps run at the settled clock")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD, choices=list(wl.WORKLOADS) + list(wl.VARIANTS))
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the host oracle timing")
    ap.add_argument("--multistep", type=int, default=0, metavar="N",
                    help="also time N denoising steps: one full step, then N-1 steps that recompute only the "
                         "target block against the cached prefix K/V; adds a 'multistep' object to the line")
    ap.add_argument("--shard-heads", type=int, default=1, metavar="K",
                    help="run one GPU's share of a K-way head-sharded job: heads and kv_heads divided by K")
    ap.add_argument("--text-padding", default="none", choices=["none", "right", "random"],
                    help="pad the text per sample (seeded text mask: 'right' keeps a random-length prefix, "
                         "'random' a coin per token) and run the padded attention entry points")
    ap.add_argument("--cfg", default=None, choices=list(wl.CFG_WORKLOADS),
                    help="benchmark the norm-rescaled guidance step on this workload instead (own JSON line)")
    ap.add_argument("--unfused-q", action="store_true",
                    help="two-kernel form: the norm kernel writes Q' and the attention reads it (default for bf16 "
                         "with the per-head RMSNorm: Q's norm and rotation inside the attention kernel)")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the step and attention timings of the other bf16 workloads (the line's `configs`)")
    ap.add_argument("--no-gemm-reference", action="store_true",
                    help="skip the library bf16 GEMM timed beside the attention (the line's `library_gemm`)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB five times (the reference "
                         "kernel that scales the FETCH_SIZE / WRITE_SIZE counters) and exit")
    ap.add_argument("--summarize-counters", metavar="DIR", default=None,
                    help="CPU only: read rocprofv3 --pmc outputs under DIR and write the HBM-traffic record")
    args = ap.parse_args(argv)

    if args.summarize_counters:
        if args.cfg:
            return summarize_cfg_counters(args.summarize_counters, args.copy_calibration or 256, args.cfg)
        return summarize_counters(args.summarize_counters, args.copy_calibration or 256, args.workload)
    if args.gpus != 1:
        print("bench.py runs on exactly one GPU: this build has no multi-GPU path "
              "(--gpus %d requested)" % args.gpus, file=sys.stderr)
        return 2
    import torch
    if not torch.cuda.is_available():
        print("bench.py needs an MI355X GPU (none visible)", file=sys.stderr)
        return 2

    if args.cfg:
        print(json.dumps(bench_cfg(args.cfg, args.steps, args.warmup, args.cpu_budget, args.no_cpu_baseline,
                                   args.clock_ramp_s)),
              flush=True)
        return 0

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("copied %d bytes five times" % n)
        return 0

    clocks_before = read_clocks()
    w = wl.get(args.workload)
    if args.shard_heads > 1:
        K = args.shard_heads
        if w.heads % K or w.kv_heads % K:
            print("--shard-heads %d does not divide %d/%d heads" % (K, w.heads, w.kv_heads), file=sys.stderr)
            return 2
        w = dataclasses.replace(w, name="%s_heads_div%d" % (w.name, K), heads=w.heads // K,
                                kv_heads=w.kv_heads // K)
    if args.text_padding != "none":
        if wl.n_text_tokens(w) == 0:
            print("--text-padding needs a workload with text tokens", file=sys.stderr)
            return 2
        w = dataclasses.replace(w, name="%s_textpad_%s" % (w.name, args.text_padding))
    log("workload %s: B=%d H=%d/%d D=%d S=%d (queries %d) mask=%s dtype=%s" % (
        w.name, w.batch, w.heads, w.kv_heads, w.head_dim, w.seq_len, w.n_new, w.mask_mode, w.dtype))
    step = Step(w, "cuda", args.text_padding, fuse_q=not args.unfused_q)
    step.run()
    torch.cuda.synchronize()
    step.meta.check()
    valid = None
    if step.kv is not None:
        step.kv.check()
        valid = text_valid_keys(wl.sequence_inputs(w)[0], step.tv)
        log("valid text tokens per sample: %s of %d" % (step.tv.sum(axis=1).tolist(), step.tv.shape[1]))
    kv_limit = step.meta.kv_limit.cpu().numpy()
    pairs = useful_pairs(kv_limit, w, valid)
    flops = 4.0 * w.head_dim * pairs * w.heads
    log("useful pairs per head (batch summed) %d  useful FLOPs/step %.4e" % (pairs, flops))

    t = time_gpu(step, args.steps, args.warmup, args.clock_ramp_s)
    log("timing: %s" % json.dumps(t))
    clocks_load = clocks_under_load(torch, step.run)
    log("clocks under load: %s" % json.dumps(clocks_load))
    cold = time_norm_cold(step, ramp_s=args.clock_ramp_s)
    log("norm/rope with rotated inputs: %s" % json.dumps(cold))
    props = torch.cuda.get_device_properties(0)
    value = flops / (t["step_ms"] * 1e-3) / 1e12
    attn_tflops = flops / (t["attn_ms_mean"] * 1e-3) / 1e12
    elem = 2 if w.dtype == "bf16" else 4
    # Norm kernel traffic: read + write of the heads it norms.
    normed_heads = w.kv_heads if step.fused else w.heads + w.kv_heads
    norm_bytes = 2 * w.batch * w.n_new * normed_heads * w.head_dim * elem

    roofline = {"bound": "mfma", "achieved": attn_tflops, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": attn_tflops / PEAK_BF16_TFLOPS, "traffic": measured_traffic(w),
                "kernel": kernel_label(w.head_dim, step.kv is not None, step.fused),
                "launch_ms_mean": t["attn_ms_mean"],
                "launch_ms_min": t["attn_ms_min"], "flops_per_launch": flops}
    line = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": t["step_ms"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "batch": w.batch, "heads": w.heads, "kv_heads": w.kv_heads,
                   "head_dim": w.head_dim, "seq_len": w.seq_len, "queries": w.n_new, "mask": w.mask_mode,
                   "rope_axes": list(w.axes), "qk_norm": w.qk_norm, "rope_linear_factor": w.rope_linear,
                   "rope_ntk_factor": w.rope_ntk,
                   "step": "token metadata + qk-%s/rope + attention" % (
                       "rmsnorm" if w.qk_norm == "rms_per_head" else "layernorm-across-heads"),
                   "q_norm": "inside the attention kernel" if step.fused else "norm kernel (Q' through HBM)"},
        "pct_bf16_peak": 100.0 * value / PEAK_BF16_TFLOPS,
        "attention_only": {"tflops": attn_tflops, "pct_bf16_peak": 100.0 * attn_tflops / PEAK_BF16_TFLOPS,
                           "mfma_work_frac": attn_tflops * padded_work_factor(w.head_dim) / PEAK_BF16_TFLOPS,
                           "ms_mean": t["attn_ms_mean"], "ms_median": t["attn_ms_median"],
                           "ms_min": t["attn_ms_min"]},
        "qknorm_rope": {"heads": "k only" if step.fused else "q and k", "ms": t["norm_ms"], "gbs": norm_bytes / (t["norm_ms"] * 1e-3) / 1e9,
                        "frac_hbm": norm_bytes / (t["norm_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS,
                        "bytes": norm_bytes,
                        "rotated_inputs": {"copies": 3, "ms_mean": cold["ms_mean"], "ms_median": cold["ms_median"],
                                           "gbs": norm_bytes / (cold["ms_mean"] * 1e-3) / 1e9,
                                           "frac_hbm": norm_bytes / (cold["ms_mean"] * 1e-3) / 1e9 / PEAK_HBM_GBS}},
        "device": {"name": props.name, "arch": getattr(props, "gcnArchName", ""),
                   "compute_units": props.multi_processor_count},
        "token_metadata_ms": t["meta_ms"],
        "step_timing": {"host_wall_ms_per_step": t["wall_ms_per_step"],
                        "clock_ramp": {"seconds": args.clock_ramp_s, "steps": t["ramp_steps"]},
                        "ms_per_step_with_kernel_events": t["step_ms_with_kernel_events"]},
        "roofline": roofline,
        "cpu_baseline": None,
    }
    if step.tv is not None:
        line["config"]["text_padding"] = {"kind": args.text_padding, "text_tokens": int(step.tv.shape[1]),
                                          "valid_per_sample": step.tv.sum(axis=1).tolist()}
        line["config"]["step"] = "token metadata + key validity + qk-rmsnorm/rope + padded attention"
    other = (not args.no_other_configs and args.workload == DEFAULT_WORKLOAD and args.shard_heads == 1
             and args.text_padding == "none" and not args.unfused_q)
    if other:
        line["configs"] = {}
        for name in OTHER_CONFIGS:
            c = measure_config(name, args.steps, args.warmup, args.clock_ramp_s)
            log("config %s: %s" % (name, json.dumps(c)))
            line["configs"][name] = c
    line["clocks"] = {"before": clocks_before, "under_load": clocks_load, "after": read_clocks()}
    sclk = clocks_load.get("sclk_mhz") if isinstance(clocks_load, dict) else None
    if sclk:
        # The published peak assumes 2.4 GHz; under load the card holds a lower
        # shader clock (power limit), so this is the fraction of the peak that
        # the measured clock allows.
        ghz = sum(sclk) / len(sclk) / 1000.0
        line["attention_only"]["frac_of_peak_at_measured_sclk"] = attn_tflops / (PEAK_BF16_TFLOPS * ghz / PEAK_SCLK_GHZ)
    if other and not args.no_gemm_reference:
        g = library_gemm_reference(torch)
        g["attention_vs_gemm"] = attn_tflops / g["tflops"]
        log("library gemm: %s" % json.dumps(g))
        line["library_gemm"] = g
    line["host"] = {"cpu_model": cpu_model(), "cores": len(os.sched_getaffinity(0))}
    if args.multistep:
        ms = multistep(step, args.multistep, args.steps, args.warmup, t["step_ms"], args.clock_ramp_s)
        log("multistep: %s" % json.dumps(ms))
        line["multistep"] = ms
    if not args.no_cpu_baseline:
        log("cpu baseline: oracle on host cores, ~%.0f s" % args.cpu_budget)
        cb = cpu_baseline(w, step.drawn, args.cpu_budget, step.tv)
        line["cpu_baseline"] = {k: cb[k] for k in ("value", "unit", "cores", "kind", "sample")}
        line["cpu_baseline"]["single_thread"] = cpu_single_thread()
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
