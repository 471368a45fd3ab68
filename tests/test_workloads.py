"""The seeded input generator: bf16 rounding and the sequence layouts."""
import numpy as np
import torch

import workloads as wl


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 3
    x = np.concatenate([x, np.float32([1.00390625, 1.01171875, -1.00390625, 0.0, 65504.0])])
    ours = wl.bf16_round_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(wl.bf16_bits_to_f64(ours), torch.from_numpy(x).to(torch.bfloat16).double().numpy())


def test_layouts_and_sizes():
    sizes = {name: w.seq_len for name, w in wl.WORKLOADS.items()}
    assert list(sizes.values()) == [32, 4096, 5120, 6656, 21504]
    w5 = wl.get(4)
    assert w5.prefix_len == 5120 and w5.n_new == 16384
    for w in wl.WORKLOADS.values():
        mask, shapes = wl.sequence_inputs(w)
        assert mask.size == w.seq_len
        assert int(mask.sum()) == sum(f * h * ww for f, h, ww in shapes)
        assert sum(w.axes) == w.head_dim and all(a % 2 == 0 for a in w.axes)
        assert w.heads % w.kv_heads == 0


def test_draw_is_seeded_and_prefix_stable():
    w = wl.small_workload("t", 1, 2, 1, 8, (("T", 3), ("I", 1, 2, 2)), (4, 2, 2), seed=5)
    a = wl.draw(w)
    b = wl.draw(w, parts=("v",))
    assert np.array_equal(a.bits["v"], b.bits["v"])
    assert a.bits["q"].dtype == np.uint16 and a.vals["q"].dtype == np.float64
    assert a.vals["q"].shape == (1, 7, 2, 8) and a.vals["k"].shape == (1, 7, 1, 8)


def test_text_mask_recipes():
    w = wl.get("qwen_image21_t1024_i64x64")
    assert wl.n_text_tokens(w) == 1024
    a = wl.text_mask(w, 3, "right")
    assert a.shape == (2, 1024) and a.dtype == np.uint8
    assert np.array_equal(a, wl.text_mask(w, 3, "right"))
    for row in a:  # a valid prefix, then padding
        L = int(row.sum())
        assert L >= 1 and np.all(row[:L] == 1) and np.all(row[L:] == 0)
    r = wl.text_mask(w, 4, "random")
    assert set(np.unique(r)) <= {0, 1} and 0.4 < r.mean() < 0.6
    assert wl.text_mask(w, 5, "none").all()
    assert wl.text_mask(wl.get("lumina_next_full_gqa"), 1, "right").shape == (2, 0)
