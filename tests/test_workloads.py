"""Seeded input generators: bf16 rounding and workload structure (CPU only)."""
import numpy as np
import torch

from mixture_experts_layer_17_amd import workloads as wl
from oracle import moe_oracle as mo


def test_bf16_round_to_nearest_even_matches_torch():
    r = np.random.default_rng(0)
    a = np.concatenate([r.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.00390625, 1.01171875, -1.00390625, 0.0, -0.0], np.float32)])
    bits = wl.f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, ref)
    back = wl.bf16_bits_to_f32(bits)
    np.testing.assert_array_equal(back, torch.from_numpy(a).to(torch.bfloat16).float().numpy())


def test_inputs_are_deterministic_and_shaped():
    w = wl.scaled(wl.WORKLOADS[3], T=64, d=64, f=64, E=16)
    a = wl.make_inputs(w)
    b = wl.make_inputs(w)
    for key in ("x", "w_gate", "w_up", "w_down", "dout", "logits"):
        np.testing.assert_array_equal(a[key], b[key])
    assert a["w_gate"].shape == (16, 64, 64) and a["w_down"].shape == (16, 64, 64)
    assert abs(float(a["w_gate"].std()) - 0.02) < 0.002


def test_zipf_routing_is_skewed_with_empty_experts():
    w = wl.WORKLOADS[4]
    bias = wl.zipf_bias(w.E, wl.DEFAULT_SEED, w.wid)
    assert sorted(np.round(np.exp(-bias / 3)).astype(int)) == list(range(1, w.E + 1))
    T = 4096
    logits = wl.normal((T, w.E), 1.0, wl.DEFAULT_SEED, w.wid, wl.TID_LOGITS) + bias[None, :]
    idx = mo.topk_select(logits, w.k)
    counts = np.bincount(idx.ravel(), minlength=w.E)
    assert counts.max() >= 8 * counts.mean() and (counts == 0).sum() >= 5
