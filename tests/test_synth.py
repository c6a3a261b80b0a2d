"""The seeded input generator: bf16 rounding and the workload recipes."""

import numpy as np
import pytest

from linear_cross_entropy_03_amd import synth


def test_bf16_rounding_matches_torch_nearest_even():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    a = np.concatenate([rng.standard_normal(4096).astype(np.float32) * 3,
                        np.array([1.00390625, 1.01171875, -2.00781250, 0.0, -0.0,
                                  3.4e38, 1e-40], dtype=np.float32)])
    bits = synth.f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bits, ref)
    back = synth.bf16_bits_to_f32(bits)
    np.testing.assert_array_equal(back, torch.from_numpy(a).to(torch.bfloat16).float().numpy())


def test_f16_storage_matches_torch_nearest_even():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(1)
    a = np.concatenate([rng.standard_normal(4096).astype(np.float32) * 3,
                        np.array([1.00048828125, 1.00146484375, 65504.0, 70000.0, 6e-8, -0.0],
                                 dtype=np.float32)])
    inp = synth.make_ce_inputs(4, 8, "f16")  # exercises the f16 branch end to end
    assert inp["logits"].dtype == np.uint16
    with np.errstate(over="ignore"):   # 70000 rounds to inf, as in torch
        bits, exact = synth._store(a, "f16")
    ref = torch.from_numpy(a).to(torch.float16)
    np.testing.assert_array_equal(bits, ref.view(torch.int16).numpy().view(np.uint16))
    np.testing.assert_array_equal(exact, ref.float().numpy())


def test_ignore_counts_and_ranges():
    inp = synth.make_flce_inputs(256, 64, 1024, "f32", ignore_frac=0.1)
    y = inp["targets"]
    assert y.dtype == np.int32 and int((y == -100).sum()) == 26
    assert np.all((y == -100) | ((y >= 0) & (y < 1024)))
    ce = synth.make_ce_inputs(1024, 4096, "bf16", ignore_frac=0.05)
    assert int((ce["targets"] == -100).sum()) == 51


def test_zipf_head_frequency():
    inp = synth.make_flce_inputs(32768, 8, 128256, "bf16", target_dist="zipf")
    y = inp["targets"]
    top = float((y == 0).sum()) / float((y != -100).sum())
    # P(rank 1) = 1 / H_{V,1.1} ~= 0.133 for V = 128256.
    assert 0.12 < top < 0.146


def test_deterministic_by_seed():
    a = synth.make_flce_inputs(16, 8, 32, "bf16", bias_std=0.01, seed=3)
    b = synth.make_flce_inputs(16, 8, 32, "bf16", bias_std=0.01, seed=3)
    for k in ("X", "W", "bias", "targets"):
        np.testing.assert_array_equal(a[k], b[k])
