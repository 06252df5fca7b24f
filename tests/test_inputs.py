"""The seeded input generator: determinism, the A recipe and bf16 encoding."""
import numpy as np
import torch

import ssm_inputs


def test_seeded_and_deterministic():
    a = ssm_inputs.make_scan_inputs(2, 8, 16, 32, io_dtype="bf16", gate=True, seed=0)
    b = ssm_inputs.make_scan_inputs(2, 8, 16, 32, io_dtype="bf16", gate=True, seed=0)
    c = ssm_inputs.make_scan_inputs(2, 8, 16, 32, io_dtype="bf16", gate=True, seed=1)
    for k in ("u", "delta", "B", "C", "z", "A", "D", "delta_bias"):
        assert np.array_equal(a[k], b[k])
    assert not np.array_equal(a["u"], c["u"])


def test_a_is_minus_n_plus_one():
    A = ssm_inputs.a_matrix(5, 256)
    assert A.dtype == np.float32
    assert np.array_equal(A, -np.broadcast_to(np.arange(1, 257, dtype=np.float32), (5, 256)))


def test_bf16_round_to_nearest_even_matches_torch():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(100000).astype(np.float32) * np.float32(100)
    # ties: values exactly halfway between two bf16 numbers
    ties = (np.arange(1, 2000, dtype=np.uint32) << 16 | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties, np.array([0.0, -0.0, np.inf, -np.inf], np.float32)])
    ours = ssm_inputs.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = ssm_inputs.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_step_size_bias_range():
    inp = ssm_inputs.make_scan_inputs(1, 4096, 16, 1, seed=0)
    bias = inp["delta_bias"].astype(np.float64)
    dt0 = np.log1p(np.exp(bias))
    assert dt0.min() >= 1e-3 * (1 - 1e-5) and dt0.max() <= 1e-1 * (1 + 1e-5)


def test_update_inputs_shapes():
    inp = ssm_inputs.make_update_inputs(3, 10, 16, io_dtype="bf16")
    assert inp["state"].shape == (3, 10, 16) and inp["state"].dtype == np.float32
    assert inp["u"].dtype == np.uint16 and inp["u"].shape == (3, 10)
    d = ssm_inputs.to_f64(inp["delta"])
    assert (d > 0).all()
