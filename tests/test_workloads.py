"""Seeded input generators: determinism, shapes and bf16 rounding (CPU only)."""
import numpy as np
import torch

import workloads as W


def test_bf16_round_matches_torch():
    rng = np.random.default_rng(0)
    a = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.005859375, 3.4e38, 1e-40], np.float32)])
    ours = W.bf16_round(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(ours.view(np.uint32), ref.view(np.uint32))
    bits = W.bf16_bits(ours)
    assert np.array_equal(bits, torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


def test_generators_deterministic_and_shaped():
    spec = W.WORKLOADS["tiny"]
    a = W.gen_scan_inputs(spec)
    b = W.gen_scan_inputs(spec)
    for k in a:
        assert np.array_equal(a[k], b[k]), k
    assert a["x"].shape == (1, 64, 8) and a["B"].shape == (1, 64, 4) and a["A"].shape == (8, 4)
    assert np.array_equal(a["A"], -np.tile(np.arange(1, 5, dtype=np.float32), (8, 1)))
    assert np.all(a["D"] == 1.0) and np.all(a["conv_b"] == 0.0)
    # the bias is the inverse softplus of a step size in [1e-3, 1e-1]
    s = np.logaddexp(0.0, a["delta_bias"].astype(np.float64))
    assert np.all((s > 0.99e-3) & (s < 1.01e-1))


def test_bf16_workload_values_are_bf16():
    spec = W.WORKLOADS["train"]
    a = W.gen_scan_inputs(spec, batch=1, seqlen=32, d_inner=64)
    for k in ("x", "delta", "z", "B", "C"):
        assert np.all((a[k].view(np.uint32) & 0xFFFF) == 0), k
    s = np.logaddexp(0.0, a["delta"].astype(np.float64))
    assert np.all((s > 0.97e-3) & (s < 1.03e-1))
    assert np.all(a["delta_bias"] == 0.0)


def test_decode_inputs():
    spec = W.DECODE
    p0 = W.gen_decode_layer_params(spec, 0)
    p1 = W.gen_decode_layer_params(spec, 1)
    assert not np.array_equal(p0["conv_w"], p1["conv_w"])
    s = W.gen_decode_step_inputs(spec, 3, 5, streams=2)
    assert s["x"].shape == (2, 8192) and s["B"].shape == (2, 16)
    s2 = W.gen_decode_step_inputs(spec, 3, 5, streams=2)
    assert np.array_equal(s["delta"], s2["delta"])
