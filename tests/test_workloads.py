"""Seeded input generators: determinism, shapes and the bf16 rounding (CPU only)."""
import numpy as np
import pytest

import workloads as W


def test_round_bf16_matches_torch():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 100000),
                        np.array([0.0, -0.0, 1.0, 65504.0, 3.0e38, 1e-40, np.inf, -np.inf], np.float32)])
    x = x.astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(W.round_bf16(x), ref)


def test_generators_deterministic_and_shaped():
    w = W.WORKLOADS["gla_340m"]
    a = W.gla_inputs(w, B=1, L=128)
    b = W.gla_inputs(w, B=1, L=128)
    for n in ("q", "k", "v", "g", "do", "dht"):
        np.testing.assert_array_equal(a[n], b[n])
    assert a["q"].shape == (1, 4, 128, 128) and a["v"].shape == (1, 4, 128, 256)
    assert np.all(a["g"] <= 0) and a["h0"] is None
    # bf16-exact values
    np.testing.assert_array_equal(W.round_bf16(a["k"]), a["k"])
    s = W.gsa_inputs(W.WORKLOADS["gsa_340m"], B=1, L=64)
    assert s["g"].shape == (1, 4, 64, 64) and np.all(s["g"] <= 0)
    d = W.decode_inputs(W.WORKLOADS["decode"], T=3, B=2)
    assert d["q"].shape == (3, 2, 4, 128) and d["state"].shape == (2, 4, 128, 256)


def test_long_sequence_bias_channels():
    """13 of 128 channels per head biased toward alpha ~ 1 (mean gate ~ -2e-3 vs ~ -0.05)."""
    w = W.WORKLOADS["gla_long"]
    x = W.gla_inputs(w, L=512, with_grad=False)
    mean = x["g"].mean(axis=(0, 2))            # [H, Dk]
    slow = (mean > -0.01).sum(axis=1)
    assert np.all(slow == 13), slow
