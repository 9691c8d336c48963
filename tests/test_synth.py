"""The seeded input generator: shapes, determinism, rounding and value ranges (CPU only)."""
import numpy as np

from delta_rule_sequence_chunkwise_amd import synth


def test_round_bf16_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -9, 1.0 + 2 ** -9, -2.5, 3.0e-3,
                  1.0 + 2 ** -7 + 2 ** -8], dtype=np.float32)
    y = synth.round_bf16(x)
    # bf16 keeps 7 mantissa bits: 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even (1.0);
    # 1 + 2^-7 + 2^-8 is a tie between 1 + 2^-7 and 1 + 2^-6 -> even (1 + 2^-6)
    assert y[0] == 1.0 and y[1] == 1.0 and y[3] == 1.0
    assert y[2] == np.float32(1.0 + 2 ** -7)
    assert y[6] == np.float32(1.0 + 2 ** -6)
    assert y[4] == -2.5
    assert (y.view(np.uint32) & 0xFFFF).max() == 0
    assert np.all(np.abs(y - x) <= np.abs(x) * 2 ** -8)


def test_tiny_workload_shapes_and_determinism():
    w = synth.WORKLOADS["tiny"]
    a = synth.make_inputs(w)
    b = synth.make_inputs(w)
    assert a["q"].shape == (1, 2, 256, 64) and a["v"].shape == (1, 2, 256, 64)
    assert a["beta"].shape == (1, 2, 256) and a["alpha"] is None and a["S0"] is None
    for name in ("q", "k", "v", "beta", "d"):
        assert a[name].dtype == np.float32
        assert np.array_equal(a[name], b[name])
    assert np.allclose(np.linalg.norm(a["q"], axis=-1), 1.0, atol=1e-6)
    assert np.all((a["beta"] > 0) & (a["beta"] < 1))
    assert np.all(a["d"] > 0)


def test_bf16_workload_values_are_bf16_exact():
    w = synth.Workload("t", B=1, H=2, T=64, dk=128, dv=128)
    x = synth.make_inputs(w)
    for name in ("q", "k", "v"):
        assert (x[name].view(np.uint32) & 0xFFFF).max() == 0
    a = x["alpha"]
    assert np.all((a > 0.85) & (a < 0.9951))


def test_regime_shift_changes_log_d_spread():
    w = synth.Workload("t", B=1, H=4, T=512, dk=128, dv=128, sigma_d_late=0.75)
    x = synth.make_inputs(w)
    ld = np.log(x["d"])
    early, late = ld[:, :, :256].std(), ld[:, :, 256:].std()
    assert abs(early - 0.25) < 0.01 and abs(late - 0.75) < 0.02


def test_decode_inputs():
    w = synth.WORKLOADS["decode"]
    x = synth.make_decode_inputs(w, steps=3, B=2, H=3)
    assert x["S0"].shape == (2, 3, 128, 128)
    assert x["q"].shape == (3, 2, 3, 128) and x["beta"].shape == (3, 2, 3)
    assert abs(x["S0"].std() - 0.02) < 0.002


def test_precond_gates():
    a = synth.make_precond_gates(2, 3, 50, 64, seed=5)
    b = synth.make_precond_gates(2, 3, 50, 64, seed=5)
    assert a["r"].shape == (2, 3, 50) and a["d1"].shape == (2, 3, 64)
    assert np.array_equal(a["r"], b["r"]) and np.array_equal(a["d1"], b["d1"])
    assert a["r"].dtype == np.float32 and np.all((a["r"] > 0.9) & (a["r"] <= 1.0))
    assert np.all(a["d1"] > 0)
