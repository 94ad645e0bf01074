"""The seeded input generator: determinism, prefix stability, distributions, bf16 rounding."""
import numpy as np

import gen


def test_deterministic_and_prefix_stable():
    a = gen.fill(10001, "f32", 1234, 0.5, 2.0)
    b = gen.fill(10001, "f32", 1234, 0.5, 2.0)
    c = gen.fill(333, "f32", 1234, 0.5, 2.0)
    assert np.array_equal(a, b)
    assert np.array_equal(a[:333], c)
    assert not np.array_equal(a, gen.fill(10001, "f32", 1235, 0.5, 2.0))


def test_moments():
    a = gen.fill(1 << 20, "f32", 99, 0.5, 2.0).astype(np.float64)
    assert abs(a.mean() - 0.5) < 0.01
    assert abs(a.std() - 2.0) < 0.01
    z = (a - 0.5) / 2.0
    assert abs(np.mean(z ** 4) - 3.0) < 0.05  # Gaussian kurtosis


def test_bf16_is_rounded_f32():
    f = gen.fill(1 << 16, "f32", 7, 1.0, 0.1)
    b = gen.fill(1 << 16, "bf16", 7, 1.0, 0.1)
    assert np.array_equal(b, gen.round_bf16(f))


def test_round_bf16_nearest_even():
    vals = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20,
                     -2.5, 65504.0, np.inf, -np.inf], dtype=np.float32)
    got = gen.bf16_to_f32(gen.round_bf16(vals))
    want = np.array([1.0, 1.0, 1.0 + 2 ** -6, 1.0 + 2 ** -7, -2.5, 65536.0, np.inf, -np.inf],
                    dtype=np.float32)
    assert np.array_equal(got, want)
    nan = gen.round_bf16(np.array([np.nan], dtype=np.float32))
    assert np.isnan(gen.bf16_to_f32(nan))[0]


def test_outlier_mask():
    n = 1 << 20
    base = gen.fill(n, "f32", 42, 0.0, 1.0)
    out = gen.fill(n, "f32", 42, 0.0, 1.0, outlier_p=0.01, outlier_scale=50.0)
    scaled = out != base
    frac = scaled.mean()
    assert 0.009 < frac < 0.011
    assert np.allclose(out[scaled], base[scaled] * 50.0, rtol=1e-6)


def test_workload_inputs():
    w = gen.WORKLOADS["ln2"].scaled(8)
    d = gen.make_inputs(w)
    assert d["x"].shape == (8, 4096) and d["x"].dtype == np.uint16
    assert d["beta"].shape == (4096,)
    full_prefix = gen.make_inputs(gen.WORKLOADS["ln2"], rows=8)
    assert np.array_equal(d["x"], full_prefix["x"])
    assert gen.sweep_workload("rms", "f32", 384).M == 349525
