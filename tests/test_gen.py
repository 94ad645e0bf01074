"""The seeded input generator: determinism, prefix stability, distributions, bf16 and fp16
rounding, parameter types."""
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


def test_f16_is_rounded_f32():
    f = gen.fill(1 << 16, "f32", 7, 1.0, 0.1)
    h = gen.fill(1 << 16, "f16", 7, 1.0, 0.1)
    assert h.dtype == np.float16
    assert np.array_equal(h.view(np.uint16), gen.round_f16(f).view(np.uint16))


def test_round_f16_matches_numpy():
    """The binary16 encoder against numpy's float32 -> float16 conversion (IEEE round to
    nearest even): normals over many decades, subnormals, ties, overflow, signed zeros."""
    rng = np.random.default_rng(0)
    scale = np.float32(10.0) ** rng.integers(-9, 6, 200000).astype(np.float32)
    vals = np.concatenate([
        rng.standard_normal(200000).astype(np.float32) * scale,
        np.array([0.0, -0.0, np.inf, -np.inf, 65504.0, 65519.99, 65520.0, 65536.0, 2.0 ** -14,
                  2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -25, 2.0 ** -26, 1 - 2.0 ** -12,
                  1 + 2.0 ** -11, 1 + 3 * 2.0 ** -11, -(2.0 ** -15) * 1.5], dtype=np.float32)])
    with np.errstate(over="ignore"):
        want = vals.astype(np.float16)
    assert np.array_equal(gen.round_f16(vals).view(np.uint16), want.view(np.uint16))
    assert np.isnan(gen.round_f16(np.array([np.nan], dtype=np.float32)))[0]


def test_mixed_parameter_type():
    w = gen.Workload("t", "ln", "bf16", 4, 64, 1e-5, config=9, pdtype="f32")
    d = gen.make_inputs(w)
    assert d["x"].dtype == np.uint16 and d["gamma"].dtype == np.float32
    assert d["beta"].dtype == np.float32
    # the same seeds in bf16 round the fp32 parameters
    same = gen.make_inputs(gen.Workload("t", "ln", "bf16", 4, 64, 1e-5, config=9))
    assert np.array_equal(same["gamma"], gen.round_bf16(d["gamma"]))
    assert np.array_equal(same["x"], d["x"])


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
