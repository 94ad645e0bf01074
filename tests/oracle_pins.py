"""Pins for the fp64 oracle: checks against what the pages and mathematics fix.

Each ``pin_*`` takes an :class:`oracle.Oracle` and raises ``AssertionError`` when the
oracle disagrees.  ``test_oracle_pins.py`` runs them on the real oracle (all must pass)
and ``test_oracle_mutants.py`` runs them on deliberately broken copies of the oracle's
source (at least one must fail for every planted mistake).

What pins what:
  * hand-derived worked examples (tests/golden/hand_examples.json) -- forward values,
    eps placement, gamma/beta indexing, row indexing, degenerate rows, backward values,
    and the root-sum-square magnitudes that size the dgamma/dbeta parity bound;
  * invariants: RMS of y is 1 at gamma=1, eps=0; LayerNorm y has mean 0 and variance 1;
    scale (and, for LayerNorm, shift) invariance; dx orthogonality relations at eps=0;
  * central finite differences of the forward for dx, dgamma, dbeta;
  * torch.nn.functional.rms_norm / layer_norm with autograd in float64 on the CPU, an
    independent library implementation;
  * consistency of the bf16 decode and of row selection;
  * the binary16 decode against numpy's float16 (an independent implementation), and
    fp16 / mixed-precision inputs against the same values widened to fp32.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

import gen

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "hand_examples.json")


def _expr(s) -> float:
    """Evaluate one closed-form expression from the golden file (sqrt only)."""
    if isinstance(s, (int, float)):
        return float(s)
    return float(eval(s, {"__builtins__": {}}, {"sqrt": math.sqrt}))


def _exprs(a):
    return np.array([[_expr(v) for v in row] for row in a]) if isinstance(a[0], list) \
        else np.array([_expr(v) for v in a])


def _as_dtype(values, dtype):
    """Exact host bits for small integer / dyadic values."""
    v = np.asarray(values, dtype=np.float64)
    f = v.astype(np.float32)
    assert np.array_equal(f.astype(np.float64), v), "golden inputs must be exact in fp32"
    if dtype == "bf16":
        b = gen.round_bf16(f)
        assert np.array_equal(gen.bf16_to_f32(b).astype(np.float64), v), "must be exact in bf16"
        return b
    return f


def _close(got, want, tol, what):
    got = np.asarray(got, np.float64)
    want = np.asarray(want, np.float64)
    assert got.shape == want.shape, f"{what}: shape {got.shape} != {want.shape}"
    err = np.max(np.abs(got - want) / np.maximum(1.0, np.abs(want))) if got.size else 0.0
    assert err <= tol, f"{what}: max scaled error {err:.3e} > {tol:.1e}"


# ------------------------------------------------------------------ golden examples
def pin_golden_forward(orc):
    cases = json.load(open(GOLDEN))["forward"]
    for c in cases:
        for dtype in ("f32", "bf16"):
            x = _as_dtype(c["x"], dtype)
            g = _as_dtype(c["gamma"], dtype)
            if c["kind"] == "rms":
                y, rstd = orc.rms_fwd(x, g, c["eps"])
            else:
                y, mean, rstd = orc.ln_fwd(x, g, _as_dtype(c["beta"], dtype), c["eps"])
                _close(mean, _exprs(c["mean"]), 1e-14, f"{c['name']} mean")
            _close(rstd, _exprs(c["rstd"]), 1e-14, f"{c['name']} rstd")
            _close(y, _exprs(c["y"]), 1e-14, f"{c['name']} y ({dtype})")


def pin_golden_backward(orc):
    cases = json.load(open(GOLDEN))["backward"]
    for c in cases:
        for dtype in ("f32", "bf16"):
            x = _as_dtype(c["x"], dtype)
            g = _as_dtype(c["gamma"], dtype)
            dy = _as_dtype(c["dy"], dtype)
            if c["kind"] == "rms":
                dx = orc.rms_bwd_dx(dy, x, g, c["eps"])
                dg, sg = orc.rms_dgamma(dy, x, c["eps"])
            else:
                dx = orc.ln_bwd_dx(dy, x, g, c["eps"])
                dg, db, sg, sb = orc.ln_dgamma_dbeta(dy, x, c["eps"])
                _close(db, _exprs(c["dbeta"]), 1e-14, f"{c['name']} dbeta")
                # the size of the dbeta parity bound: root-sum-square of the summed dy
                _close(sb, _exprs(c["dbeta_scale"]), 1e-14, f"{c['name']} dbeta_scale")
            _close(dx, _exprs(c["dx"]), 1e-14, f"{c['name']} dx ({dtype})")
            _close(dg, _exprs(c["dgamma"]), 1e-14, f"{c['name']} dgamma")
            # the size of the dgamma parity bound: root-sum-square of the summed dy * xhat
            _close(sg, _exprs(c["dgamma_scale"]), 1e-14, f"{c['name']} dgamma_scale")


# ------------------------------------------------------------------------ invariants
def _random_rows(M, N, seed, mean=0.0, std=1.0, dtype="f32"):
    return gen.fill(M * N, dtype, seed, mean, std).reshape(M, N)


def pin_rms_unit_rms(orc):
    """gamma = 1, eps = 0: mean(y^2) = ms / (ms + 0) = 1 for every row."""
    for dtype, N in (("f32", 37), ("bf16", 256), ("f32", 1)):
        x = _random_rows(5, N, 11 + N, 0.3, 2.0, dtype)
        ones = _as_dtype(np.ones(N), dtype)
        y, _ = orc.rms_fwd(x, ones, 0.0)
        ms = np.mean(y * y, axis=1)
        assert np.max(np.abs(ms - 1.0)) < 1e-12, f"RMS of y != 1 (N={N}, {dtype})"


def pin_ln_moments(orc):
    """gamma = 1, beta = 0, eps = 0: each row of y has mean 0 and (biased) variance 1."""
    for dtype, N in (("f32", 33), ("bf16", 512)):
        x = _random_rows(6, N, 23 + N, 0.5, 2.0, dtype)
        ones = _as_dtype(np.ones(N), dtype)
        zeros = _as_dtype(np.zeros(N), dtype)
        y, mean, _ = orc.ln_fwd(x, ones, zeros, 0.0)
        assert np.max(np.abs(y.mean(axis=1))) < 1e-12, "LayerNorm output mean != 0"
        assert np.max(np.abs(y.var(axis=1) - 1.0)) < 1e-12, "LayerNorm output variance != 1"
        xd = gen.bf16_to_f32(x) if dtype == "bf16" else x
        assert np.max(np.abs(mean - xd.astype(np.float64).mean(axis=1))) < 1e-12


def pin_invariance(orc):
    """eps = 0: RMS y(a x) = y(x) for a > 0; LayerNorm y(a x + c) = y(x).  Scaling by a
    power of two and shifting small integers keep the fp32 inputs exact."""
    N = 24
    rng = np.random.default_rng(5)
    x = (rng.integers(-64, 64, size=(4, N)) / 16.0).astype(np.float32)
    g = (1.0 + rng.integers(-8, 8, size=N) / 32.0).astype(np.float32)
    b = (rng.integers(-8, 8, size=N) / 32.0).astype(np.float32)
    y1, _ = orc.rms_fwd(x, g, 0.0)
    y2, _ = orc.rms_fwd((x * 4.0).astype(np.float32), g, 0.0)
    assert np.max(np.abs(y1 - y2)) < 1e-12, "RMSNorm not scale invariant"
    z1, _, _ = orc.ln_fwd(x, g, b, 0.0)
    z2, _, _ = orc.ln_fwd((x * 0.25 + 3.0).astype(np.float32), g, b, 0.0)
    assert np.max(np.abs(z1 - z2)) < 1e-12, "LayerNorm not scale/shift invariant"


def pin_dx_orthogonality(orc):
    """eps = 0: RMS sum_j dx_j x_j = 0 (scale invariance); LayerNorm sum_j dx_j = 0 and
    sum_j dx_j x_j = 0 (shift and scale invariance), for any dy and gamma."""
    M, N = 4, 19
    x = _random_rows(M, N, 101, 0.2, 1.5)
    dy = _random_rows(M, N, 102)
    g = gen.fill(N, "f32", 103, 1.0, 0.3)
    xd = x.astype(np.float64)
    dx = orc.rms_bwd_dx(dy, x, g, 0.0)
    assert np.max(np.abs(np.sum(dx * xd, axis=1))) < 1e-11, "RMS: sum dx*x != 0"
    dx = orc.ln_bwd_dx(dy, x, g, 0.0)
    assert np.max(np.abs(np.sum(dx, axis=1))) < 1e-11, "LN: sum dx != 0"
    assert np.max(np.abs(np.sum(dx * xd, axis=1))) < 1e-11, "LN: sum dx*x != 0"


# ---------------------------------------------------------------- finite differences
def _loss(orc, kind, x, g, b, dy, eps):
    if kind == "rms":
        y, _ = orc.rms_fwd(x, g, eps)
    else:
        y, _, _ = orc.ln_fwd(x, g, b, eps)
    return float(np.sum(dy.astype(np.float64) * y))


def _dyadic(rng, shape, lo, hi, scale=64):
    return (rng.integers(int(lo * scale), int(hi * scale), size=shape) / scale).astype(np.float32)


def pin_finite_differences(orc):
    """Central differences of L = sum(dy * y) with respect to x, gamma and beta.
    Inputs are multiples of 2^-6 and the step is 2^-12, so x +- h is exact in fp32."""
    h = 2.0 ** -12
    rng = np.random.default_rng(7)
    for kind in ("rms", "ln"):
        for eps in (0.0, 1e-5, 0.25):
            M, N = 3, 7
            x = _dyadic(rng, (M, N), -3, 3)
            x[:, 0] += 0.5  # keep rows away from zero
            g = _dyadic(rng, N, 0.5, 1.5)
            b = _dyadic(rng, N, -0.5, 0.5)
            dy = _dyadic(rng, (M, N), -1, 1)
            if kind == "rms":
                dx = orc.rms_bwd_dx(dy, x, g, eps)
                dg, _ = orc.rms_dgamma(dy, x, eps)
                db = None
            else:
                dx = orc.ln_bwd_dx(dy, x, g, eps)
                dg, db, _, _ = orc.ln_dgamma_dbeta(dy, x, eps)
            for i in range(M):
                for j in range(N):
                    xp = x.copy(); xp[i, j] += h
                    xm = x.copy(); xm[i, j] -= h
                    fd = (_loss(orc, kind, xp, g, b, dy, eps) - _loss(orc, kind, xm, g, b, dy, eps)) / (2 * h)
                    assert abs(fd - dx[i, j]) < 1e-6 * max(1.0, abs(fd)), \
                        f"{kind} eps={eps}: dx[{i},{j}] {dx[i, j]} vs finite difference {fd}"
            for j in range(N):
                gp = g.copy(); gp[j] += h
                gm = g.copy(); gm[j] -= h
                fd = (_loss(orc, kind, x, gp, b, dy, eps) - _loss(orc, kind, x, gm, b, dy, eps)) / (2 * h)
                assert abs(fd - dg[j]) < 1e-6 * max(1.0, abs(fd)), \
                    f"{kind} eps={eps}: dgamma[{j}] {dg[j]} vs finite difference {fd}"
                if db is not None:
                    bp = b.copy(); bp[j] += h
                    bm = b.copy(); bm[j] -= h
                    fd = (_loss(orc, kind, x, g, bp, dy, eps) - _loss(orc, kind, x, g, bm, dy, eps)) / (2 * h)
                    assert abs(fd - db[j]) < 1e-6 * max(1.0, abs(fd)), \
                        f"ln eps={eps}: dbeta[{j}] {db[j]} vs finite difference {fd}"


# ------------------------------------------------------------ library cross-check
def pin_torch_float64(orc):
    """torch.nn.functional.rms_norm / layer_norm and autograd, float64 on the CPU."""
    import torch
    import torch.nn.functional as F

    for (M, N, eps) in ((5, 48, 1e-6), (3, 33, 0.1), (2, 1, 1e-3)):
        x = _random_rows(M, N, 201 + N, 0.4, 1.7)
        g = gen.fill(N, "f32", 202 + N, 1.0, 0.2)
        b = gen.fill(N, "f32", 203 + N, 0.0, 0.2)
        dy = _random_rows(M, N, 204 + N)
        for kind in ("rms", "ln"):
            xt = torch.tensor(x, dtype=torch.float64, requires_grad=True)
            gt = torch.tensor(g, dtype=torch.float64, requires_grad=True)
            bt = torch.tensor(b, dtype=torch.float64, requires_grad=True)
            if kind == "rms":
                yt = F.rms_norm(xt, (N,), weight=gt, eps=eps)
                y, _ = orc.rms_fwd(x, g, eps)
                dx = orc.rms_bwd_dx(dy, x, g, eps)
                dg, _ = orc.rms_dgamma(dy, x, eps)
            else:
                yt = F.layer_norm(xt, (N,), weight=gt, bias=bt, eps=eps)
                y, _, _ = orc.ln_fwd(x, g, b, eps)
                dx = orc.ln_bwd_dx(dy, x, g, eps)
                dg, db, _, _ = orc.ln_dgamma_dbeta(dy, x, eps)
            yt.backward(torch.tensor(dy, dtype=torch.float64))
            _close(y, yt.detach().numpy(), 1e-12, f"torch {kind} y M={M} N={N}")
            _close(dx, xt.grad.numpy(), 1e-10, f"torch {kind} dx M={M} N={N}")
            _close(dg, gt.grad.numpy(), 1e-10, f"torch {kind} dgamma M={M} N={N}")
            if kind == "ln":
                _close(db, bt.grad.numpy(), 1e-10, f"torch ln dbeta M={M} N={N}")


# ------------------------------------------------------------------ consistency
def pin_bf16_decode_and_rows(orc):
    """bf16 bits and the same values as fp32 give identical results; a row subset gives
    the same rows as the full evaluation."""
    M, N = 9, 40
    xb = _random_rows(M, N, 301, 0.1, 1.3, "bf16")
    gb = gen.fill(N, "bf16", 302, 1.0, 0.1)
    bb = gen.fill(N, "bf16", 303, 0.0, 0.1)
    dyb = _random_rows(M, N, 304, dtype="bf16")
    xf, gf, bf, dyf = (gen.bf16_to_f32(a) for a in (xb, gb, bb, dyb))
    rows = np.array([7, 0, 3])
    for kind in ("rms", "ln"):
        if kind == "rms":
            y_b, r_b = orc.rms_fwd(xb, gb, 1e-6)
            y_f, r_f = orc.rms_fwd(xf, gf, 1e-6)
            y_s, r_s = orc.rms_fwd(xb, gb, 1e-6, rows=rows)
            dx_b = orc.rms_bwd_dx(dyb, xb, gb, 1e-6)
            dx_s = orc.rms_bwd_dx(dyb, xb, gb, 1e-6, rows=rows)
        else:
            y_b, _, r_b = orc.ln_fwd(xb, gb, bb, 1e-6)
            y_f, _, r_f = orc.ln_fwd(xf, gf, bf, 1e-6)
            y_s, _, r_s = orc.ln_fwd(xb, gb, bb, 1e-6, rows=rows)
            dx_b = orc.ln_bwd_dx(dyb, xb, gb, 1e-6)
            dx_s = orc.ln_bwd_dx(dyb, xb, gb, 1e-6, rows=rows)
        assert np.array_equal(y_b, y_f) and np.array_equal(r_b, r_f), f"{kind}: bf16 decode"
        assert np.array_equal(y_s, y_b[rows]) and np.array_equal(r_s, r_b[rows]), f"{kind}: rows"
        assert np.array_equal(dx_s, dx_b[rows]), f"{kind}: dx rows"
    # dgamma over all rows equals the sum of per-row-block dgammas (rows are independent)
    dg_all, _ = orc.rms_dgamma(dyb, xb, 1e-6)
    dg_a, _ = orc.rms_dgamma(dyb[:4], xb[:4], 1e-6)
    dg_b, _ = orc.rms_dgamma(dyb[4:], xb[4:], 1e-6)
    assert np.max(np.abs(dg_all - (dg_a + dg_b))) < 1e-12, "dgamma is not a sum over rows"


def pin_f16_decode(orc):
    """binary16 bits decode to numpy's float16 values: LayerNorm of the two-element row
    [h, 0] has mean h/2 exactly.  Normals, subnormals, the largest finite value, signed
    zero and negative values."""
    bits = np.array([0x3C00, 0xC000, 0x7BFF, 0x0400, 0x03FF, 0x0001, 0x8001, 0x3555, 0x0000,
                     0x8000, 0x4248, 0xFBFF, 0x1234, 0x5678, 0x2E66], dtype=np.uint16)
    h = bits.view(np.float16)
    x = np.stack([h, np.zeros_like(h)], axis=1)
    g = np.ones(2, np.float16)
    b = np.zeros(2, np.float16)
    _, mean, _ = orc.ln_fwd(x, g, b, 1e-5)
    want = h.astype(np.float64) / 2.0
    assert np.array_equal(mean, want), f"fp16 decode: {mean} vs {want}"


def pin_f16_and_mixed_params(orc):
    """fp16 activations, and bf16 / fp16 activations with fp32 gamma and beta, give the
    results of the same values widened exactly to fp32 (the oracle works in double from
    the decoded values, so any mix-up of which buffer has which type shows)."""
    M, N = 6, 24
    rng = np.random.default_rng(311)
    for act in ("bf16", "f16"):
        xv = (rng.standard_normal((M, N)) * 1.7 + 0.3).astype(np.float32)
        dyv = rng.standard_normal((M, N)).astype(np.float32)
        x = gen.round_to(xv, act)
        dy = gen.round_to(dyv, act)
        # fp32 parameters that are not representable in the 16-bit type
        g32 = (1.0 + 0.1 * rng.standard_normal(N)).astype(np.float32) + np.float32(2.0 ** -13)
        b32 = (0.1 * rng.standard_normal(N)).astype(np.float32) + np.float32(2.0 ** -14)
        wide = (lambda a: gen.bf16_to_f32(a)) if act == "bf16" else (lambda a: a.astype(np.float32))
        xf, dyf = wide(x), wide(dy)
        for eps in (1e-5, 0.0):
            got = orc.ln_fwd(x, g32, b32, eps)
            want = orc.ln_fwd(xf, g32, b32, eps)
            for a, w in zip(got, want):
                assert np.array_equal(a, w), f"{act}+f32 LayerNorm forward"
            got = orc.rms_fwd(x, g32, eps)
            want = orc.rms_fwd(xf, g32, eps)
            for a, w in zip(got, want):
                assert np.array_equal(a, w), f"{act}+f32 RMSNorm forward"
            assert np.array_equal(orc.ln_bwd_dx(dy, x, g32, eps), orc.ln_bwd_dx(dyf, xf, g32, eps))
            assert np.array_equal(orc.rms_bwd_dx(dy, x, g32, eps),
                                  orc.rms_bwd_dx(dyf, xf, g32, eps))
        # same-type parameters: fp16 gamma equals its fp32 widening
        g16 = gen.round_to(g32, act)
        assert np.array_equal(orc.rms_fwd(x, g16, 1e-6)[0], orc.rms_fwd(xf, wide(g16), 1e-6)[0])
        dg, _ = orc.rms_dgamma(dy, x, 1e-6)
        dgf, _ = orc.rms_dgamma(dyf, xf, 1e-6)
        assert np.array_equal(dg, dgf), f"{act} dgamma decode"


def pin_residual_sum(orc):
    """The residual sum rounded to the activation type: numpy's float64 -> float32 and
    float64 -> float16 conversions (round to nearest, ties to even) for fp32 and fp16; for
    bf16, sums exact in fp32 rounded by the generator's bf16 encoder, and hand-made ties,
    overflow and subnormal cases for all three."""
    rng = np.random.default_rng(404)
    M, N = 8, 64
    scale = 2.0 ** rng.integers(-20, 20, (M, N))
    a32 = (rng.standard_normal((M, N)) * scale).astype(np.float32)
    b32 = (rng.standard_normal((M, N)) * scale[:, ::-1]).astype(np.float32)
    want = (a32.astype(np.float64) + b32.astype(np.float64)).astype(np.float32)
    assert np.array_equal(orc.residual_sum(a32, b32), want.astype(np.float64)), "fp32 sum"
    a16 = (rng.standard_normal((M, N)) * 2.0 ** rng.integers(-12, 10, (M, N))).astype(np.float16)
    b16 = (rng.standard_normal((M, N)) * 2.0 ** rng.integers(-12, 10, (M, N))).astype(np.float16)
    with np.errstate(over="ignore"):
        want = (a16.astype(np.float64) + b16.astype(np.float64)).astype(np.float16)
    assert np.array_equal(orc.residual_sum(a16, b16), want.astype(np.float64)), "fp16 sum"
    ab = gen.round_bf16(rng.standard_normal((M, N)).astype(np.float32) * 3)
    bb = gen.round_bf16(rng.standard_normal((M, N)).astype(np.float32))
    exact = gen.bf16_to_f32(ab) + gen.bf16_to_f32(bb)  # exact: exponents close
    want = gen.bf16_to_f32(gen.round_bf16(exact)).astype(np.float64)
    assert np.array_equal(orc.residual_sum(ab, bb), want), "bf16 sum"
    # hand cases: (a, b, bf16 result, fp16 result)
    cases = [(1.0, 2.0 ** -8, 1.0, 1.0 + 2.0 ** -8),            # bf16 tie -> even
             (1.0 + 2.0 ** -7, 2.0 ** -8, 1.0 + 2.0 ** -6, 1.0 + 2.0 ** -7 + 2.0 ** -8),
             (1.0, 2.0 ** -11, 1.0, 1.0),                       # fp16 tie -> even
             (1.0 + 2.0 ** -10, 2.0 ** -11, 1.0, 1.0 + 2.0 ** -9),
             (65504.0, 16.0, 65536.0, np.inf),                  # fp16 overflow
             (65504.0, 8.0, 65536.0, 65504.0),
             (2.0 ** -24, 2.0 ** -24, 2.0 ** -23, 2.0 ** -23),   # fp16 subnormals
             (-3.0, 3.0, 0.0, 0.0)]
    for a, b, want_b, want_h in cases:
        xa = gen.round_bf16(np.array([[a]], np.float32))
        xb = gen.round_bf16(np.array([[b]], np.float32))
        assert orc.residual_sum(xa, xb)[0, 0] == want_b, f"bf16 {a} + {b}"
        ha = np.array([[a]], np.float16)
        hb = np.array([[b]], np.float16)
        assert orc.residual_sum(ha, hb)[0, 0] == want_h, f"fp16 {a} + {b}"
    big = gen.round_bf16(np.array([[3.38e38]], np.float32))
    assert np.isinf(orc.residual_sum(big, big)[0, 0]), "bf16 overflow"


ALL_PINS = [pin_golden_forward, pin_golden_backward, pin_rms_unit_rms, pin_ln_moments,
            pin_invariance, pin_dx_orthogonality, pin_finite_differences, pin_torch_float64,
            pin_bf16_decode_and_rows, pin_f16_decode, pin_f16_and_mixed_params,
            pin_residual_sum]
