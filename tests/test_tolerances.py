"""The parity bounds where the plain relative rules cannot hold, checked on the CPU against
an fp32 evaluation of the definitions (numpy float32, the operations in the order the
definitions give them) and against planted mistakes:

* ill-conditioned fp32 dx elements (every LayerNorm row of two elements: dx =
  rstd*(g_0 - g_1)/2 * (1 - xhat^2); now and then an element of a short LayerNorm row;
  rows whose mean is large next to their spread): fp32 arithmetic misses the literal
  1e-5 * max(1, |ref|) there but meets 1e-5 of the element's sensitivity S to its terms
  and to the row's mean; well-conditioned elements stay on the literal rule, and a
  dropped term still fails.
* fp32 LayerNorm y of rows whose mean is large next to their spread: y = (x - mean) *
  rstd * gamma + beta carries the mean's rounding times rstd; held to 1e-5 of its
  sensitivity there, the literal rule elsewhere.
* LayerNorm dgamma of a column whose x sits at its row's mean: the term dy * xhat is
  near zero and carries the mean's rounding, so the 1e-4 relative rule fails for fp32
  arithmetic; the floor from the mean's own bound admits it, and a dgamma computed
  without subtracting the mean still fails.

The backward is the derivative of the forward (the torch.compile page, "Why Is Peak
Vectorization Your New Best Friend?"); LayerNorm's statistics as on the "Fused RMSNorm"
page, "What it is"."""
import numpy as np

import gen
import oracle
from parity import (KAPPA, TOL_DGAMMA, TOL_F32, dgamma_scale, dx_terms, fp32_dx_scale,
                    fp32_y_scale, y_terms)
from test_gpu_parity import small_workload

F = np.float32


def _ln_bwd_fp32(x, dy, gamma, eps):
    """fp32 evaluation of LayerNorm's dx and dgamma terms, row by row."""
    x, dy, gamma = x.astype(F), dy.astype(F), gamma.astype(F)
    n = F(x.shape[1])
    mu = (x.sum(axis=1, dtype=F) / n).astype(F)
    d = x - mu[:, None]
    var = ((d * d).sum(axis=1, dtype=F) / n).astype(F)
    r = (F(1) / np.sqrt(var + F(eps))).astype(F)
    xh = d * r[:, None]
    g = dy * gamma[None, :]
    c1 = ((g * xh).sum(axis=1, dtype=F) / n).astype(F)
    c2 = (g.sum(axis=1, dtype=F) / n).astype(F)
    dx = r[:, None] * (g - c2[:, None] - xh * c1[:, None])
    return dx.astype(np.float64), xh, c1, c2, r, g


def _fp32_dx_case(w):
    inp = gen.make_inputs(w)
    orc = oracle.get()
    ref = orc.ln_bwd_dx(inp["dy"], inp["x"], inp["gamma"], w.eps)
    dx, xh, c1, c2, r, g = _ln_bwd_fp32(inp["x"], inp["dy"], inp["gamma"], w.eps)
    rows = np.arange(w.M)
    return inp, orc, ref, dx, rows, (r, g, c2)


def test_ln_two_element_rows_need_the_term_scale():
    w = gen.Workload("ln_f32_590x2", "ln", "f32", 590, 2, 1e-6, config=9)
    inp, orc, ref, dx, rows, (r, g, c2) = _fp32_dx_case(w)
    err = np.abs(dx - ref)
    literal = TOL_F32 * np.maximum(1.0, np.abs(ref))
    miss = err > literal
    assert np.count_nonzero(miss) > 0, "the literal rule holds here: no exception"
    # the elements that miss it are differences of terms more than KAPPA times larger
    terms = dx_terms(w, inp, rows, orc)
    assert np.all(terms[miss] > KAPPA * np.maximum(1.0, np.abs(ref[miss])))
    bound = TOL_F32 * fp32_dx_scale(w, inp, rows, dx, ref, orc)
    assert np.all(err <= bound), float(np.max(err / bound))
    # dropping xhat * c1 (a plausible slip) fails
    wrong = (r[:, None] * (g - c2[:, None])).astype(np.float64)
    bw = TOL_F32 * fp32_dx_scale(w, inp, rows, wrong, ref, orc)
    assert np.count_nonzero(np.abs(wrong - ref) > bw) > w.M // 2


def _check_rule(w, min_miss, max_miss=None):
    """fp32 evaluation against the rule: some elements miss the literal bound, all of them
    ill-conditioned, none misses the rule, and an error of twice the literal bound planted
    on a well-conditioned element is caught."""
    inp, orc, ref, dx, rows, _ = _fp32_dx_case(w)
    err = np.abs(dx - ref)
    literal = TOL_F32 * np.maximum(1.0, np.abs(ref))
    miss = err > literal
    assert np.count_nonzero(miss) >= min_miss
    if max_miss is not None:
        assert np.count_nonzero(miss) <= max_miss
    scale = fp32_dx_scale(w, inp, rows, dx, ref, orc)
    assert np.all(err <= TOL_F32 * scale), float(np.max(err / (TOL_F32 * scale)))
    sens = dx_terms(w, inp, rows, orc)
    ill = sens > KAPPA * np.maximum(1.0, np.abs(ref))
    assert np.all(ill[miss])
    assert np.all(err[~ill] <= 0.5 * literal[~ill]), "little margin left on the literal rule"
    i, j = np.argwhere(~ill)[len(np.argwhere(~ill)) // 2]
    bad = dx.copy()
    bad[i, j] = ref[i, j] + 2 * literal[i, j]
    sb = fp32_dx_scale(w, inp, rows, bad, ref, orc)
    assert abs(bad[i, j] - ref[i, j]) > TOL_F32 * sb[i, j]
    return np.count_nonzero(ill), ill.size


def test_short_rows_keep_the_literal_rule_where_well_conditioned():
    # a GPU parity case (LayerNorm fp32, N = 3): two elements of 4593 are differences of
    # terms two hundred times larger
    n_ill, n = _check_rule(small_workload("ln", "f32", 3, x_mean=0.25, x_std=1.5), 1, 10)
    assert n_ill < n // 10, "most elements stay on the literal rule"
    # a row of two whose values are close: the mean's rounding, amplified by rstd, is most
    # of dx's error (found by a seeded random search over forced plans)
    _check_rule(gen.Workload("ln_f32_429x2", "ln", "f32", 429, 2, 1e-6, x_mean=0.3,
                             config=9), 1)


def test_rows_with_a_large_mean_are_ill_conditioned():
    # mean 5, spread 0.05: x - mean loses 7 bits before rstd scales it up by 20
    w = gen.Workload("ln_f32_4096x64", "ln", "f32", 4096, 64, 1e-5, x_mean=5.0, x_std=0.05,
                     config=9)
    n_ill, n = _check_rule(w, 100)
    # the same rows with mean 0 are well-conditioned nearly everywhere
    w0 = gen.Workload("ln_f32_4096x64", "ln", "f32", 4096, 64, 1e-5, x_mean=0.0, x_std=0.05,
                      config=9)
    inp, orc, ref, dx, rows, _ = _fp32_dx_case(w0)
    assert np.all(np.abs(dx - ref) <= TOL_F32 * np.maximum(1.0, np.abs(ref)))


def test_ln_dgamma_floor_admits_the_means_rounding_only():
    # one row; x_1 is the exact mean of the row, which fp32 cannot hold exactly
    x = np.array([[0.1, 0.2, 0.3, 0.2]], np.float32)
    dy = np.array([[0.5, -1.25, 2.0, 0.75]], np.float32)
    gamma = np.ones(4, np.float32)
    beta = np.zeros(4, np.float32)
    w = gen.Workload("ln_f32_1x4", "ln", "f32", 1, 4, 1e-5, config=9)
    inp = {"x": x, "dy": dy, "gamma": gamma, "beta": beta}
    orc = oracle.get()
    ref, _, sg, _ = orc.ln_dgamma_dbeta(dy, x, w.eps)
    _, xh, _, _, _, _ = _ln_bwd_fp32(x, dy, gamma, w.eps)
    got = (dy * xh)[0].astype(np.float64)
    plain = TOL_DGAMMA * np.maximum(np.abs(ref), sg)
    assert np.any(np.abs(got - ref) > plain), "fp32 meets the plain rule: no floor needed"
    scale = dgamma_scale(w, inp, got, ref, sg, orc)
    assert np.all(np.abs(got - ref) <= TOL_DGAMMA * scale)
    # columns the plain rule already covers keep its scale
    ok = np.abs(got - ref) <= plain
    assert np.array_equal(scale[ok], np.maximum(np.abs(ref), sg)[ok])
    # forgetting to subtract the mean is far outside the floor
    r = 1.0 / np.sqrt(np.var(x[0].astype(np.float64)) + w.eps)
    wrong = dy[0].astype(np.float64) * x[0].astype(np.float64) * r
    assert np.all(np.abs(wrong - ref) > TOL_DGAMMA * dgamma_scale(w, inp, wrong, ref, sg, orc))
    # RMSNorm's dgamma has no mean: its scale is the plain one
    wr = gen.Workload("rms_f32_1x4", "rms", "f32", 1, 4, 1e-5, config=9)
    assert np.array_equal(dgamma_scale(wr, inp, wrong, ref, sg, orc), np.maximum(np.abs(ref), sg))


def _ln_fwd_fp32(x, gamma, beta, eps):
    x, gamma, beta = x.astype(F), gamma.astype(F), beta.astype(F)
    n = F(x.shape[1])
    mu = (x.sum(axis=1, dtype=F) / n).astype(F)
    d = x - mu[:, None]
    var = ((d * d).sum(axis=1, dtype=F) / n).astype(F)
    r = (F(1) / np.sqrt(var + F(eps))).astype(F)
    return (d * r[:, None] * gamma[None, :] + beta[None, :]).astype(np.float64)


def test_ln_forward_rows_with_a_large_mean():
    w = gen.Workload("ln_f32_4096x64", "ln", "f32", 4096, 64, 1e-5, x_mean=5.0, x_std=0.05,
                     config=9)
    inp = gen.make_inputs(w)
    orc = oracle.get()
    rows = np.arange(w.M)
    ref, _, _ = orc.ln_fwd(inp["x"], inp["gamma"], inp["beta"], w.eps)
    y = _ln_fwd_fp32(inp["x"], inp["gamma"], inp["beta"], w.eps)
    err = np.abs(y - ref)
    literal = TOL_F32 * np.maximum(1.0, np.abs(ref))
    miss = err > literal
    assert np.count_nonzero(miss) > 100
    scale = fp32_y_scale(w, inp, rows, y, ref, orc)
    assert np.all(err <= TOL_F32 * scale)
    sens = y_terms(w, inp, rows, orc)
    ill = sens > KAPPA * np.maximum(1.0, np.abs(ref))
    assert np.all(ill[miss])
    # the unbiased variance (a plausible slip: rstd off by sqrt(64/63)) is caught, and so is
    # a dropped beta
    x64 = inp["x"].astype(np.float64)
    xc = x64 - x64.mean(axis=1, keepdims=True)
    r_unb = 1.0 / np.sqrt((xc * xc).sum(axis=1, keepdims=True) / (w.N - 1) + w.eps)
    for bad in (xc * r_unb * inp["gamma"] + inp["beta"], y - inp["beta"][None, :]):
        sb = fp32_y_scale(w, inp, rows, bad, ref, orc)
        assert np.count_nonzero(np.abs(bad - ref) > TOL_F32 * sb) > bad.size // 2
    # centred rows of the same spread are well-conditioned: the literal rule holds
    w0 = gen.Workload("ln_f32_4096x64", "ln", "f32", 4096, 64, 1e-5, x_mean=0.0, x_std=0.05,
                      config=9)
    i0 = gen.make_inputs(w0)
    r0, _, _ = orc.ln_fwd(i0["x"], i0["gamma"], i0["beta"], w0.eps)
    y0 = _ln_fwd_fp32(i0["x"], i0["gamma"], i0["beta"], w0.eps)
    assert np.all(np.abs(y0 - r0) <= 0.5 * TOL_F32 * np.maximum(1.0, np.abs(r0)))
