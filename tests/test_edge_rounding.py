"""Rounding of the edge terms' closed form in float32 (host arithmetic, no GPU).

The bf16 forward forms the two terms of an edge (i, i+1) of eq. (10) in the p-form
R = ((p_r - p_l)/y - c p_l)/y and L = (c p_r - (p_r - p_l)/y)/y (c = ln 2, p = 2^alpha,
y = alpha_r - alpha_l), which cancels as |y| -> 0.  The kernels replace it by the degree-1
series below a threshold: 0.07 on the diagonal tiles, 0.02 on the others.  This test
evaluates the closed form in float32 with exp2 results perturbed by up to one ulp (the
accuracy of the hardware's exp2) and checks the relative error of R and L against float64:
above 0.02 it stays under 2^-8, the largest relative rounding error of a bf16 weight, which
every weight takes before the P V product; at 0.01 it does not, which is why the threshold
is not lower.  It also checks that the degree-1 series is within 2e-4 below 0.07.
"""

import numpy as np

C = np.log(2.0)


def _closed_form_rel_err(lo, hi, n=200_000, seed=0):
    rng = np.random.default_rng(seed)
    al = rng.uniform(-20.0, 0.0, n).astype(np.float32)
    ar = (al + (rng.uniform(lo, hi, n) * rng.choice([-1.0, 1.0], n)).astype(np.float32)).astype(np.float32)
    y = (ar - al).astype(np.float32)  # exact: Sterbenz

    def exp2_1ulp(a):
        p = np.exp2(a.astype(np.float64))
        ulp = np.spacing(p.astype(np.float32)).astype(np.float64)
        return (p + rng.uniform(-1.0, 1.0, a.shape) * ulp).astype(np.float32)

    pl, pr = exp2_1ulp(al), exp2_1ulp(ar)
    u = (1.0 / y.astype(np.float64)).astype(np.float32)
    c = np.float32(C)
    du = ((pr - pl) * u).astype(np.float32)
    R = ((du - c * pl).astype(np.float32) * u).astype(np.float32)
    L = ((c * pr - du).astype(np.float32) * u).astype(np.float32)
    yd = y.astype(np.float64)
    pld, prd = np.exp2(al.astype(np.float64)), np.exp2(ar.astype(np.float64))
    Rt = ((prd - pld) / yd - C * pld) / yd
    Lt = (C * prd - (prd - pld) / yd) / yd
    return max(np.abs(R / Rt - 1.0).max(), np.abs(L / Lt - 1.0).max())


def test_closed_form_above_threshold_within_bf16_rounding():
    bound = 2.0 ** -8
    assert _closed_form_rel_err(0.02, 0.03) < bound
    assert _closed_form_rel_err(0.03, 0.07) < bound / 2
    # a lower threshold would let the closed form exceed the bf16 rounding of the weights
    assert _closed_form_rel_err(0.01, 0.012) > bound


def test_degree_one_series_below_diagonal_threshold():
    # c^2 phi_2(c y) = c^2/2 + c^3 y/6 + O(y^2); relative truncation error ~ c^2 y^2 / 12
    y = np.linspace(-0.07, 0.07, 2001)
    y = y[y != 0.0]
    x = C * y
    exact = C * C * (np.expm1(x) - x) / (x * x)  # c^2 (e^x - 1 - x)/x^2
    series = C * C / 2.0 + C ** 3 * y / 6.0
    assert np.abs(series / exact - 1.0).max() < 2e-4
