"""The CPU reference pinned to what the pages and the mathematics fix.

Source: J. Su, "Continuous Softmax Attention" -- eq. (2)-(3) (definition),
eq. (6) and the limits after it, identity eq. (7), eq. (8) (what the
reference evaluates), eq. (10)-(11) (the simplified form), eq. (12)
(standard attention) and eq. (13) (Taylor expansion of b); the gradient of the
forward (the backward reference) against finite differences of the defining
integral and two symmetries of eq. (2).
"""

import json
import math
import os

import mpmath as mp
import numpy as np
import pytest

import pins
from oracle import csa1_reference, csa_backward_reference, csa_half_reference, seg_integrals, csa_reference, dphi1, dphi2, phi1, phi2, std_reference

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_phi_limits_at_zero():
    # limits stated right after eq. (6)
    assert phi1(0.0) == 1.0
    assert phi2(0.0) == 0.5
    assert phi1(np.array([0.0, -0.0])).tolist() == [1.0, 1.0]
    assert phi2(np.array([0.0, -0.0])).tolist() == [0.5, 0.5]


def _grid():
    xs = [0.0, 1e-300, -1e-300, 1e-12, -1e-12, 1e-6, -3e-5, 0.01, -0.1, 0.2499999, -0.2499999,
          0.25, -0.25, 0.2500001, -0.2500001, 0.3, -0.7, 1.0, -1.0, 3.3, -5.0, 12.0, -20.0, 40.0, -60.0, 60.0]
    return np.array(xs + list(np.linspace(-30, 30, 241)))


def test_phi_against_50_digit_integrals():
    # eq. (6): the integral definitions, evaluated independently in mpmath
    xs = _grid()
    f1, f2 = phi1(xs), phi2(xs)
    with mp.workdps(50):
        for x, a, b in zip(xs, f1, f2):
            X = mp.mpf(float(x))
            e1 = mp.quad(lambda s: mp.exp(s * X), [0, 1])
            e2 = mp.quad(lambda s: mp.exp(s * X) * (1 - s), [0, 1])
            assert abs(a - float(e1)) <= 2e-15 * float(e1), x
            assert abs(b - float(e2)) <= 2e-15 * float(e2), x


def test_phi_positive_and_continuous_across_series_switch():
    # positivity noted after eq. (7); no jump where the evaluation switches form
    xs = _grid()
    assert np.all(phi1(xs) > 0) and np.all(phi2(xs) > 0)
    for r in (0.25, -0.25):
        lo, hi = np.nextafter(r, 0.0), r
        assert abs(phi2(lo) - phi2(hi)) < 1e-15
        assert abs(phi1(lo) - phi1(hi)) < 1e-15


def test_identity_7():
    # eq. (7): phi_1(x) - phi_2(x) = e^x phi_2(-x)
    xs = np.linspace(-60, 60, 2401)
    lhs = phi1(xs) - phi2(xs)
    rhs = np.exp(xs) * phi2(-xs)
    assert np.all(np.abs(lhs - rhs) <= 1e-12 * np.abs(rhs))


@pytest.mark.parametrize("seed,scale", [(0, 1.0), (5, 3.0), (6, 0.05)])
def test_against_quadrature_of_definition(seed, scale):
    # eq. (2)-(3) integrated numerically
    assert pins.dev_vs_quadrature(csa_reference, seed=seed, scale=scale) < 1e-12


@pytest.mark.parametrize("seed,scale", [(1, 1.5), (7, 6.0)])
def test_against_simplified_form_in_mpmath(seed, scale):
    # eq. (10)-(11) in 50-digit arithmetic: also exercises identity (7) and the regrouping (9)
    assert pins.dev_vs_simplified(csa_reference, seed=seed, scale=scale) < 1e-12


def test_trapezoid_weights_for_equal_logits():
    assert pins.dev_trapezoid(csa_reference) < 1e-13


@pytest.mark.parametrize("beta", [0.7, -1.3, 1e-3, 4.0])
def test_linear_ramp_closed_form(beta):
    assert pins.dev_linear_ramp(csa_reference, beta=beta) < 1e-11


def test_taylor_of_correction_b():
    # eq. (13) first order (interior constant 0), extended to second order;
    # the residual must shrink like eps^3
    devs = [pins.dev_taylor_b(csa_reference, eps) for eps in (0.08, 0.04, 0.02, 0.01)]
    for big, small in zip(devs, devs[1:]):
        assert 5.0 < big / small < 11.0, devs
    assert devs[-1] < 1e-5


def test_first_order_b_is_a_second_difference():
    # eq. (13): b_i = (a_{i-1} + a_{i+1} - 2 a_i)/6 + ... for interior i
    rng = np.random.default_rng(11)
    t, eps = 5, 1e-3
    q_t = rng.standard_normal(3) * eps
    k_hat = rng.standard_normal((t + 1, 3))
    b, a = pins.implied_b(csa_reference, q_t, k_hat, t)
    for i in range(1, t):
        assert abs(b[i] - (a[i - 1] + a[i + 1] - 2 * a[i]) / 6) < 50 * eps ** 2


def test_copied_sink_first_segment_is_flat():
    assert pins.dev_copied_sink(csa_reference) < 1e-13


def test_constant_values_and_key_shift():
    q, k, v, k0, v0 = pins.random_case(8, T=10, scale=2.0)
    c = np.array([0.5, -2.0, 3.0, 1.0])
    o, _ = csa_reference(q, k, np.broadcast_to(c, v.shape), k0, np.broadcast_to(c, v0.shape))
    assert np.abs(o - c).max() < 1e-13
    # k_i -> k_i + w for every position including 0: o unchanged, lse += q.w
    w = np.array([0.3, -0.4, 0.9])
    o1, l1 = csa_reference(q, k, v, k0, v0)
    o2, l2 = csa_reference(q, k + w, v, k0 + w, v0)
    assert np.abs(o1 - o2).max() < 1e-12
    assert np.abs((l2 - l1) - (q[0, 0] @ w)).max() < 1e-12


def test_weights_positive_and_bounded_by_neighbours():
    # e^{a_i + b_i} <= max(e^{a_{i-1}}, e^{a_i}, e^{a_{i+1}}) follows from eq. (4)'s integrand
    rng = np.random.default_rng(12)
    for t in (1, 2, 7):
        q_t = rng.standard_normal(3) * 3
        k_hat = rng.standard_normal((t + 1, 3))
        b, a = pins.implied_b(csa_reference, q_t, k_hat, t)
        w = a + b
        assert np.all(np.isfinite(w))
        for i in range(t + 1):
            nb = [a[j] for j in (i - 1, i, i + 1) if 0 <= j <= t]
            assert w[i] <= max(nb) + 1e-12


def test_rows_subset_matches_full():
    q, k, v, k0, v0 = pins.random_case(9, T=12)
    o, l = csa_reference(q, k, v, k0, v0)
    rows = [0, 5, 11]
    o2, l2 = csa_reference(q, k, v, k0, v0, rows=rows)
    assert np.array_equal(o[:, :, rows], o2) and np.array_equal(l[:, :, rows], l2)


def test_std_reference_against_library_softmax_attention():
    # eq. (12), checked against torch's attention routine in float64 (scale 1, causal)
    import torch

    g = torch.Generator().manual_seed(0)
    q, k, v = (torch.randn(2, 3, 17, 5, generator=g, dtype=torch.float64) for _ in range(3))
    o, lse = std_reference(q, k, v)
    ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=1.0)
    assert np.abs(o - ref.numpy()).max() < 1e-13
    s = (q @ k.transpose(-1, -2)).numpy()
    mask = np.triu(np.ones((17, 17), bool), 1)
    s[..., mask] = -np.inf
    lse_lib = np.log(np.exp(s).sum(-1))
    assert np.abs(lse - lse_lib).max() < 1e-12


def test_golden_fixture():
    # a stored regression case written by tests/golden/make_golden.py (oracle only)
    with open(os.path.join(GOLDEN, "csa_small.json")) as f:
        g = json.load(f)
    o, lse = csa_reference(np.array(g["q"]), np.array(g["k"]), np.array(g["v"]),
                           np.array(g["k0"]), np.array(g["v0"]))
    assert np.abs(o - np.array(g["o"])).max() < 1e-14
    assert np.abs(lse - np.array(g["lse"])).max() < 1e-14
    # and the same case against the definition by quadrature
    qq, kh, vh = pins.hat(np.array(g["q"]), np.array(g["k"]), np.array(g["v"]),
                          np.array(g["k0"]), np.array(g["v0"]))
    for r in range(qq.shape[0]):
        oq, lq = pins.quadrature_row(qq[r], kh, vh, r + 1)
        assert np.abs(np.array(g["o"])[0, 0, r] - oq).max() < 1e-12
        assert abs(g["lse"][0][0][r] - lq) < 1e-12


# ---------------------------------------------------------------- first-order variant

def test_first_order_trapezoid_for_equal_logits():
    # equal logits: interior b = 0, ends -ln 2 -> the same 1/2, 1, ..., 1, 1/2 weights
    assert pins.dev_trapezoid(csa1_reference) < 1e-13


@pytest.mark.parametrize("beta", [0.7, -1.3, 2.5, 1e-3])
def test_first_order_linear_logits_closed_form(beta):
    assert pins.dev1_linear(csa1_reference, beta=beta) < 1e-11


def test_first_order_agrees_with_exact_to_second_order():
    devs = [pins.dev1_vs_exact(csa1_reference, eps) for eps in (0.08, 0.04, 0.02, 0.01)]
    for big, small in zip(devs, devs[1:]):
        assert 3.0 < big / small < 5.5, devs   # ~4: second order
    assert devs[-1] < 1e-3


def test_first_order_key_shift_invariance():
    # k_i -> k_i + w for every position (k_0 included) adds q.w to every logit:
    # b (a difference of logits) is unchanged, o is unchanged, lse moves by q.w
    q, k, v, k0, v0 = pins.random_case(21, T=7)
    w = np.array([0.4, -1.1, 0.25])
    o, lse = csa1_reference(q, k, v, k0, v0)
    o2, lse2 = csa1_reference(q, k + w, v, k0 + w, v0)
    assert np.abs(o2 - o).max() < 1e-12
    assert np.abs(lse2 - lse - (q @ w)).max() < 1e-12


# ---------------------------------------------------------------- backward (gradient)

@pytest.mark.parametrize("seed,scale", [(11, 1.0), (14, 0.05), (15, 3.0)])
def test_backward_against_finite_differences_of_the_definition(seed, scale):
    # scale 0.05 keeps every neighbour difference inside the series branch of phi_1', phi_2'
    assert pins.dev_grad_fd(csa_backward_reference, seed=seed, scale=scale) < 1e-8


def test_backward_shift_invariants():
    assert pins.dev_grad_shift(csa_backward_reference) < 1e-12


def test_backward_trapezoid_values():
    assert pins.dev_grad_trapezoid(csa_backward_reference) < 1e-14


def test_dphi_are_the_derivatives_of_phi():
    x = np.concatenate([np.linspace(-6, 6, 49), [-0.26, -0.2499, 0.2499, 0.26, 1e-9, 0.0]])
    h = 1e-6
    for f, df in ((phi1, dphi1), (phi2, dphi2)):
        fd = (f(x + h) - f(x - h)) / (2 * h)
        assert (np.abs(df(x) - fd) / np.maximum(1.0, np.abs(fd))).max() < 1e-8
    assert dphi1(0.0) == 0.5 and abs(float(dphi2(0.0)) - 1.0 / 6.0) < 1e-17


# ---------------------------------------------------------------- interval [1/2, t + 1/2]

@pytest.mark.parametrize("seed,scale", [(0, 1.0), (3, 0.05), (4, 3.0)])
def test_half_interval_against_quadrature_of_definition(seed, scale):
    # scale 0.05 keeps every segment's difference inside the series branch
    assert pins.dev_half_vs_quadrature(csa_half_reference, seed=seed, scale=scale) < 1e-12


def test_half_interval_trapezoid_for_equal_logits():
    assert pins.dev_half_trapezoid(csa_half_reference) < 1e-14


@pytest.mark.parametrize("beta", [0.7, -1.3, 0.01])
def test_half_interval_linear_ramp_closed_form(beta):
    assert pins.dev_half_linear_ramp(csa_half_reference, beta=beta) < 1e-11


def test_segment_integrals_reduce_to_phi_on_the_unit_segment():
    x = np.concatenate([np.linspace(-6, 6, 49), [-0.51, -0.4999, 0.4999, 0.51, 0.0]])
    f0, f1 = seg_integrals(x, 0.0, 1.0)
    assert np.abs(f0 - phi1(x)).max() < 1e-13
    assert np.abs((f0 - f1) - phi2(x)).max() < 1e-13
    # additivity over [0, 1/2] + [1/2, 1]
    a0, a1 = seg_integrals(x, 0.0, 0.5)
    b0, b1 = seg_integrals(x, 0.5, 1.0)
    assert np.abs(a0 + b0 - f0).max() < 1e-13 and np.abs(a1 + b1 - f1).max() < 1e-13
