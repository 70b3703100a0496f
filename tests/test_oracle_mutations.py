"""Plant plausible mistakes in a copy of the CPU reference and show the pins catch each.

The reference's source text is edited in memory (never on disk), executed as a
throw-away module, and run through the checks of ``pins``.  A mutant passes
only if every check stays within its tolerance -- which must never happen.
"""

import inspect

import pytest

import oracle.backward as oracle_backward
import oracle.csa as oracle_csa
import oracle.first_order as oracle_first_order
import oracle.half_interval as oracle_half
import pins

MUTATIONS = {
    "sign of delta": ("delta = a[1:] - a_left", "delta = a_left - a[1:]"),
    "sign of the phi_2 term": ("(v_im1 - v_i))", "(v_i - v_im1))"),
    "dropped phi_2 term": ("f1[:, None] * v_i + f2[:, None] * (v_im1 - v_i)", "f1[:, None] * v_i"),
    "phi_2 in the denominator": ("seg_den = e_left * f1", "seg_den = e_left * f2"),
    "value index shifted": ("v_i = V[1:]", "v_i = V[:-1]"),
    "exponent on the right end": ("e_left = np.exp(a_left - shift)", "e_left = np.exp(a[1:] - shift)"),
    "phi_2 series coefficients": ("math.factorial(n + 2)", "math.factorial(n + 1)"),
    "phi_2 closed form sign": ("(np.expm1(safe) - safe)", "(np.expm1(safe) + safe)"),
    "lse without the shift": ("lse = shift + math.log(den)", "lse = math.log(den)"),
    "position 0 dropped": ("K = k_hat[: t + 1]", "K = np.concatenate([k_hat[1:2], k_hat[1 : t + 1]])"),
    "value at position 0 dropped": ("V = v_hat[: t + 1]",
                                    "V = np.concatenate([0 * v_hat[:1], v_hat[1 : t + 1]])"),
}

CHECKS = [
    (pins.dev_vs_quadrature, 1e-12),
    (pins.dev_trapezoid, 1e-13),
    (pins.dev_linear_ramp, 1e-11),
    (pins.dev_vs_simplified, 1e-12),
    (pins.dev_copied_sink, 1e-13),
    (lambda ref: pins.dev_vs_quadrature(ref, seed=6, scale=0.05), 1e-12),
]


def _mutant(old, new, fn="csa_reference", module=oracle_csa):
    src = inspect.getsource(module)
    if module is not oracle_csa:  # the module imports helpers relatively
        src = src.replace("from .csa import ", "from oracle.csa import ")
    assert src.count(old) == 1, f"mutation anchor not unique: {old!r}"
    ns = {"__name__": "oracle_mutant"}
    exec(compile(src.replace(old, new), "<oracle mutant>", "exec"), ns)
    return ns[fn]


def test_unmutated_reference_passes_every_check():
    for check, tol in CHECKS:
        assert check(oracle_csa.csa_reference) < tol


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutant_is_caught(name):
    ref = _mutant(*MUTATIONS[name])
    caught = []
    for check, tol in CHECKS:
        try:
            caught.append(not (check(ref) < tol))
        except Exception:
            caught.append(True)
    assert any(caught), f"mutation '{name}' escaped every pin"


# ---------------------------------------------------------------- first-order variant

MUTATIONS1 = {
    "interior coefficient": ("- 2.0 * a[1:t]) / 6.0", "- 2.0 * a[1:t]) / 3.0"),
    "interior own-logit weight": ("- 2.0 * a[1:t]) / 6.0", "- 1.0 * a[1:t]) / 6.0"),
    "end slope sign at position 0": ("(a[1] - a[0]) / 3.0", "(a[0] - a[1]) / 3.0"),
    "end slope sign at position t": ("(a[t - 1] - a[t]) / 3.0", "(a[t] - a[t - 1]) / 3.0"),
    "end constant dropped": ("b[t] = -math.log(2.0) + ", "b[t] = 0.0 + "),
    "values shifted by one position": ("o = (w @ V) / den", "o = (w @ np.roll(V, 1, axis=0)) / den"),
    "lse without the shift": ("lse = shift + math.log(den)", "lse = math.log(den)"),
}

CHECKS1 = [
    (pins.dev_trapezoid, 1e-13),
    (pins.dev1_linear, 1e-11),
    (lambda ref: pins.dev1_linear(ref, beta=-1.3), 1e-11),
    (lambda ref: pins.dev1_vs_exact(ref, 0.01), 1e-3),
]


def test_unmutated_first_order_reference_passes_every_check():
    for check, tol in CHECKS1:
        assert check(oracle_first_order.csa1_reference) < tol


@pytest.mark.parametrize("name", sorted(MUTATIONS1))
def test_first_order_mutant_is_caught(name):
    ref = _mutant(*MUTATIONS1[name], fn="csa1_reference", module=oracle_first_order)
    caught = []
    for check, tol in CHECKS1:
        try:
            caught.append(not (check(ref) < tol))
        except Exception:
            caught.append(True)
    assert any(caught), f"mutation '{name}' escaped every pin"


# ---------------------------------------------------------------- backward reference

MUTATIONS_BWD = {
    "sign of the denominator term": ("h = (dlse_t - float(do_t @ o)) / den", "h = (dlse_t + float(do_t @ o)) / den"),
    "lse gradient dropped": ("h = (dlse_t - float(do_t @ o)) / den", "h = (0.0 - float(do_t @ o)) / den"),
    "derivatives swapped": ("d_right = E * (dphi1(delta) * A + dphi2(delta) * Bc)",
                            "d_right = E * (dphi2(delta) * A + dphi1(delta) * Bc)"),
    "left derivative sign": ("d_left = f_seg - d_right", "d_left = d_right - f_seg"),
    "left derivative without f": ("d_left = f_seg - d_right", "d_left = -d_right"),
    "value gradients swapped": ("dv[1:] += np.outer(E * (f1 - f2), g)", "dv[1:] += np.outer(E * f2, g)"),
    "dphi_2 series coefficients": ("(n + 1) / math.factorial(n + 3)", "(n + 1) / math.factorial(n + 2) / 3"),
    "dphi_2 closed form sign": ("+ 2.0 * safe) / (safe * safe * safe)", "- 2.0 * safe) / (safe * safe * safe)"),
    "dphi_1 closed form": ("(safe * np.exp(safe) - np.expm1(safe))", "(safe * np.exp(safe) - np.exp(safe))"),
    "dq from shifted keys": ("dq = dS @ K", "dq = dS @ np.roll(K, 1, axis=0)"),
    "segment numerator B term": ("Bc = (v_im1 - v_i) @ g", "Bc = (v_i - v_im1) @ g"),
}

CHECKS_BWD = [
    (lambda ref: pins.dev_grad_fd(ref, seed=21, T=4, d=2, dv=2), 1e-8),
    (lambda ref: pins.dev_grad_fd(ref, seed=22, T=4, d=2, dv=2, scale=0.05), 1e-8),
    (pins.dev_grad_shift, 1e-12),
    (pins.dev_grad_trapezoid, 1e-14),
]


def test_unmutated_backward_reference_passes_every_check():
    for check, tol in CHECKS_BWD:
        assert check(oracle_backward.csa_backward_reference) < tol


@pytest.mark.parametrize("name", sorted(MUTATIONS_BWD))
def test_backward_mutant_is_caught(name):
    ref = _mutant(*MUTATIONS_BWD[name], fn="csa_backward_reference", module=oracle_backward)
    caught = []
    for check, tol in CHECKS_BWD:
        try:
            caught.append(not (check(ref) < tol))
        except Exception:
            caught.append(True)
    assert any(caught), f"mutation '{name}' escaped every pin"


# ---------------------------------------------------------------- interval [1/2, t + 1/2]

MUTATIONS_HALF = {
    "left half taken as the whole segment": ("lo = np.where(i == 1, 0.5, 0.0)", "lo = np.zeros(i.shape)"),
    "right half taken as the whole segment": ("hi = np.where(i == t + 1, 0.5, 1.0)", "hi = np.ones(i.shape)"),
    "right half segment dropped": ("i = np.arange(1, t + 2)", "i = np.arange(1, t + 1)"),
    "halves swapped": ("lo = np.where(i == 1, 0.5, 0.0)", "lo = np.where(i == t + 1, 0.5, 0.0)"),
    "weights of the two ends swapped": ("(e * (f0 - f1))[:, None] * V[i - 1] + (e * f1)[:, None] * V[i]",
                                        "(e * f1)[:, None] * V[i - 1] + (e * (f0 - f1))[:, None] * V[i]"),
    "series antiderivative power": ("(hi ** (n + 2) - lo ** (n + 2)) / (n + 2)", "(hi ** (n + 1) - lo ** (n + 1)) / (n + 2)"),
    "closed form of F1": ("(ehi * (hi * safe - 1.0) - elo * (lo * safe - 1.0))", "(ehi * (hi * safe + 1.0) - elo * (lo * safe + 1.0))"),
    "last query without the copied position": ("k[b, h, -1:]], axis=0)", "0 * k[b, h, -1:]], axis=0)"),
}

CHECKS_HALF = [
    (pins.dev_half_vs_quadrature, 1e-12),
    (lambda ref: pins.dev_half_vs_quadrature(ref, seed=3, scale=0.05), 1e-12),
    (pins.dev_half_trapezoid, 1e-14),
    (pins.dev_half_linear_ramp, 1e-11),
]


def test_unmutated_half_interval_reference_passes_every_check():
    for check, tol in CHECKS_HALF:
        assert check(oracle_half.csa_half_reference) < tol


@pytest.mark.parametrize("name", sorted(MUTATIONS_HALF))
def test_half_interval_mutant_is_caught(name):
    ref = _mutant(*MUTATIONS_HALF[name], fn="csa_half_reference", module=oracle_half)
    caught = []
    for check, tol in CHECKS_HALF:
        try:
            caught.append(not (check(ref) < tol))
        except Exception:
            caught.append(True)
    assert any(caught), f"mutation '{name}' escaped every pin"
