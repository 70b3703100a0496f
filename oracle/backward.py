"""Float64 CPU reference for the gradient of the causal CSA forward.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing in the product
path may import this module.

The pages train every model with the method (Experiments), so the backward pass
is the plain derivative of the forward.  This module differentiates the forward
exactly as ``oracle.csa`` evaluates it -- eq. (8) of J. Su, "Continuous Softmax
Attention" (Assembly and Simplification), segment by segment -- for the scalar

    loss = sum_t dO_t . o_t + sum_t dlse_t lse_t,

and returns its gradient with respect to q, k, v and the two extra vectors
k_0, v_0 (which the pages suggest may be trainable, Analysis of the Result).

Derivation (written here because the pages give none).  For query t, segment
i = 1..t joins positions i-1 and i, with delta_i = a_i - a_{i-1} and
E_i = e^{a_{i-1}}.  By eq. (4)-(5) its numerator is
E_i [phi_1(delta_i) v_i + phi_2(delta_i) (v_{i-1} - v_i)] and its denominator
E_i phi_1(delta_i).  With g = dO_t / den and h = (dlse_t - dO_t . o_t) / den,
the loss changes with the segment's two quantities through

    f_i = E_i [phi_1(delta_i) A_i + phi_2(delta_i) B_i],
    A_i = g . v_i + h,   B_i = g . (v_{i-1} - v_i),

so  d f_i / d a_i     = E_i [phi_1'(delta_i) A_i + phi_2'(delta_i) B_i]  and
    d f_i / d a_{i-1} = f_i - (d f_i / d a_i),
where phi_1'(x) = integral_0^1 s e^{s x} ds and phi_2'(x) = integral_0^1
s (1 - s) e^{s x} ds are the derivatives of the functions of eq. (6).  The
logit gradients dS_{t,j} = d loss / d a_{t,j} then give dq_t = sum_j dS_{t,j} k_j
and dk_j += dS_{t,j} q_t; the values enter the numerator linearly, so
dv_i += g E_i (phi_1 - phi_2)(delta_i) from segment i and
dv_{i-1} += g E_i phi_2(delta_i).
"""

from __future__ import annotations

import math

import numpy as np

from .csa import _as_f64, phi1, phi2

# Same switch as phi_1, phi_2: the closed forms below lose digits to cancellation
# near 0, where the Taylor series of the integral definitions is summed instead.
#   phi_1'(x) = sum_n (n+1) x^n/(n+2)!,  phi_2'(x) = sum_n (n+1) x^n/(n+3)!
# 15 terms at |x| < 0.25 leave a truncation error below 1e-20.
_SERIES_RADIUS = 0.25
_SERIES_TERMS = 15
_DPHI1_COEF = np.array([(n + 1) / math.factorial(n + 2) for n in range(_SERIES_TERMS)])
_DPHI2_COEF = np.array([(n + 1) / math.factorial(n + 3) for n in range(_SERIES_TERMS)])


def _series(x: np.ndarray, coef: np.ndarray) -> np.ndarray:
    acc = np.zeros_like(x)
    for c in coef[::-1]:
        acc = acc * x + c
    return acc


def dphi1(x) -> np.ndarray:
    """phi_1'(x) = integral_0^1 s e^{s x} ds = ((x - 1) e^x + 1)/x^2, value 1/2 at 0.

    Derivative of phi_1 of Preliminaries, eq. (6).
    """
    x = np.asarray(x, dtype=np.float64)
    small = np.abs(x) < _SERIES_RADIUS
    safe = np.where(small, 1.0, x)
    with np.errstate(over="ignore"):
        # (x - 1) e^x + 1 = x e^x - (e^x - 1)
        closed = (safe * np.exp(safe) - np.expm1(safe)) / (safe * safe)
    return np.where(small, _series(x, _DPHI1_COEF), closed)


def dphi2(x) -> np.ndarray:
    """phi_2'(x) = integral_0^1 s (1 - s) e^{s x} ds = ((x - 2) e^x + x + 2)/x^3, 1/6 at 0.

    Derivative of phi_2 of Preliminaries, eq. (6).
    """
    x = np.asarray(x, dtype=np.float64)
    small = np.abs(x) < _SERIES_RADIUS
    safe = np.where(small, 1.0, x)
    with np.errstate(over="ignore"):
        # (x - 2) e^x + x + 2 = (x - 2)(e^x - 1) + 2 x
        closed = ((safe - 2.0) * np.expm1(safe) + 2.0 * safe) / (safe * safe * safe)
    return np.where(small, _series(x, _DPHI2_COEF), closed)


def csa_backward_row(q_t, k_hat, v_hat, t, do_t, dlse_t=0.0):
    """Gradient of dO_t . o_t + dlse_t lse_t for one query t by differentiating eq. (8).

    q_t: (d,);  k_hat, v_hat: (>= t+1, d) / (>= t+1, d_v), row 0 = k_0 / v_0;
    t >= 1;  do_t: (d_v,);  dlse_t: scalar.
    Returns (dq_t (d,), dk_hat (t+1, d), dv_hat (t+1, d_v)) for positions 0..t.
    """
    if t < 1:
        raise ValueError("query position t starts at 1")
    K = k_hat[: t + 1]
    V = v_hat[: t + 1]
    a = K @ q_t                       # a_{t,i}, i = 0..t
    shift = float(a.max())
    a_left = a[:-1]                   # a_{t,i-1}, i = 1..t
    delta = a[1:] - a_left            # delta_{t,i}
    E = np.exp(a_left - shift)        # e^{a_{t,i-1}}, shifted (cancels with den)
    f1, f2 = phi1(delta), phi2(delta)
    v_i, v_im1 = V[1:], V[:-1]
    num = (E[:, None] * (f1[:, None] * v_i + f2[:, None] * (v_im1 - v_i))).sum(axis=0)
    den = float((E * f1).sum())
    o = num / den
    g = do_t / den                              # d loss / d num
    h = (dlse_t - float(do_t @ o)) / den        # d loss / d den
    A = v_i @ g + h
    Bc = (v_im1 - v_i) @ g
    f_seg = E * (f1 * A + f2 * Bc)
    d_right = E * (dphi1(delta) * A + dphi2(delta) * Bc)   # d f_i / d a_i
    d_left = f_seg - d_right                               # d f_i / d a_{i-1}
    dS = np.zeros(t + 1)
    dS[1:] += d_right
    dS[:-1] += d_left
    dq = dS @ K
    dk = np.outer(dS, q_t)
    dv = np.zeros_like(V)
    dv[1:] += np.outer(E * (f1 - f2), g)
    dv[:-1] += np.outer(E * f2, g)
    return dq, dk, dv


def csa_backward_reference(q, k, v, do, k0=None, v0=None, dlse=None):
    """Gradient of sum_t dO_t . o_t + dlse_t lse_t through the causal CSA forward, float64.

    q, k: [B, H, T, d];  v, do: [B, H, T, d_v];  k0: [B, H, d] or None (zeros);
    v0: [B, H, d_v] or None (zeros);  dlse: [B, H, T] or None (zeros).  Conventions
    as ``csa_reference`` (query row r is t = r + 1; key row r is position r + 1).

    Returns (dq, dk, dv, dk0, dv0) as float64 numpy arrays of the input shapes.
    """
    q, k, v, do = _as_f64(q), _as_f64(k), _as_f64(v), _as_f64(do)
    B, H, T, d = q.shape
    dvd = v.shape[-1]
    k0 = np.zeros((B, H, d)) if k0 is None else _as_f64(k0)
    v0 = np.zeros((B, H, dvd)) if v0 is None else _as_f64(v0)
    dlse = np.zeros((B, H, T)) if dlse is None else _as_f64(dlse)
    dq = np.zeros_like(q)
    dkh = np.zeros((B, H, T + 1, d))
    dvh = np.zeros((B, H, T + 1, dvd))
    for b in range(B):
        for h in range(H):
            k_hat = np.concatenate([k0[b, h][None], k[b, h]], axis=0)
            v_hat = np.concatenate([v0[b, h][None], v[b, h]], axis=0)
            for r in range(T):
                t = r + 1
                gq, gk, gv = csa_backward_row(q[b, h, r], k_hat, v_hat, t, do[b, h, r], float(dlse[b, h, r]))
                dq[b, h, r] = gq
                dkh[b, h, : t + 1] += gk
                dvh[b, h, : t + 1] += gv
    return dq, dkh[:, :, 1:], dvh[:, :, 1:], dkh[:, :, 0], dvh[:, :, 0]
