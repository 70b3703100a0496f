"""Float64 CPU reference for the causal forward pass of continuous softmax attention.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing in the product
path may import this module.

What is computed -- J. Su, "Continuous Softmax Attention":

* Problem Statement, eq. (2)-(3): the output of query t is the ratio of two
  integrals over s in [0, t] of e^{q_t . k_s}, with k_s and v_s linearly
  interpolated between integer positions; positions 0..t are k_0 (an extra
  vector) followed by the first t keys.
* Preliminaries, eq. (4)-(6): each unit segment [i-1, i] integrates in closed
  form through phi_1(x) = (e^x - 1)/x and phi_2(x) = (e^x - 1 - x)/x^2, with
  phi_1(0) = 1 and phi_2(0) = 1/2.
* Assembly and Simplification, eq. (8): o_t is the sum of the segment
  numerators over the sum of the segment denominators.

This module evaluates eq. (8) exactly as written -- segment by segment -- and
deliberately does NOT use the correction-weight form eq. (10)-(11) that the
GPU kernels implement.  The extra log-sum-exp output is the natural log of the
denominator integral of eq. (2), lse_t = ln of the integral of e^{q_t . k_s}
over [0, t] (the pages define no lse; this is the plain reading).

Index conventions (the pages number positions from 0 with k_0 first; arrays
are 0-based):  key position i >= 1 is array row i-1 of ``k``/``v``; position 0
is ``k0``/``v0``; query t = 1..T is array row t-1 of ``q``; no 1/sqrt(d)
scale is applied inside (eq. (1)-(2) use the bare dot product).
"""

from __future__ import annotations

import math

import numpy as np

# Below this |x| the closed forms of eq. (6) lose digits to cancellation, so
# the Taylor series of the integral definitions is summed instead:
#   phi_1(x) = sum_n x^n/(n+1)!,  phi_2(x) = sum_n x^n/(n+2)!.
# 15 terms at |x| < 0.25 leave a truncation error below 1e-21.
_SERIES_RADIUS = 0.25
_SERIES_TERMS = 15
_PHI1_COEF = np.array([1.0 / math.factorial(n + 1) for n in range(_SERIES_TERMS)])
_PHI2_COEF = np.array([1.0 / math.factorial(n + 2) for n in range(_SERIES_TERMS)])


def _series(x: np.ndarray, coef: np.ndarray) -> np.ndarray:
    acc = np.zeros_like(x)
    for c in coef[::-1]:
        acc = acc * x + c
    return acc


def phi1(x) -> np.ndarray:
    """phi_1(x) = integral_0^1 e^{s x} ds = (e^x - 1)/x, phi_1(0) = 1.

    Preliminaries, eq. (6) and the limit stated right after it.
    """
    x = np.asarray(x, dtype=np.float64)
    small = np.abs(x) < _SERIES_RADIUS
    safe = np.where(small, 1.0, x)
    with np.errstate(over="ignore"):
        closed = np.expm1(safe) / safe
    return np.where(small, _series(x, _PHI1_COEF), closed)


def phi2(x) -> np.ndarray:
    """phi_2(x) = integral_0^1 e^{s x} (1 - s) ds = (e^x - 1 - x)/x^2, phi_2(0) = 1/2.

    Preliminaries, eq. (6) and the limit stated right after it.
    """
    x = np.asarray(x, dtype=np.float64)
    small = np.abs(x) < _SERIES_RADIUS
    safe = np.where(small, 1.0, x)
    with np.errstate(over="ignore"):
        closed = (np.expm1(safe) - safe) / (safe * safe)
    return np.where(small, _series(x, _PHI2_COEF), closed)


def csa_row(q_t: np.ndarray, k_hat: np.ndarray, v_hat: np.ndarray, t: int):
    """o_t and lse_t for one query by eq. (8) (Assembly and Simplification).

    q_t:   (d,) query t.
    k_hat: (>= t+1, d) keys at positions 0, 1, ..., with row 0 = k_0.
    v_hat: (>= t+1, d_v) values at the same positions, row 0 = v_0.
    t:     query position, t >= 1 (integration interval [0, t]).
    """
    if t < 1:
        raise ValueError("query position t starts at 1")
    K = k_hat[: t + 1]
    V = v_hat[: t + 1]
    a = K @ q_t                       # a_{t,i} = q_t . k_i, i = 0..t
    shift = float(a.max())            # common factor e^{shift}; cancels in the ratio
    a_left = a[:-1]                   # a_{t,i-1}, i = 1..t
    delta = a[1:] - a_left            # delta_{t,i} = a_{t,i} - a_{t,i-1}
    e_left = np.exp(a_left - shift)   # e^{a_{t,i-1}}, shifted
    f1 = phi1(delta)
    f2 = phi2(delta)
    v_i = V[1:]                       # v_i,     i = 1..t
    v_im1 = V[:-1]                    # v_{i-1}, i = 1..t
    # eq. (4): segment numerator  e^{a_{i-1}} [phi_1 v_i + phi_2 (v_{i-1} - v_i)]
    seg_num = e_left[:, None] * (f1[:, None] * v_i + f2[:, None] * (v_im1 - v_i))
    # eq. (5): segment denominator e^{a_{i-1}} phi_1
    seg_den = e_left * f1
    num = seg_num.sum(axis=0)
    den = seg_den.sum()
    o = num / den
    lse = shift + math.log(den)
    if not (np.all(np.isfinite(o)) and math.isfinite(lse)):
        raise FloatingPointError(f"non-finite oracle result at t={t}")
    return o, lse


def _as_f64(x):
    try:  # torch tensors (any dtype, incl. bfloat16) are upcast exactly
        import torch

        if isinstance(x, torch.Tensor):
            return x.detach().to("cpu", torch.float64).numpy()
    except ImportError:  # pragma: no cover
        pass
    return np.asarray(x, dtype=np.float64)


def csa_reference(q, k, v, k0=None, v0=None, rows=None):
    """Causal continuous-softmax-attention forward, eq. (8), in float64.

    q, k: [B, H, T, d];  v: [B, H, T, d_v];  k0: [B, H, d] or None (zeros);
    v0: [B, H, d_v] or None (zeros) -- the three choices for k_0, v_0 are
    discussed under Analysis of the Result; "all zeros" is the default here.
    rows: optional iterable of 0-based query rows (row r is query t = r + 1);
    all T rows when None.

    Returns (o [B, H, R, d_v], lse [B, H, R]) as float64 numpy arrays.
    """
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, H, T, d = q.shape
    dv = v.shape[-1]
    k0 = np.zeros((B, H, d)) if k0 is None else _as_f64(k0)
    v0 = np.zeros((B, H, dv)) if v0 is None else _as_f64(v0)
    rows = np.arange(T) if rows is None else np.asarray(list(rows), dtype=np.int64)
    if rows.size and (rows.min() < 0 or rows.max() >= T):
        raise ValueError("query row out of range")
    o = np.empty((B, H, rows.size, dv))
    lse = np.empty((B, H, rows.size))
    for b in range(B):
        for h in range(H):
            k_hat = np.concatenate([k0[b, h][None], k[b, h]], axis=0)
            v_hat = np.concatenate([v0[b, h][None], v[b, h]], axis=0)
            for j, r in enumerate(rows):
                o[b, h, j], lse[b, h, j] = csa_row(q[b, h, r], k_hat, v_hat, int(r) + 1)
    return o, lse


def std_row(q_t: np.ndarray, k: np.ndarray, v: np.ndarray, t: int):
    """Standard causal softmax attention for query t, eq. (12) (Analysis of the Result).

    Keys/values at positions 1..t are array rows 0..t-1; no k_0, no correction.
    """
    a = k[:t] @ q_t
    shift = float(a.max())
    e = np.exp(a - shift)
    den = e.sum()
    return (e @ v[:t]) / den, shift + math.log(den)


def std_reference(q, k, v, rows=None):
    """Row-by-row float64 eq. (12); same shapes and conventions as csa_reference."""
    q, k, v = _as_f64(q), _as_f64(k), _as_f64(v)
    B, H, T, _ = q.shape
    rows = np.arange(T) if rows is None else np.asarray(list(rows), dtype=np.int64)
    o = np.empty((B, H, rows.size, v.shape[-1]))
    lse = np.empty((B, H, rows.size))
    for b in range(B):
        for h in range(H):
            for j, r in enumerate(rows):
                o[b, h, j], lse[b, h, j] = std_row(q[b, h, r], k[b, h], v[b, h], int(r) + 1)
    return o, lse
