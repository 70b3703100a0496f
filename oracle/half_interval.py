"""Float64 CPU reference for the interval variant [1/2, t + 1/2] of continuous softmax attention.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing in the product
path may import this module.

J. Su, "Continuous Softmax Attention", Problem Statement: the original paper
integrates eq. (2) over [1/2, t + 1/2] instead of [0, t] (for symmetry; the page
finds it less natural for causal attention and keeps [0, t]).  Reading taken
here (the page says no more): eq. (2) with the interpolation of eq. (3)
unchanged, integrated over [1/2, t + 1/2].  Query t therefore covers half of
segment [0, 1] (s in [1/2, 1], between k_0 and k_1), the whole segments
[1, 2] .. [t-1, t], and half of segment [t, t+1] (s in [t, t + 1/2], between
k_t and k_{t+1}): it reaches half a step toward position t+1.  For the last
query t = T, position T+1 does not exist; it is taken equal to position T
(k_{T+1} = k_T, v_{T+1} = v_T), the counterpart at the right end of the
"copy" choice for k_0, v_0 (Analysis of the Result) -- its half segment is
then flat.

Evaluation: as ``oracle.csa`` (eq. (4)-(5), segment by segment), with each
segment's integrals taken over the covered part [alpha, beta] of its local
coordinate sigma in [0, 1]:
    numerator   e^{a_{i-1}} [(F0 - F1)(delta) v_{i-1} + F1(delta) v_i],
    denominator e^{a_{i-1}} F0(delta),
    F0(x) = integral_alpha^beta e^{sigma x} d sigma,
    F1(x) = integral_alpha^beta sigma e^{sigma x} d sigma
(for [alpha, beta] = [0, 1]: F0 = phi_1, F0 - F1 = phi_2 of eq. (6)).
"""

from __future__ import annotations

import math

import numpy as np

from .csa import _as_f64

# Below this |x| the closed forms lose digits to cancellation; the Taylor series of
# the integrals is summed instead: F0 = sum_n x^n/n! (b^{n+1} - a^{n+1})/(n+1),
# F1 = sum_n x^n/n! (b^{n+2} - a^{n+2})/(n+2).  20 terms at |x| < 0.5 leave < 1e-22.
_SERIES_RADIUS = 0.5
_SERIES_TERMS = 20


def seg_integrals(x, lo, hi):
    """(F0, F1) = (integral_lo^hi e^{s x} ds, integral_lo^hi s e^{s x} ds), elementwise in x
    (lo, hi: scalars or arrays broadcast against x)."""
    x = np.asarray(x, dtype=np.float64)
    lo = np.asarray(lo, dtype=np.float64)
    hi = np.asarray(hi, dtype=np.float64)
    small = np.abs(x) < _SERIES_RADIUS
    safe = np.where(small, 1.0, x)
    with np.errstate(over="ignore"):
        ehi, elo = np.exp(hi * safe), np.exp(lo * safe)
        f0 = (ehi - elo) / safe
        # antiderivative of s e^{s x}: e^{s x} (s x - 1) / x^2
        f1 = (ehi * (hi * safe - 1.0) - elo * (lo * safe - 1.0)) / (safe * safe)
    s0 = np.zeros_like(x)
    s1 = np.zeros_like(x)
    for n in range(_SERIES_TERMS - 1, -1, -1):
        c = 1.0 / math.factorial(n)
        s0 = s0 * x + c * (hi ** (n + 1) - lo ** (n + 1)) / (n + 1)
        s1 = s1 * x + c * (hi ** (n + 2) - lo ** (n + 2)) / (n + 2)
    return np.where(small, s0, f0), np.where(small, s1, f1)


def csa_half_row(q_t, k_hat, v_hat, t: int):
    """o_t and lse_t over [1/2, t + 1/2].

    k_hat, v_hat: (>= t+2, d) rows for positions 0, 1, ..., t+1 (row 0 = k_0).
    """
    if t < 1:
        raise ValueError("query position t starts at 1")
    K = k_hat[: t + 2]
    V = v_hat[: t + 2]
    a = K @ q_t                         # positions 0..t+1
    shift = float(a.max())
    i = np.arange(1, t + 2)             # segments [i-1, i], i = 1..t+1
    lo = np.where(i == 1, 0.5, 0.0)     # covered part [lo, hi] of each segment's sigma
    hi = np.where(i == t + 1, 0.5, 1.0)
    delta = a[i] - a[i - 1]
    f0, f1 = seg_integrals(delta, lo, hi)
    e = np.exp(a[i - 1] - shift)
    num = ((e * (f0 - f1))[:, None] * V[i - 1] + (e * f1)[:, None] * V[i]).sum(axis=0)
    den = float((e * f0).sum())
    o = num / den
    lse = shift + math.log(den)
    if not (np.all(np.isfinite(o)) and math.isfinite(lse)):
        raise FloatingPointError(f"non-finite result at t={t}")
    return o, lse


def csa_half_reference(q, k, v, k0=None, v0=None, rows=None):
    """The [1/2, t + 1/2] variant for every query row (or ``rows``), float64.

    Shapes and conventions as ``csa_reference``; position T+1 (needed by the last
    query only) repeats position T.  Returns (o [B, H, R, d_v], lse [B, H, R]).
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
            k_hat = np.concatenate([k0[b, h][None], k[b, h], k[b, h, -1:]], axis=0)
            v_hat = np.concatenate([v0[b, h][None], v[b, h], v[b, h, -1:]], axis=0)
            for j, r in enumerate(rows):
                o[b, h, j], lse[b, h, j] = csa_half_row(q[b, h, r], k_hat, v_hat, int(r) + 1)
    return o, lse
