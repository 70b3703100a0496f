"""Float64 CPU reference for the first-order variant of the forward pass.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing in the product
path may import this module.

J. Su, "Continuous Softmax Attention", Analysis of the Result, eq. (13): the
correction b_{t,i} of eq. (10) expands, for an interior position, to the
second difference (a_{t,i-1} + a_{t,i+1} - 2 a_{t,i})/6 of the logits -- the
"short convolution" reading of the method.  This module computes eq. (11) with
b replaced by that first-order term (and the matching first-order term at the
two end positions), written out directly; it shares nothing with the kernels.
"""

from __future__ import annotations

import math

import numpy as np

from .csa import _as_f64


def csa1_row(q_t: np.ndarray, k_hat: np.ndarray, v_hat: np.ndarray, t: int):
    """o_t and lse_t with the correction b replaced by its first-order expansion.

    Analysis of the Result, eq. (13): for an interior position 1 <= i <= t-1,
    b_{t,i} = ln(phi_2(a_{i-1} - a_i) + phi_2(a_{i+1} - a_i)) expands to the
    second difference (a_{i-1} + a_{i+1} - 2 a_i)/6.  The two end positions of
    eq. (10) keep a single phi_2 term; with phi_2(x) = 1/2 + x/6 + O(x^2) the same
    expansion gives ln phi_2(x) = -ln 2 + x/3, x the difference to the one
    neighbour (a_1 - a_0 at i = 0, a_{t-1} - a_t at i = t).  The output is then
    the weighted average of eq. (11) with weights e^{a_i + b_i}; lse is the
    natural log of their sum.  Same arguments as csa_row.
    """
    if t < 1:
        raise ValueError("query position t starts at 1")
    K = k_hat[: t + 1]
    V = v_hat[: t + 1]
    a = K @ q_t                                        # a_{t,i}, i = 0..t
    b = np.empty(t + 1)
    b[1:t] = (a[: t - 1] + a[2:] - 2.0 * a[1:t]) / 6.0  # interior second difference
    b[0] = -math.log(2.0) + (a[1] - a[0]) / 3.0        # end i = 0
    b[t] = -math.log(2.0) + (a[t - 1] - a[t]) / 3.0    # end i = t
    z = a + b
    shift = float(z.max())
    w = np.exp(z - shift)
    den = w.sum()
    o = (w @ V) / den
    lse = shift + math.log(den)
    if not (np.all(np.isfinite(o)) and math.isfinite(lse)):
        raise FloatingPointError(f"non-finite oracle result at t={t}")
    return o, lse


def csa1_reference(q, k, v, k0=None, v0=None, rows=None):
    """First-order variant of the forward (csa1_row), same shapes and conventions as
    csa_reference."""
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
                o[b, h, j], lse[b, h, j] = csa1_row(q[b, h, r], k_hat, v_hat, int(r) + 1)
    return o, lse
