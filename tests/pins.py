"""Independent checks ("pins") of the CPU reference.

Each check computes the expected value by a route that does not go through
the reference's own formula, eq. (8) of J. Su, "Continuous Softmax Attention":

* ``quadrature_row``  -- Gauss-Legendre integration of the defining integrals,
  eq. (2) with the interpolation eq. (3) (Problem Statement);
* ``simplified_row_mp`` -- eq. (10)-(11) (Assembly and Simplification) in
  50-digit mpmath arithmetic;
* closed forms derived from eq. (2): equal logits (trapezoid rule), a linear
  ramp of keys and values, the copied sink at t = 1;
* the Taylor expansion of the correction b, eq. (13) (Analysis of the
  Result), taken to second order.

Every function returns the maximum deviation so that mutation tests can
assert that a planted mistake in the reference is caught.
"""

from __future__ import annotations

import math

import mpmath as mp
import numpy as np

_GL_X, _GL_W = np.polynomial.legendre.leggauss(48)
_GL_S = 0.5 * (_GL_X + 1.0)   # nodes on [0, 1]
_GL_W01 = 0.5 * _GL_W


def quadrature_row(q_t, k_hat, v_hat, t):
    """(o_t, lse_t) by integrating e^{q.k_s} and e^{q.k_s} v_s over [0, t].

    k_s and v_s are built by linear interpolation (eq. (3)); each unit segment
    is integrated with a 48-point Gauss-Legendre rule on a fine sub-grid.
    """
    num = np.zeros(v_hat.shape[1])
    den = 0.0
    terms = []
    for i in range(1, t + 1):
        for sub in range(4):  # 4 sub-intervals per unit segment
            s_local = (sub + _GL_S) / 4.0          # position inside [i-1, i], 0..1
            w = _GL_W01 / 4.0
            k_s = (1.0 - s_local)[:, None] * k_hat[i - 1] + s_local[:, None] * k_hat[i]
            v_s = (1.0 - s_local)[:, None] * v_hat[i - 1] + s_local[:, None] * v_hat[i]
            terms.append((k_s @ q_t, w, v_s))
    shift = max(float(x.max()) for x, _, _ in terms)
    for logits, w, v_s in terms:
        e = np.exp(logits - shift) * w
        den += e.sum()
        num += e @ v_s
    return num / den, shift + math.log(den)


def _phi2_mp(x):
    if x == 0:
        return mp.mpf(1) / 2
    return (mp.exp(x) - 1 - x) / (x * x)


def simplified_row_mp(q_t, k_hat, v_hat, t, dps=50):
    """(o_t, lse_t) by eq. (10)-(11) in mpmath: weights e^{a_i + b_i}, i = 0..t."""
    with mp.workdps(dps):
        q = [mp.mpf(float(x)) for x in q_t]
        a = [mp.fsum(mp.mpf(float(kk)) * qq for kk, qq in zip(k_hat[i], q)) for i in range(t + 1)]
        eb = []
        for i in range(t + 1):
            s = mp.mpf(0)
            if i >= 1:
                s += _phi2_mp(a[i - 1] - a[i])
            if i <= t - 1:
                s += _phi2_mp(a[i + 1] - a[i])
            eb.append(s)
        wts = [mp.exp(a[i]) * eb[i] for i in range(t + 1)]
        den = mp.fsum(wts)
        o = [mp.fsum(wts[i] * mp.mpf(float(v_hat[i][c])) for i in range(t + 1)) / den
             for c in range(v_hat.shape[1])]
        return np.array([float(x) for x in o]), float(mp.log(den))


def hat(q, k, v, k0, v0, b=0, h=0):
    k_hat = np.concatenate([k0[b, h][None], k[b, h]], axis=0)
    v_hat = np.concatenate([v0[b, h][None], v[b, h]], axis=0)
    return q[b, h], k_hat, v_hat


def random_case(seed, T=9, d=3, dv=4, scale=1.0, sink=True):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((1, 1, T, d)) * scale
    k = rng.standard_normal((1, 1, T, d))
    v = rng.standard_normal((1, 1, T, dv))
    k0 = rng.standard_normal((1, 1, d)) if sink else np.zeros((1, 1, d))
    v0 = rng.standard_normal((1, 1, dv)) if sink else np.zeros((1, 1, dv))
    return q, k, v, k0, v0


def dev_vs_quadrature(ref, seed=0, scale=1.0):
    """Max |reference - quadrature| over all rows of a small random case."""
    q, k, v, k0, v0 = random_case(seed, scale=scale)
    o, lse = ref(q, k, v, k0, v0)
    qq, kh, vh = hat(q, k, v, k0, v0)
    worst = 0.0
    for r in range(q.shape[2]):
        oq, lq = quadrature_row(qq[r], kh, vh, r + 1)
        worst = max(worst, float(np.abs(o[0, 0, r] - oq).max()), abs(float(lse[0, 0, r]) - lq))
    return worst


def dev_vs_simplified(ref, seed=1, scale=1.5):
    """Max |reference - mpmath eq. (10)-(11)| over all rows of a small random case."""
    q, k, v, k0, v0 = random_case(seed, T=8, scale=scale)
    o, lse = ref(q, k, v, k0, v0)
    qq, kh, vh = hat(q, k, v, k0, v0)
    worst = 0.0
    for r in range(q.shape[2]):
        om, lm = simplified_row_mp(qq[r], kh, vh, r + 1)
        worst = max(worst, float(np.abs(o[0, 0, r] - om).max()), abs(float(lse[0, 0, r]) - lm))
    return worst


def dev_trapezoid(ref, seed=2, T=7):
    """Equal logits (q = 0): weights 1/2, 1, ..., 1, 1/2 and lse = ln t."""
    _, k, v, k0, v0 = random_case(seed, T=T)
    q = np.zeros((1, 1, T, k.shape[-1]))
    o, lse = ref(q, k, v, k0, v0)
    vh = np.concatenate([v0[0, 0][None], v[0, 0]], axis=0)
    worst = 0.0
    for r in range(T):
        t = r + 1
        expect = (0.5 * vh[0] + vh[1:t].sum(axis=0) + 0.5 * vh[t]) / t
        worst = max(worst, float(np.abs(o[0, 0, r] - expect).max()), abs(float(lse[0, 0, r]) - math.log(t)))
    return worst


def dev_linear_ramp(ref, beta=0.7, T=6):
    """k_i = i w, v_i = i c with k_0 = v_0 = 0: q.k_s = beta s, v_s = s c exactly.

    o_t = c (e^{beta t}(beta t - 1) + 1) / (beta (e^{beta t} - 1)),
    lse_t = ln((e^{beta t} - 1)/beta).
    """
    d, dv = 3, 2
    w = np.array([0.3, -0.2, 0.5])
    qv = w * (beta / float(w @ w))          # q . w = beta
    c = np.array([1.5, -0.25])
    pos = np.arange(1, T + 1, dtype=np.float64)
    q = np.broadcast_to(qv, (1, 1, T, d)).copy()
    k = (pos[:, None] * w[None, :])[None, None]
    v = (pos[:, None] * c[None, :])[None, None]
    o, lse = ref(q, k, v, np.zeros((1, 1, d)), np.zeros((1, 1, dv)))
    worst = 0.0
    for r in range(T):
        t = r + 1
        with mp.workdps(40):  # the closed forms cancel for small beta*t; evaluate them exactly
            bt = mp.mpf(beta) * t
            ratio = (mp.exp(bt) * (bt - 1) + 1) / (mp.mpf(beta) * mp.expm1(bt))
            o_exp = c * float(ratio)
            l_exp = float(mp.log(mp.expm1(bt) / mp.mpf(beta)))
        worst = max(worst, float(np.abs(o[0, 0, r] - o_exp).max()), abs(float(lse[0, 0, r]) - l_exp))
    return worst


def implied_b(ref, q_t, k_hat, t):
    """Correction b_{t,i} recovered from the reference with one-hot values.

    With v_i = e_i (the i-th unit vector, i = 0..t) the output is the vector of
    normalised weights e^{a_i + b_i - lse}; so b_i = ln o_i + lse - a_i.
    """
    d = q_t.shape[0]
    q = q_t[None, None, None, :].repeat(t, axis=2)
    k = k_hat[1 : t + 1][None, None]
    eye = np.eye(t + 1)
    o, lse = ref(q, k, eye[1:][None, None], k_hat[0][None, None], eye[0][None, None], rows=[t - 1])
    a = k_hat[: t + 1] @ q_t
    return np.log(o[0, 0, 0]) + lse[0, 0, 0] - a, a


def dev_taylor_b(ref, eps, seed=3, t=6):
    """|b - second-order Taylor| for logits of size eps (should scale as eps^3).

    Interior: b = (L + R)/6 + (L^2 - L R + R^2)/36 + O(3), L = a_{i-1} - a_i,
    R = a_{i+1} - a_i (first order: eq. (13)).  Ends: b = -ln 2 + x/3 + x^2/36
    + O(3) with x the single neighbour difference.
    """
    rng = np.random.default_rng(seed)
    d = 4
    q_t = rng.standard_normal(d) * eps
    k_hat = rng.standard_normal((t + 1, d))
    b, a = implied_b(ref, q_t, k_hat, t)
    worst = 0.0
    for i in range(t + 1):
        if i == 0 or i == t:
            x = a[1] - a[0] if i == 0 else a[t - 1] - a[t]
            approx = -math.log(2.0) + x / 3 + x * x / 36
        else:
            L, R = a[i - 1] - a[i], a[i + 1] - a[i]
            approx = (L + R) / 6 + (L * L - L * R + R * R) / 36
        worst = max(worst, abs(b[i] - approx))
    return worst


def dev_copied_sink(ref, seed=4):
    """k_0 = k_1, v_0 = v_1: the first segment is flat, so o_1 = v_1, lse_1 = a_1."""
    q, k, v, _, _ = random_case(seed)
    k0, v0 = k[:, :, 0].copy(), v[:, :, 0].copy()
    o, lse = ref(q, k, v, k0, v0, rows=[0])
    a1 = float(q[0, 0, 0] @ k[0, 0, 0])
    return max(float(np.abs(o[0, 0, 0] - v[0, 0, 0]).max()), abs(float(lse[0, 0, 0]) - a1))


# ---------------------------------------------------------------- first-order variant

def dev1_linear(ref, beta=0.7, T=6):
    """First-order variant on linear logits a_i = beta i (k_0 = v_0 = 0, v_i = i c).

    The second difference vanishes, so interior weights are e^{beta i}; the ends
    carry e^{-ln 2 + x/3} with x = beta at i = 0 and x = -beta at i = t.  The sums
    are taken in closed form (geometric and arithmetic-geometric series):
    den = e^{beta/3}/2 + r (r^{t-1} - 1)/(r - 1) + e^{beta t - beta/3}/2,
    num = c [ r (1 - t r^{t-1} + (t-1) r^t)/(1 - r)^2 + t e^{beta t - beta/3}/2 ],
    r = e^beta.
    """
    d, dv = 3, 2
    w = np.array([0.3, -0.2, 0.5])
    qv = w * (beta / float(w @ w))
    c = np.array([1.5, -0.25])
    pos = np.arange(1, T + 1, dtype=np.float64)
    q = np.broadcast_to(qv, (1, 1, T, d)).copy()
    k = (pos[:, None] * w[None, :])[None, None]
    v = (pos[:, None] * c[None, :])[None, None]
    o, lse = ref(q, k, v, np.zeros((1, 1, d)), np.zeros((1, 1, dv)))
    worst = 0.0
    with mp.workdps(40):
        bb = mp.mpf(beta)
        r = mp.exp(bb)
        for row in range(T):
            t = row + 1
            geo = r * (r ** (t - 1) - 1) / (r - 1) if t > 1 else mp.mpf(0)
            ageo = r * (1 - t * r ** (t - 1) + (t - 1) * r ** t) / (1 - r) ** 2 if t > 1 else mp.mpf(0)
            end_t = mp.exp(bb * t - bb / 3) / 2
            den = mp.exp(bb / 3) / 2 + geo + end_t
            ratio = (ageo + t * end_t) / den
            o_exp = c * float(ratio)
            l_exp = float(mp.log(den))
            worst = max(worst, float(np.abs(o[0, 0, row] - o_exp).max()), abs(float(lse[0, 0, row]) - l_exp))
    return worst


def dev1_vs_exact(ref, eps, seed=3, t=6):
    """max_i |b_i(first-order reference) - b_i(exact reference)| for logits of size eps.

    eq. (13) is the first-order term of the exact b, so the gap is second order:
    it must shrink like eps^2 (a wrong coefficient, sign or end constant leaves an
    O(eps) or O(1) gap).
    """
    from oracle import csa_reference

    rng = np.random.default_rng(seed)
    q_t = rng.standard_normal(4) * eps
    k_hat = rng.standard_normal((t + 1, 4))
    b1, _ = implied_b(ref, q_t, k_hat, t)
    b, _ = implied_b(csa_reference, q_t, k_hat, t)
    return float(np.abs(b1 - b).max())


# ---------------------------------------------------------------- backward (gradient)

def _loss_by_quadrature(q, k, v, k0, v0, do, dlse):
    """sum_t dO_t . o_t + dlse_t lse_t with (o_t, lse_t) from the defining integral, eq. (2)."""
    qq, kh, vh = hat(q, k, v, k0, v0)
    total = 0.0
    for r in range(q.shape[2]):
        o, lse = quadrature_row(qq[r], kh, vh, r + 1)
        total += float(do[0, 0, r] @ o) + float(dlse[0, 0, r]) * lse
    return total


def grad_case(seed, T=5, d=3, dv=3, scale=1.0):
    q, k, v, k0, v0 = random_case(seed, T=T, d=d, dv=dv, scale=scale)
    rng = np.random.default_rng(seed + 1000)
    do = rng.standard_normal((1, 1, T, dv))
    dlse = rng.standard_normal((1, 1, T))
    return q, k, v, k0, v0, do, dlse


def dev_grad_fd(ref_bwd, seed=11, scale=1.0, h=1e-5, T=5, d=3, dv=3):
    """max |gradient - central difference of the quadrature loss| / max |gradient|.

    Every entry of q, k, v, k_0, v_0 is perturbed by +-h and the loss re-evaluated
    from the defining integral (Gauss-Legendre), never through eq. (8).  The
    truncation error is O(h^2) and the rounding error O(1e-16/h), ~1e-10 relative.
    """
    q, k, v, k0, v0, do, dlse = grad_case(seed, T=T, d=d, dv=dv, scale=scale)
    got = ref_bwd(q, k, v, do, k0, v0, dlse)
    inputs = [q, k, v, k0, v0]
    worst, scale_g = 0.0, max(float(np.abs(g).max()) for g in got)
    for x, g in zip(inputs, got):
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + h
            lp = _loss_by_quadrature(*inputs, do, dlse)
            x[idx] = old - h
            lm = _loss_by_quadrature(*inputs, do, dlse)
            x[idx] = old
            worst = max(worst, abs((lp - lm) / (2 * h) - float(g[idx])))
    return worst / scale_g


def dev_grad_shift(ref_bwd, seed=12, T=24, d=5, dv=4, scale=1.5):
    """Two symmetries of eq. (2) seen in the gradient.

    v_s -> v_s + c for every position moves every o_t by c, so sum over positions
    0..T of dv equals sum_t dO_t; k_s -> k_s + w moves every logit of query t by
    q_t . w, which leaves o_t unchanged and moves lse_t by q_t . w, so the sum of dk
    over positions equals sum_t dlse_t q_t.
    """
    q, k, v, k0, v0, do, dlse = grad_case(seed, T=T, d=d, dv=dv, scale=scale)
    dq, dk, dv_, dk0, dv0 = ref_bwd(q, k, v, do, k0, v0, dlse)
    sum_v = dv_[0, 0].sum(axis=0) + dv0[0, 0] - do[0, 0].sum(axis=0)
    sum_k = dk[0, 0].sum(axis=0) + dk0[0, 0] - dlse[0, 0] @ q[0, 0]
    return max(float(np.abs(sum_v).max()), float(np.abs(sum_k).max()))


def dev_grad_trapezoid(ref_bwd, seed=13, T=7):
    """q = 0 (equal logits): o_t is the trapezoid average, so dv has the closed form
    dv_j = sum_t w_{t,j} dO_t / t with w_{t,0} = w_{t,t} = 1/2 and 1 in between."""
    _, k, v, k0, v0, do, dlse = grad_case(seed, T=T)
    q = np.zeros((1, 1, T, k.shape[-1]))
    _, _, dv_, _, dv0 = ref_bwd(q, k, v, do, k0, v0, dlse)
    expect = np.zeros((T + 1, v.shape[-1]))
    for r in range(T):
        t = r + 1
        w = np.ones(t + 1)
        w[0] = w[t] = 0.5
        expect[: t + 1] += np.outer(w / t, do[0, 0, r])
    got = np.concatenate([dv0[0, 0][None], dv_[0, 0]], axis=0)
    return float(np.abs(got - expect).max())


# ---------------------------------------------------------------- interval [1/2, t + 1/2]

def quadrature_half_row(q_t, k_hat, v_hat, t):
    """(o_t, lse_t) integrating eq. (2) over [1/2, t + 1/2] with the interpolation of eq. (3).

    k_hat, v_hat hold positions 0..t+1.  Each covered piece of a unit segment is integrated
    with the 48-point Gauss-Legendre rule on 4 sub-intervals, as ``quadrature_row``.
    """
    pieces = [(1, 0.5, 1.0)] + [(i, 0.0, 1.0) for i in range(2, t + 1)] + [(t + 1, 0.0, 0.5)]
    terms = []
    for i, lo, hi in pieces:
        for sub in range(4):
            a, b = lo + (hi - lo) * sub / 4, lo + (hi - lo) * (sub + 1) / 4
            s_local = a + (b - a) * _GL_S
            w = _GL_W01 * (b - a)
            k_s = (1.0 - s_local)[:, None] * k_hat[i - 1] + s_local[:, None] * k_hat[i]
            v_s = (1.0 - s_local)[:, None] * v_hat[i - 1] + s_local[:, None] * v_hat[i]
            terms.append((k_s @ q_t, w, v_s))
    shift = max(float(x.max()) for x, _, _ in terms)
    num = np.zeros(v_hat.shape[1])
    den = 0.0
    for logits, w, v_s in terms:
        e = np.exp(logits - shift) * w
        den += e.sum()
        num += e @ v_s
    return num / den, shift + math.log(den)


def _half_hat(q, k, v, k0, v0):
    """Positions 0..T+1 with position T+1 repeating position T (the last query's convention)."""
    qq, kh, vh = hat(q, k, v, k0, v0)
    return qq, np.concatenate([kh, kh[-1:]]), np.concatenate([vh, vh[-1:]])


def dev_half_vs_quadrature(ref, seed=0, scale=1.0):
    """Max |reference - quadrature over [1/2, t + 1/2]| over all rows (incl. the last)."""
    q, k, v, k0, v0 = random_case(seed, scale=scale)
    o, lse = ref(q, k, v, k0, v0)
    qq, kh, vh = _half_hat(q, k, v, k0, v0)
    worst = 0.0
    for r in range(q.shape[2]):
        oq, lq = quadrature_half_row(qq[r], kh, vh, r + 1)
        worst = max(worst, float(np.abs(o[0, 0, r] - oq).max()), abs(float(lse[0, 0, r]) - lq))
    return worst


def dev_half_trapezoid(ref, seed=2, T=7):
    """Equal logits (q = 0): o_t is the average of v_s over [1/2, t + 1/2], i.e. weights
    1/8, 7/8, 1, ..., 1, 7/8, 1/8 on positions 0..t+1 (t = 1: 1/8, 3/4, 1/8); lse = ln t."""
    _, k, v, k0, v0 = random_case(seed, T=T)
    q = np.zeros((1, 1, T, k.shape[-1]))
    o, lse = ref(q, k, v, k0, v0)
    _, _, vh = _half_hat(q, k, v, k0, v0)
    worst = 0.0
    for r in range(T):
        t = r + 1
        w = np.ones(t + 2)
        w[0] = w[t + 1] = 1.0 / 8.0
        if t == 1:
            w[1] = 0.75
        else:
            w[1] = w[t] = 7.0 / 8.0
        expect = (w @ vh[: t + 2]) / t
        worst = max(worst, float(np.abs(o[0, 0, r] - expect).max()), abs(float(lse[0, 0, r]) - math.log(t)))
    return worst


def dev_half_linear_ramp(ref, beta=0.7, T=6):
    """k_i = i w, v_i = i c (k_0 = v_0 = 0): q.k_s = beta s and v_s = s c on [0, T], so for
    t < T (position t+1 is a real key)
    o_t = c [s e^{beta s}/beta - e^{beta s}/beta^2] / [e^{beta s}/beta] over [1/2, t + 1/2],
    lse_t = ln((e^{beta (t+1/2)} - e^{beta/2})/beta)."""
    d, dv = 3, 2
    w = np.array([0.3, -0.2, 0.5])
    qv = w * (beta / float(w @ w))
    c = np.array([1.5, -0.25])
    pos = np.arange(1, T + 1, dtype=np.float64)
    q = np.broadcast_to(qv, (1, 1, T, d)).copy()
    k = (pos[:, None] * w[None, :])[None, None]
    v = (pos[:, None] * c[None, :])[None, None]
    o, lse = ref(q, k, v, np.zeros((1, 1, d)), np.zeros((1, 1, dv)))
    worst = 0.0
    with mp.workdps(40):
        bb = mp.mpf(beta)
        for r in range(T - 1):
            t = r + 1
            lo, hi = mp.mpf(1) / 2, mp.mpf(t) + mp.mpf(1) / 2
            den = (mp.exp(bb * hi) - mp.exp(bb * lo)) / bb
            num = (mp.exp(bb * hi) * (bb * hi - 1) - mp.exp(bb * lo) * (bb * lo - 1)) / (bb * bb)
            o_exp = c * float(num / den)
            worst = max(worst, float(np.abs(o[0, 0, r] - o_exp).max()), abs(float(lse[0, 0, r]) - float(mp.log(den))))
    return worst
