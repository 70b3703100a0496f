"""GPU parity of the interval variant [1/2, t + 1/2] (csa_forward_half_interval, bf16)
against its float64 CPU reference (oracle.half_interval).

Tolerance: max abs error on o and lse of 2e-2 (bfloat16 inputs, float32 accumulation),
as for the exact forward.  Small cases on every row; the large workloads on sampled
rows plus properties of every row.
"""

import math

import numpy as np
import pytest
import torch

import continuous_softmax_attention_amd as csa
from oracle import csa_half_reference
from workloads import WORKLOADS, make_inputs, sample_rows

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TOL = 2e-2


def _gpu(*ts):
    return [None if t is None else t.to(DEV) for t in ts]


def _run(q, k, v, k0=None, v0=None):
    o, lse = csa.csa_forward_half_interval(*_gpu(q, k, v, k0, v0))
    torch.cuda.synchronize()
    return o.float().cpu().double().numpy(), lse.cpu().double().numpy()


def _errs(o, lse, o_ref, l_ref):
    return float(np.abs(o - o_ref).max()), float(np.abs(lse - l_ref).max())


def _report(tag, eo, el):
    print(f"[parity half-interval] {tag}: max|o-ref| = {eo:.3e}  max|lse-ref| = {el:.3e}", flush=True)


def _random_case(B, H, T, d, seed, q_mult=1.0, sink=True):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, H, T, d, generator=g) * (q_mult / math.sqrt(d))
    k = torch.randn(B, H, T, d, generator=g)
    v = torch.randn(B, H, T, d, generator=g)
    k0 = torch.randn(B, H, d, generator=g) if sink else None
    v0 = torch.randn(B, H, d, generator=g) if sink else None
    cast = (lambda t: None if t is None else t.bfloat16())
    return cast(q), cast(k), cast(v), cast(k0), cast(v0)


@pytest.mark.parametrize("d", [16, 64, 128])
@pytest.mark.parametrize("T", [1, 2, 3, 15, 16, 17, 31, 63, 64, 65, 127, 128, 129, 200, 257])
def test_edge_shapes_with_random_sink(T, d):
    q, k, v, k0, v0 = _random_case(1, 2, T, d, seed=9100 * T + d)
    o, lse = _run(q, k, v, k0, v0)
    o_ref, l_ref = csa_half_reference(q, k, v, k0, v0)
    eo, el = _errs(o, lse, o_ref, l_ref)
    assert eo <= TOL and el <= TOL, (eo, el)


def test_many_heads_no_sink():
    q, k, v, _, _ = _random_case(3, 5, 300, 128, seed=16, sink=False)
    o, lse = _run(q, k, v)
    o_ref, l_ref = csa_half_reference(q, k, v)
    eo, el = _errs(o, lse, o_ref, l_ref)
    _report("B3 H5 T300", eo, el)
    assert eo <= TOL and el <= TOL


@pytest.mark.parametrize("q_mult", [4.0, 8.0, 12.0])
def test_large_logits_copied_sink(q_mult):
    q, k, v, _, _ = _random_case(1, 3, 333, 128, seed=81, q_mult=q_mult, sink=False)
    k0, v0 = k[:, :, 0].clone(), v[:, :, 0].clone()
    o, lse = _run(q, k, v, k0, v0)
    o_ref, l_ref = csa_half_reference(q, k, v, k0, v0)
    eo, el = _errs(o, lse, o_ref, l_ref)
    _report(f"large logits x{q_mult}", eo, el)
    assert eo <= TOL and el <= TOL


def test_one_hot_values_give_the_weights():
    # v_i = e_i: o_t is the normalised weight of every position 1..t+1 in turn
    T, d = 127, 128
    q, k, _, _, _ = _random_case(1, 1, T, d, seed=82, q_mult=8.0, sink=False)
    v = torch.zeros(1, 1, T, d)
    v[0, 0, torch.arange(T), torch.arange(T)] = 1.0
    v = v.bfloat16()
    o, lse = _run(q, k, v)
    o_ref, l_ref = csa_half_reference(q, k, v)
    eo, el = _errs(o, lse, o_ref, l_ref)
    _report("one-hot weights, logit std 8", eo, el)
    assert eo <= TOL and el <= TOL


def test_trapezoid_closed_form_through_kernel():
    # q = 0: the integrand of eq. (2) is the interpolated v over [1/2, t + 1/2], so the
    # weights are 1/8 (position 0), 3/8 + 1/2 (position 1), 1 (interior), 1/2 + 3/8
    # (position t), 1/8 (position t + 1; for t = T it falls on position T), lse = ln t
    T, d = 130, 64
    _, k, v, k0, v0 = _random_case(1, 1, T, d, seed=5)
    q = torch.zeros(1, 1, T, d, dtype=torch.bfloat16)
    o, lse = _run(q, k, v, k0, v0)
    vh = torch.cat([v0[0, 0][None], v[0, 0], v[0, 0, -1:]]).double().numpy()
    for r in range(T):
        t = r + 1
        w = np.zeros(t + 2)
        w[0] += 1 / 8
        w[1] += 3 / 8
        w[1:t] += 1 / 2
        w[2:t + 1] += 1 / 2
        w[t] += 3 / 8
        w[t + 1] += 1 / 8
        expect = (w[:, None] * vh[:t + 2]).sum(0) / t
        assert abs(w.sum() - t) < 1e-12
        assert np.abs(o[0, 0, r] - expect).max() < 1e-2
        # the row sums add the bf16-rounded weights (c^2/8, 3c^2/8, ... are not exact in
        # bf16): each is off by at most 2^-9 relatively, so lse by at most ~2^-9 < 2e-3 + slack
        assert abs(lse[0, 0, r] - math.log(t)) < 4e-3


def test_linear_logits_exact_in_bf16():
    # k_i = i w, v_i = i c with w, c powers of two: every input is exact in bf16 and the
    # logits are exactly beta i
    T, d = 200, 64
    w = torch.zeros(d)
    w[3] = 2.0 ** -6
    q = torch.zeros(1, 1, T, d)
    q[..., 3] = 1.0
    pos = torch.arange(1, T + 1, dtype=torch.float32)
    k = (pos[:, None] * w[None, :])[None, None]
    c = torch.full((d,), 2.0 ** -8)
    v = (pos[:, None] * c[None, :])[None, None]
    q, k, v = q.bfloat16(), k.bfloat16(), v.bfloat16()
    o, lse = _run(q, k, v)
    o_ref, l_ref = csa_half_reference(q, k, v)
    eo, el = _errs(o, lse, o_ref, l_ref)
    _report("linear logits", eo, el)
    assert eo <= TOL and el <= TOL


def test_unsupported_dtype_and_head_dim_are_rejected():
    q, k, v, _, _ = _random_case(1, 1, 64, 64, seed=6)
    with pytest.raises(csa.CsaError) as err:
        csa.csa_forward_half_interval(*_gpu(q.float(), k.float(), v.float()))
    assert err.value.status == csa.CSA_ERR_UNSUPPORTED
    q, k, v, _, _ = _random_case(1, 1, 64, 32, seed=6)
    with pytest.raises(csa.CsaError) as err:
        csa.csa_forward_half_interval(*_gpu(q, k, v))
    assert err.value.status == csa.CSA_ERR_UNSUPPORTED


@pytest.mark.parametrize("name", ["lm", "long", "stress"])
def test_large_workloads_sampled_rows(name):
    w = WORKLOADS[name]
    print(f"[parity half-interval] {name}: generating B{w.B} H{w.H} T{w.T} d{w.d} {w.dtype}", flush=True)
    q, k, v, k0, v0 = make_inputs(w)
    o_dev, lse_dev = csa.csa_forward_half_interval(*_gpu(q, k, v, k0, v0))
    torch.cuda.synchronize()
    assert bool(torch.isfinite(lse_dev).all()) and bool(torch.isfinite(o_dev.float()).all())
    vmax = float(v.float().abs().max())
    assert float(o_dev.float().abs().max()) <= vmax * (1 + 1e-2)
    rows = sample_rows(w.T, seed=w.seed, n_random=16)
    o = o_dev[:, :, rows].float().cpu().double().numpy()
    lse = lse_dev[:, :, rows].cpu().double().numpy()
    del o_dev, lse_dev
    o_ref, l_ref = csa_half_reference(q, k, v, k0, v0, rows=rows)
    eo, el = _errs(o, lse, o_ref, l_ref)
    _report(f"{name} ({len(rows)} rows x {w.B * w.H} heads)", eo, el)
    assert eo <= TOL and el <= TOL
