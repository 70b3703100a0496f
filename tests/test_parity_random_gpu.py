"""GPU parity on a seeded sweep of random shapes: every forward rule (exact weights, eq. (13)'s
first-order form, the [1/2, t+1/2] interval variant) and the backward, each against its float64
reference on every row.  The shapes are drawn once from a fixed seed: batch and head counts that
are and are not multiples of the work-group grouping, lengths scattered over 1..520 with extra
weight on the 64-row tile edges, the three head dimensions, the three sink choices (none, random,
copied) and two logit scales.  Bars as everywhere: 1e-5 (float32) and 2e-2 (bf16) max abs error
on o and lse; gradients 2e-2 x max(1, max|G_ref|) per tensor (1e-5 x for float32).
"""

import math

import numpy as np
import pytest
import torch

import continuous_softmax_attention_amd as csa
from oracle import csa1_reference, csa_backward_reference, csa_half_reference, csa_reference

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2}
GRAD_NAMES = ("dq", "dk", "dv", "dk0", "dv0")


def _draw_cases(n, seed):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        B = int(rng.choice([1, 2, 3]))
        H = int(rng.choice([1, 2, 3, 5]))
        if rng.random() < 0.4:  # near a tile edge
            T = int(max(1, 64 * rng.integers(1, 9) + rng.integers(-2, 3)))
        else:
            T = int(rng.integers(1, 521))
        d = int(rng.choice([16, 64, 128]))
        sink = str(rng.choice(["none", "random", "copy"]))
        q_mult = float(rng.choice([1.0, 4.0]))
        cases.append((i, B, H, T, d, sink, q_mult))
    return cases


def _inputs(B, H, T, d, sink, q_mult, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    q = torch.randn(B, H, T, d, generator=g) * (q_mult / math.sqrt(d))
    k = torch.randn(B, H, T, d, generator=g)
    v = torch.randn(B, H, T, d, generator=g)
    k0 = v0 = None
    if sink == "random":
        k0 = torch.randn(B, H, d, generator=g)
        v0 = torch.randn(B, H, d, generator=g)
    q, k, v = q.to(dtype), k.to(dtype), v.to(dtype)
    if sink == "copy":
        k0, v0 = k[:, :, 0].clone(), v[:, :, 0].clone()
    elif sink == "random":
        k0, v0 = k0.to(dtype), v0.to(dtype)
    return q, k, v, k0, v0


def _gpu(*ts):
    return [None if t is None else t.to(DEV) for t in ts]


FWD_CASES = _draw_cases(36, seed=20261)
RULES = {
    "exact": (csa.csa_forward, csa_reference),
    "first_order": (csa.csa_forward_first_order, csa1_reference),
    "half_interval": (csa.csa_forward_half_interval, csa_half_reference),
}


@pytest.mark.parametrize("rule", list(RULES))
@pytest.mark.parametrize("case", FWD_CASES, ids=lambda c: "c{}-B{}H{}T{}d{}-{}-x{:g}".format(*c))
def test_forward_random_shapes(case, rule):
    i, B, H, T, d, sink, q_mult = case
    fn, ref = RULES[rule]
    dtype = torch.float32 if (rule == "exact" and i % 3 == 0) else torch.bfloat16
    q, k, v, k0, v0 = _inputs(B, H, T, d, sink, q_mult, dtype, seed=7000 + i)
    o, lse = fn(*_gpu(q, k, v, k0, v0))
    torch.cuda.synchronize()
    o = o.float().cpu().double().numpy()
    lse = lse.cpu().double().numpy()
    o_ref, l_ref = ref(q, k, v, k0, v0)
    eo, el = float(np.abs(o - o_ref).max()), float(np.abs(lse - l_ref).max())
    tol = TOL[dtype] * (4.0 if dtype == torch.float32 and q_mult > 1.0 else 1.0)
    print(f"[parity random] {rule} {case} {dtype}: o {eo:.3e} lse {el:.3e}", flush=True)
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    assert eo <= tol and el <= tol, (eo, el)


BWD_CASES = _draw_cases(16, seed=20262)


@pytest.mark.parametrize("case", BWD_CASES, ids=lambda c: "c{}-B{}H{}T{}d{}-{}-x{:g}".format(*c))
def test_backward_random_shapes(case):
    i, B, H, T, d, sink, q_mult = case
    dtype = torch.float32 if i % 4 == 0 else torch.bfloat16
    q, k, v, k0, v0 = _inputs(B, H, T, d, sink, q_mult, dtype, seed=8000 + i)
    g = torch.Generator().manual_seed(9000 + i)
    do = torch.randn(B, H, T, d, generator=g).to(dtype)
    qg, kg, vg, k0g, v0g, dog = _gpu(q, k, v, k0, v0, do)
    o, lse = csa.csa_forward(qg, kg, vg, k0g, v0g)
    got = [None if x is None else x.float().cpu().double().numpy()
           for x in csa.csa_backward(qg, kg, vg, o, lse, dog, k0g, v0g)]
    torch.cuda.synchronize()
    ref = csa_backward_reference(q, k, v, do, k0, v0)
    bar = 1e-5 * (4.0 if q_mult > 1.0 else 1.0) if dtype == torch.float32 else 2e-2
    for name, x, r in zip(GRAD_NAMES, got, ref):
        if x is None or r is None:
            continue
        r = np.asarray(r, dtype=np.float64)
        assert np.all(np.isfinite(x)), name
        e = float(np.abs(x - r).max()) / max(1.0, float(np.abs(r).max()))
        print(f"[parity random] backward {case} {dtype} {name}: {e:.3e}", flush=True)
        assert e <= bar, (name, e)
