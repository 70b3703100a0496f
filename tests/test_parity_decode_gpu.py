"""GPU parity of csa_decode (few new queries against a key/value cache) against the
float64 CPU reference: the decode queries are the last Tq rows of the forward, so the
reference is csa_reference on a q whose last Tq rows are the decode queries, evaluated
on exactly those rows.

Tolerances (max abs error on o and lse): 1e-5 for float32, 2e-2 for bfloat16.
"""

import math

import numpy as np
import pytest
import torch

import continuous_softmax_attention_amd as csa
from oracle import csa_reference
from workloads import DECODE_WORKLOADS, make_decode_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TOL = {torch.float32: 1e-5, torch.bfloat16: 2e-2}


def _gpu(*ts):
    return [None if t is None else t.to(DEV) for t in ts]


def _run(q, k, v, k0=None, v0=None, workspace=None):
    o, lse = csa.csa_decode(*_gpu(q, k, v, k0, v0), workspace=workspace)
    torch.cuda.synchronize()
    return o.float().cpu().double().numpy(), lse.cpu().double().numpy()


def _reference(q, k, v, k0=None, v0=None):
    B, H, Tq, d = q.shape
    T = k.shape[2]
    qf = torch.zeros(B, H, T, d, dtype=torch.float64)
    qf[:, :, T - Tq:] = q.double()
    return csa_reference(qf, k, v, k0, v0, rows=range(T - Tq, T))


def _errs(o, lse, o_ref, l_ref):
    return float(np.abs(o - o_ref).max()), float(np.abs(lse - l_ref).max())


def _report(tag, eo, el):
    print(f"[parity decode] {tag}: max|o-ref| = {eo:.3e}  max|lse-ref| = {el:.3e}", flush=True)


CASES = [(T, Tq) for T in (1, 2, 3, 63, 64, 65, 511, 512, 513, 1023, 1025, 2000) for Tq in (1, 2, 5, 8) if Tq <= T]


@pytest.mark.parametrize("T,Tq", CASES)
def test_bf16_d128_random_sink(T, Tq):
    q, k, v, k0, v0 = make_decode_inputs("decode", B=1, H=2, Tq=Tq, T=T, seed=100 * T + Tq, sink="random")
    o, lse = _run(q, k, v, k0, v0)
    o_ref, l_ref = _reference(q, k, v, k0, v0)
    eo, el = _errs(o, lse, o_ref, l_ref)
    assert eo <= TOL[torch.bfloat16] and el <= TOL[torch.bfloat16], (eo, el)


@pytest.mark.parametrize("d", [16, 64, 128])
@pytest.mark.parametrize("T,Tq", [(1, 1), (65, 3), (600, 8), (1025, 1)])
def test_f32_all_head_dims(T, Tq, d):
    q, k, v, k0, v0 = make_decode_inputs("decode", B=2, H=1, Tq=Tq, T=T, d=d, dtype="f32", seed=7 * T + d,
                                         sink="random")
    o, lse = _run(q, k, v, k0, v0)
    o_ref, l_ref = _reference(q, k, v, k0, v0)
    eo, el = _errs(o, lse, o_ref, l_ref)
    assert eo <= TOL[torch.float32] and el <= TOL[torch.float32], (eo, el)


@pytest.mark.parametrize("d", [16, 64])
def test_bf16_small_head_dims_no_sink(d):
    q, k, v, _, _ = make_decode_inputs("decode", B=2, H=3, Tq=4, T=777, d=d, seed=d)
    o, lse = _run(q, k, v)
    o_ref, l_ref = _reference(q, k, v)
    eo, el = _errs(o, lse, o_ref, l_ref)
    assert eo <= TOL[torch.bfloat16] and el <= TOL[torch.bfloat16], (eo, el)


@pytest.mark.parametrize("sink", ["random", "zero"])
@pytest.mark.parametrize("T,Tq", [(1, 1), (8, 8), (64, 3), (65, 8), (129, 1), (1000, 5)])
def test_bf16_d64_lengths_and_queries(T, Tq, sink):
    q, k, v, k0, v0 = make_decode_inputs("decode", B=1, H=3, Tq=Tq, T=T, d=64, seed=31 * T + Tq, sink=sink)
    o, lse = _run(q, k, v, k0, v0)
    o_ref, l_ref = _reference(q, k, v, k0, v0)
    eo, el = _errs(o, lse, o_ref, l_ref)
    assert eo <= TOL[torch.bfloat16] and el <= TOL[torch.bfloat16], (eo, el)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("T,Tq", [(3000, 5), (3074, 5), (2049, 8), (2500, 1)])
def test_many_heads_every_head(T, Tq, d):
    # enough heads that a split spans several 64-key tiles; T = 3074 puts the last five
    # queries on both sides of a split boundary when splits are 128 (or 64) rows long
    q, k, v, k0, v0 = make_decode_inputs("decode", B=4, H=16, Tq=Tq, T=T, d=d, seed=T + d, sink="random")
    o, lse = _run(q, k, v, k0, v0)
    o_ref, l_ref = _reference(q, k, v, k0, v0)
    eo, el = _errs(o, lse, o_ref, l_ref)
    _report(f"B4 H16 T{T} Tq{Tq} d{d}", eo, el)
    assert eo <= TOL[torch.bfloat16] and el <= TOL[torch.bfloat16], (eo, el)


@pytest.mark.parametrize("Tq", [1, 3])
def test_long_cache_one_head(Tq):
    # one head of a 131072-position cache: hundreds of splits, merged 16 at a time
    q, k, v, k0, v0 = make_decode_inputs("decode", B=1, H=1, Tq=Tq, T=131072, seed=40 + Tq, sink="random")
    o, lse = _run(q, k, v, k0, v0)
    o_ref, l_ref = _reference(q, k, v, k0, v0)
    eo, el = _errs(o, lse, o_ref, l_ref)
    _report(f"one head T131072 Tq{Tq}", eo, el)
    assert eo <= TOL[torch.bfloat16] and el <= TOL[torch.bfloat16], (eo, el)


@pytest.mark.parametrize("q_mult", [4.0, 8.0, 12.0])
def test_large_logits_copied_sink(q_mult):
    q, k, v, k0, v0 = make_decode_inputs("decode", B=1, H=3, Tq=8, T=1500, seed=9, sink="copy")
    q = (q.float() * q_mult).bfloat16()
    o, lse = _run(q, k, v, k0, v0)
    o_ref, l_ref = _reference(q, k, v, k0, v0)
    eo, el = _errs(o, lse, o_ref, l_ref)
    _report(f"large logits x{q_mult}", eo, el)
    assert eo <= TOL[torch.bfloat16] and el <= TOL[torch.bfloat16]


def test_trapezoid_closed_form():
    # q = 0: weights 1/2, 1, ..., 1, 1/2 over positions 0..t and lse = ln t
    T, Tq, d = 700, 3, 64
    _, k, v, k0, v0 = make_decode_inputs("decode", B=1, H=1, Tq=Tq, T=T, d=d, dtype="f32", seed=2, sink="random")
    q = torch.zeros(1, 1, Tq, d)
    o, lse = _run(q, k, v, k0, v0)
    vh = torch.cat([v0[0, 0][None], v[0, 0]]).double().numpy()
    for j in range(Tq):
        t = T - Tq + 1 + j
        expect = (0.5 * vh[0] + vh[1:t].sum(0) + 0.5 * vh[t]) / t
        assert np.abs(o[0, 0, j] - expect).max() < 1e-5
        assert abs(lse[0, 0, j] - math.log(t)) < 1e-5


def test_matches_the_forward_rows():
    # the decode of the last Tq queries equals those rows of csa_forward
    T, Tq, d = 1000, 8, 128
    q, k, v, k0, v0 = make_decode_inputs("decode", B=2, H=2, Tq=Tq, T=T, seed=11, sink="random")
    qf = torch.randn(2, 2, T, d).bfloat16()
    qf[:, :, T - Tq:] = q
    of, lf = csa.csa_forward(*_gpu(qf, k, v, k0, v0))
    od, ld = csa.csa_decode(*_gpu(q, k, v, k0, v0))
    torch.cuda.synchronize()
    assert float((of[:, :, T - Tq:].float() - od.float()).abs().max()) <= 2e-2
    assert float((lf[:, :, T - Tq:] - ld).abs().max()) <= 2e-2


def test_workspace_reused_across_calls():
    # a second call with a smaller cache reuses (and fully overwrites) the workspace it needs
    q1, k1, v1, a1, b1 = make_decode_inputs("decode", B=2, H=2, Tq=4, T=1500, seed=12, sink="random")
    q2, k2, v2, a2, b2 = make_decode_inputs("decode", B=2, H=2, Tq=2, T=300, seed=13, sink="random")
    ws = torch.empty(csa.csa_decode_workspace_bytes(2, 2, 4, 1500, 128), dtype=torch.uint8, device=DEV)
    for (q, k, v, k0, v0) in ((q1, k1, v1, a1, b1), (q2, k2, v2, a2, b2)):
        o, lse = _run(q, k, v, k0, v0, workspace=ws)
        o_ref, l_ref = _reference(q, k, v, k0, v0)
        eo, el = _errs(o, lse, o_ref, l_ref)
        assert eo <= TOL[torch.bfloat16] and el <= TOL[torch.bfloat16]


def test_invalid_arguments_raise():
    q, k, v, _, _ = make_decode_inputs("decode", B=1, H=1, Tq=8, T=100, seed=1)
    with pytest.raises(csa.CsaError):
        csa.csa_decode(*_gpu(q, k[:, :, :5].contiguous(), v[:, :, :5].contiguous()))  # Tq > T
    with pytest.raises(csa.CsaError):
        csa.csa_decode(*_gpu(q, k, v), workspace=torch.empty(16, dtype=torch.uint8, device=DEV))


@pytest.mark.parametrize("name", ["decode", "decode_spec"])
def test_decode_workloads_sampled_heads(name):
    w = DECODE_WORKLOADS[name]
    print(f"[parity decode] {name}: generating B{w.B} H{w.H} Tq{w.Tq} T{w.T} d{w.d} {w.dtype}", flush=True)
    q, k, v, k0, v0 = make_decode_inputs(w)
    o_dev, lse_dev = csa.csa_decode(*_gpu(q, k, v, k0, v0))
    torch.cuda.synchronize()
    # every head: finite, and each output a convex combination of the values
    assert bool(torch.isfinite(lse_dev).all()) and bool(torch.isfinite(o_dev.float()).all())
    assert float(o_dev.float().abs().max()) <= float(v.float().abs().max()) * (1 + 1e-2)
    # eight seeded heads against the reference, every query
    rng = np.random.default_rng(w.seed)
    heads = rng.choice(w.B * w.H, size=8, replace=False)
    worst_o = worst_l = 0.0
    for bh in heads:
        b, h = int(bh) // w.H, int(bh) % w.H
        sl = (slice(b, b + 1), slice(h, h + 1))
        o_ref, l_ref = _reference(q[sl], k[sl], v[sl])
        eo, el = _errs(o_dev[sl].float().cpu().double().numpy(), lse_dev[sl].cpu().double().numpy(), o_ref, l_ref)
        worst_o, worst_l = max(worst_o, eo), max(worst_l, el)
    _report(f"{name} (8 of {w.B * w.H} heads x {w.Tq} queries)", worst_o, worst_l)
    assert worst_o <= TOL[torch.bfloat16] and worst_l <= TOL[torch.bfloat16]
