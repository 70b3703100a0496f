"""csa_decode_noalloc (the decode entry point whose workspace is the library's static device
scratch) against csa_decode with a caller-provided workspace, through the C-ABI: two calls in
a row on one GPU, the second with smaller sizes (and another head dimension and dtype), then
the first again.  The two entry points run the same kernels with the same split plan, so
their outputs must agree bit for bit; the first case is also held to the bf16 bar (2e-2)
against the float64 CPU reference.
"""

import numpy as np
import pytest
import torch

import continuous_softmax_attention_amd as csa
from oracle import csa_reference
from workloads import make_decode_inputs

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")


def _gpu(*ts):
    return [None if t is None else t.to(DEV) for t in ts]


def _noalloc_raw(q, k, v, k0, v0):
    """One csa_decode_noalloc call through the C-ABI with preallocated outputs."""
    B, H, Tq, d = q.shape
    T = k.shape[2]
    out = torch.empty_like(q)
    lse = torch.empty((B, H, Tq), dtype=torch.float32, device=DEV)
    dt = csa.CSA_BF16 if q.dtype == torch.bfloat16 else csa.CSA_F32
    st = csa.csa_decode_noalloc_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                    0 if k0 is None else k0.data_ptr(), 0 if v0 is None else v0.data_ptr(),
                                    out.data_ptr(), lse.data_ptr(), B, H, Tq, T, d, dt,
                                    torch.cuda.current_stream(DEV).cuda_stream)
    assert st == csa.CSA_OK, csa.status_string(st)
    return out, lse


def _case(B, H, Tq, T, d, dtype, seed):
    q, k, v, k0, v0 = make_decode_inputs("decode", B=B, H=H, Tq=Tq, T=T, d=d, dtype=dtype, seed=seed,
                                         sink="random")
    return (q, k, v, k0, v0), _gpu(q, k, v, k0, v0)


def _compare(host, dev_args, tag):
    o_n, l_n = _noalloc_raw(*dev_args)
    o_w, l_w = csa.csa_decode(*dev_args)
    torch.cuda.synchronize()
    print(f"[no-alloc decode] {tag}: max|o_noalloc - o_decode| = {float((o_n.float() - o_w.float()).abs().max()):.3e}",
          flush=True)
    assert torch.equal(o_n, o_w) and torch.equal(l_n, l_w), tag
    return o_n, l_n


def test_noalloc_matches_decode_two_calls_second_smaller():
    # first call: B2 H4, 8 queries against 3000 cached positions, bf16 d128 (several splits)
    host1, dev1 = _case(2, 4, 8, 3000, 128, "bf16", seed=11)
    o1, l1 = _compare(host1, dev1, "B2 H4 Tq8 T3000 d128 bf16")
    q, k, v, k0, v0 = host1
    B, H, Tq, d = q.shape
    T = k.shape[2]
    qf = torch.zeros(B, H, T, d, dtype=torch.float64)
    qf[:, :, T - Tq:] = q.double()
    o_ref, l_ref = csa_reference(qf, k, v, k0, v0, rows=range(T - Tq, T))
    eo = float(np.abs(o1.float().cpu().double().numpy() - o_ref).max())
    el = float(np.abs(l1.cpu().double().numpy() - l_ref).max())
    print(f"[no-alloc decode] vs reference: max|o-ref| = {eo:.3e}  max|lse-ref| = {el:.3e}", flush=True)
    assert eo <= 2e-2 and el <= 2e-2
    # second call, smaller: B1 H2, 3 queries against 500 positions, float32 d64
    host2, dev2 = _case(1, 2, 3, 500, 64, "f32", seed=12)
    _compare(host2, dev2, "B1 H2 Tq3 T500 d64 f32")
    # the first sizes again: the scratch keeps the smaller call's records, none of which may leak
    o3, l3 = _compare(host1, dev1, "B2 H4 Tq8 T3000 d128 bf16 (again)")
    assert torch.equal(o3, o1) and torch.equal(l3, l1)


def test_noalloc_single_query_long_cache():
    # one query against 20000 positions: the longest splits of the plan
    host, dev = _case(1, 3, 1, 20000, 128, "bf16", seed=13)
    _compare(host, dev, "B1 H3 Tq1 T20000 d128 bf16")
