"""GPU: the SIMD micro-benchmarks of libcsa_bench (csa_probe) run through the C-ABI.

Measurement code only (bench.py --probes and the MFMA-only ceiling in the bench line): every kind
launches, returns CSA_OK, raises the cycle counter above zero and leaves finite values in the
sink.  Rates are not checked here: they are what bench.py reports.
"""

import math

import pytest
import torch

import continuous_softmax_attention_amd as csa

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
KINDS = range(13)  # include/csa_bench.h: kinds 0 .. 12


@pytest.mark.parametrize("kind", KINDS)
def test_probe_kind_runs(kind):
    waves, iters = 64, 32
    sink = torch.full(((waves + 3) // 4,), float("nan"), dtype=torch.float32, device=DEV)
    cyc = torch.zeros(1, dtype=torch.int64, device=DEV)
    stream = torch.cuda.current_stream(DEV)
    print(f"[probe] kind {kind} waves {waves} iters {iters}", flush=True)
    st = csa.csa_probe_raw(kind, waves, iters, sink.data_ptr(), cyc.data_ptr(), stream.cuda_stream)
    assert st == 0, st
    torch.cuda.synchronize()
    assert int(cyc.item()) > 0
    vals = sink.cpu().tolist()
    assert all(math.isfinite(x) for x in vals), vals


def test_probe_cycles_grow_with_iterations():
    # the longest wave's loop cycles: a launch with 8x the iterations takes more of them
    sink = torch.zeros(16, dtype=torch.float32, device=DEV)
    cyc = torch.zeros(1, dtype=torch.int64, device=DEV)
    stream = torch.cuda.current_stream(DEV)
    got = []
    for iters in (256, 2048):
        cyc.zero_()
        assert csa.csa_probe_raw(1, 64, iters, sink.data_ptr(), cyc.data_ptr(), stream.cuda_stream) == 0
        torch.cuda.synchronize()
        got.append(int(cyc.item()))
    assert got[1] > 4 * got[0], got
