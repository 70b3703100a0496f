"""The entry points under HIP graph capture: csa_forward, csa_backward, csa_decode and
csa_decode_noalloc recorded into one graph (explicit outputs and workspaces, so nothing is
allocated or cleared by a memory API inside the capture), replayed several times with new
input values copied in by eager work between the replays, and every replay compared bit for
bit with the same calls run eagerly.  The library itself allocates nothing and clears its
workspaces with kernels, so its launches are what the graph holds.
"""

import math

import pytest
import torch

import continuous_softmax_attention_amd as csa

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
B, H, T, D, TQ = 2, 3, 300, 128, 4


def _fill(bufs, seed):
    g = torch.Generator().manual_seed(seed)
    for name, t in bufs.items():
        x = torch.randn(t.shape, generator=g)
        if name in ("q", "qd"):
            x = x / math.sqrt(D)
        t.copy_(x.to(t.dtype).to(DEV))  # eager host-to-device copies between replays


def test_graph_replays_match_eager_calls():
    bf = torch.bfloat16
    bufs = {
        "q": torch.empty(B, H, T, D, dtype=bf, device=DEV),
        "k": torch.empty(B, H, T, D, dtype=bf, device=DEV),
        "v": torch.empty(B, H, T, D, dtype=bf, device=DEV),
        "k0": torch.empty(B, H, D, dtype=bf, device=DEV),
        "v0": torch.empty(B, H, D, dtype=bf, device=DEV),
        "do": torch.empty(B, H, T, D, dtype=bf, device=DEV),
        "qd": torch.empty(B, H, TQ, D, dtype=bf, device=DEV),
    }
    q, k, v, k0, v0, do, qd = (bufs[n] for n in ("q", "k", "v", "k0", "v0", "do", "qd"))
    out = torch.empty_like(q)
    lse = torch.empty(B, H, T, dtype=torch.float32, device=DEV)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    ws_b = torch.empty(csa.csa_backward_workspace_bytes_fast(B, H, T, D), dtype=torch.uint8, device=DEV)
    dec_out = torch.empty_like(qd)
    dec_lse = torch.empty(B, H, TQ, dtype=torch.float32, device=DEV)
    ws_d = torch.empty(csa.csa_decode_workspace_bytes(B, H, TQ, T, D), dtype=torch.uint8, device=DEV)
    na_out = torch.empty_like(qd)
    na_lse = torch.empty_like(dec_lse)

    def calls():
        csa.csa_forward(q, k, v, k0, v0, out=out, lse=lse)
        grads = csa.csa_backward(q, k, v, out, lse, do, k0, v0, dq=dq, dk=dk, dv=dv, workspace=ws_b)
        csa.csa_decode(qd, k, v, k0, v0, out=dec_out, lse=dec_lse, workspace=ws_d)
        csa.csa_decode_noalloc(qd, k, v, k0, v0, out=na_out, lse=na_lse)
        return grads[3], grads[4]  # dk0, dv0 (allocated by the wrapper)

    _fill(bufs, seed=1)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm-up off the capture (library load, scratch set-up)
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        dk0, dv0 = calls()

    for rep in range(3):
        _fill(bufs, seed=100 + rep)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (out, lse, dq, dk, dv, dk0, dv0, dec_out, dec_lse, na_out, na_lse)]
        # the same calls eagerly, into fresh buffers
        o_e, l_e = csa.csa_forward(q, k, v, k0, v0)
        g_e = csa.csa_backward(q, k, v, o_e, l_e, do, k0, v0,
                               workspace=torch.empty_like(ws_b))
        d_e, dl_e = csa.csa_decode(qd, k, v, k0, v0, workspace=torch.empty_like(ws_d))
        n_e, nl_e = csa.csa_decode_noalloc(qd, k, v, k0, v0)
        torch.cuda.synchronize()
        want = [o_e, l_e, *g_e, d_e, dl_e, n_e, nl_e]
        names = ("out", "lse", "dq", "dk", "dv", "dk0", "dv0", "decode out", "decode lse",
                 "noalloc out", "noalloc lse")
        for name, a, b in zip(names, got, want):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager call"
        assert bool(torch.isfinite(got[0].float()).all()) and bool(torch.isfinite(got[2].float()).all())
        print(f"[graph] replay {rep}: all {len(names)} results identical to the eager calls", flush=True)
