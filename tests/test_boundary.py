"""The C-ABI boundary on the CPU: the libraries load, export every declared
symbol, and validate arguments before touching the GPU.

No kernel is launched here: ``*_check`` entry points run the validation alone,
and every ``csa_forward`` call below is made with arguments the validation
rejects, so it returns before any HIP call.
"""

import ctypes
import os

import pytest

import continuous_softmax_attention_amd as csa
from continuous_softmax_attention_amd import build as csa_build

OK, INV, UNS = csa.CSA_OK, csa.CSA_ERR_INVALID_ARG, csa.CSA_ERR_UNSUPPORTED


@pytest.fixture(scope="module", autouse=True)
def built():
    missing = [n for n in csa_build.LIBS if not os.path.exists(csa.library_path(n))]
    if missing:  # the libraries cross-compile on a machine without a GPU
        csa_build.build()


@pytest.mark.parametrize("lib,header", [("libcsa.so", "csa.h"), ("libcsa_bench.so", "csa_bench.h")])
def test_exports_every_declared_symbol(lib, header):
    names = csa.header_functions(header)
    assert names, header
    handle = ctypes.CDLL(csa.library_path(lib))
    for n in names:
        assert hasattr(handle, n), f"{lib} does not export {n} declared in {header}"


def test_header_declares_the_entry_points():
    assert {"csa_forward", "csa_forward_check", "csa_forward_first_order", "csa_forward_first_order_check",
            "csa_forward_half_interval", "csa_forward_half_interval_check",
            "csa_decode", "csa_decode_check", "csa_decode_workspace_bytes",
            "csa_decode_noalloc", "csa_decode_noalloc_check",
            "csa_backward", "csa_backward_check", "csa_backward_workspace_bytes",
            "csa_status_string"} <= set(csa.header_functions("csa.h"))
    assert {"std_fwd", "std_fwd_check", "csa_probe"} <= set(csa.header_functions("csa_bench.h"))


def test_probe_rejects_bad_arguments_before_launching():
    # unknown kind, sizes out of range, null buffers: refused before any HIP call
    for kind, waves, iters, sink, cyc in ((-1, 64, 1, A, A), (13, 64, 1, A, A), (0, 0, 1, A, A),
                                          (0, 1 << 25, 1, A, A), (0, 64, 0, A, A), (0, 64, 1 << 31, A, A),
                                          (0, 64, 1, None, A), (0, 64, 1, A, None)):
        assert csa.csa_probe_raw(kind, waves, iters, sink, cyc) == INV


A = 0x10000  # fake, 16-byte-aligned addresses: validation never dereferences them
MB = 1 << 20


def _args(**kw):
    a = dict(q=A, k=A + 64 * MB, v=A + 128 * MB, k0=None, v0=None, out=A + 192 * MB, lse=A + 256 * MB,
             B=2, H=3, T=100, d=64, dtype=csa.CSA_BF16)
    a.update(kw)
    return a


def _check(**kw):
    a = _args(**kw)
    return csa.csa_forward_check(a["q"], a["k"], a["v"], a["k0"], a["v0"], a["out"], a["lse"],
                                 a["B"], a["H"], a["T"], a["d"], a["dtype"])


def test_valid_arguments_pass():
    assert _check() == OK
    assert _check(k0=A + 300 * MB, v0=A + 301 * MB) == OK
    assert _check(lse=None) == OK
    for d in (16, 64, 128):
        for dt in (csa.CSA_F32, csa.CSA_BF16):
            assert _check(d=d, dtype=dt) == OK
    assert _check(T=1, B=1, H=1) == OK


@pytest.mark.parametrize("field", ["q", "k", "v", "out"])
def test_null_required_pointer(field):
    assert _check(**{field: None}) == INV


@pytest.mark.parametrize("d", [0, 1, 8, 32, 96, 256])
def test_unsupported_head_dim(d):
    assert _check(d=d) == UNS


@pytest.mark.parametrize("dt", [-1, 2, 7])
def test_unsupported_dtype(dt):
    assert _check(dtype=dt) == UNS


@pytest.mark.parametrize("kw", [dict(B=0), dict(H=0), dict(T=0), dict(T=-5), dict(B=-1)])
def test_non_positive_sizes(kw):
    assert _check(**kw) == INV


@pytest.mark.parametrize("field,off", [("q", 8), ("k", 4), ("v", 2), ("out", 8), ("k0", 8), ("v0", 4), ("lse", 2)])
def test_misaligned(field, off):
    base = _args(k0=A + 300 * MB, v0=A + 301 * MB)
    assert _check(**{**base, field: base[field] + off}) == INV


def test_overlapping_output():
    assert _check(out=A + 64 * MB + 4096) == INV            # out inside k
    assert _check(lse=A + 1024) == INV                      # lse inside q
    assert _check(lse=A + 192 * MB + 16) == INV             # lse inside out
    assert _check(k0=A + 300 * MB, out=A + 300 * MB - 16) == INV  # out runs into k0


def test_size_overflow_rejected():
    assert _check(B=1 << 31) == INV
    assert _check(T=1 << 40) == INV


def test_forward_rejects_before_any_hip_call():
    # an invalid call must return its code without touching the (absent) GPU
    assert csa.csa_forward_raw(None, A, A, None, None, A + MB, None, 1, 1, 8, 64, csa.CSA_F32) == INV
    assert csa.csa_forward_raw(A, A + MB, A + 2 * MB, None, None, A + 3 * MB, None, 1, 1, 8, 48, csa.CSA_F32) == UNS
    assert csa.std_fwd_raw(A, A + MB, A + 2 * MB, A + 3 * MB, None, 1, 1, 0, 64, csa.CSA_F32) == INV


def test_std_check_matches_rules():
    assert csa.std_fwd_check(A, A + MB, A + 2 * MB, A + 3 * MB, None, 1, 2, 64, 128, csa.CSA_BF16) == OK
    assert csa.std_fwd_check(A, A + MB, A + 2 * MB, A + MB, None, 1, 2, 64, 128, csa.CSA_BF16) == INV
    assert csa.std_fwd_check(A, A + MB, A + 2 * MB, A + 3 * MB, None, 1, 2, 64, 100, csa.CSA_BF16) == UNS


def _check1(**kw):
    a = _args(**kw)
    return csa.csa_forward_first_order_check(a["q"], a["k"], a["v"], a["k0"], a["v0"], a["out"], a["lse"],
                                             a["B"], a["H"], a["T"], a["d"], a["dtype"])


def test_first_order_check_rules():
    # same validation as csa_forward, and bf16 only
    assert _check1() == OK
    assert _check1(k0=A + 300 * MB, v0=A + 301 * MB, lse=None) == OK
    for d in (16, 64, 128):
        assert _check1(d=d) == OK
        assert _check1(d=d, dtype=csa.CSA_F32) == UNS
    assert _check1(d=96) == UNS
    assert _check1(q=None) == INV
    assert _check1(T=0) == INV
    assert _check1(out=A + 64 * MB + 4096) == INV
    assert _check1(k0=A + 300 * MB + 8) == INV
    # the launching entry point rejects the same calls before any HIP call
    assert csa.csa_forward_first_order_raw(None, A, A, None, None, A + MB, None, 1, 1, 8, 64, csa.CSA_BF16) == INV
    assert csa.csa_forward_first_order_raw(A, A + MB, A + 2 * MB, None, None, A + 3 * MB, None, 1, 1, 8, 64,
                                           csa.CSA_F32) == UNS


def _checkh(**kw):
    a = _args(**kw)
    return csa.csa_forward_half_interval_check(a["q"], a["k"], a["v"], a["k0"], a["v0"], a["out"], a["lse"],
                                               a["B"], a["H"], a["T"], a["d"], a["dtype"])


def test_half_interval_check_rules():
    # same validation as csa_forward; bf16 only
    assert _checkh() == OK
    assert _checkh(k0=A + 300 * MB, v0=A + 301 * MB, lse=None) == OK
    for d in (16, 64, 128):
        assert _checkh(d=d) == OK
        assert _checkh(d=d, dtype=csa.CSA_F32) == UNS
    assert _checkh(d=32) == UNS
    assert _checkh(d=96) == UNS
    assert _checkh(q=None) == INV
    assert _checkh(T=0) == INV
    assert _checkh(out=A + 64 * MB + 4096) == INV
    assert _checkh(v0=A + 301 * MB + 4) == INV
    # the launching entry point rejects the same calls before any HIP call
    assert csa.csa_forward_half_interval_raw(None, A, A, None, None, A + MB, None, 1, 1, 8, 64, csa.CSA_BF16) == INV
    assert csa.csa_forward_half_interval_raw(A, A + MB, A + 2 * MB, None, None, A + 3 * MB, None, 1, 1, 8, 32,
                                             csa.CSA_BF16) == UNS


def _dargs(**kw):
    a = dict(q=A, k=A + 64 * MB, v=A + 128 * MB, k0=None, v0=None, out=A + 192 * MB, lse=A + 193 * MB,
             ws=A + 256 * MB, wsb=None, B=2, H=3, Tq=4, T=1000, d=128, dtype=csa.CSA_BF16)
    a.update(kw)
    if a["wsb"] is None:
        a["wsb"] = max(0, csa.csa_decode_workspace_bytes(a["B"], a["H"], a["Tq"], a["T"], a["d"]))
    return a


def _dcheck(**kw):
    a = _dargs(**kw)
    return csa.csa_decode_check(a["q"], a["k"], a["v"], a["k0"], a["v0"], a["out"], a["lse"], a["ws"], a["wsb"],
                                a["B"], a["H"], a["Tq"], a["T"], a["d"], a["dtype"])


def test_decode_workspace_size():
    # one (O[d], m, l) float32 record per (head, split, query), with room for one split per
    # 64 of the T + 1 positions (the call picks the split length)
    assert csa.csa_decode_workspace_bytes(2, 3, 4, 1000, 128) == 2 * 3 * 16 * 4 * 130 * 4
    assert csa.csa_decode_workspace_bytes(1, 1, 1, 255, 64) == 4 * 66 * 4
    assert csa.csa_decode_workspace_bytes(1, 1, 1, 256, 64) == 5 * 66 * 4
    for bad in (dict(Tq=0), dict(Tq=9), dict(Tq=5, T=4), dict(d=32), dict(B=0), dict(T=0)):
        a = dict(B=1, H=1, Tq=1, T=100, d=64)
        a.update(bad)
        assert csa.csa_decode_workspace_bytes(a["B"], a["H"], a["Tq"], a["T"], a["d"]) == -1


def test_decode_check_rules():
    assert _dcheck() == OK
    assert _dcheck(k0=A + 300 * MB, v0=A + 301 * MB, lse=None) == OK
    assert _dcheck(Tq=1, T=1) == OK
    for d in (16, 64, 128):
        for dt in (csa.CSA_F32, csa.CSA_BF16):
            assert _dcheck(d=d, dtype=dt) == OK
    assert _dcheck(d=96) == UNS
    assert _dcheck(dtype=5) == UNS
    for bad in (dict(Tq=0), dict(Tq=9), dict(Tq=8, T=7), dict(ws=None), dict(wsb=16), dict(q=None),
                dict(ws=A + 256 * MB + 8), dict(out=A + 192 * MB + 2), dict(lse=A + 193 * MB + 2),
                dict(ws=A + 64 * MB + 4096),                    # workspace inside k
                dict(out=A + 256 * MB + 64),                    # out inside the workspace
                dict(lse=A + 192 * MB + 16)):                   # lse inside out
        assert _dcheck(**bad) == INV, bad
    # the launching entry point rejects the same calls before any HIP call
    a = _dargs(Tq=9)
    assert csa.csa_decode_raw(a["q"], a["k"], a["v"], None, None, a["out"], None, a["ws"], 1 << 20,
                              a["B"], a["H"], 9, a["T"], a["d"], a["dtype"]) == INV


def _ncheck(**kw):
    a = _dargs(**kw)
    return csa.csa_decode_noalloc_check(a["q"], a["k"], a["v"], a["k0"], a["v0"], a["out"], a["lse"],
                                        a["B"], a["H"], a["Tq"], a["T"], a["d"], a["dtype"])


def test_decode_noalloc_check_rules():
    # csa_decode's rules without the workspace arguments, and a size limit: the workspace
    # csa_decode would need must fit the static scratch
    cap = csa.CSA_DECODE_NOALLOC_SCRATCH_BYTES
    assert cap == 64 << 20
    assert _ncheck() == OK
    assert _ncheck(k0=A + 300 * MB, v0=A + 301 * MB, lse=None) == OK
    for d in (16, 64, 128):
        for dt in (csa.CSA_F32, csa.CSA_BF16):
            assert _ncheck(d=d, dtype=dt) == OK
    assert _ncheck(d=96) == UNS
    for bad in (dict(Tq=0), dict(Tq=9), dict(q=None), dict(out=A + 192 * MB + 2), dict(lse=A + 192 * MB + 16)):
        assert _ncheck(**bad) == INV, bad
    # the largest T that fits, and one past it (B16 H8 Tq8 d128: 128 heads x 130 floats x 8 queries)
    rec = 16 * 8 * 8 * 130 * 4
    t_fit = (cap // rec) * 64 - 1
    assert csa.csa_decode_workspace_bytes(16, 8, 8, t_fit, 128) <= cap
    assert csa.csa_decode_workspace_bytes(16, 8, 8, t_fit + 1, 128) > cap
    big = dict(B=16, H=8, Tq=8, d=128, k=A + 1024 * MB, v=A + 2048 * MB, out=A + 4096 * MB, lse=A + 4097 * MB)
    assert _ncheck(T=t_fit, **big) == OK
    assert _ncheck(T=t_fit + 1, **big) == csa.CSA_ERR_SCRATCH_TOO_SMALL
    assert "scratch" in csa.status_string(csa.CSA_ERR_SCRATCH_TOO_SMALL)
    # the launching entry point returns the same codes before any HIP call
    a = _dargs(T=t_fit + 1, **big)
    assert csa.csa_decode_noalloc_raw(a["q"], a["k"], a["v"], None, None, a["out"], None, a["B"], a["H"], a["Tq"],
                                      a["T"], a["d"], a["dtype"]) == csa.CSA_ERR_SCRATCH_TOO_SMALL
    a = _dargs(Tq=9)
    assert csa.csa_decode_noalloc_raw(a["q"], a["k"], a["v"], None, None, a["out"], None, a["B"], a["H"], 9,
                                      a["T"], a["d"], a["dtype"]) == INV


def _bargs(**kw):
    big = 2 * 3 * 100 * 64 * 2  # B*H*T*d bf16 bytes of the default sizes (< 1 MB)
    a = dict(q=A, k=A + 1 * MB, v=A + 2 * MB, k0=None, v0=None, o=A + 3 * MB, lse=A + 4 * MB, dout=A + 5 * MB,
             dq=A + 6 * MB, dk=A + 7 * MB, dv=A + 8 * MB, dk0=A + 9 * MB, dv0=A + 10 * MB, ws=A + 11 * MB,
             wsb=1 << 20, B=2, H=3, T=100, d=64, dtype=csa.CSA_BF16)
    assert big < MB
    a.update(kw)
    return a


def _bcheck(**kw):
    a = _bargs(**kw)
    return csa.csa_backward_check(a["q"], a["k"], a["v"], a["k0"], a["v0"], a["o"], a["lse"], a["dout"],
                                  a["dq"], a["dk"], a["dv"], a["dk0"], a["dv0"], a["ws"], a["wsb"],
                                  a["B"], a["H"], a["T"], a["d"], a["dtype"])


def test_backward_workspace_size():
    # 512 zero bytes, then D_t, mu_t, dS_{t,0}, P_{t,0} as float32 per (b, h, t), then
    # 16 partial sums of dk_0 and dv_0 (2 x 128 float32) per (b, h); then, 256-byte aligned,
    # Q^T and dO^T per (b, h) as d rows of T rounded up to 128 bf16
    def expect(B, H, T, d):
        head = 512 + 16 * B * H * T + B * H * 16 * 1024
        return (head + 255) // 256 * 256 + 2 * B * H * d * ((T + 127) // 128 * 128) * 2
    assert csa.csa_backward_workspace_bytes(2, 3, 100, 64) == expect(2, 3, 100, 64)
    assert csa.csa_backward_workspace_bytes(4, 16, 4096, 128) == expect(4, 16, 4096, 128)
    assert expect(4, 16, 4096, 128) - 2 * 4 * 16 * 4096 * 128 * 2 < 6 << 20  # the rest is O(B H T)
    assert csa.csa_backward_workspace_bytes(1, 2, 100, 16) == expect(1, 2, 100, 16)
    for bad in (dict(d=32), dict(d=96), dict(B=0), dict(T=0), dict(H=-1)):
        a = dict(B=1, H=1, T=100, d=64)
        a.update(bad)
        assert csa.csa_backward_workspace_bytes(a["B"], a["H"], a["T"], a["d"]) == -1


def _ds_tiles_brute(T):
    # (query block of 128 rows, key tile of 64 keys) pairs with the key tile at or before the
    # tile holding the block's last row
    nqb = (T + 127) // 128
    return sum(min(qb * 128 + 127, T - 1) // 64 + 1 for qb in range(nqb))


@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 127, 128, 129, 191, 192, 193, 255, 256, 257, 1000, 4096, 16384])
def test_backward_fast_workspace_size(T):
    base = csa.csa_backward_workspace_bytes(2, 3, T, 128)
    fast = csa.csa_backward_workspace_bytes_fast(2, 3, T, 128)
    off = (base + 255) // 256 * 256
    assert fast == off + 2 * 3 * _ds_tiles_brute(T) * 8 * 64 * 32
    assert csa.csa_backward_workspace_bytes_fast(1, 1, T, 16) == -1


def test_backward_check_accepts_either_workspace():
    a = _bargs()
    lo = csa.csa_backward_workspace_bytes(a["B"], a["H"], a["T"], a["d"])
    hi = csa.csa_backward_workspace_bytes_fast(a["B"], a["H"], a["T"], a["d"])
    assert hi > lo
    assert _bcheck(wsb=lo) == OK and _bcheck(wsb=hi) == OK and _bcheck(wsb=lo - 16) == INV


def test_backward_check_rules():
    assert _bcheck() == OK
    assert _bcheck(d=128) == OK
    assert _bcheck(dk0=None, dv0=None) == OK
    assert _bcheck(k0=A + 12 * MB, v0=A + 13 * MB) == OK
    assert _bcheck(dtype=csa.CSA_F32) == OK    # float32: the VALU kernels
    assert _bcheck(d=16) == OK                 # bf16 at d = 16: the VALU kernels
    assert _bcheck(d=16, dtype=csa.CSA_F32) == OK
    assert _bcheck(d=32) == UNS
    assert _bcheck(d=96) == UNS
    assert _bcheck(dtype=7) == UNS
    for field in ("q", "k", "v", "o", "lse", "dout", "dq", "dk", "dv", "ws"):
        assert _bcheck(**{field: None}) == INV, field
    for bad in (dict(wsb=512 + 16 * 600 + 6 * 16 * 1024 - 1),   # one byte short
                dict(B=0), dict(T=0),
                dict(q=A + 8), dict(dq=A + 6 * MB + 8), dict(ws=A + 11 * MB + 4), dict(lse=A + 4 * MB + 2),
                dict(dk0=A + 9 * MB + 2),
                dict(dq=A + 64),                          # dq inside q
                dict(dk=A + 6 * MB + 16),                 # dk inside dq
                dict(ws=A + 5 * MB + 4096),               # workspace inside dout
                dict(dv0=A + 9 * MB + 16),                # dv0 inside dk0
                dict(dk0=A + 4 * MB)):                    # dk0 inside lse
        assert _bcheck(**bad) == INV, bad
    # the launching entry point rejects the same calls before any HIP call
    for bad, code in ((dict(d=32), UNS), (dict(dtype=7), UNS), (dict(q=A + 8), INV)):
        a = _bargs(**bad)
        assert csa.csa_backward_raw(a["q"], a["k"], a["v"], None, None, a["o"], a["lse"], a["dout"], a["dq"], a["dk"],
                                    a["dv"], None, None, a["ws"], a["wsb"], a["B"], a["H"], a["T"], a["d"],
                                    a["dtype"]) == code, bad


def test_status_strings():
    for s in (OK, INV, UNS, csa.CSA_ERR_HIP, csa.CSA_ERR_SCRATCH_TOO_SMALL, 99):
        assert isinstance(csa.status_string(s), str) and csa.status_string(s)


def test_python_binding_refuses_cpu_tensors():
    import torch

    q = torch.zeros(1, 1, 4, 16)
    with pytest.raises(ValueError):
        csa.csa_forward(q, q, q)
    with pytest.raises(ValueError):
        csa.std_fwd(q, q, q)
    with pytest.raises(ValueError):
        csa.csa_backward(q, q, q, q, torch.zeros(1, 1, 4), q)
