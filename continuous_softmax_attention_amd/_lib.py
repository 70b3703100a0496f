"""ctypes binding of the C-ABI in include/csa.h and include/csa_bench.h.

Argument marshalling only: tensors are checked and turned into device
pointers, the call runs on the caller's (or torch's current) HIP stream, and
a non-zero status becomes a ``CsaError``.  All arithmetic happens in the HIP
kernels; if the libraries are missing the calls raise instead of falling back
to anything else.
"""

from __future__ import annotations

import ctypes
import os
import re

PKG = os.path.dirname(os.path.abspath(__file__))
INCLUDE = os.path.join(os.path.dirname(PKG), "include")

CSA_F32 = 0
CSA_BF16 = 1
CSA_OK = 0
CSA_ERR_INVALID_ARG = 1
CSA_ERR_UNSUPPORTED = 2
CSA_ERR_HIP = 3
CSA_ERR_SCRATCH_TOO_SMALL = 4
CSA_DECODE_NOALLOC_SCRATCH_BYTES = 64 << 20  # the static scratch of csa_decode_noalloc (include/csa.h)


class CsaError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what} failed with status {status}: {status_string(status)}")


_vp = ctypes.c_void_p
_i64 = ctypes.c_int64
_SIGS = {
    "csa_forward": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, ctypes.c_int, _vp]),
    "csa_forward_check": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, ctypes.c_int]),
    "csa_forward_first_order": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, ctypes.c_int, _vp]),
    "csa_forward_first_order_check": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, ctypes.c_int]),
    "csa_forward_half_interval": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, ctypes.c_int, _vp]),
    "csa_forward_half_interval_check": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, ctypes.c_int]),
    "csa_decode": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64,
                                  ctypes.c_int, _vp]),
    "csa_decode_check": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, _i64, _i64,
                                        ctypes.c_int]),
    "csa_decode_workspace_bytes": (_i64, [_i64, _i64, _i64, _i64, _i64]),
    "csa_decode_noalloc": (ctypes.c_int, [_vp] * 7 + [_i64] * 5 + [ctypes.c_int, _vp]),
    "csa_decode_noalloc_check": (ctypes.c_int, [_vp] * 7 + [_i64] * 5 + [ctypes.c_int]),
    "csa_backward": (ctypes.c_int, [_vp] * 14 + [_i64] * 5 + [ctypes.c_int, _vp]),
    "csa_backward_check": (ctypes.c_int, [_vp] * 14 + [_i64] * 5 + [ctypes.c_int]),
    "csa_backward_workspace_bytes": (_i64, [_i64] * 4),
    "csa_backward_workspace_bytes_fast": (_i64, [_i64] * 4),
    "csa_backward_workspace_bytes_kept": (_i64, [_i64] * 5),
    "csa_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "std_fwd": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, ctypes.c_int, _vp]),
    "std_fwd_check": (ctypes.c_int, [_vp, _vp, _vp, _vp, _vp, _i64, _i64, _i64, _i64, ctypes.c_int]),
    "csa_probe": (ctypes.c_int, [ctypes.c_int, _i64, _i64, _vp, _vp, _vp]),
}

_handles: dict[str, ctypes.CDLL] = {}


def library_path(name: str = "libcsa.so") -> str:
    return os.path.join(PKG, name)


def load(name: str = "libcsa.so") -> ctypes.CDLL:
    """Load an in-tree library (built by ``continuous_softmax_attention_amd.build``)."""
    if name in _handles:
        return _handles[name]
    path = library_path(name)
    if not os.path.exists(path):
        raise RuntimeError(
            f"{path} is not built; run `python -m continuous_softmax_attention_amd.build` "
            "(the HIP path has no fallback)")
    lib = ctypes.CDLL(path)
    for sym, (res, args) in _SIGS.items():
        if hasattr(lib, sym):
            fn = getattr(lib, sym)
            fn.restype = res
            fn.argtypes = args
    _handles[name] = lib
    return lib


def header_functions(header: str) -> list[str]:
    """Names of the functions a public header declares."""
    with open(os.path.join(INCLUDE, header)) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)


def status_string(status: int) -> str:
    try:
        return load().csa_status_string(int(status)).decode()
    except Exception:  # library missing: still give a readable message
        return {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "HIP launch failure",
                4: "sizes exceed the static decode scratch"}.get(status, "unknown")


# ---------------------------------------------------------------- raw pointers

def csa_forward_raw(q, k, v, k0, v0, out, lse, B, H, T, d, dtype, stream=0) -> int:
    """Direct C-ABI call with integer device pointers; returns the status code."""
    return load().csa_forward(q, k, v, k0 or None, v0 or None, out, lse or None, B, H, T, d, dtype, stream or None)


def csa_forward_first_order_raw(q, k, v, k0, v0, out, lse, B, H, T, d, dtype, stream=0) -> int:
    return load().csa_forward_first_order(q, k, v, k0 or None, v0 or None, out, lse or None, B, H, T, d, dtype,
                                          stream or None)


def csa_forward_half_interval_raw(q, k, v, k0, v0, out, lse, B, H, T, d, dtype, stream=0) -> int:
    return load().csa_forward_half_interval(q, k, v, k0 or None, v0 or None, out, lse or None, B, H, T, d, dtype,
                                            stream or None)


def csa_decode_raw(q, k, v, k0, v0, out, lse, ws, ws_bytes, B, H, Tq, T, d, dtype, stream=0) -> int:
    return load().csa_decode(q, k, v, k0 or None, v0 or None, out, lse or None, ws, ws_bytes, B, H, Tq, T, d, dtype,
                             stream or None)


def csa_decode_check(q, k, v, k0, v0, out, lse, ws, ws_bytes, B, H, Tq, T, d, dtype) -> int:
    return load().csa_decode_check(q, k, v, k0, v0, out, lse, ws, ws_bytes, B, H, Tq, T, d, dtype)


def csa_decode_noalloc_raw(q, k, v, k0, v0, out, lse, B, H, Tq, T, d, dtype, stream=0) -> int:
    return load().csa_decode_noalloc(q, k, v, k0 or None, v0 or None, out, lse or None, B, H, Tq, T, d, dtype,
                                     stream or None)


def csa_decode_noalloc_check(q, k, v, k0, v0, out, lse, B, H, Tq, T, d, dtype) -> int:
    return load().csa_decode_noalloc_check(q, k, v, k0, v0, out, lse, B, H, Tq, T, d, dtype)


def csa_decode_workspace_bytes(B, H, Tq, T, d) -> int:
    """Bytes of workspace csa_decode needs (-1 for invalid sizes)."""
    return int(load().csa_decode_workspace_bytes(B, H, Tq, T, d))


def csa_backward_raw(q, k, v, k0, v0, o, lse, dout, dq, dk, dv, dk0, dv0, ws, ws_bytes, B, H, T, d, dtype,
                     stream=0) -> int:
    return load().csa_backward(q, k, v, k0 or None, v0 or None, o, lse, dout, dq, dk, dv, dk0 or None,
                               dv0 or None, ws, ws_bytes, B, H, T, d, dtype, stream)


def csa_backward_check(q, k, v, k0, v0, o, lse, dout, dq, dk, dv, dk0, dv0, ws, ws_bytes, B, H, T, d,
                       dtype) -> int:
    return load().csa_backward_check(q, k, v, k0, v0, o, lse, dout, dq, dk, dv, dk0, dv0, ws, ws_bytes,
                                     B, H, T, d, dtype)


def csa_backward_workspace_bytes(B, H, T, d) -> int:
    """Bytes of workspace csa_backward needs (-1 for invalid sizes)."""
    return int(load().csa_backward_workspace_bytes(B, H, T, d))


def csa_backward_workspace_bytes_kept(B, H, T, d, heads_per_group) -> int:
    """Bytes with which csa_backward keeps dS for heads_per_group heads at a time (-1: invalid)."""
    return int(load().csa_backward_workspace_bytes_kept(B, H, T, d, heads_per_group))


# default budget of the kept-dS workspace the binding allocates (dS grows as T^2 per head)
KEPT_DS_BUDGET_BYTES = 2 << 30


def csa_backward_workspace_bytes_fast(B, H, T, d) -> int:
    """Bytes of workspace with which csa_backward keeps dS between its kernels (-1 for invalid
    sizes); grows as T^2."""
    return int(load().csa_backward_workspace_bytes_fast(B, H, T, d))


def std_fwd_raw(q, k, v, out, lse, B, H, T, d, dtype, stream=0) -> int:
    return load("libcsa_bench.so").std_fwd(q, k, v, out, lse or None, B, H, T, d, dtype, stream or None)


def csa_forward_check(q, k, v, k0, v0, out, lse, B, H, T, d, dtype) -> int:
    return load().csa_forward_check(q, k, v, k0, v0, out, lse, B, H, T, d, dtype)


def csa_forward_first_order_check(q, k, v, k0, v0, out, lse, B, H, T, d, dtype) -> int:
    return load().csa_forward_first_order_check(q, k, v, k0, v0, out, lse, B, H, T, d, dtype)


def csa_forward_half_interval_check(q, k, v, k0, v0, out, lse, B, H, T, d, dtype) -> int:
    return load().csa_forward_half_interval_check(q, k, v, k0, v0, out, lse, B, H, T, d, dtype)


def std_fwd_check(q, k, v, out, lse, B, H, T, d, dtype) -> int:
    return load("libcsa_bench.so").std_fwd_check(q, k, v, out, lse, B, H, T, d, dtype)


def csa_probe_raw(kind, waves, iters, sink, cycles, stream=0) -> int:
    """One SIMD micro-benchmark launch (include/csa_bench.h): kind 0 MFMA, 1 fp32 FMA,
    2 exp, 3 rcp, 4 MFMA and FMA together; sink and cycles are device addresses."""
    return load("libcsa_bench.so").csa_probe(kind, waves, iters, sink, cycles, stream or None)


# ---------------------------------------------------------------- torch tensors

def _dtype_code(t):
    import torch

    if t.dtype == torch.float32:
        return CSA_F32
    if t.dtype == torch.bfloat16:
        return CSA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}; expected float32 or bfloat16")


def _check(name, t, shape, dtype, device):
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream_handle(stream, device):
    import torch

    if stream is None:
        stream = torch.cuda.current_stream(device)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def csa_forward(q, k, v, k0=None, v0=None, *, out=None, lse=None, return_lse=True, stream=None):
    """Continuous softmax attention forward (causal) through libcsa.

    q, k, v: [B, H, T, d] float32 or bfloat16 device tensors (same dtype);
    k0, v0: [B, H, d] or None (zeros).  Returns (out, lse) -- lse is float32
    [B, H, T] (None when return_lse is False and no lse buffer is given).
    """
    return _csa_call("csa_forward", q, k, v, k0, v0, out, lse, return_lse, stream)


def csa_forward_first_order(q, k, v, k0=None, v0=None, *, out=None, lse=None, return_lse=True, stream=None):
    """The first-order variant (b as the second difference of the logits, eq. (13)) through
    libcsa; bfloat16 only.  Same arguments and results as csa_forward."""
    return _csa_call("csa_forward_first_order", q, k, v, k0, v0, out, lse, return_lse, stream)


def csa_forward_half_interval(q, k, v, k0=None, v0=None, *, out=None, lse=None, return_lse=True, stream=None):
    """The interval variant [1/2, t + 1/2] (the original paper's choice, Problem Statement) through
    libcsa; bfloat16, d in {64, 128}.  Same arguments and results as csa_forward."""
    return _csa_call("csa_forward_half_interval", q, k, v, k0, v0, out, lse, return_lse, stream)


def _csa_call(symbol, q, k, v, k0, v0, out, lse, return_lse, stream):
    import torch

    if q.dim() != 4:
        raise ValueError("q must be [B, H, T, d]")
    B, H, T, d = q.shape
    dt = q.dtype
    dev = q.device
    if dev.type != "cuda":
        raise ValueError(f"{symbol} runs on the GPU only; inputs must be device tensors")
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(name, t, (B, H, T, d), dt, dev)
    for name, t in (("k0", k0), ("v0", v0)):
        if t is not None:
            _check(name, t, (B, H, d), dt, dev)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check("out", out, (B, H, T, d), dt, dev)
    if lse is None and return_lse:
        lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    elif lse is not None:
        _check("lse", lse, (B, H, T), torch.float32, dev)
    st = getattr(load(), symbol)(
        q.data_ptr(), k.data_ptr(), v.data_ptr(),
        k0.data_ptr() if k0 is not None else None, v0.data_ptr() if v0 is not None else None,
        out.data_ptr(), lse.data_ptr() if lse is not None else None,
        B, H, T, d, _dtype_code(q), _stream_handle(stream, dev))
    if st != CSA_OK:
        raise CsaError(st, symbol)
    return out, lse


def std_fwd(q, k, v, *, out=None, lse=None, return_lse=True, stream=None):
    """Standard causal softmax attention (the comparator) through libcsa_bench."""
    import torch

    B, H, T, d = q.shape
    dt, dev = q.dtype, q.device
    if dev.type != "cuda":
        raise ValueError("std_fwd runs on the GPU only; inputs must be device tensors")
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check(name, t, (B, H, T, d), dt, dev)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check("out", out, (B, H, T, d), dt, dev)
    if lse is None and return_lse:
        lse = torch.empty((B, H, T), dtype=torch.float32, device=dev)
    elif lse is not None:
        _check("lse", lse, (B, H, T), torch.float32, dev)
    st = load("libcsa_bench.so").std_fwd(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
        lse.data_ptr() if lse is not None else None, B, H, T, d, _dtype_code(q), _stream_handle(stream, dev))
    if st != CSA_OK:
        raise CsaError(st, "std_fwd")
    return out, lse


def _decode_args(q, k, v, k0, v0, out, lse, return_lse, what):
    import torch

    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, H, Tq, d] and k, v [B, H, T, d]")
    B, H, Tq, d = q.shape
    T = k.shape[2]
    dt, dev = q.dtype, q.device
    if dev.type != "cuda":
        raise ValueError(f"{what} runs on the GPU only; inputs must be device tensors")
    _check("q", q, (B, H, Tq, d), dt, dev)
    for name, t in (("k", k), ("v", v)):
        _check(name, t, (B, H, T, d), dt, dev)
    for name, t in (("k0", k0), ("v0", v0)):
        if t is not None:
            _check(name, t, (B, H, d), dt, dev)
    if out is None:
        out = torch.empty_like(q)
    else:
        _check("out", out, (B, H, Tq, d), dt, dev)
    if lse is None and return_lse:
        lse = torch.empty((B, H, Tq), dtype=torch.float32, device=dev)
    elif lse is not None:
        _check("lse", lse, (B, H, Tq), torch.float32, dev)
    return B, H, Tq, T, d, out, lse


def csa_decode(q, k, v, k0=None, v0=None, *, out=None, lse=None, return_lse=True, workspace=None, stream=None):
    """Forward of a few new queries against a key/value cache through libcsa.

    q: [B, H, Tq, d] (the queries at positions T-Tq+1..T, 1 <= Tq <= 8); k, v: [B, H, T, d];
    k0, v0: [B, H, d] or None.  ``workspace`` is a device tensor of at least
    csa_decode_workspace_bytes(B, H, Tq, T, d) bytes (allocated here when None).
    Returns (out [B, H, Tq, d], lse [B, H, Tq] float32 or None).
    """
    import torch

    B, H, Tq, T, d, out, lse = _decode_args(q, k, v, k0, v0, out, lse, return_lse, "csa_decode")
    need = csa_decode_workspace_bytes(B, H, Tq, T, d)
    if need < 0:
        raise CsaError(CSA_ERR_INVALID_ARG, "csa_decode (sizes)")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    st = load().csa_decode(
        q.data_ptr(), k.data_ptr(), v.data_ptr(),
        k0.data_ptr() if k0 is not None else None, v0.data_ptr() if v0 is not None else None,
        out.data_ptr(), lse.data_ptr() if lse is not None else None,
        workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        B, H, Tq, T, d, _dtype_code(q), _stream_handle(stream, q.device))
    if st != CSA_OK:
        raise CsaError(st, "csa_decode")
    return out, lse


def csa_decode_noalloc(q, k, v, k0=None, v0=None, *, out=None, lse=None, return_lse=True, stream=None):
    """csa_decode with the library's static device scratch as its workspace (the entry point
    allocates nothing; pass ``out`` and ``lse`` to keep this wrapper from allocating them).
    Calls on one GPU share that scratch: calls that can overlap must be ordered by the caller.
    """
    B, H, Tq, T, d, out, lse = _decode_args(q, k, v, k0, v0, out, lse, return_lse, "csa_decode_noalloc")
    st = load().csa_decode_noalloc(
        q.data_ptr(), k.data_ptr(), v.data_ptr(),
        k0.data_ptr() if k0 is not None else None, v0.data_ptr() if v0 is not None else None,
        out.data_ptr(), lse.data_ptr() if lse is not None else None,
        B, H, Tq, T, d, _dtype_code(q), _stream_handle(stream, q.device))
    if st != CSA_OK:
        raise CsaError(st, "csa_decode_noalloc")
    return out, lse


def csa_backward(q, k, v, o, lse, dout, k0=None, v0=None, *, sink_grads=True, dq=None, dk=None, dv=None,
                 workspace=None, stream=None):
    """Gradients of the causal CSA forward through libcsa (bfloat16 or float32, d in {16, 64, 128}).

    q, k, v, o (the forward's output), dout: [B, H, T, d] device tensors of one dtype; lse: the
    forward's [B, H, T] float32 lse; k0, v0: [B, H, d] or None (zeros).  Returns
    (dq, dk, dv, dk0, dv0) -- dk0 and dv0 ([B, H, d]) are None when sink_grads is False.
    ``workspace``: a device tensor of at least csa_backward_workspace_bytes(B, H, T, d) bytes;
    with csa_backward_workspace_bytes_fast(B, H, T, d) bytes or more dS is computed once
    (allocated here when None: the larger size while it is at most a quarter of the free device
    memory, else the smaller).
    """
    import torch

    if q.dim() != 4:
        raise ValueError("q must be [B, H, T, d]")
    B, H, T, d = q.shape
    dt, dev = q.dtype, q.device
    if dev.type != "cuda":
        raise ValueError("csa_backward runs on the GPU only; inputs must be device tensors")
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout)):
        _check(name, t, (B, H, T, d), dt, dev)
    _check("lse", lse, (B, H, T), torch.float32, dev)
    for name, t in (("k0", k0), ("v0", v0)):
        if t is not None:
            _check(name, t, (B, H, d), dt, dev)
    need = csa_backward_workspace_bytes(B, H, T, d)
    if need < 0:
        raise CsaError(CSA_ERR_UNSUPPORTED if d not in (16, 64, 128) else CSA_ERR_INVALID_ARG, "csa_backward (sizes)")
    if workspace is None:
        # dS kept for as many heads at a time as fit min(2 GiB, a quarter of the free device
        # memory) -- it grows as T^2 per head -- else the O(B H T) workspace (dS recomputed);
        # the results are identical either way
        free, _ = torch.cuda.mem_get_info(dev)
        budget = min(KEPT_DS_BUDGET_BYTES, free // 4)
        one = csa_backward_workspace_bytes_kept(B, H, T, d, 1) if dt == torch.bfloat16 else -1
        size = need
        if 0 < one <= budget:
            per_head = csa_backward_workspace_bytes_kept(B, H, T, d, 2) - one if B * H > 1 else 0
            heads = B * H if per_head == 0 else min(B * H, 1 + (budget - one) // per_head)
            size = csa_backward_workspace_bytes_kept(B, H, T, d, heads)
        workspace = torch.empty(size, dtype=torch.uint8, device=dev)
    grads = []
    for name, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        if t is None:
            t = torch.empty_like(q)
        else:
            _check(name, t, (B, H, T, d), dt, dev)
        grads.append(t)
    dk0 = torch.empty((B, H, d), dtype=dt, device=dev) if sink_grads else None
    dv0 = torch.empty((B, H, d), dtype=dt, device=dev) if sink_grads else None
    st = load().csa_backward(
        q.data_ptr(), k.data_ptr(), v.data_ptr(),
        k0.data_ptr() if k0 is not None else None, v0.data_ptr() if v0 is not None else None,
        o.data_ptr(), lse.data_ptr(), dout.data_ptr(),
        grads[0].data_ptr(), grads[1].data_ptr(), grads[2].data_ptr(),
        dk0.data_ptr() if dk0 is not None else None, dv0.data_ptr() if dv0 is not None else None,
        workspace.data_ptr(), workspace.numel() * workspace.element_size(),
        B, H, T, d, _dtype_code(q), _stream_handle(stream, dev))
    if st != CSA_OK:
        raise CsaError(st, "csa_backward")
    return grads[0], grads[1], grads[2], dk0, dv0
