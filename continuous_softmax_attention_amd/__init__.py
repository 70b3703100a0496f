"""Causal continuous softmax attention forward for AMD MI355X (gfx950).

The compute path is the C-ABI library ``libcsa.so`` (hand-written HIP
kernels, include/csa.h); this package only marshals arguments to it.
``std_fwd`` (``libcsa_bench.so``) is standard softmax attention on the same
tiling, kept as a throughput comparison point.

Method: J. Su, "Continuous Softmax Attention" -- keys and values linearly
interpolated between positions with an extra k_0, v_0 (eq. (2)-(3)), reduced
to softmax attention with a neighbour-dependent correction (eq. (10)-(11)).
"""

from ._lib import (  # noqa: F401
    CSA_BF16,
    CSA_ERR_HIP,
    CSA_DECODE_NOALLOC_SCRATCH_BYTES,
    CSA_ERR_INVALID_ARG,
    CSA_ERR_SCRATCH_TOO_SMALL,
    CSA_ERR_UNSUPPORTED,
    CSA_F32,
    CSA_OK,
    CsaError,
    csa_backward,
    csa_backward_check,
    csa_backward_raw,
    csa_backward_workspace_bytes,
    csa_backward_workspace_bytes_fast,
    csa_backward_workspace_bytes_kept,
    csa_decode,
    csa_decode_check,
    csa_decode_noalloc,
    csa_decode_noalloc_check,
    csa_decode_noalloc_raw,
    csa_decode_raw,
    csa_decode_workspace_bytes,
    csa_forward,
    csa_forward_check,
    csa_forward_first_order,
    csa_forward_first_order_check,
    csa_forward_first_order_raw,
    csa_forward_half_interval,
    csa_forward_half_interval_check,
    csa_forward_half_interval_raw,
    csa_forward_raw,
    csa_probe_raw,
    header_functions,
    library_path,
    load,
    status_string,
    std_fwd,
    std_fwd_check,
    std_fwd_raw,
)
