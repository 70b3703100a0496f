"""Compile the HIP libraries in-tree for gfx950 (MI355X).

    python -m continuous_softmax_attention_amd.build

produces ``libcsa.so`` (csa_forward) and ``libcsa_bench.so`` (std_fwd, the
standard-attention comparator on the same tiling) next to this file.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")

LIBS = {
    "libcsa.so": "csa_api.hip",
    "libcsa_bench.so": "std_api.hip",
}

# -packed-fp32-ops: no v_pk_{add,mul,fma}_f32 in the generated code.
# -fno-honor-nans: without it every fmaxf on a value the compiler cannot prove canonical
# (MFMA results, cross-lane moves) gets an extra v_max_f32 x, x to quiet signalling NaNs.
# One NaN does arise by design: where two neighbouring logits are exactly equal the
# reciprocal of their difference is infinite and the closed-form edge terms are 0 * inf;
# a select on |difference| < threshold (compare, then v_cndmask) always discards that value
# for the series form, and no NaN is compared, maximised or stored.  Exactly-equal-logit
# cases run through the kernels in the tests (q = 0: the trapezoid closed form, fp32 and bf16).
HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fno-honor-nans",
    "-fPIC",
    "-shared",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I" + INCLUDE,
    "-I" + CSRC,
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the HIP libraries cannot be built")
    return path


def build(verbose: bool = False) -> list[str]:
    """Build every library (always recompiles); returns the output paths."""
    cc = hipcc()
    procs = []
    for lib, src in LIBS.items():
        out = os.path.join(PKG, lib)
        tmp = out + ".tmp"
        cmd = [cc, *HIPCC_FLAGS, os.path.join(CSRC, src), "-o", tmp]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((out, tmp, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)))
    outs = []
    failed = []
    for out, tmp, p in procs:
        log, _ = p.communicate()
        log = "\n".join(ln for ln in log.splitlines() if "packed-fp32-ops' is not a recognized feature" not in ln)
        if p.returncode != 0:
            failed.append(f"{os.path.basename(out)}:\n{log}")
            continue
        if verbose and log.strip():
            print(log)
        os.replace(tmp, out)
        outs.append(out)
    if failed:
        raise RuntimeError("HIP build failed:\n" + "\n".join(failed))
    return outs


if __name__ == "__main__":
    for p in build(verbose="-v" in sys.argv):
        print("built", p)
