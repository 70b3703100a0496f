"""Throughput of the causal continuous-softmax-attention forward on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload lm] [--no-cpu-baseline]

One step = one csa_forward call over the whole workload (every query row of
every batch and head); inputs are resident in HBM before the timed region.  Each
leg's untimed warm-up is W calls and at least --settle-s seconds of calls (default
0.3 s): the GPU's clocks take ~50-100 ms of sustained load to ramp up.
Metric: TFLOP/s counting 4 T^2 d / 2 FLOP per (batch, head) -- QK^T plus PV
over the causal half, the convention under which the pages call continuous
and standard attention "essentially the same" in FLOPs -- and the fraction of
the MI355X dense bf16 MFMA peak.  The standard-attention kernel built on the
same tiling (std_fwd) runs on the same inputs for the ratio, and so does the
first-order variant (csa_forward_first_order, b as the second difference of the
logits) -- the same kernel without the exact correction weights -- and the interval
variant [1/2, t + 1/2] (csa_forward_half_interval), under the same FLOP count.  The ``decode``
object times csa_decode (a few new queries against a key/value cache, bound by HBM
bandwidth) on the decode workloads, and ``backward`` times csa_backward (the gradients
dq, dk, dv, dk0, dv0 from the forward's o and lse and a seeded dO) on the same workload,
counting 2.5 times the forward's FLOP (five matrix products of the forward's size against
its two: S recomputed, dP, dV, dK, dQ).

Prints ONE JSON line.  `cpu_baseline` times the float64 CPU reference on a
bounded sample of query rows of the same workload (process pool over host
cores), scaled to TFLOP/s by the same FLOP convention.  `mfma_ceiling` runs an
MFMA-only micro-benchmark (csa_probe in libcsa_bench) on the same GPU: the bf16
MFMA rate the chip sustains under that load, the shader clock it ran at, and the
forward's fraction of that rate.  `--probes` prints the full set of SIMD
micro-benchmarks instead (VALU, exp and rcp issue cost; MFMA and VALU together).
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA, published
PEAK_F32_TFLOPS = 157.3     # MI355X dense fp32 MFMA, published
PEAK_HBM_GBS = 8000.0

METRIC = "continuous-attn fwd TFLOP/s + % bf16 MFMA peak, B4 H16 T4096 d128"


# ------------------------------------------------------------------ CPU leg

_CPU = {}


def _cpu_task(args):
    import numpy as np

    from oracle import csa_reference

    b, h, rows = args
    q, k, v = _CPU["q"], _CPU["k"], _CPU["v"]
    sl = (slice(b, b + 1), slice(h, h + 1))
    csa_reference(q[sl], k[sl], v[sl], None if _CPU["k0"] is None else _CPU["k0"][sl],
                  None if _CPU["v0"] is None else _CPU["v0"][sl], rows=rows)
    return int(np.sum(rows + 1))


# Worker processes of the CPU leg: one GPU's share of the host is 16 cores, whatever
# os.sched_getaffinity shows (it may list every core of the host), so the pool takes at most 16;
# the affinity mask's own count is reported beside it.
CPU_WORKERS_MAX = 16


def cpu_baseline(w, q, k, v, k0, v0, heads=64, rows_per_head=320, seed=123):
    """Time the float64 reference on a seeded sample of (head, row) pairs.

    Runs before any GPU work (the pool forks).  Returns the cpu_baseline object.
    """
    import multiprocessing as mp

    import numpy as np

    rng = np.random.default_rng(seed)
    nheads = w.B * w.H
    pick = rng.choice(nheads, size=min(heads, nheads), replace=False)
    tasks = []
    for bh in pick:
        rows = np.sort(rng.choice(w.T, size=rows_per_head, replace=False))
        tasks.append((int(bh) // w.H, int(bh) % w.H, rows))
    _CPU.update(q=q.float().numpy(), k=k.float().numpy(), v=v.float().numpy(),
                k0=None if k0 is None else k0.float().numpy(), v0=None if v0 is None else v0.float().numpy())
    host_cores = len(os.sched_getaffinity(0))
    workers = max(1, min(CPU_WORKERS_MAX, host_cores))
    os.environ.setdefault("OMP_NUM_THREADS", "1")
    ctx = mp.get_context("fork")
    t0 = time.perf_counter()
    with ctx.Pool(workers) as pool:
        done = pool.map(_cpu_task, tasks, chunksize=1)
    dt = time.perf_counter() - t0
    _CPU.clear()
    positions = sum(done)                      # sum over sampled rows of (t + 1)
    flop = 4.0 * w.d * positions               # same convention as the metric
    total_rows = w.B * w.H * w.T
    rate = flop / dt
    return {
        "value": rate / 1e12,
        "unit": "TFLOP/s",
        "cores": workers,
        "host_cores": host_cores,
        "kind": "oracle",
        "sample": (f"{len(tasks)} of {nheads} heads x {rows_per_head} seeded query rows "
                   f"({len(tasks) * rows_per_head} of {total_rows} rows), float64 eq. (8), "
                   f"{workers} worker processes (of {host_cores} cores in the affinity mask; "
                   f"one GPU's share of the host is {CPU_WORKERS_MAX}), {dt:.1f} s wall"),
        "sample_s": round(dt, 2),
        # the whole workload at the sampled rate (row cost grows with t + 1, counted in the FLOP)
        "extrapolated_full_s": round(float(w.flop) / rate, 1),
        "extrapolation": "full-workload seconds = metric FLOP / (FLOP of the sampled rows / sample_s); "
                         "a row's cost grows with t + 1, which the FLOP of a row counts",
    }


# the other bf16 configurations, timed after the headline: (workload, oracle heads, rows per head)
OTHER_CONFIGS = (("long", 32, 40), ("stress", 16, 80))


# ------------------------------------------------------------------ HBM traffic

TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn16_lm_B4H16T4096d128_hbm_traffic.txt")


def _profile_values(path):
    """The `key = value` lines of a committed rocprofv3 summary, or None when the file is
    missing or the kernel sources it names have changed since the counters were taken (their
    sha256 is recorded in the summary)."""
    import hashlib

    if not os.path.exists(path):
        return None
    import re

    kv = {}
    with open(path) as f:
        for line in f:
            m = re.match(r"([a-z0-9_]+) = (.*)$", line.strip())
            if m:
                kv[m.group(1)] = m.group(2).strip()
    h = hashlib.sha256()
    for rel in kv.get("kernel_sources", "").split():
        src = os.path.join(ROOT, rel)
        if not os.path.exists(src):
            return None
        with open(src, "rb") as f:
            h.update(f.read())
    if h.hexdigest() != kv.get("kernel_source_sha256"):
        return None
    return kv


def measured_traffic(workload_name):
    """HBM bytes per csa_forward launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary (lm only), or None when it does not apply to the current kernel."""
    kv = _profile_values(TRAFFIC_FILE) if workload_name == "lm" else None
    if kv is None:
        return None
    return int(kv["csa_fetch_bytes"]) + int(kv["csa_write_bytes"])


ISSUE_FILE = os.path.join(ROOT, "profiles", "attn16_lm_B4H16T4096d128_issue_counters.md")
# Plain VALU issue peak of the chip: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz, one unpacked
# fp32 operation per lane and cycle (a wave64 instruction takes a SIMD for 4 cycles).  The
# SIMD probes measure an exp or rcp at about three times an FMA's issue time.
VALU_PEAK_LANE_OPS = 256 * 4 * 16 * 2.4e9
TRANS_ISSUE_WEIGHT = 3


def measured_valu(workload_name, avg_ms):
    """VALU issue of the csa_forward kernel from the committed SQ_INSTS_* counters (lm only):
    lane operations per second against the plain VALU peak, with the transcendentals counted
    once (`frac`) and at their measured issue cost (`frac_trans_weighted`), or None when the
    counters do not apply to the current kernel."""
    kv = _profile_values(ISSUE_FILE) if workload_name == "lm" else None
    if kv is None:
        return None
    valu = int(kv["csa_insts_valu"]) - int(kv["csa_insts_mfma"])  # wave instructions besides MFMA
    trans = int(kv["csa_insts_trans"])
    secs = avg_ms * 1e-3
    ops = 64.0 * valu / secs
    weighted = 64.0 * (valu + (TRANS_ISSUE_WEIGHT - 1) * trans) / secs
    return {"bound": "alu", "insts_per_launch": valu, "transcendental_per_launch": trans,
            "achieved": round(ops / 1e12, 2), "peak": round(VALU_PEAK_LANE_OPS / 1e12, 2),
            "unit": "T lane-ops/s", "frac": round(ops / VALU_PEAK_LANE_OPS, 4),
            "frac_trans_weighted": round(weighted / VALU_PEAK_LANE_OPS, 4)}


# ------------------------------------------------------------------ GPU leg

SETTLE_S = 0.3  # untimed warm-up time per leg, at least (see time_kernel)


def time_kernel(fn, steps, warmup, stream, settle_s=None):
    """Average per-launch duration (ms) from HIP events on the launch stream, and
    the wall time (ms) of the whole timed region bracketed by synchronisations.

    Warm-up: ``warmup`` untimed calls, continued (untimed) until at least ``settle_s``
    seconds of them have run.  The GPU's clocks ramp up over the first ~50-100 ms of
    sustained load (measured on the MI355X: 0.58 ms per lm call at the start, 0.46 ms
    after ~100 calls); a handful of warm-up calls would time the ramp, not the kernel."""
    import torch

    settle_s = SETTLE_S if settle_s is None else settle_s
    t_start = time.perf_counter()
    n = 0
    while n < warmup or (time.perf_counter() - t_start < settle_s and n < 20000):
        fn()
        n += 1
        if n % 50 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        fn()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    per = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    return sum(per) / len(per), min(per), wall_ms


# iterations per probe launch: ~2-3 ms each at four waves per SIMD
_PROBE_ITERS = {0: 20000, 1: 40000, 2: 20000, 3: 20000, 4: 10000, 5: 20000, 6: 10000, 7: 10000, 8: 10000,
                9: 3000, 10: 30000, 11: 30000, 12: 10000}
_PROBE_PER_ITER = {0: 4, 1: 8, 2: 8, 3: 8, 5: 2}  # instructions of the kind per iteration
_PROBE_WAVES = 4096  # four per SIMD of the 256 CUs


def simd_probes(kinds, stream, waves=_PROBE_WAVES):
    """SIMD micro-benchmarks (csa_probe in libcsa_bench), `waves` / 1024 waves per SIMD: per
    kind the launch duration, the issue cost per instruction per SIMD (single-instruction
    kinds) and the SIMD cycles per wave-iteration; kind 0 gives the MFMA-only ceiling the
    kernels are compared with.  The shader clock comes from the fp32 FMA kernel (kind 1): the
    longest-running wave's s_memtime cycles over the launch's duration."""
    import torch

    import continuous_softmax_attention_amd as csa

    dev = torch.device("cuda:0")
    sink = torch.empty((waves + 3) // 4, dtype=torch.float32, device=dev)
    cyc = torch.zeros(1, dtype=torch.int64, device=dev)
    per_simd = waves / 1024.0  # waves per SIMD
    ms, cycles = {}, {}
    for kind in sorted(set(kinds) | {1}):
        it = _PROBE_ITERS[kind]

        def launch(kind=kind, it=it):
            cyc.zero_()
            st = csa.csa_probe_raw(kind, waves, it, sink.data_ptr(), cyc.data_ptr(), stream.cuda_stream)
            if st != 0:
                raise RuntimeError(f"csa_probe({kind}) returned {st}")

        _, ms[kind], _ = time_kernel(launch, 3, 2, stream)
        cycles[kind] = int(cyc.item())
    ghz = cycles[1] / (ms[1] * 1e-3) / 1e9
    res = {"shader_clock_ghz": round(ghz, 3)}
    for kind in kinds:
        it, t = _PROBE_ITERS[kind], ms[kind] * 1e-3
        r = {"ms": round(ms[kind], 4), "cycles_per_wave_iteration": round(t * ghz * 1e9 / (per_simd * it), 1)}
        if kind in _PROBE_PER_ITER:
            r["cycles_per_instruction"] = round(t * ghz * 1e9 / (per_simd * it * _PROBE_PER_ITER[kind]), 2)
        if kind in (0, 5):
            r["tflops"] = round(waves * it * 65536.0 / t / 1e12, 1)
        res[kind] = r
    return res


def decode_legs(steps, warmup):
    """csa_decode on the decode workloads: HBM bandwidth of the whole call (both launches),
    counting the key/value cache read once (the algorithmic bytes; q, out and lse are
    under 0.1% of them)."""
    import torch

    import continuous_softmax_attention_amd as csa
    from workloads import DECODE_WORKLOADS, make_decode_inputs

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    legs = {}
    for name, w in DECODE_WORKLOADS.items():
        q, k, v, k0, v0 = make_decode_inputs(w)
        qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
        del q, k, v
        out = torch.empty_like(qd)
        lse = torch.empty((w.B, w.H, w.Tq), dtype=torch.float32, device=dev)
        ws = torch.empty(csa.csa_decode_workspace_bytes(w.B, w.H, w.Tq, w.T, w.d), dtype=torch.uint8, device=dev)

        def step():
            csa.csa_decode(qd, kd, vd, None, None, out=out, lse=lse, workspace=ws, stream=stream)

        avg_ms, min_ms, _ = time_kernel(step, steps, warmup, stream)
        gbs = w.cache_bytes / (avg_ms * 1e-3) / 1e9
        legs[name] = {"workload": f"B{w.B} H{w.H} Tq{w.Tq} T{w.T} d{w.d} {w.dtype}", "value": round(gbs, 1),
                      "unit": "GB/s", "ms": round(avg_ms, 4), "min_ms": round(min_ms, 4),
                      "bytes": w.cache_bytes, "frac_hbm": round(gbs / PEAK_HBM_GBS, 4)}
        del qd, kd, vd, out, lse, ws
        torch.cuda.empty_cache()
    return legs


def counters_mode(w, q, k, v, k0, v0):
    """One launch of each kernel plus a 256 MiB device-to-device copy whose HBM bytes
    are known (256 MiB read + 256 MiB written), to scale FETCH_SIZE/WRITE_SIZE; then (bf16
    workloads) a forward and one csa_backward call, and one csa_decode call on the decode
    workload."""
    import torch

    import continuous_softmax_attention_amd as csa

    dev = torch.device("cuda:0")
    src = torch.ones(1 << 26, dtype=torch.float32, device=dev)   # 256 MiB
    dst = torch.empty_like(src)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    k0d = None if k0 is None else k0.to(dev)
    v0d = None if v0 is None else v0.to(dev)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    csa.csa_forward(qd, kd, vd, k0d, v0d)
    torch.cuda.synchronize()
    csa.std_fwd(qd, kd, vd)
    torch.cuda.synchronize()
    if w.dtype == "bf16":
        csa.csa_forward_first_order(qd, kd, vd, k0d, v0d)
        torch.cuda.synchronize()
        if w.d in (64, 128):
            csa.csa_forward_half_interval(qd, kd, vd, k0d, v0d)
            torch.cuda.synchronize()
        from workloads import make_grad_output

        o, lse = csa.csa_forward(qd, kd, vd, k0d, v0d)
        dod = make_grad_output(q.shape, q.dtype, w.seed).to(dev)
        torch.cuda.synchronize()
        csa.csa_backward(qd, kd, vd, o, lse, dod, k0d, v0d)
        torch.cuda.synchronize()
        del o, lse, dod
    del qd, kd, vd
    from workloads import make_decode_inputs

    dq, dk, dv, _, _ = make_decode_inputs("decode")
    dq, dk, dv = dq.to(dev), dk.to(dev), dv.to(dev)
    csa.csa_decode(dq, dk, dv)
    torch.cuda.synchronize()
    print(json.dumps({"counters_run": w.name, "copy_bytes": 2 * src.numel() * 4}), flush=True)


def probes_mode():
    """All SIMD micro-benchmarks, one JSON line: the MFMA-only ceiling (16x16x32 and 32x32x16),
    the issue cost of fp32 FMA, exp and rcp, MFMA with VALU work in the same waves against the
    two alone, and the forward's per-key weight arithmetic alone and beside 16x16x32 or
    32x32x16 MFMAs at the forward's ratio, at 2, 4 and 8 waves per SIMD (the tiling choice)."""
    import torch

    stream = torch.cuda.current_stream(torch.device("cuda:0"))
    r = simd_probes([0, 1, 2, 3, 4, 5], stream)
    # the mixed kernel does half the MFMA iterations of kind 0 and half the FMAs of kind 1
    parts = (0.5 * r[0]["ms"], 0.5 * r[1]["ms"])
    out = {"probes": "gfx950 SIMD, 4 waves per SIMD, 256 threads per work-group",
           "shader_clock_ghz": r["shader_clock_ghz"],
           "mfma_only": r[0], "fma": r[1], "exp": r[2], "rcp": r[3], "mfma_and_fma": r[4],
           "mix_over_sum_of_parts": round(r[4]["ms"] / sum(parts), 3),
           "mix_over_larger_part": round(r[4]["ms"] / max(parts), 3),
           "mfma32_only": r[5]}
    # weight arithmetic (2 keys per wave-iteration) with 4 16x16x32 or 2 32x32x16 MFMAs
    tiling = {}
    for wps in (2, 4, 8):
        w = simd_probes([6, 7, 8], stream, waves=1024 * wps)
        tiling[f"{wps}_waves_per_simd"] = {
            "cycles_per_wave_iteration": {"weights": w[6]["cycles_per_wave_iteration"],
                                          "weights_mfma16x16x32": w[7]["cycles_per_wave_iteration"],
                                          "weights_mfma32x32x16": w[8]["cycles_per_wave_iteration"]},
            "mfma32_over_mfma16": round(w[8]["ms"] / w[7]["ms"], 3)}
    out["weights_and_mfma"] = tiling
    # does a transcendental take issue slots of the plain VALU?  8 FMA chains alone (kind 1) and
    # with 2 exp / rcp chains beside them (kinds 10, 11), cycles per wave-iteration
    mix = simd_probes([1, 2, 3, 10, 11], stream)
    c = {k: mix[k]["cycles_per_wave_iteration"] for k in (1, 10, 11)}
    out["fma_with_transcendentals"] = {
        "fma8": c[1], "fma8_exp2": c[10], "fma8_rcp2": c[11],
        "exp2_alone": round(mix[2]["cycles_per_wave_iteration"] / 4, 1),
        "rcp2_alone": round(mix[3]["cycles_per_wave_iteration"] / 4, 1)}
    # the weights by three routes, two keys per wave-iteration at 4 waves per SIMD: the p-form of
    # the kernels (kind 6), the log-domain form of eq. (13) (kind 9), and the p-form with the
    # reciprocal replaced by an LDS table (kind 12)
    wr = simd_probes([6, 9, 12], stream)
    cw = {k: wr[k]["cycles_per_wave_iteration"] for k in (6, 9, 12)}
    out["weight_routes"] = {"cycles_per_wave_iteration": {"p_form": cw[6], "log_domain": cw[9], "lds_table": cw[12]},
                            "log_domain_over_p_form": round(cw[9] / cw[6], 3),
                            "lds_table_over_p_form": round(cw[12] / cw[6], 3)}
    print(json.dumps(out), flush=True)


def main():
    global SETTLE_S
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="lm")
    ap.add_argument("--settle-s", type=float, default=SETTLE_S,
                    help="untimed warm-up per leg lasts at least this long (GPU clock ramp)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-std", action="store_true")
    ap.add_argument("--no-first-order", action="store_true")
    ap.add_argument("--no-half-interval", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-other-configs", action="store_true",
                    help="skip the long and stress configurations (extra keys of the JSON line)")
    ap.add_argument("--probes", action="store_true",
                    help="print the SIMD micro-benchmarks (MFMA-only ceiling, VALU / exp / rcp issue cost, "
                         "MFMA and VALU in one wave) as one JSON line and exit")
    ap.add_argument("--no-ceiling", action="store_true")
    ap.add_argument("--counters", action="store_true",
                    help="for rocprofv3 --pmc passes: one plain device copy of 256 MiB (counter "
                         "calibration), one csa_forward and one std_fwd launch, then exit")
    args = ap.parse_args()
    SETTLE_S = args.settle_s
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: there is no multi-GPU path "
              "(independent (batch, head) shards need no communication); run with --gpus 1",
              file=sys.stderr)
        sys.exit(2)

    if args.probes:
        return probes_mode()

    from workloads import WORKLOADS, make_inputs

    w = WORKLOADS[args.workload]
    q, k, v, k0, v0 = make_inputs(w)
    if args.counters:
        return counters_mode(w, q, k, v, k0, v0)
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(w, q, k, v, k0, v0)
    others = {}
    if not args.no_other_configs and args.workload == "lm":
        for name, heads, rows in OTHER_CONFIGS:  # inputs and oracle time before any GPU work
            wo = WORKLOADS[name]
            inp = make_inputs(wo)
            others[name] = (wo, inp, None if args.no_cpu_baseline else cpu_baseline(wo, *inp, heads=heads,
                                                                                      rows_per_head=rows))

    import torch

    import continuous_softmax_attention_amd as csa

    dev = torch.device("cuda:0")
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    k0d = None if k0 is None else k0.to(dev)
    v0d = None if v0 is None else v0.to(dev)
    out = torch.empty_like(qd)
    lse = torch.empty((w.B, w.H, w.T), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        csa.csa_forward(qd, kd, vd, k0d, v0d, out=out, lse=lse, stream=stream)

    avg_ms, min_ms, wall_ms = time_kernel(step, args.steps, args.warmup, stream)
    flop = float(w.flop)
    tflops = flop / (avg_ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS

    res = {
        "metric": METRIC,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": f"{w.name}: causal CSA forward B{w.B} H{w.H} T{w.T} d{w.d} {w.dtype}"
                               + (", RoPE on q,k" if w.rope else "") + f", k0/v0 {w.sink}",
                   "B": w.B, "H": w.H, "T": w.T, "d": w.d},
        "pct_peak": round(100.0 * tflops / peak, 2),
        "kernel_ms": {"avg": round(avg_ms, 4), "min": round(min_ms, 4)},
        "roofline": {
            "bound": "mfma",
            "achieved": round(tflops, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(tflops / peak, 4),
            "traffic": measured_traffic(w.name),
        },
        "valu": measured_valu(w.name, avg_ms),
    }
    if not args.no_std:
        sout = torch.empty_like(qd)
        slse = torch.empty_like(lse)

        def std_step():
            csa.std_fwd(qd, kd, vd, out=sout, lse=slse, stream=stream)

        s_avg, _, _ = time_kernel(std_step, args.steps, args.warmup, stream)
        s_tflops = flop / (s_avg * 1e-3) / 1e12
        res["std_attention"] = {"value": round(s_tflops, 2), "unit": "TFLOP/s", "kernel_ms": round(s_avg, 4),
                                "pct_peak": round(100.0 * s_tflops / peak, 2)}
        res["ratio_vs_std"] = round(tflops / s_tflops, 4)
    if not args.no_first_order and w.dtype == "bf16":
        fout = torch.empty_like(qd)
        flse = torch.empty_like(lse)

        def first_step():
            csa.csa_forward_first_order(qd, kd, vd, k0d, v0d, out=fout, lse=flse, stream=stream)

        f_avg, _, _ = time_kernel(first_step, args.steps, args.warmup, stream)
        f_tflops = flop / (f_avg * 1e-3) / 1e12
        res["first_order"] = {"value": round(f_tflops, 2), "unit": "TFLOP/s", "kernel_ms": round(f_avg, 4),
                              "pct_peak": round(100.0 * f_tflops / peak, 2),
                              "exact_over_first_order": round(tflops / f_tflops, 4)}
    if not args.no_half_interval and w.dtype == "bf16":
        hout = torch.empty_like(qd)
        hlse = torch.empty_like(lse)

        def half_step():
            csa.csa_forward_half_interval(qd, kd, vd, k0d, v0d, out=hout, lse=hlse, stream=stream)

        h_avg, _, _ = time_kernel(half_step, args.steps, args.warmup, stream)
        h_tflops = flop / (h_avg * 1e-3) / 1e12
        res["half_interval"] = {"value": round(h_tflops, 2), "unit": "TFLOP/s", "kernel_ms": round(h_avg, 4),
                                "pct_peak": round(100.0 * h_tflops / peak, 2)}
    if not args.no_backward and w.dtype == "bf16":
        from workloads import make_grad_output

        dod = make_grad_output(q.shape, q.dtype, w.seed).to(dev)
        grads = [torch.empty_like(qd) for _ in range(3)]
        bws = torch.empty(csa.csa_backward_workspace_bytes_fast(w.B, w.H, w.T, w.d), dtype=torch.uint8,
                          device=dev)
        csa.csa_forward(qd, kd, vd, k0d, v0d, out=out, lse=lse, stream=stream)

        def bwd_step():
            csa.csa_backward(qd, kd, vd, out, lse, dod, k0d, v0d, dq=grads[0], dk=grads[1], dv=grads[2],
                             workspace=bws, stream=stream)

        b_avg, b_min, _ = time_kernel(bwd_step, args.steps, args.warmup, stream)
        b_tflops = 2.5 * flop / (b_avg * 1e-3) / 1e12
        res["backward"] = {"value": round(b_tflops, 2), "unit": "TFLOP/s", "kernel_ms": round(b_avg, 4),
                           "min_ms": round(b_min, 4), "pct_peak": round(100.0 * b_tflops / peak, 2),
                           "flop": "2.5 x forward", "fwd_plus_bwd_ms": round(avg_ms + b_avg, 4)}
        del dod, grads, bws
    if not args.no_decode:
        res["decode"] = decode_legs(args.steps, args.warmup)
    if not args.no_ceiling and w.dtype == "bf16":
        pr = simd_probes([0], stream)
        res["mfma_ceiling"] = {"mfma_only_tflops": pr[0]["tflops"], "frac_of_mfma_only": round(tflops / pr[0]["tflops"], 4)}
    if others:
        del qd, kd, vd, out, lse
        torch.cuda.empty_cache()
        res["other_configs"] = {name: other_config_leg(wo, inp, ocpu, args, stream)
                                for name, (wo, inp, ocpu) in others.items()}
    if cpu is not None:
        res["cpu_baseline"] = cpu
    print(json.dumps(res), flush=True)


def other_config_leg(w, inp, cpu, args, stream):
    """csa_forward and std_fwd on another bf16 configuration (same FLOP convention as the
    metric), with the oracle's time on a sample of its rows."""
    import torch

    import continuous_softmax_attention_amd as csa

    dev = torch.device("cuda:0")
    q, k, v, k0, v0 = inp
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    k0d = None if k0 is None else k0.to(dev)
    v0d = None if v0 is None else v0.to(dev)
    out = torch.empty_like(qd)
    lse = torch.empty((w.B, w.H, w.T), dtype=torch.float32, device=dev)

    def step():
        csa.csa_forward(qd, kd, vd, k0d, v0d, out=out, lse=lse, stream=stream)

    def std_step():
        csa.std_fwd(qd, kd, vd, out=out, lse=lse, stream=stream)

    avg, mn, _ = time_kernel(step, args.steps, args.warmup, stream)
    s_avg, _, _ = time_kernel(std_step, args.steps, args.warmup, stream)
    flop = float(w.flop)
    tf, s_tf = flop / (avg * 1e-3) / 1e12, flop / (s_avg * 1e-3) / 1e12
    leg = {"workload": f"{w.name}: causal CSA forward B{w.B} H{w.H} T{w.T} d{w.d} {w.dtype}"
                       + f", q scaled by {w.q_scale * math.sqrt(w.d):g}/sqrt(d)"
                       + f", k0/v0 {w.sink}",
           "value": round(tf, 2), "unit": "TFLOP/s", "pct_peak": round(100.0 * tf / PEAK_BF16_TFLOPS, 2),
           "frac": round(tf / PEAK_BF16_TFLOPS, 4), "kernel_ms": {"avg": round(avg, 4), "min": round(mn, 4)},
           "std_attention": {"value": round(s_tf, 2), "kernel_ms": round(s_avg, 4)},
           "ratio_vs_std": round(tf / s_tf, 4), "flop": flop}
    if cpu is not None:
        leg["cpu_baseline"] = cpu
        leg["gpu_over_oracle"] = round(tf / cpu["value"], 1)
    del qd, kd, vd, out, lse
    torch.cuda.empty_cache()
    return leg


if __name__ == "__main__":
    main()
