"""Seeded synthetic inputs for continuous softmax attention (tests and bench).

This module holds input generation only -- shapes, seeds, random draws, the
1/sqrt(d) query pre-scaling, rotary position embedding applied before the
call, and the choice of k_0/v_0 -- and none of the attention arithmetic.  It
is the one module that both the CPU reference and the HIP path consume.

Workloads (all causal; q, k, v drawn in that order from N(0, 1) with
``torch.Generator('cpu').manual_seed(seed)`` as float32 [B, H, T, d];
transforms in float32; one final cast to the workload dtype):

=========  ====  ==========================  =====  ==========================================
name       seed  B, H, T, d                  dtype  transforms / k_0, v_0
=========  ====  ==========================  =====  ==========================================
tiny       1     1, 1, 64, 16                f32    q *= 1/sqrt(d);  k_0 = v_0 = 0
tile       2     1, 4, 1024, 64              f32    q *= 1/sqrt(d);  k_0 = v_0 = 0
tail       2     1, 4, 1000, 64              f32    q *= 1/sqrt(d);  k_0 = v_0 = 0 (own draw)
lm         3     4, 16, 4096, 128            bf16   q *= 1/sqrt(d); RoPE(q, k), base 10000
long       4     1, 32, 16384, 128           bf16   q *= 1/sqrt(d);  k_0 = v_0 = 0
stress     5     2, 8, 8192, 128             bf16   q *= 8/sqrt(d) (logit std ~ 8);
                                                    k_0 = k_1, v_0 = v_1 (after the cast)
=========  ====  ==========================  =====  ==========================================

Decode workloads (few new queries against a key/value cache of T positions; the
queries are the last Tq positions T-Tq+1..T; q [B, H, Tq, d], then k and v
[B, H, T, d], drawn in that order with the same generator rule):

===========  ====  =============================  =====  ===========================
name         seed  B, H, Tq, T, d                 dtype  transforms / k_0, v_0
===========  ====  =============================  =====  ===========================
decode       6     16, 8, 1, 8192, 128            bf16   q *= 1/sqrt(d); zeros
decode_spec  7     16, 8, 8, 8192, 128            bf16   q *= 1/sqrt(d); zeros
===========  ====  =============================  =====  ===========================

Backward pass: the same (q, k, v, k_0, v_0) as the workload, plus an upstream
gradient dO ~ N(0, 1) of the output's shape drawn from its own generator seeded
``seed + 1000`` (``make_grad_output``).

The pages fix no shapes; their experiments are language-model training runs
with rotary embeddings, which ``lm`` stands in for.  "All zeros" and "copy
the first key/value" are two of the k_0/v_0 choices listed under Analysis of
the Result of J. Su, "Continuous Softmax Attention".
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

# torch is used only as a seeded random-number source and as a container.
import torch


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int
    H: int
    T: int
    d: int
    dtype: str          # "f32" or "bf16"
    q_scale: float      # multiplier applied to q before the cast
    rope: bool          # rotary embedding on q and k (before the cast)
    sink: str           # "zero" or "copy" (k_0 = k_1, v_0 = v_1)

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def elements(self) -> int:
        """Causal score entries: query t sees positions 0..t, so sum_t (t + 1)."""
        return self.B * self.H * (self.T * (self.T + 1) // 2 + self.T)

    @property
    def flop(self) -> int:
        """Metric FLOP: 4 T^2 d / 2 per head (QK^T plus PV, causal half)."""
        return self.B * self.H * 2 * self.T * self.T * self.d


def _w(name, seed, B, H, T, d, dtype, q_mult=1.0, rope=False, sink="zero"):
    return Workload(name, seed, B, H, T, d, dtype, q_mult / math.sqrt(d), rope, sink)


WORKLOADS = {
    "tiny": _w("tiny", 1, 1, 1, 64, 16, "f32"),
    "tile": _w("tile", 2, 1, 4, 1024, 64, "f32"),
    "tail": _w("tail", 2, 1, 4, 1000, 64, "f32"),
    "lm": _w("lm", 3, 4, 16, 4096, 128, "bf16", rope=True),
    "long": _w("long", 4, 1, 32, 16384, 128, "bf16"),
    "stress": _w("stress", 5, 2, 8, 8192, 128, "bf16", q_mult=8.0, sink="copy"),
}


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    seed: int
    B: int
    H: int
    Tq: int             # new queries, at positions T-Tq+1..T
    T: int              # cached positions (keys/values 1..T)
    d: int
    dtype: str
    q_scale: float
    sink: str

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    @property
    def cache_bytes(self) -> int:
        """Bytes of k and v read once per call (the algorithmic HBM traffic that dominates)."""
        return 2 * self.B * self.H * self.T * self.d * (4 if self.dtype == "f32" else 2)


DECODE_WORKLOADS = {
    "decode": DecodeWorkload("decode", 6, 16, 8, 1, 8192, 128, "bf16", 1 / math.sqrt(128), "zero"),
    "decode_spec": DecodeWorkload("decode_spec", 7, 16, 8, 8, 8192, 128, "bf16", 1 / math.sqrt(128), "zero"),
}


def make_decode_inputs(w: DecodeWorkload | str, *, B=None, H=None, Tq=None, T=None, d=None, dtype=None,
                       seed=None, sink=None):
    """Draw (q, k, v, k0, v0) for a decode call: q [B, H, Tq, d], k and v [B, H, T, d].

    Keyword overrides give smaller variants; sink is "zero" (k0 = v0 = None), "copy"
    (k_0 = k_1, v_0 = v_1) or "random" (k0, v0 drawn after v).
    """
    if isinstance(w, str):
        w = DECODE_WORKLOADS[w]
    B = w.B if B is None else B
    H = w.H if H is None else H
    Tq = w.Tq if Tq is None else Tq
    T = w.T if T is None else T
    d = w.d if d is None else d
    dt = w.torch_dtype if dtype is None else {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]
    seed = w.seed if seed is None else seed
    sink = w.sink if sink is None else sink
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn((B, H, Tq, d), generator=g, dtype=torch.float32) / math.sqrt(d)
    k = torch.randn((B, H, T, d), generator=g, dtype=torch.float32)
    v = torch.randn((B, H, T, d), generator=g, dtype=torch.float32)
    q, k, v = q.to(dt), k.to(dt), v.to(dt)
    if sink == "copy":
        k0, v0 = k[:, :, 0, :].clone(), v[:, :, 0, :].clone()
    elif sink == "random":
        k0 = torch.randn((B, H, d), generator=g, dtype=torch.float32).to(dt)
        v0 = torch.randn((B, H, d), generator=g, dtype=torch.float32).to(dt)
    else:
        k0 = v0 = None
    return q, k, v, k0, v0


def rope_interleaved(x: torch.Tensor, base: float = 10000.0) -> torch.Tensor:
    """Rotary embedding on interleaved pairs (2j, 2j+1), angle pos * base^(-2j/d).

    x: float32 [B, H, T, d]; the position is the array row index 0..T-1.
    """
    B, H, T, d = x.shape
    j = torch.arange(d // 2, dtype=torch.float64)
    inv = base ** (-2.0 * j / d)
    ang = torch.arange(T, dtype=torch.float64)[:, None] * inv[None, :]
    cos = torch.cos(ang).to(torch.float32)
    sin = torch.sin(ang).to(torch.float32)
    pairs = x.reshape(B, H, T, d // 2, 2)
    x0 = pairs[..., 0]
    x1 = pairs[..., 1]
    return torch.stack((x0 * cos - x1 * sin, x0 * sin + x1 * cos), dim=-1).reshape(B, H, T, d)


def make_inputs(w: Workload | str, *, B=None, H=None, T=None, d=None, dtype=None, seed=None):
    """Draw (q, k, v, k0, v0) on the CPU for a workload.

    Keyword overrides give smaller variants of the same recipe (same
    transforms and k_0/v_0 rule).  k0/v0 are None for the all-zeros choice.
    """
    if isinstance(w, str):
        w = WORKLOADS[w]
    B = w.B if B is None else B
    H = w.H if H is None else H
    T = w.T if T is None else T
    d = w.d if d is None else d
    dt = w.torch_dtype if dtype is None else {"f32": torch.float32, "bf16": torch.bfloat16}[dtype]
    seed = w.seed if seed is None else seed
    q_scale = w.q_scale * math.sqrt(w.d) / math.sqrt(d)
    g = torch.Generator("cpu").manual_seed(seed)
    q = torch.randn((B, H, T, d), generator=g, dtype=torch.float32)
    k = torch.randn((B, H, T, d), generator=g, dtype=torch.float32)
    v = torch.randn((B, H, T, d), generator=g, dtype=torch.float32)
    q = q * q_scale
    if w.rope:
        q = rope_interleaved(q)
        k = rope_interleaved(k)
    q, k, v = q.to(dt), k.to(dt), v.to(dt)
    if w.sink == "copy":
        k0 = k[:, :, 0, :].clone()
        v0 = v[:, :, 0, :].clone()
    else:
        k0 = v0 = None
    return q, k, v, k0, v0


def make_grad_output(shape, dtype, seed: int):
    """Upstream gradient dO for the backward pass: N(0, 1) of ``shape`` from its own
    generator (``seed + 1000``), cast once to ``dtype`` (a torch dtype)."""
    g = torch.Generator("cpu").manual_seed(seed + 1000)
    return torch.randn(tuple(shape), generator=g, dtype=torch.float32).to(dtype)


def sample_rows(T: int, seed: int, n_random: int = 48, tile: int = 64, n_edges: int = 4):
    """0-based query rows checked on large workloads.

    Queries t = 1..4 and T-3..T, three rows around each of ``n_edges`` evenly
    spaced multiples of ``tile``, and ``n_random`` seeded-uniform rows.
    """
    ts = set(range(1, min(4, T) + 1)) | set(range(max(1, T - 3), T + 1))
    for j in range(1, n_edges + 1):
        m = (j * (T // tile)) // (n_edges + 1)
        for t in (m * tile - 1, m * tile, m * tile + 1):
            if 1 <= t <= T:
                ts.add(t)
    rng = np.random.default_rng(seed)
    ts |= set(int(x) for x in rng.integers(1, T + 1, size=n_random))
    return np.array(sorted(t - 1 for t in ts), dtype=np.int64)
