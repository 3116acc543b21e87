"""Seeded synthetic inputs for the chunked GDN/KDA prefill workloads.

This module draws random numbers and lays them out; it holds none of the method's
arithmetic, so both the HIP path and the fp64 oracle can be fed from it. Every array is
produced on the CPU with ``numpy.random.default_rng`` in float32 and, for bf16 workloads,
rounded to bfloat16 by torch (round to nearest even).

Layouts (all row-major, rows = tokens of every stream back to back):

* ``x``          [alloc, 2*Hqk*dk + H*dv]  packed ``[q | k | v]`` rows (raw conv input
  when the front end is on, otherwise q, k, v themselves), dtype f32 or bf16; Hqk = H
  unless the spec sets fewer q/k heads.
* ``g``          [alloc, H] (GDN, one log-gate per head) or [alloc, H, dk] (KDA), f32.
* ``beta``       [alloc, H] f32, already through the sigmoid.
* ``h0``         [B, H, dk, dv] f32 initial state per stream.
* ``conv_w``     [cd, K] f32 and ``conv_state`` [B, cd, K-1] in the dtype of ``x``
  (front end only).
* ``cu_seqlens`` [B+1] int32.
* ``z`` [alloc, H, dv] in the dtype of ``x`` and ``norm_w`` [dv] f32 (output gate only).

``alloc`` = round_up(N, chunk) + chunk rows; rows ``[N, alloc)`` of every per-token array
hold ``pad_fill`` (0, NaN, 1e30, ...), so a kernel that read past a stream's end would
see it.

Distributions (second parameter of N(.,.) is the standard deviation):
q, k, v ~ N(0,1); conv weights ~ N(0, 0.5); carried conv state ~ N(0, 1);
beta = sigmoid(N(0,1)); g = -softplus(N(0,1)) or Uniform(-0.5, -0.01);
h0 = 0 or N(0, 0.1); output gate: z ~ N(0, 1), norm_w ~ Uniform(0.5, 1.5).
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np
import torch


@dataclasses.dataclass
class Spec:
    """Shape and distribution of one synthetic workload."""
    name: str
    lengths: Sequence[int]            # tokens per stream
    H: int = 32
    dk: int = 128
    dv: int = 128
    chunk: int = 64
    dtype: str = "bf16"               # "bf16" | "f32" (q/k/v, conv state, o)
    gate: str = "gdn"                 # "gdn" (per head) | "kda" (per key channel)
    # "softplus": -softplus(N(0,1)); "uniform": U(-0.5,-0.01); "slow": U(-0.02,-1e-4), a
    # decay weak enough that the state carries over many chunks
    gate_dist: str = "softplus"
    front_end: bool = False           # raw packed QKV + conv1d(K) + SiLU
    conv_k: int = 4
    h0_std: float = 0.1               # 0 -> zero initial state
    seed: int = 0
    pad_fill: float = 0.0
    eps: float = 1e-6
    out_gate: bool = False            # gated RMSNorm of o with z (z, norm_w drawn last)
    norm_eps: float = 1e-6
    Hqk: int = 0                      # q/k heads (0 = H); value head h reads h // (H // Hqk)

    @property
    def B(self) -> int:
        return len(self.lengths)

    @property
    def N(self) -> int:
        return int(sum(self.lengths))

    @property
    def qk_heads(self) -> int:
        return self.Hqk or self.H

    @property
    def cd(self) -> int:
        return 2 * self.qk_heads * self.dk + self.H * self.dv

    @property
    def alloc(self) -> int:
        c = self.chunk
        return ((self.N + c - 1) // c) * c + c

    @property
    def torch_dtype(self):
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.dk)


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.logaddexp(0.0, x).astype(np.float32)


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


def _normal(rng, shape, std=1.0) -> np.ndarray:
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def make(spec: Spec) -> dict:
    """Draw every input of ``spec``; returns CPU torch tensors (see module docstring)."""
    rng = np.random.default_rng(spec.seed)
    N, alloc, H, dk, dv, cd = spec.N, spec.alloc, spec.H, spec.dk, spec.dv, spec.cd
    td = spec.torch_dtype
    out = {"spec": spec}

    x = torch.from_numpy(_normal(rng, (N, cd))).to(td)
    xt = torch.full((alloc, cd), spec.pad_fill, dtype=td)
    xt[:N] = x
    out["x"] = xt

    gshape = (N, H) if spec.gate == "gdn" else (N, H, dk)
    if spec.gate_dist == "softplus":
        g = -_softplus(_normal(rng, gshape))
    elif spec.gate_dist == "slow":
        g = rng.uniform(-0.02, -1e-4, size=gshape).astype(np.float32)
    else:
        g = rng.uniform(-0.5, -0.01, size=gshape).astype(np.float32)
    gt = torch.full((alloc,) + gshape[1:], spec.pad_fill, dtype=torch.float32)
    gt[:N] = torch.from_numpy(g)
    out["g"] = gt

    b = _sigmoid(_normal(rng, (N, H)))
    bt = torch.full((alloc, H), spec.pad_fill, dtype=torch.float32)
    bt[:N] = torch.from_numpy(b)
    out["beta"] = bt

    if spec.h0_std > 0:
        out["h0"] = torch.from_numpy(_normal(rng, (spec.B, H, dk, dv), spec.h0_std))
    else:
        out["h0"] = torch.zeros((spec.B, H, dk, dv), dtype=torch.float32)

    if spec.front_end:
        out["conv_w"] = torch.from_numpy(_normal(rng, (cd, spec.conv_k), 0.5))
        out["conv_state"] = torch.from_numpy(
            _normal(rng, (spec.B, cd, spec.conv_k - 1))).to(td)
    else:
        out["conv_w"] = None
        out["conv_state"] = None

    if spec.out_gate:
        z = torch.from_numpy(_normal(rng, (N, H, dv))).to(td)
        zt = torch.full((alloc, H, dv), spec.pad_fill, dtype=td)
        zt[:N] = z
        out["z"] = zt
        out["norm_w"] = torch.from_numpy(rng.uniform(0.5, 1.5, size=dv).astype(np.float32))
    else:
        out["z"] = None
        out["norm_w"] = None

    cu = np.zeros(spec.B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(spec.lengths, dtype=np.int64))
    out["cu_seqlens"] = torch.from_numpy(cu)
    return out


def refill_tails(inp: dict, value: float) -> dict:
    """Copy of ``inp`` whose rows at or past N of every per-token array hold ``value``."""
    spec = dataclasses.replace(inp["spec"], pad_fill=value)
    res = dict(inp)
    res["spec"] = spec
    N = spec.N
    for key in ("x", "g", "beta", "z"):
        if inp.get(key) is None:
            continue
        t = inp[key].clone()
        t[N:] = value
        res[key] = t
    return res


# ----------------------------------------------------------------------------------------
# The five workloads. Small variants (same distributions, smaller shapes) are built by
# the tests with dataclasses.replace(spec, ...).


def varlen_lengths(seed: int = 4, B: int = 16, max_len: int = 8192,
                   forced: Sequence[int] = (1, 63, 64, 65),
                   total_range=(61440, 69632)) -> List[int]:
    """B lengths from U[1, max_len] with ``forced`` values at seeded positions.

    Attempt i draws from ``default_rng([seed, i])``; the first attempt whose total lies
    in ``total_range`` is kept, so the result is a pure function of the arguments.
    """
    for attempt in range(100000):
        rng = np.random.default_rng([seed, attempt])
        lens = rng.integers(1, max_len + 1, size=B)
        pos = rng.choice(B, size=len(forced), replace=False)
        lens[pos] = np.asarray(forced)
        if total_range[0] <= int(lens.sum()) <= total_range[1]:
            return [int(v) for v in lens]
    raise RuntimeError("no qualifying length draw")


def config(i: int, pad_fill: float = 0.0) -> Spec:
    """Workload ``i`` (1..5) at full size."""
    if i == 1:
        return Spec("gdn-core-T256-H2-d64-f32", [256], H=2, dk=64, dv=64, dtype="f32",
                    gate_dist="uniform", h0_std=0.0, seed=1, pad_fill=pad_fill)
    if i == 2:
        return Spec("gdn-frontend-T4096-H32-d128-bf16", [4096], front_end=True, seed=2,
                    pad_fill=pad_fill)
    if i == 3:
        return Spec("gdn-batched-B8xT2048-H32-d128-bf16", [2048] * 8, seed=3,
                    pad_fill=pad_fill)
    if i == 4:
        return Spec("gdn-varlen-B16-N%d-H32-d128-bf16" % sum(varlen_lengths()),
                    varlen_lengths(), seed=4, pad_fill=pad_fill)
    if i == 5:
        return Spec("kda-frontend-T16384-H32-d128-bf16", [16384], gate="kda",
                    front_end=True, seed=5, pad_fill=pad_fill)
    raise ValueError(i)


def decode_config(B: int = 64, gate: str = "gdn", pad_fill: float = 0.0) -> Spec:
    """A decode batch: B streams with one new token each (row b is stream b's token), the
    front end on, H=32, dk=dv=128, bf16, carried states h0 ~ N(0, 0.1)."""
    return Spec("%s-decode-B%d-H32-d128-bf16" % (gate, B), [1] * B, gate=gate,
                front_end=True, seed=6, pad_fill=pad_fill)
