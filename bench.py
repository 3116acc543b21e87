#!/usr/bin/env python3
"""Throughput of the chunked GDN/KDA prefill on one MI355X, printed as one JSON line.

A step is one call of the C ABI over one batch of synthetic input: the whole path (front
end when the workload has one, L2, chunk preparation, inter-chunk scan, state write-back).
The default workload is GDN with the conv front end, 1 stream of T=4096 tokens, H=32,
dk=dv=128, chunk 64 (seeded synthetic bf16 inputs). Inputs are resident in HBM when timing
starts; several input copies are rotated so that a step never finds its inputs in the
256 MB Infinity Cache from the previous step. The GPU's clocks reach their sustained level
only after some tens of milliseconds of load, so by default the warm-up runs about 100 ms
of steps and the timed region about 100 ms (at least 20 and 40 steps); ``--warmup`` and
``--steps`` fix the counts instead, and the JSON line reports the counts used.

``--decode gdn|kda`` times the decode step instead: one call advances 64 streams by one
token each (front end, one recurrence step on each stream's 2 MiB state, window update);
the value is decoded tokens/s.

Extra fields: ``roofline`` (the call's algorithmic bytes -- every input read once, o written
once in the input dtype, the states read and written once -- over the call's duration from
hipEvents the library records on the call's stream during the timed steps, against the HBM
peak; the same ratio over the wall-clock step; the call's algorithmic MFMA work against the
dense fp16 peak; per-stage times) and ``cpu_baseline`` (the fp64 oracle on a bounded
sample, on this host's cores).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0       # MI355X HBM3E
MFMA_PEAK_TFLOPS = 2500.0    # MI355X dense fp16/bf16 MFMA
FP32_PEAK_TFLOPS = 157.3     # MI355X fp32 (vector and MFMA)
METRIC = "prefill tokens/s per GDN/KDA layer (H=32, d=128) + % of MFMA/HBM roofline"
DECODE_METRIC = ("decode tokens/s per GDN/KDA layer (one token per stream, H=32, d=128) "
                 "+ % of HBM roofline")
CSRC = os.path.join(ROOT, "gated_delta_rule_depthwise_amd", "csrc")
# the sources a kernel's traffic depends on (device code and the host code launching it)
KERNEL_SOURCES = {"prefill": ("gdn_kernels.hip", "gdn_api.cpp", "gdn_internal.h"),
                  "decode": ("gdn_decode.hip", "gdn_api.cpp", "gdn_internal.h")}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_hash(which: str = "prefill") -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[which]:
        h.update(open(os.path.join(CSRC, f), "rb").read())
    return h.hexdigest()[:16]


def gate_fused(spec) -> bool:
    """The output gate rides in the chunk kernel's o flush except for the per-key-channel
    instances at dk = dv = 128 and in fp32, which gate in a pass of their own."""
    return not (spec.gate == "kda" and (spec.dk == 128 or spec.dtype == "f32"))


def algorithmic_bytes(spec) -> int:
    """Bytes a call must move at least: the q/k/v (or raw) rows read once, the gates and
    betas read once, o written once in the input dtype, every state read and written once,
    the conv taps and windows (read and written) once, and with the output gate z and its
    weights read once. With bf16 rows, H=32 and d=128 this is 34,132 bytes per token on the
    4096-token single stream."""
    N, H, dk, dv, B = spec.N, spec.H, spec.dk, spec.dv, spec.B
    es = 2 if spec.dtype == "bf16" else 4
    n = N * spec.cd * es                                         # q|k|v or raw rows
    n += N * H * (dk if spec.gate == "kda" else 1) * 4           # log-gates
    n += N * H * 4                                               # beta
    n += N * H * dv * es                                         # o (input dtype)
    n += 2 * B * H * dk * dv * 4                                 # h in and out
    if spec.front_end:
        n += spec.cd * spec.conv_k * 4 + 2 * B * spec.cd * (spec.conv_k - 1) * es
    if spec.out_gate:
        n += N * H * dv * es + dv * 4                            # z and the norm weights
    return n


def algorithmic_flops(spec) -> int:
    """MFMA work of the chunked algorithm per call: per token and head the strict-lower
    K K^T, the triangular solve, the triangular T K and T V, Q K^T and P U over the chunk,
    and the three state products W h, Q h and K^T U: 2 H [(C-1)/2 dk + C^2/6 + 4 (C+1)/2 d
    + 3 dk dv] per token (4.512 MFLOP at H=32, d=128, C=64)."""
    C, d = spec.chunk, spec.dv
    per_tok = 2 * spec.H * ((C - 1) / 2 * spec.dk + C * C / 6 + 4 * (C + 1) / 2 * d +
                            3 * spec.dk * spec.dv)
    return int(spec.N * per_tok)


def decode_bytes(spec) -> dict:
    """Bytes one decode launch must move: every state read and written once, the token
    rows, windows (read + written), taps, gates, beta and o."""
    B, H, dk, dv, cd = spec.B, spec.H, spec.dk, spec.dv, spec.cd
    es = 2 if spec.dtype == "bf16" else 4
    n = 2 * B * H * dk * dv * 4 + B * cd * es + B * H * (dk if spec.gate == "kda" else 1) * 4
    n += B * H * 4 + B * H * dv * 4
    if spec.out_gate:
        n += B * H * dv * es + dv * 4
    if spec.front_end:
        n += 2 * B * cd * (spec.conv_k - 1) * es + cd * spec.conv_k * 4
    return {"recur": n}


def cpu_baseline(spec, inp, budget_s: float) -> dict:
    """The oracle as it stands, on a bounded sample of the same workload."""
    import oracle
    H = spec.H
    cu = inp["cu_seqlens"].numpy()

    def run(heads):
        r = oracle.prefill(inp["x"], inp["g"], inp["beta"], inp["h0"], H=H, dk=spec.dk,
                           dv=spec.dv, cu_seqlens=cu, conv_w=inp["conv_w"],
                           conv_state=inp["conv_state"], heads=heads, Hqk=spec.qk_heads)
        if spec.out_gate:
            oracle.gated_rmsnorm(r["o"], inp["z"][:spec.N][:, heads], inp["norm_w"],
                                 spec.norm_eps)

    t0 = time.perf_counter()
    run([0])
    t1 = time.perf_counter() - t0
    n = int(max(1, min(H, math.floor(budget_s / max(t1, 1e-3)))))
    heads = list(range(n))
    t0 = time.perf_counter()
    run(heads)
    dt = time.perf_counter() - t0
    if n == H and dt < budget_s / 3:
        # a small workload (a decode batch): repeat the whole layer to fill the budget
        reps = int(min(1000, math.floor(budget_s / max(dt, 1e-3))))
        t0 = time.perf_counter()
        for _ in range(reps):
            run(heads)
        dt = (time.perf_counter() - t0) / reps
        return {"value": spec.N / dt, "unit": "tokens/s", "cores": oracle.num_threads(),
                "kind": "oracle",
                "sample": "the whole workload (%d tokens, %d heads, fp64) %d times, %.1f s"
                          % (spec.N, H, reps, dt * reps)}
    # every head is independent and costs the same: the full layer takes dt * H / n
    return {"value": spec.N / (dt * H / n), "unit": "tokens/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": "all %d tokens of the workload, %d of %d heads (fp64, %.1f s); "
                      "full-layer time scaled by %d/%d" % (spec.N, n, H, dt, H, n)}


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=0,
                    help="timed steps (0: about 100 ms of them, at least 40)")
    ap.add_argument("--warmup", type=int, default=-1,
                    help="untimed steps first (-1: about 100 ms of them, at least 20)")
    ap.add_argument("--config", type=int, default=2, help="workload 1..5 (default 2)")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--profile-every", type=int, default=0,
                    help="record the stage events on every n-th timed step (1 = all; "
                         "0 = about 5 of the timed steps)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration)")
    ap.add_argument("--decode", choices=("gdn", "kda"), default=None,
                    help="time the decode step (64 streams, one token each) instead")
    ap.add_argument("--gate", action="store_true",
                    help="with the output gate (gated RMSNorm of o with z)")
    ap.add_argument("--qk-heads", type=int, default=0,
                    help="q/k heads shared by the value heads (0 = as many as value heads)")
    ap.add_argument("--chunk", type=int, default=64,
                    help="rows per chunk (32 runs on the instances that have it)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(requested --gpus %d)" % args.gpus, file=sys.stderr)
        return 2

    import torch
    from gated_delta_rule_depthwise_amd import binding as B
    from gated_delta_rule_depthwise_amd import inputs
    from gated_delta_rule_depthwise_amd.runner import Decode, Prefill

    import dataclasses

    def variant(spec):
        if args.gate:
            spec = dataclasses.replace(spec, out_gate=True, name=spec.name + "-gated")
        if args.qk_heads:
            spec = dataclasses.replace(spec, Hqk=args.qk_heads,
                                       name=spec.name + "-qk%d" % args.qk_heads)
        if args.chunk != 64:
            spec = dataclasses.replace(spec, chunk=args.chunk,
                                       name=spec.name + "-c%d" % args.chunk)
        return spec

    dev = "cuda"
    if args.decode:
        spec = variant(inputs.decode_config(64, gate=args.decode))
        inp = inputs.make(spec)
        first = Decode(inp, dev)
        per_copy = sum(t.numel() * t.element_size() for t in
                       (first.x, first.g, first.beta, first.o, first.h))
    else:
        spec = variant(inputs.config(args.config))
        inp = inputs.make(spec)
        first = Prefill(inp, dev)
        per_copy = sum(t.numel() * t.element_size() for t in
                       (first.x, first.g, first.beta, first.o, first.ws))
    copies = max(1, min(8, math.ceil((1 << 30) / per_copy)))
    calls = [first] + [type(first)(inp, dev) for _ in range(copies - 1)]
    torch.cuda.synchronize()

    def run_steps(n, first_step=0):
        for i in range(first_step, first_step + n):
            rc = calls[i % copies]()
            if rc != 0:
                raise RuntimeError("libgdn status %d (%s)" % (rc, B.gdn_status_string(rc)))

    done = 0
    if args.warmup < 0 or args.steps <= 0:
        # step counts from the duration of 5 steps (clocks not yet ramped: an overestimate)
        run_steps(5)
        torch.cuda.synchronize()
        tp = time.perf_counter()
        run_steps(5, 5)
        torch.cuda.synchronize()
        done = 10
        n100 = math.ceil(0.1 / max((time.perf_counter() - tp) / 5, 1e-6))
        if args.warmup < 0:
            args.warmup = max(20, 10 + n100)
        if args.steps <= 0:
            args.steps = max(40, n100)
    run_steps(max(0, args.warmup - done), done)
    args.warmup = max(args.warmup, done)  # untimed steps run
    if args.profile_every <= 0:
        args.profile_every = max(1, args.steps // 5)
    torch.cuda.synchronize()
    B.gdn_profile_read()          # drop anything recorded so far
    torch.cuda.synchronize()
    # Stage events are recorded on every PROFILE_EVERY-th step of the timed loop: each
    # recorded event leaves the stream idle for several microseconds between two kernels,
    # which would otherwise be counted in every step's wall time.
    t0 = time.perf_counter()
    for i in range(args.steps):
        B.gdn_profile_enable(i % args.profile_every == 0)
        rc = calls[i % copies]()
        if rc != 0:
            raise RuntimeError("libgdn status %d" % rc)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    B.gdn_profile_enable(False)
    rc, ms, launches = B.gdn_profile_read()
    assert rc == 0

    if args.copy_probe:
        a = torch.empty(1 << 28, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()

    segs = 0
    if not args.decode and first.kind != B.GDN_KIND_VARLEN:
        segs = B.gdn_segments(first.params, first.plan_kind, spec.B, spec.N // spec.B,
                              first.ws_bytes)
    names = {B.GDN_PROF_FRONT: "front", B.GDN_PROF_RECUR: "recur", B.GDN_PROF_STATE: "state",
             B.GDN_PROF_GATE: "gate"}
    avg_ms = {names[i]: ms[i] / launches[i] for i in names if launches[i]}
    launches_of = {names[i]: launches[i] for i in names if launches[i]}
    call_ms = sum(avg_ms.values())  # every kernel of a call, one event pair per stage
    ms_per_step = elapsed * 1e3 / args.steps
    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        tr = json.load(open(TRAFFIC_FILE))
        ent = tr.get(spec.name, {}).get("call")
        if ent and ent.get("kernel_hash") == kernel_hash("decode" if args.decode else
                                                         "prefill"):
            traffic = ent["bytes_per_launch"]
    if args.decode:
        alg = decode_bytes(spec)["recur"]
        flops = 0
        kname = ("the whole call: decode_kernel (front end + one recurrence step + window "
                 "update, fused)")
    else:
        alg = algorithmic_bytes(spec)
        flops = algorithmic_flops(spec)
        parts = []
        if "front" in avg_ms:
            parts.append("front_kernel (float32 rows)")
        if spec.front_end and spec.dtype == "bf16":
            parts.append("chunk_kernel with the front end fused")
        else:
            parts.append("chunk_kernel")
        if segs:
            parts.append("segmented scan of %d segments: warm_boundary_kernel + pass 1 + "
                         "pass 2 (the chain of segment maps in its first workgroups); warm "
                         "starts where the gates allow" % segs)
        if "gate" in avg_ms:
            parts.append("gate_kernel")
        kname = "the whole call: " + "; ".join(parts)
    achieved = alg / (call_ms * 1e-3) / 1e9
    fp32 = spec.dtype == "f32"
    mfma_peak = FP32_PEAK_TFLOPS if fp32 else MFMA_PEAK_TFLOPS

    line = {
        "metric": DECODE_METRIC if args.decode else METRIC,
        "value": spec.N / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("%s in; fp32 arithmetic; fp32 o" % spec.dtype) if args.decode else
                 "f32 in; fp32 MFMA and VALU; fp32 o" if fp32 else
                 "bf16 in; fp16 MFMA operands (hi + lo pairs where a single rounding would "
                 "show), fp32 accumulate and VALU; fp32 o",
        "data": "synthetic (seeded; distributions of the workload description)",
        "config": {"workload": spec.name, "tokens": spec.N, "streams": spec.B, "H": spec.H,
                   "dk": spec.dk, "dv": spec.dv, "chunk": spec.chunk, "gate": spec.gate,
                   "front_end": spec.front_end, "output_gate": spec.out_gate,
                   "qk_heads": spec.qk_heads,
                   "input_copies_rotated": copies},
        "roofline": {"bound": "hbm",
                     "kernel": kname,
                     "achieved": achieved,
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic, "algorithmic_bytes_per_launch": alg,
                     "avg_launch_ms": call_ms,
                     "timed_launches": max(launches_of.values()),
                     "frac_wall": alg / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
                     "mfma": {"algorithmic_flops_per_launch": flops,
                              "achieved_tflops": flops / (call_ms * 1e-3) / 1e12,
                              "peak_tflops": mfma_peak,
                              "frac": flops / (call_ms * 1e-3) / 1e12 / mfma_peak},
                     "stage_ms": avg_ms},
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(spec, inp, args.cpu_budget)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
