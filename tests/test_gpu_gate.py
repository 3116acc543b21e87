"""Parity of the output gate (gated RMSNorm of o with z) with the oracle.

The reference output is the oracle's o passed through the oracle's gated RMSNorm. Where the
chunk kernel stages whole o rows the gate runs in its o flush, with z from an LDS tile or,
in the scalar gate's fused front end, from registers; the per-key-channel instances at
dk = dv = 128 and in fp32 run it as its own pass (gate_kernel); the decode kernel applies
it to the row it finishes. Every kind is covered below.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
from gated_delta_rule_depthwise_amd import binding as B
from gated_delta_rule_depthwise_amd import inputs
from gated_delta_rule_depthwise_amd.runner import Decode
from tests.gpu_util import compare, rel_err, run_gpu, run_oracle, spec_small

pytestmark = pytest.mark.gpu


def gated(inp, ref, heads=None):
    """``ref`` with o replaced by the oracle's gated RMSNorm of it; ``o_metric`` is the
    error measure for the gated rows (see gated_err)."""
    spec = inp["spec"]
    heads = list(range(spec.H)) if heads is None else list(heads)
    z = inp["z"][:spec.N][:, heads]
    out = dict(ref)
    out["o"] = oracle.gated_rmsnorm(ref["o"], z, inp["norm_w"], spec.norm_eps)
    out["o_metric"] = lambda got, want: gated_err(got, want, ref["o"], z, inp["norm_w"],
                                                  spec.norm_eps)
    return out


def gated_err(y, y_ref, o_ref, z, w, eps):
    """The o bar carried through the gate. If |o - o_ref| <= e RMS(o_ref) elementwise, then
    to first order the gated row y = o / rms_r * c (c = w silu(z), rms_r the row's root mean
    square) moves by at most e RMS(o_ref) / rms_r (|c| + |y|): the first term from the
    element itself, the second from the row's rms. This returns the smallest e that covers
    every element, to be held to the same bar as o. (max|dy| / RMS(y) is no fit here: the
    gate multiplies by |w silu(z)| up to about 7 while dividing rows of small rms by it.)"""
    o_ref = np.asarray(o_ref, np.float64)
    y = np.asarray(y, np.float64)
    if not np.all(np.isfinite(y)):
        return float("inf")
    zz = z.double().numpy() if hasattr(z, "double") else np.asarray(z, np.float64)
    c = np.asarray(w.double().numpy() if hasattr(w, "double") else w, np.float64) * \
        zz / (1.0 + np.exp(-zz))
    rms_r = np.sqrt((o_ref * o_ref).mean(-1, keepdims=True) + eps)
    scale = np.sqrt((o_ref * o_ref).mean()) / rms_r * (np.abs(c) + np.abs(y_ref))
    d = np.abs(y - y_ref)
    # where the gate factor is 0 (z = 0) the gated value must be exactly 0
    err = np.where(scale > 0, d / np.where(scale > 0, scale, 1.0), np.where(d == 0, 0.0, np.inf))
    return float(np.max(err))


CASES = {
    "gdn-bf16-front-d128": dict(base=2, lengths=[777], H=4),
    "gdn-bf16-front-d64": dict(base=2, lengths=[777], H=4, dk=64, dv=64),
    "gdn-bf16-d128": dict(base=3, lengths=[300], H=3),
    "gdn-f32-d64": dict(base=1, lengths=[333], H=2, h0_std=0.1),
    "kda-bf16-front-d128": dict(base=5, lengths=[500], H=2),
    "kda-bf16-d64": dict(base=5, lengths=[400], H=2, dk=64, dv=64, front_end=False),
    "kda-f32-d64": dict(base=1, lengths=[300], H=2, gate="kda"),
    "gdn-bf16-batched": dict(base=3, lengths=[256] * 3, H=2),
    "gdn-bf16-varlen": dict(base=4, lengths=[1, 63, 64, 65, 200], H=2),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_gated_prefill_matches_oracle(name):
    kw = dict(CASES[name])
    base = kw.pop("base")
    spec = spec_small(base, out_gate=True, seed=21, **kw)
    inp = inputs.make(spec)
    if len(set(spec.lengths)) > 1:   # NaN in every per-token array past the last row
        inp = inputs.refill_tails(inp, float("nan"))
    call = run_gpu(inp)
    ref = gated(inp, run_oracle(inp))
    compare(call, ref, o_metric=ref["o_metric"])


def test_gate_pass_only_where_o_is_not_staged():
    """The per-key-channel instances at 128 columns and in fp32, and calls whose front end
    runs inside the scan with the per-key-channel gate, gate in a pass of their own; the
    others gate in the o flush (with the scalar gate's fused front end, z in registers: its
    tiles leave no room for a z tile) and record nothing in that profile bucket."""
    for base, kw, want in ((5, dict(lengths=[200], H=2), 1),
                           (5, dict(lengths=[200], H=2, front_end=False), 1),
                           (1, dict(lengths=[200], H=2, gate="kda"), 1),
                           (1, dict(lengths=[200], H=2), 0),
                           (3, dict(lengths=[200], H=2), 0),
                           (2, dict(lengths=[200], H=2), 0),
                           (2, dict(lengths=[200], H=2, dk=64, dv=64), 0)):
        spec = spec_small(base, out_gate=True, seed=22, **kw)
        inp = inputs.make(spec)
        B.gdn_profile_read()
        B.gdn_profile_enable(True)
        call = run_gpu(inp)
        B.gdn_profile_enable(False)
        rc, _, launches = B.gdn_profile_read()
        assert rc == 0 and launches[B.GDN_PROF_GATE] == want
        ref = gated(inp, run_oracle(inp))
        compare(call, ref, o_metric=ref["o_metric"])


def test_gated_segmented_scan():
    """A long single stream takes the segmented scan (two chunk-kernel passes that both
    write o); the gate applies in both."""
    spec = spec_small(2, lengths=[4096], H=4, out_gate=True, gate_dist="slow", seed=23)
    inp = inputs.make(spec)
    call = run_gpu(inp)
    assert B.gdn_segments(call.params, call.plan_kind, 1, 4096, call.ws_bytes) >= 3
    ref = gated(inp, run_oracle(inp))
    compare(call, ref, o_metric=ref["o_metric"])


def test_gated_full_size_sampled_heads():
    """The default prefill workload (T=4096, H=32, front end) with the gate, heads sampled."""
    spec = dataclasses.replace(inputs.config(2), out_gate=True)
    inp = inputs.make(spec)
    call = run_gpu(inp)
    heads = [0, 31]
    ref = gated(inp, run_oracle(inp, heads=heads), heads)
    compare(call, ref, heads=heads, o_metric=ref["o_metric"])


DECODE = [dict(), dict(gate="kda"), dict(dk=64, dv=64, dtype="f32", front_end=False)]


@pytest.mark.parametrize("kw", DECODE, ids=["gdn", "kda", "f32-d64"])
def test_gated_decode_matches_oracle(kw):
    spec = dataclasses.replace(inputs.decode_config(6), H=3, out_gate=True, seed=25, **kw)
    inp = inputs.make(spec)
    dec = Decode(inp, "cuda")
    assert dec() == 0
    torch.cuda.synchronize()
    ref = gated(inp, run_oracle(inp))
    assert ref["o_metric"](dec.o.cpu().numpy(), ref["o"]) <= 1e-4
    assert rel_err(dec.h.cpu().numpy(), ref["h"]) <= 1e-4


def test_gated_decode_steps_equal_gated_prefill():
    """T gated decode calls give the gated o rows of a T-token prefill."""
    Bn, T, H = 2, 16, 2
    pre = dataclasses.replace(inputs.config(3), name="steps", lengths=[T] * Bn, H=H,
                              front_end=True, gate_dist="slow", out_gate=True, seed=26)
    inp = inputs.make(pre)
    ref = gated(inp, run_oracle(inp))
    dinp = dict(inp)
    dinp["spec"] = dataclasses.replace(pre, lengths=[1] * Bn)
    dec = Decode(dinp, "cuda")
    x = inp["x"].cuda()
    N = Bn * T
    g = inp["g"][:N].reshape(Bn, T, H)
    beta = inp["beta"][:N].reshape(Bn, T, H)
    o = np.empty((Bn, T, H, pre.dv))
    for t in range(T):
        assert dec.step(x, t, T, g[:, t].contiguous().cuda(),
                        beta[:, t].contiguous().cuda()) == 0
        o[:, t] = dec.o.cpu().numpy()
    assert ref["o_metric"](o.reshape(N, H, pre.dv), ref["o"]) <= 1e-4
