"""Helpers shared by the GPU parity tests: run a workload through the C ABI and through the
oracle on the same seeded inputs, and compare."""
import dataclasses

import numpy as np
import torch

import oracle
from gated_delta_rule_depthwise_amd import inputs
from gated_delta_rule_depthwise_amd.runner import Prefill

TOL = {"f32": 1e-4, "bf16": 2e-2}  # max |gpu - oracle| / RMS(oracle)
SENTINEL = -12345.0                 # o rows the call must not write


def rel_err(got, ref):
    """max |got - ref| / RMS(ref) over the given entries; inf if got has NaN/Inf."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if not np.all(np.isfinite(got)):
        return float("inf")
    rms = np.sqrt(np.mean(ref * ref))
    return float(np.max(np.abs(got - ref)) / max(rms, 1e-30))


def spec_small(base: int, **kw):
    """Workload ``base`` with some fields replaced; the name records the changes."""
    tag = ",".join("%s=%s" % (k, v if k != "lengths" else (v if len(v) < 5 else "%d streams" % len(v)))
                   for k, v in sorted(kw.items()) if k != "seed")
    spec = dataclasses.replace(inputs.config(base), **kw)
    return dataclasses.replace(spec, name="cfg%d[%s]" % (base, tag))


def run_gpu(inp, mode=None, o_fill=SENTINEL, **kw):
    call = Prefill(inp, "cuda", mode=mode, o_fill=o_fill, **kw)
    rc = call()
    torch.cuda.synchronize()
    assert rc == 0, "libgdn status %d" % rc
    return call


def run_oracle(inp, heads=None, eps=None, scale=None, l2=None):
    spec = inp["spec"]
    eps = spec.eps if eps is None else eps
    return oracle.prefill(
        inp["x"], inp["g"], inp["beta"], inp["h0"], H=spec.H, dk=spec.dk, dv=spec.dv,
        cu_seqlens=inp["cu_seqlens"].numpy(), conv_w=inp["conv_w"],
        conv_state=inp["conv_state"], l2=(eps >= 0) if l2 is None else l2, eps=max(eps, 0.0),
        scale=spec.scale if scale is None else scale, heads=heads, Hqk=spec.qk_heads)


def compare(call, ref, heads=None, tol=None, o_metric=None):
    """Parity of o (real rows), every final h and the conv windows; returns the errors.
    ``o_metric(got, ref)`` replaces max|got - ref| / RMS(ref) for o."""
    spec = call.spec
    heads = list(range(spec.H)) if heads is None else list(heads)
    tol = TOL[spec.dtype] if tol is None else tol
    N = spec.N
    o = call.o[:N, heads].float().cpu().numpy()
    e_o = (o_metric or rel_err)(o, ref["o"])
    h = call.h[:, heads].cpu().numpy()
    e_h = rel_err(h, ref["h"])
    assert e_o <= tol, "o error %.3g > %.3g" % (e_o, tol)
    assert e_h <= tol, "h error %.3g > %.3g" % (e_h, tol)
    # rows the call must not write keep the sentinel bit for bit
    tail = call.o[N:].float()
    assert bool((tail == SENTINEL).all()), "o written past the last real row"
    if ref["conv_state"] is not None:
        cs = call.conv_state[:, torch.as_tensor(ref["channels"], device=call.conv_state.device)]
        want = torch.from_numpy(ref["conv_state"]).to(cs.dtype)
        assert torch.equal(cs.cpu(), want), "conv window differs"
    return e_o, e_h
