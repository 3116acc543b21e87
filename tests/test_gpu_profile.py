"""Stage timers: with profiling on, each stage of a call files exactly one start/end event
pair, every pair reads a positive time no longer than the call's wall time, and the results
are bit-identical to an untimed call."""
import time

import pytest
import torch

from gated_delta_rule_depthwise_amd import binding as B
from gated_delta_rule_depthwise_amd import inputs
from gated_delta_rule_depthwise_amd.runner import Decode, Prefill
from tests.gpu_util import spec_small

pytestmark = pytest.mark.gpu


def timed(call):
    B.gdn_profile_read()
    B.gdn_profile_enable(True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    rc = call()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3
    B.gdn_profile_enable(False)
    prc, ms, launches = B.gdn_profile_read()
    assert rc == 0 and prc == 0
    return ms, launches, wall_ms


@pytest.mark.parametrize("case", ["segmented-front", "f32-front", "varlen", "gated-pass"])
def test_prefill_stage_timers(case):
    if case == "segmented-front":   # bf16 rows: warm plan, chunk passes (front end fused), chain
        spec = spec_small(2, lengths=[2048], H=4, seed=61)
        stages = {B.GDN_PROF_RECUR}
    elif case == "f32-front":       # float32 rows: the front kernel, then the chunk kernel
        spec = spec_small(2, lengths=[300], H=2, dk=64, dv=64, dtype="f32", seed=64)
        stages = {B.GDN_PROF_FRONT, B.GDN_PROF_RECUR}
    elif case == "varlen":          # stream ranking + chunk kernel, no front end
        spec = spec_small(4, lengths=[1, 300, 64, 129], H=2, seed=62)
        stages = {B.GDN_PROF_RECUR}
    else:                           # output gate in its own pass (per-channel gate, d=128)
        spec = spec_small(5, lengths=[200], H=2, out_gate=True, seed=63)
        stages = {B.GDN_PROF_RECUR, B.GDN_PROF_GATE}
    inp = inputs.make(spec)
    ref = Prefill(inp, "cuda")
    assert ref() == 0
    call = Prefill(inp, "cuda")
    ms, launches, wall_ms = timed(call)
    for s in range(B.GDN_PROF_BUCKETS):
        assert launches[s] == (1 if s in stages else 0), (s, launches)
        if s in stages:
            assert 0.0 < ms[s] <= wall_ms, (s, ms[s], wall_ms)
    torch.cuda.synchronize()
    assert torch.equal(call.o, ref.o) and torch.equal(call.h, ref.h)
    if ref.conv_state is not None:
        assert torch.equal(call.conv_state, ref.conv_state)


@pytest.mark.parametrize("shared", [False, True])
def test_decode_stage_timer(shared):
    """Decode is one stage of one kernel, or two with shared q/k heads (the q/k window
    pass): one pair either way."""
    import dataclasses
    spec = dataclasses.replace(inputs.decode_config(4), H=4, Hqk=2 if shared else 0, seed=64)
    inp = inputs.make(spec)
    ref = Decode(inp, "cuda")
    assert ref() == 0
    dec = Decode(inp, "cuda")
    ms, launches, wall_ms = timed(dec)
    assert launches[B.GDN_PROF_RECUR] == 1 and sum(launches) == 1
    assert 0.0 < ms[B.GDN_PROF_RECUR] <= wall_ms
    torch.cuda.synchronize()
    assert torch.equal(dec.o, ref.o) and torch.equal(dec.h, ref.h)
