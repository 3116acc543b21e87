"""Shared q/k heads (Hqk < H): value head h reads q/k head h // (H / Hqk), through every
entry point, against the oracle (which gathers the same q/k columns for each value head)."""
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

CASES = {
    "gdn-bf16-front-H8-qk2": dict(base=2, lengths=[300], H=8, Hqk=2),
    "gdn-bf16-H6-qk3": dict(base=3, lengths=[200], H=6, Hqk=3),
    "gdn-f32-d64-H4-qk1": dict(base=1, lengths=[150], H=4, Hqk=1),
    "kda-bf16-front-H4-qk2": dict(base=5, lengths=[200], H=4, Hqk=2),
    "gdn-bf16-batched-front": dict(base=2, lengths=[128] * 3, H=4, Hqk=2),
    "gdn-bf16-varlen-front": dict(base=2, lengths=[1, 64, 65, 130], H=4, Hqk=2),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_shared_qk_prefill_matches_oracle(name):
    kw = dict(CASES[name])
    base = kw.pop("base")
    spec = spec_small(base, seed=31, **kw)
    inp = inputs.make(spec)
    if len(set(spec.lengths)) > 1:
        inp = inputs.refill_tails(inp, float("nan"))
    call = run_gpu(inp)
    compare(call, run_oracle(inp))


def test_shared_qk_segmented_scan():
    spec = spec_small(2, lengths=[4096], H=4, Hqk=2, gate_dist="slow", seed=32)
    inp = inputs.make(spec)
    call = run_gpu(inp)
    assert B.gdn_segments(call.params, call.plan_kind, 1, 4096, call.ws_bytes) >= 3
    compare(call, run_oracle(inp))


def test_shared_qk_full_size_sampled_heads():
    """T=4096 with the front end, 16 q/k heads for 32 value heads; heads sampled so that
    two value heads share a q/k head."""
    spec = dataclasses.replace(inputs.config(2), Hqk=16, seed=33)
    inp = inputs.make(spec)
    call = run_gpu(inp)
    heads = [0, 1, 30]
    compare(call, run_oracle(inp, heads=heads), heads=heads)


@pytest.mark.parametrize("kw", [dict(), dict(gate="kda"), dict(front_end=False)],
                         ids=["gdn-front", "kda-front", "gdn"])
def test_shared_qk_decode_matches_oracle(kw):
    """The q/k windows are read by every value head of a group and advanced by a pass of
    their own after the step; compared bit for bit."""
    spec = dataclasses.replace(inputs.decode_config(5), H=8, Hqk=2, seed=34, **kw)
    inp = inputs.make(spec)
    dec = Decode(inp, "cuda")
    assert dec() == 0
    torch.cuda.synchronize()
    ref = run_oracle(inp)
    assert rel_err(dec.o.cpu().numpy(), ref["o"]) <= 1e-4
    assert rel_err(dec.h.cpu().numpy(), ref["h"]) <= 1e-4
    if ref["conv_state"] is not None:
        cs = dec.conv_state[:, torch.as_tensor(ref["channels"], device="cuda")]
        assert torch.equal(cs.cpu(), torch.from_numpy(ref["conv_state"]).to(cs.dtype))


def test_shared_qk_decode_steps_equal_prefill():
    Bn, T, H = 3, 12, 4
    pre = dataclasses.replace(inputs.config(3), name="steps", lengths=[T] * Bn, H=H, Hqk=2,
                              front_end=True, gate_dist="slow", seed=35)
    inp = inputs.make(pre)
    ref = run_oracle(inp)
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
    assert rel_err(o.reshape(N, H, pre.dv), ref["o"]) <= 1e-4
    assert rel_err(dec.h.cpu().numpy(), ref["h"]) <= 1e-4
    cs = dec.conv_state[:, torch.as_tensor(ref["channels"], device="cuda")]
    assert torch.equal(cs.cpu(), torch.from_numpy(ref["conv_state"]).to(cs.dtype))
