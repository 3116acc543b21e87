"""dv = 2 dk: value heads twice as wide as key heads (the chunk kernel covers one (stream,
head) with two column slices; the scan runs unsegmented and the output gate runs as its
own pass), against the oracle."""
import dataclasses

import pytest
import torch

from gated_delta_rule_depthwise_amd import binding as B
from gated_delta_rule_depthwise_amd import inputs
from gated_delta_rule_depthwise_amd.runner import Decode
from tests.gpu_util import compare, rel_err, run_gpu, run_oracle, spec_small
from tests.test_gpu_gate import gated

pytestmark = pytest.mark.gpu

CASES = {
    "gdn-bf16-front-128x256": dict(base=2, lengths=[333], H=2, dk=128, dv=256),
    "gdn-bf16-128x256-qk1": dict(base=3, lengths=[200], H=2, Hqk=1, dk=128, dv=256),
    "kda-bf16-front-128x256": dict(base=5, lengths=[200], H=2, dk=128, dv=256),
    "gdn-bf16-varlen-128x256": dict(base=4, lengths=[1, 65, 130], H=2, dk=128, dv=256),
    "gdn-f32-64x128": dict(base=1, lengths=[300], H=2, dk=64, dv=128),
    "kda-f32-front-64x128": dict(base=1, lengths=[200], H=2, dk=64, dv=128, gate="kda",
                                 front_end=True),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_wide_values_match_oracle(name):
    kw = dict(CASES[name])
    base = kw.pop("base")
    spec = spec_small(base, seed=41, **kw)
    inp = inputs.make(spec)
    if len(set(spec.lengths)) > 1:
        inp = inputs.refill_tails(inp, float("nan"))
    call = run_gpu(inp)
    if call.kind != B.GDN_KIND_VARLEN:
        assert B.gdn_segments(call.params, call.plan_kind, spec.B, spec.N // spec.B,
                              call.ws_bytes) == 0
    compare(call, run_oracle(inp))


def test_wide_values_long_stream_unsegmented():
    """A stream long enough to segment at dk = dv runs serially here, and matches."""
    spec = spec_small(2, lengths=[2048], H=2, dk=128, dv=256, gate_dist="slow", seed=42)
    inp = inputs.make(spec)
    call = run_gpu(inp)
    compare(call, run_oracle(inp))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_wide_values_gated(dtype):
    kw = dict(dk=128, dv=256) if dtype == "bf16" else dict(dk=64, dv=128, dtype="f32")
    spec = spec_small(2, lengths=[200], H=2, out_gate=True, seed=43, **kw)
    inp = inputs.make(spec)
    B.gdn_profile_read()
    B.gdn_profile_enable(True)
    call = run_gpu(inp)
    B.gdn_profile_enable(False)
    rc, _, launches = B.gdn_profile_read()
    assert rc == 0 and launches[B.GDN_PROF_GATE] == 1
    ref = gated(inp, run_oracle(inp))
    compare(call, ref, o_metric=ref["o_metric"])


@pytest.mark.parametrize("kw", [dict(dk=128, dv=256), dict(dk=128, dv=256, gate="kda"),
                                dict(dk=64, dv=128, dtype="f32", front_end=False),
                                dict(dk=128, dv=256, out_gate=True)],
                         ids=["gdn-128x256", "kda-128x256", "gdn-f32-64x128", "gated-128x256"])
def test_wide_values_decode(kw):
    spec = dataclasses.replace(inputs.decode_config(5), H=3, seed=44, **kw)
    inp = inputs.make(spec)
    dec = Decode(inp, "cuda")
    assert dec() == 0
    torch.cuda.synchronize()
    ref = run_oracle(inp)
    if spec.out_gate:
        ref = gated(inp, ref)
        assert ref["o_metric"](dec.o.cpu().numpy(), ref["o"]) <= 1e-4
    else:
        assert rel_err(dec.o.cpu().numpy(), ref["o"]) <= 1e-4
    assert rel_err(dec.h.cpu().numpy(), ref["h"]) <= 1e-4
    if ref["conv_state"] is not None:
        cs = dec.conv_state[:, torch.as_tensor(ref["channels"], device="cuda")]
        assert torch.equal(cs.cpu(), torch.from_numpy(ref["conv_state"]).to(cs.dtype))
