"""A call captured in a HIP graph (torch.cuda.CUDAGraph) and replayed gives the eager
result on every replay. The library records nothing but kernel launches on the call's
stream (no memsets, no allocation, no host synchronisation), so a serving loop can
capture a prefill or a decode step once and replay it. Between replays the states are
restored eagerly and the program does other GPU work."""
import dataclasses

import pytest
import torch

from gated_delta_rule_depthwise_amd import inputs
from gated_delta_rule_depthwise_amd.runner import Decode, Prefill
from tests.gpu_util import spec_small

pytestmark = pytest.mark.gpu


def _capture_and_replay(call, outputs, replays=3):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call.reset()
        assert call() == 0                      # warm-up (first-use setup) outside capture
    torch.cuda.synchronize()
    want = [t.clone() for t in outputs()]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        rc = call()
    assert rc == 0
    for i in range(replays):
        for t in outputs():                     # scribble over the outputs eagerly
            t.fill_(float("nan")) if t.is_floating_point() else t.zero_()
        call.reset()
        torch.cuda.synchronize()
        torch.randn(1 << 20, device="cuda").sum()   # unrelated eager work in between
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(outputs(), want):
            assert torch.equal(a, b), "replay %d differs" % i


@pytest.mark.parametrize("base,kw", [
    (2, dict(lengths=[4096], H=4, gate_dist="slow")),     # front end + segmented scan
    (5, dict(lengths=[300], H=2, out_gate=True)),         # KDA + gate pass
    (4, dict(lengths=[1, 64, 65, 200], H=2)),             # varlen
], ids=["gdn-front-segmented", "kda-gated", "varlen"])
def test_prefill_graph_replay(base, kw):
    spec = spec_small(base, seed=51, **kw)
    call = Prefill(inputs.make(spec), "cuda")

    def outputs():  # o rows past the last real row are never written
        out = [call.o[:spec.N], call.h]
        return out + ([call.conv_state] if call.conv_state is not None else [])
    _capture_and_replay(call, outputs)


def test_decode_graph_replay():
    spec = dataclasses.replace(inputs.decode_config(16), H=4, Hqk=2, out_gate=True, seed=52)
    dec = Decode(inputs.make(spec), "cuda")
    _capture_and_replay(dec, lambda: [dec.o, dec.h, dec.conv_state])
