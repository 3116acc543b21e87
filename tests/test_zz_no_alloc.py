"""gdn_prefill_noalloc, the allocation-free variant of gdn_prefill, through the C ABI.

Two calls in a row on one device, the second smaller than the first: each must give what
gdn_prefill gives on the same inputs (bit for bit: the same launches on the same data, its
workspace being the library's device array instead of the caller's) and match the oracle.
"""
import pytest
import torch

from gated_delta_rule_depthwise_amd import binding as B
from gated_delta_rule_depthwise_amd import inputs
from gated_delta_rule_depthwise_amd.runner import Prefill
from tests.gpu_util import SENTINEL, compare, run_oracle, spec_small

pytestmark = pytest.mark.gpu


def _noalloc(call):
    s = torch.cuda.current_stream().cuda_stream
    return B.gdn_prefill_noalloc(call.params, call.q_ptr, call.k_ptr, call.v_ptr, call.g,
                                 call.beta, call.h, call.conv_state, call.conv_w, call.o,
                                 call.spec.N, s)


def test_noalloc_matches_prefill_on_two_calls():
    specs = (inputs.config(2),                               # T=4096, H=32: segmented scan
             spec_small(2, lengths=[700], H=2, seed=72))     # then a smaller call
    for spec in specs:
        inp = inputs.make(spec)
        want = Prefill(inp, "cuda", o_fill=SENTINEL)
        assert want() == 0
        got = Prefill(inp, "cuda", o_fill=SENTINEL)
        rc = _noalloc(got)
        torch.cuda.synchronize()
        assert rc == 0, B.gdn_status_string(rc)
        assert torch.equal(got.o, want.o), spec.name
        assert torch.equal(got.h, want.h), spec.name
        assert torch.equal(got.conv_state, want.conv_state), spec.name
        e_o, e_h = compare(got, run_oracle(inp))
        print("%s: err(o)=%.3g err(h)=%.3g" % (spec.name, e_o, e_h), flush=True)
