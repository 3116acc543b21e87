"""Debug validation of device-side inputs (gdn_debug_validate): malformed cu_seqlens and
per-key-channel log-gates that are not a decay are reported in the status word, and the
call then leaves every buffer as it was. Every malformed cu_seqlens here keeps its rows
inside the buffers, so a call that did run could not read or write outside them."""
import dataclasses

import pytest
import torch

from gated_delta_rule_depthwise_amd import binding as B
from gated_delta_rule_depthwise_amd import inputs
from gated_delta_rule_depthwise_amd.runner import Prefill
from tests.gpu_util import SENTINEL, compare, run_oracle, spec_small

pytestmark = pytest.mark.gpu


@pytest.fixture
def status():
    st = torch.zeros(1, dtype=torch.int32, device="cuda")
    B.gdn_debug_validate(st)
    yield st
    B.gdn_debug_validate(None)


def _untouched(call, before):
    for a, b in zip((call.o, call.h) + ((call.conv_state,) if call.conv_state is not None
                                        else ()), before):
        assert torch.equal(a, b)


def _snapshot(call):
    return [t.clone() for t in (call.o, call.h) +
            ((call.conv_state,) if call.conv_state is not None else ())]


@pytest.mark.parametrize("gate", ["gdn", "kda"])
def test_valid_calls_pass_and_match(status, gate):
    spec = spec_small(2, lengths=[70, 0, 130], H=2, gate=gate, seed=81)
    inp = inputs.make(spec)
    call = Prefill(inp, "cuda", o_fill=SENTINEL)
    assert call() == 0
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    compare(call, run_oracle(inp))


@pytest.mark.parametrize("case,bit", [("start", B.GDN_BAD_CU_START),
                                      ("order", B.GDN_BAD_CU_ORDER),
                                      ("total", B.GDN_BAD_CU_TOTAL),
                                      ("maxlen", B.GDN_BAD_CU_MAXLEN)])
def test_malformed_cu_seqlens(status, case, bit):
    spec = spec_small(2, lengths=[50, 80, 70], H=2, seed=82)
    inp = inputs.make(spec)
    call = Prefill(inp, "cuda", o_fill=SENTINEL)
    max_seqlen = max(spec.lengths)
    if case == "start":
        call.cu[0] = 5
    elif case == "order":
        call.cu[1] = 140   # 140 > cu[2] = 130: stream 1 runs backwards
        max_seqlen = spec.N  # (stream 0, now 140 tokens, within the bound)
    elif case == "total":
        call.cu[3] = spec.N - 10
    else:
        max_seqlen = 60    # stream 1 has 80 tokens
    torch.cuda.synchronize()
    before = _snapshot(call)
    s = torch.cuda.current_stream().cuda_stream
    rc = B.gdn_prefill_varlen(call.params, call.q_ptr, call.k_ptr, call.v_ptr, call.g,
                              call.beta, call.h_ptrs, call.cs_ptrs, call.conv_w, call.o,
                              call.cu, spec.B, spec.N, max_seqlen, call.ws, call.ws_bytes, s)
    assert rc == 0
    torch.cuda.synchronize()
    assert int(status.item()) == bit
    _untouched(call, before)


def test_kda_gate_not_a_decay(status):
    spec = spec_small(5, lengths=[150], H=2, seed=83)
    inp = inputs.make(spec)
    inp["g"][100, 1, 7] = 0.25                 # one positive log-gate in a real row
    call = Prefill(inp, "cuda", o_fill=SENTINEL)
    torch.cuda.synchronize()
    before = _snapshot(call)
    assert call() == 0
    torch.cuda.synchronize()
    assert int(status.item()) == B.GDN_BAD_KDA_GATE
    _untouched(call, before)
    # past the last real row the gates are never read, so they are not checked either
    status.zero_()
    ok = dataclasses.replace(spec, pad_fill=float("nan"))
    inp2 = inputs.make(ok)
    call2 = Prefill(inp2, "cuda", o_fill=SENTINEL)
    assert call2() == 0
    torch.cuda.synchronize()
    assert int(status.item()) == 0
    compare(call2, run_oracle(inp2))
