"""GPU parity at the workloads' full sizes, in the launch configuration bench.py times.

The whole call runs on every head; the fp64 oracle recomputes a sample of heads (each head
is independent, so its outputs are computable one head at a time) and the errors are taken
over those heads. conv windows and untouched o rows are checked on every channel/row.
"""
import numpy as np
import pytest
import torch

from gated_delta_rule_depthwise_amd import inputs
from tests.gpu_util import compare, run_gpu, run_oracle

pytestmark = pytest.mark.gpu

HEADS = [0, 13, 31]


def _full(i, heads=HEADS, fill=0.0):
    spec = inputs.config(i, pad_fill=fill)
    inp = inputs.make(spec)
    call = run_gpu(inp)
    ref = run_oracle(inp, heads=heads)
    e_o, e_h = compare(call, ref, heads=heads)
    print("%s: err(o)=%.3g err(h)=%.3g" % (spec.name, e_o, e_h), flush=True)
    return inp, call


def test_config2_front_end_T4096():
    inp, call = _full(2)
    # every channel's conv window: the last 3 raw rows
    want = inp["x"][4093:4096].t().contiguous()
    assert torch.equal(call.conv_state[0].cpu(), want)


def test_config3_batched_8x2048():
    _full(3)


@pytest.mark.parametrize("fill", [float("nan"), 1e30])
def test_config4_varlen_tails(fill):
    _full(4, heads=[0, 31], fill=fill)
