"""GPU parity of the per-key-channel gate (KDA) against the fp64 oracle."""
import dataclasses

import numpy as np
import pytest
import torch

from gated_delta_rule_depthwise_amd import inputs
from tests.gpu_util import compare, rel_err, run_gpu, run_oracle, spec_small

pytestmark = pytest.mark.gpu


def _case(spec, mode=None, heads=None):
    inp = inputs.make(spec)
    call = run_gpu(inp, mode=mode)
    ref = run_oracle(inp, heads=heads)
    errs = compare(call, ref, heads=heads)
    print("%s mode=%s err(o)=%.3g err(h)=%.3g" % (spec.name, call.mode, *errs), flush=True)
    return inp, call


@pytest.mark.parametrize("T", [1, 17, 64, 65, 200])
def test_kda_bf16_ragged(T):
    _case(spec_small(5, lengths=[T], H=2, front_end=False, seed=50 + T))


def test_kda_front_end_small():
    _case(spec_small(5, lengths=[300], H=2, seed=51))


def test_kda_f32_d64():
    _case(spec_small(1, lengths=[150], gate="kda", gate_dist="softplus", h0_std=0.1,
                     seed=52))


def test_kda_bf16_d64():
    _case(spec_small(5, lengths=[130], H=4, dk=64, dv=64, front_end=False, seed=53))


def test_kda_batched_and_varlen():
    _case(spec_small(5, lengths=[70] * 3, H=2, front_end=False, seed=54))
    _case(spec_small(5, lengths=[5, 64, 0, 100], H=2, front_end=False, seed=55,
                     pad_fill=float("nan")), mode="varlen")


def test_kda_strong_uniform_decay():
    """Per-channel gates far stronger than the workload's: still within tolerance."""
    spec = spec_small(5, lengths=[128], H=2, front_end=False, seed=56)
    inp = inputs.make(spec)
    inp["g"] = inp["g"] * 4.0
    call = run_gpu(inp)
    compare(call, run_oracle(inp))
