"""Seeded workload generators: shapes, determinism, forced lengths, tail fill (CPU)."""
import dataclasses

import numpy as np
import torch

from gated_delta_rule_depthwise_amd import inputs


def test_varlen_lengths_forced_and_total():
    lens = inputs.varlen_lengths()
    assert len(lens) == 16
    for v in (1, 63, 64, 65):
        assert v in lens
    assert 61440 <= sum(lens) <= 69632
    assert all(1 <= v <= 8192 for v in lens)
    assert inputs.varlen_lengths() == lens


def test_small_spec_shapes_and_determinism():
    spec = dataclasses.replace(inputs.config(2), lengths=[100], H=2, dk=16, dv=8)
    a, b = inputs.make(spec), inputs.make(spec)
    assert a["x"].shape == (spec.alloc, 2 * 2 * 16 + 2 * 8)
    assert a["x"].dtype == torch.bfloat16
    assert a["conv_w"].shape == (spec.cd, 4) and a["conv_state"].shape == (1, spec.cd, 3)
    assert a["g"].shape == (spec.alloc, 2) and a["beta"].shape == (spec.alloc, 2)
    assert a["h0"].shape == (1, 2, 16, 8)
    for key in ("x", "g", "beta", "h0", "conv_w", "conv_state"):
        assert torch.equal(a[key], b[key])
    assert float(a["g"][:100].max()) < 0 and float(a["beta"][:100].min()) > 0


def test_tails_hold_fill():
    spec = dataclasses.replace(inputs.config(3), lengths=[70, 5], H=2, dk=16, dv=16,
                               gate="kda")
    a = inputs.make(spec)
    n = inputs.refill_tails(a, float("nan"))
    assert torch.isnan(n["x"][75:].float()).all() and torch.isnan(n["g"][75:]).all()
    assert torch.equal(n["x"][:75], a["x"][:75])
    assert a["g"].shape == (spec.alloc, 2, 16)
    assert a["cu_seqlens"].tolist() == [0, 70, 75]


def test_full_configs_described():
    for i in range(1, 6):
        s = inputs.config(i)
        assert s.chunk == 64
    assert inputs.config(1).dtype == "f32" and inputs.config(1).H == 2
    assert inputs.config(5).gate == "kda" and inputs.config(5).N == 16384
    assert inputs.config(3).B == 8 and inputs.config(3).N == 16384
