"""Chunk-size invariance on the GPU. The chunked scan computes the token-by-token recurrence
for any chunk length, so the 32-row instances must match the oracle as the 64-row ones do,
and the two runs may differ by rounding only. The cases span several chunks and a ragged
tail: single, batched and varlen streams (with streams of 1, 31, 32, 33, 63, 64 and 65
tokens), both gates, bf16 and fp32 rows, and the fp32 front end. (32-row chunks run on the
register path; the fused bf16 front end and the fused output gate have 64-row instances
only, and a call asking for 32 rows there is refused: see test_abi.)"""
import dataclasses

import pytest
import torch

from gated_delta_rule_depthwise_amd import inputs
from tests.gpu_util import compare, rel_err, run_gpu, run_oracle, spec_small

pytestmark = pytest.mark.gpu

CASES = {
    "gdn-bf16-d128-T300": lambda: spec_small(3, lengths=[300], H=4, seed=80),
    "kda-bf16-d128-T300": lambda: spec_small(3, lengths=[300], H=4, gate="kda", seed=81),
    "gdn-f32-d64-T777": lambda: spec_small(1, lengths=[777], H=2, h0_std=0.1, seed=82),
    "kda-f32-d64-T500": lambda: spec_small(1, lengths=[500], H=2, gate="kda", h0_std=0.1,
                                           seed=83),
    "gdn-bf16-batched-3x130": lambda: spec_small(3, lengths=[130, 130, 130], H=2, seed=84),
    "gdn-bf16-varlen": lambda: spec_small(4, lengths=[1, 31, 32, 33, 63, 64, 65, 200], H=2,
                                          seed=85),
    "kda-bf16-varlen": lambda: spec_small(4, lengths=[65, 1, 97, 32], H=2, gate="kda",
                                          seed=86),
    "gdn-f32-front-T300": lambda: spec_small(1, lengths=[300], H=2, front_end=True,
                                             h0_std=0.1, seed=87),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_chunk32_matches_oracle_and_chunk64(case):
    s64 = CASES[case]()
    s32 = dataclasses.replace(s64, chunk=32)
    i64, i32 = inputs.make(s64), inputs.make(s32)
    N = s64.N
    for key in ("x", "g", "beta"):  # the same draws; only the allocated tails differ
        assert torch.equal(i64[key][:N], i32[key][:N]), key
    a, b = run_gpu(i64), run_gpu(i32)
    ref = run_oracle(i64)
    e64 = compare(a, ref)
    e32 = compare(b, ref)
    tol = 1e-4 if s64.dtype == "f32" else 2e-2
    d_o = rel_err(b.o[:N].float().cpu().numpy(), a.o[:N].float().cpu().numpy())
    d_h = rel_err(b.h.cpu().numpy(), a.h.cpu().numpy())
    print("%s chunk 64 err %.3g/%.3g, chunk 32 err %.3g/%.3g, |32 - 64| o %.3g h %.3g"
          % (s64.name, *e64, *e32, d_o, d_h), flush=True)
    assert d_o <= tol and d_h <= tol
    assert d_o > 0, "32- and 64-row chunks should round differently: did both run at 64?"
    if s64.front_end:
        assert torch.equal(a.conv_state, b.conv_state)
