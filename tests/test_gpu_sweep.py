"""A seeded sweep over the supported space: element type, gate kind, front end and its
taps, shared q/k heads, head dims, stream layout (single, batched, varlen with empty and
one-token streams), the output gate and the in-call L2 switch, each against the oracle.
Every case is small; the point is that no combination of options is left untried."""
import dataclasses

import numpy as np
import pytest

from gated_delta_rule_depthwise_amd import inputs
from tests.gpu_util import TOL, compare, run_gpu, run_oracle, spec_small
from tests.test_gpu_gate import gated

pytestmark = pytest.mark.gpu

DIMS = {"bf16": [(64, 64), (128, 128), (128, 256)], "f32": [(64, 64), (64, 128)]}


def _case(i):
    rng = np.random.default_rng([77, i])
    dtype = ["bf16", "f32"][rng.integers(2)]
    dk, dv = DIMS[dtype][rng.integers(len(DIMS[dtype]))]
    H = int(rng.integers(1, 5))
    Hqk = int(rng.choice([d for d in range(1, H + 1) if H % d == 0]))
    layout = ["single", "batched", "varlen"][rng.integers(3)]
    if layout == "single":
        lengths = [int(rng.integers(1, 400))]
    elif layout == "batched":
        lengths = [int(rng.integers(1, 200))] * int(rng.integers(2, 4))
    else:
        lengths = [int(x) for x in rng.integers(0, 200, size=int(rng.integers(2, 5)))]
        lengths[int(rng.integers(len(lengths)))] = int(rng.choice([0, 1]))
        if sum(lengths) == 0:
            lengths[0] = 5
    front = bool(rng.integers(2))
    kw = dict(lengths=lengths, H=H, Hqk=Hqk if Hqk != H else 0, dk=dk, dv=dv, dtype=dtype,
              gate=["gdn", "kda"][rng.integers(2)], front_end=front,
              conv_k=int(rng.integers(2, 5)), out_gate=bool(rng.integers(2)),
              gate_dist=["softplus", "uniform", "slow"][rng.integers(3)],
              h0_std=float(rng.choice([0.0, 0.1])), seed=1000 + i)
    # without the in-call L2 the keys must come normalised (below), which the conv would
    # undo: only cases without the front end skip the L2
    eps = -1.0 if (rng.integers(4) == 0 and not front) else None
    return kw, eps


@pytest.mark.parametrize("i", range(256))
def test_sweep_case_matches_oracle(i):
    kw, eps = _case(i)
    spec = spec_small(1, **kw)
    inp = inputs.refill_tails(inputs.make(spec), float("nan"))
    if eps is not None:  # unit q and k rows keep the recurrence well conditioned
        x = inp["x"]
        n = spec.qk_heads * spec.dk
        for off in (0, n):
            blk = x[:, off:off + n].view(-1, spec.qk_heads, spec.dk)
            blk /= blk.float().norm(dim=-1, keepdim=True).clamp_min(1e-6).to(blk.dtype)
    mode = "varlen" if len(set(spec.lengths)) > 1 or 0 in spec.lengths else None
    call = run_gpu(inp, mode=mode, eps=eps, scale=0.3 if eps is not None else None)
    ref = run_oracle(inp, eps=eps, scale=0.3 if eps is not None else None)
    if spec.out_gate:
        ref = gated(inp, ref)
        compare(call, ref, o_metric=ref["o_metric"])
    else:
        compare(call, ref)


def _seg_case(i):
    """A long single stream or two equal ones with few heads, so that the scan segments:
    per head fast or slow decay (warm-started segments, chained ones, or both in one call),
    either gate, with or without the front end and the output gate."""
    rng = np.random.default_rng([78, i])
    dtype = ["bf16", "f32"][rng.integers(2)]
    dk = [64, 128][rng.integers(2)] if dtype == "bf16" else 64
    gate = ["gdn", "kda"][rng.integers(2)]
    B = int(rng.integers(1, 3))
    T = int(rng.integers(700, 3000 if gate == "gdn" else 4000))
    kw = dict(lengths=[T] * B, H=int(rng.integers(1, 4)), dk=dk, dv=dk, dtype=dtype,
              gate=gate, front_end=bool(rng.integers(2)), conv_k=int(rng.integers(2, 5)),
              out_gate=bool(rng.integers(2)), h0_std=0.1, seed=2000 + i)
    slow = rng.integers(2, size=kw["H"]).astype(bool)  # heads that decay slowly
    return kw, slow


@pytest.mark.parametrize("i", range(96))
def test_segmented_sweep_matches_oracle(i):
    from gated_delta_rule_depthwise_amd import binding as B
    kw, slow = _seg_case(i)
    spec = spec_small(1, **kw)
    inp = inputs.make(spec)
    if spec.gate == "kda":
        inp["g"] *= 4.0  # warm windows that fit the segments of these shorter streams
    if slow.any():
        sl = inputs.make(dataclasses.replace(spec, gate_dist="slow"))["g"]
        idx = [h for h in range(spec.H) if slow[h]]
        inp["g"][:, idx] = sl[:, idx]
    call = run_gpu(inp)
    S = B.gdn_segments(call.params, call.plan_kind, spec.B, spec.N // spec.B, call.ws_bytes)
    print("%s S=%d slow heads %s" % (spec.name, S, slow.tolist()), flush=True)
    ref = run_oracle(inp)
    if spec.out_gate:
        ref = gated(inp, ref)
        compare(call, ref, o_metric=ref["o_metric"])
    else:
        compare(call, ref)


@pytest.mark.xfail(strict=False, reason="fp32 rows: the final state's largest element carries "
                   "about 3e-6 relative error (plain fp32 chunk arithmetic), and this head's "
                   "state is heavy-tailed (max 16x its RMS) while the empty stream's zero "
                   "state halves the RMS, so max|d|/RMS reaches 1.29e-4 against 1e-4")
def test_sweep_f32_heavy_tailed_state():
    """Sweep case 505 (varlen [0, 180], fp32 rows, d 64 x 128, front end), kept as a record
    of where the fp32 bar meets fp32 arithmetic."""
    test_sweep_case_matches_oracle(505)
