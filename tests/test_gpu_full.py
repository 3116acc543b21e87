"""GPU parity at the workloads' full sizes, in the launch configuration bench.py times.

The whole call runs on every head and the fp64 oracle recomputes every head, so each error
is taken over the whole o tensor and every final state (the 196608-token stream samples
two heads). conv windows and untouched o rows are checked on every channel/row.
"""
import numpy as np
import pytest
import torch

from gated_delta_rule_depthwise_amd import inputs
from tests.gpu_util import compare, rel_err, run_gpu, run_oracle, spec_small

pytestmark = pytest.mark.gpu

def _full(i, heads=None, fill=0.0):
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
    _full(4, fill=fill)


def test_config5_kda_one_shot_and_4_calls():
    """KDA, T=16384 with the front end: one call, and 4 calls of 4096 carrying the conv
    window and h; both match the oracle and each other."""
    spec = inputs.config(5)
    inp = inputs.make(spec)
    one = run_gpu(inp)
    ref = run_oracle(inp)
    e_o, e_h = compare(one, ref)
    print("%s one-shot: err(o)=%.3g err(h)=%.3g" % (spec.name, e_o, e_h), flush=True)
    import dataclasses
    h, cs = inp["h0"], inp["conv_state"]
    parts = []
    for s0 in range(0, 16384, 4096):
        sub = dataclasses.replace(spec, lengths=[4096])
        d = {"spec": sub, "x": torch.zeros(sub.alloc, spec.cd, dtype=inp["x"].dtype),
             "g": torch.zeros((sub.alloc,) + tuple(inp["g"].shape[1:])),
             "beta": torch.zeros(sub.alloc, spec.H), "h0": h, "conv_w": inp["conv_w"],
             "conv_state": cs, "cu_seqlens": torch.tensor([0, 4096], dtype=torch.int32)}
        d["x"][:4096] = inp["x"][s0:s0 + 4096]
        d["g"][:4096] = inp["g"][s0:s0 + 4096]
        d["beta"][:4096] = inp["beta"][s0:s0 + 4096]
        c = run_gpu(d)
        parts.append(c.o[:4096].cpu())
        h, cs = c.h.cpu(), c.conv_state.cpu()
    o4 = torch.cat(parts)
    assert rel_err(o4.numpy(), ref["o"]) < 2e-2
    assert rel_err(h.numpy(), ref["h"]) < 2e-2
    assert rel_err(o4.numpy(), one.o[:16384].cpu().numpy()) < 2e-2
    assert torch.equal(cs, one.conv_state.cpu())


def test_long_stream_64bit_indices():
    """One stream of 196608 tokens through the front end, C2's shapes otherwise: the raw
    rows and the activations hold 2.4 G elements (4.8 GB) and o 3.2 GB, so row offsets
    and element indices pass 2^31 and every address the kernels form must be 64-bit. The
    oracle recomputes heads 0 and 31; the new conv windows are checked on every channel."""
    T = 196608
    spec = spec_small(2, lengths=[T])
    assert T * spec.cd > 2 ** 31
    inp = inputs.make(spec)
    call = run_gpu(inp)
    ref = run_oracle(inp, heads=[0, 31])
    e_o, e_h = compare(call, ref, heads=[0, 31])
    print("%s: err(o)=%.3g err(h)=%.3g" % (spec.name, e_o, e_h), flush=True)
    want = inp["x"][T - 3:T].t().contiguous()
    assert torch.equal(call.conv_state[0].cpu(), want)


@pytest.mark.parametrize("seed", range(100, 108))
def test_config2_seed_sweep(seed):
    """The default prefill workload (T=4096 through the front end, H=32, d=128) redrawn with
    seeds 100..107: every head's o and every final state within 2e-2 of the oracle, the
    conv windows bitwise. On these seeds an fp16 hand-over of the front end's activations
    alone exceeds the bar (seed 102: err(o) 0.029; seeds 101, 104: err(h) 0.021, 0.024),
    so they check that k and v reach the scan's products with more than fp16 precision."""
    import dataclasses
    spec = dataclasses.replace(inputs.config(2), seed=seed)
    inp = inputs.make(spec)
    call = run_gpu(inp)
    e_o, e_h = compare(call, run_oracle(inp))
    print("seed %d: err(o)=%.3g err(h)=%.3g" % (seed, e_o, e_h), flush=True)
    want = inp["x"][4093:4096].t().contiguous()
    assert torch.equal(call.conv_state[0].cpu(), want)


@pytest.mark.parametrize("seed", range(100, 104))
def test_config5_seed_sweep(seed):
    """The per-key-channel workload (KDA, T=16384 through the front end, H=32, d=128)
    redrawn with seeds 100..103: every head's o and every final state within 2e-2 of the
    oracle, the conv windows bitwise."""
    import dataclasses
    spec = dataclasses.replace(inputs.config(5), seed=seed)
    inp = inputs.make(spec)
    call = run_gpu(inp)
    e_o, e_h = compare(call, run_oracle(inp))
    print("seed %d: err(o)=%.3g err(h)=%.3g" % (seed, e_o, e_h), flush=True)


def test_kda_batched_8x2048():
    """The per-key-channel gate on the batched workload's shapes: 8 streams x 2048 tokens,
    H=32, d=128, bf16 q/k/v with L2 in the call, per-stream states through h_ptrs, the
    log-gate tensor [N, H, dk] = -softplus(N(0,1)); every head against the oracle."""
    import dataclasses
    spec = dataclasses.replace(inputs.config(3), gate="kda",
                               name="kda-batched-B8xT2048-H32-d128-bf16")
    inp = inputs.make(spec)
    call = run_gpu(inp)
    e_o, e_h = compare(call, run_oracle(inp))
    print("%s: err(o)=%.3g err(h)=%.3g" % (spec.name, e_o, e_h), flush=True)


@pytest.mark.parametrize("fill", [float("nan"), 1e30])
def test_kda_varlen_tails(fill):
    """The per-key-channel gate on the varlen workload's 16 streams (lengths 1, 63, 64, 65
    among them, 67117 tokens) with NaN and 1e30 in every per-token array past the last
    token: every head and every stream's state against the oracle, o rows past the end
    untouched."""
    import dataclasses
    spec = dataclasses.replace(inputs.config(4, pad_fill=fill), gate="kda",
                               name="kda-varlen-B16-H32-d128-bf16")
    inp = inputs.make(spec)
    call = run_gpu(inp)
    e_o, e_h = compare(call, run_oracle(inp))
    print("%s tails %g: err(o)=%.3g err(h)=%.3g" % (spec.name, fill, e_o, e_h), flush=True)


def test_kda_varlen_front_end():
    """KDA varlen through the fused front end: the varlen workload's lengths with the conv
    front end and per-stream windows (each stream its own carried window)."""
    import dataclasses
    spec = dataclasses.replace(inputs.config(4, pad_fill=float("nan")), gate="kda",
                               front_end=True, name="kda-varlen-front-B16-H32-d128-bf16")
    inp = inputs.make(spec)
    call = run_gpu(inp)
    e_o, e_h = compare(call, run_oracle(inp))
    print("%s: err(o)=%.3g err(h)=%.3g" % (spec.name, e_o, e_h), flush=True)
