"""GPU parity: the HIP path through the C ABI against the fp64 oracle on the same seeded
inputs (max |gpu - oracle| / RMS(oracle) <= 1e-4 for f32 inputs, 2e-2 for bf16; conv
windows bit-exact; o rows past each stream's end untouched)."""
import dataclasses

import numpy as np
import pytest
import torch

from gated_delta_rule_depthwise_amd import inputs
from tests.gpu_util import SENTINEL, compare, rel_err, run_gpu, run_oracle, spec_small

pytestmark = pytest.mark.gpu


def _case(spec, mode=None, heads=None, **kw):
    inp = inputs.make(spec)
    call = run_gpu(inp, mode=mode, **kw)
    ref = run_oracle(inp, heads=heads, **{k: v for k, v in kw.items() if k in ("eps", "scale")})
    errs = compare(call, ref, heads=heads)
    print("%s mode=%s err(o)=%.3g err(h)=%.3g" % (spec.name, call.mode, *errs), flush=True)
    return inp, call, ref


def test_config1_full_f32():
    """GDN core, 1 stream, T=256, H=2, d=64, f32 (the smallest workload, at full size)."""
    _case(inputs.config(1))


@pytest.mark.parametrize("T", [1, 63, 64, 65, 200])
def test_f32_ragged_lengths(T):
    _case(spec_small(1, lengths=[T], h0_std=0.1, seed=10 + T))


@pytest.mark.parametrize("H", [2, 64, 128, 256])
def test_bf16_single_stream_head_counts(H):
    """From a segmented scan (2 heads) to one or more workgroups per CU (256 heads)."""
    heads = None if H <= 4 else [0, H // 2 + 1, H - 1]
    _case(spec_small(3, lengths=[130], H=H, seed=20 + H), heads=heads)


def test_bf16_d64():
    _case(spec_small(3, lengths=[150], H=4, dk=64, dv=64, seed=31))


def test_front_end_small():
    _case(spec_small(2, lengths=[300], H=2, seed=32))


@pytest.mark.parametrize("T", [1, 2, 3, 5])
def test_front_end_shorter_than_window(T):
    _case(spec_small(2, lengths=[T], H=2, seed=40 + T))


def test_no_l2_path():
    """eps < 0: q and k are used as given (only the scale multiplies q)."""
    spec = spec_small(1, lengths=[100], h0_std=0.1, seed=33)
    inp = inputs.make(spec)
    # pre-normalised keys keep the recurrence well conditioned without the in-call L2
    x = inp["x"]
    H, dk = spec.H, spec.dk
    for off in (0, H * dk):
        blk = x[:, off:off + H * dk].view(-1, H, dk)
        blk /= blk.norm(dim=-1, keepdim=True).clamp_min(1e-6)
    call = run_gpu(inp, eps=-1.0, scale=0.3)
    ref = run_oracle(inp, eps=-1.0, scale=0.3)
    compare(call, ref)


def test_batched_small():
    _case(spec_small(3, lengths=[100] * 3, H=4, seed=34))


def test_batched_front_end():
    _case(spec_small(2, lengths=[70] * 3, H=2, seed=35), mode="batched")


@pytest.mark.parametrize("fill", [0.0, float("nan"), 1e30])
def test_varlen_small_with_tails(fill):
    spec = spec_small(4, lengths=[1, 63, 64, 65, 130, 7], H=2, seed=36, pad_fill=fill)
    _case(spec)


def test_varlen_front_end_and_empty_stream():
    spec = spec_small(2, lengths=[5, 0, 64, 1, 90], H=2, seed=37, pad_fill=float("nan"))
    _case(spec, mode="varlen")


def test_varlen_equals_per_stream():
    spec = spec_small(4, lengths=[33, 64, 100, 2], H=2, seed=38)
    inp = inputs.make(spec)
    var = run_gpu(inp)
    for b, (s, e) in enumerate(zip(inp["cu_seqlens"][:-1].tolist(),
                                   inp["cu_seqlens"][1:].tolist())):
        sub = dataclasses.replace(spec, lengths=[e - s])
        one = {"spec": sub, "x": inp["x"][s:], "g": inp["g"][s:], "beta": inp["beta"][s:],
               "h0": inp["h0"][b:b + 1], "conv_w": None, "conv_state": None,
               "cu_seqlens": torch.tensor([0, e - s], dtype=torch.int32)}
        one["x"] = torch.cat([one["x"][:e - s], torch.zeros(sub.alloc - (e - s),
                                                            one["x"].shape[1],
                                                            dtype=one["x"].dtype)])
        for key in ("g", "beta"):
            one[key] = torch.cat([inp[key][s:e], torch.zeros((sub.alloc - (e - s),) +
                                                           inp[key].shape[1:])])
        single = run_gpu(one)
        # same kernels, same chunk boundaries: per-stream and varlen results are identical
        assert torch.equal(single.o[:e - s], var.o[s:e])
        assert torch.equal(single.h[0], var.h[b])


def test_split_equals_one_shot():
    spec = spec_small(2, lengths=[256], H=2, seed=39)
    inp = inputs.make(spec)
    one = run_gpu(inp)
    # the same stream as two calls of 100 and 156 tokens carrying h and the conv window
    parts = []
    h, cs = inp["h0"], inp["conv_state"]
    for a, b in [(0, 100), (100, 256)]:
        sub = dataclasses.replace(spec, lengths=[b - a])
        d = {"spec": sub, "x": torch.zeros(sub.alloc, spec.cd, dtype=inp["x"].dtype),
             "g": torch.zeros(sub.alloc, spec.H), "beta": torch.zeros(sub.alloc, spec.H),
             "h0": h, "conv_w": inp["conv_w"], "conv_state": cs,
             "cu_seqlens": torch.tensor([0, b - a], dtype=torch.int32)}
        d["x"][:b - a] = inp["x"][a:b]
        d["g"][:b - a] = inp["g"][a:b]
        d["beta"][:b - a] = inp["beta"][a:b]
        c = run_gpu(d)
        parts.append(c.o[:b - a].float().cpu())
        h, cs = c.h.cpu(), c.conv_state.cpu()
    o2 = torch.cat(parts).numpy()
    assert rel_err(o2, one.o[:256].float().cpu().numpy()) < 2e-2
    assert rel_err(h.numpy(), one.h.cpu().numpy()) < 2e-2
    assert torch.equal(cs, one.conv_state.cpu())


def test_chunk_table_exact():
    from gated_delta_rule_depthwise_amd import binding as B
    lens = inputs.varlen_lengths() + [0, 3]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    want = []
    for b, L in enumerate(lens):
        for c in range((L + 63) // 64):
            want.append([b, cu[b] + 64 * c, min(64, L - 64 * c), c])
    cu_d = torch.from_numpy(cu).cuda()
    table = torch.full((len(want) + 5, 4), -7, dtype=torch.int32, device="cuda")
    count = torch.zeros(1, dtype=torch.int32, device="cuda")
    rc = B.gdn_chunk_table(cu_d, len(lens), 64, table, table.shape[0], count,
                           torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == 0
    assert int(count) == len(want)
    assert torch.equal(table[:len(want)].cpu(), torch.tensor(want, dtype=torch.int32))
    assert bool((table[len(want):] == -7).all())


def test_deterministic_run_to_run():
    spec = spec_small(2, lengths=[200], H=4, seed=41)
    inp = inputs.make(spec)
    a = run_gpu(inp)
    b = run_gpu(inp)
    assert torch.equal(a.o, b.o) and torch.equal(a.h, b.h)


SEG_CASES = {  # slow decay, so that every segment's start state matters
    "gdn-front-T1000": lambda: spec_small(2, lengths=[1000], H=2, gate_dist="slow", seed=50),
    "gdn-front-T4096-H4": lambda: spec_small(2, lengths=[4096], H=4, gate_dist="slow", seed=55),
    "gdn-bf16-T777-H4": lambda: spec_small(3, lengths=[777], H=4, gate_dist="slow", seed=51),
    "batched-2x640": lambda: spec_small(3, lengths=[640, 640], H=2, gate_dist="slow", seed=52),
    "kda-T900": lambda: spec_small(5, lengths=[900], H=2, gate_dist="slow", seed=53),
    "f32-d64-T700": lambda: spec_small(1, lengths=[700], H=2, h0_std=0.1, gate_dist="slow",
                                       seed=54),
}


@pytest.mark.parametrize("case", sorted(SEG_CASES))
def test_segmented_scan_matches_serial_scan(case):
    """Few heads and a long stream: the call segments its scan (the segment maps chained
    into start states). It matches the oracle, as does the serial scan the same inputs
    take when the workspace has no room for segment states, and the two agree."""
    from gated_delta_rule_depthwise_amd import binding as B
    spec = SEG_CASES[case]()
    inp = inputs.make(spec)
    seg = run_gpu(inp)
    ser = run_gpu(inp, segmented=False)
    tps = spec.N // spec.B
    S = B.gdn_segments(seg.params, seg.plan_kind, spec.B, tps, seg.ws_bytes)
    assert S >= 3, "expected a segmented plan"
    assert B.gdn_segments(ser.params, ser.plan_kind, spec.B, tps, ser.ws_bytes) == 0
    ref = run_oracle(inp)
    e_seg = compare(seg, ref)
    e_ser = compare(ser, ref)
    tol = 1e-4 if spec.dtype == "f32" else 2e-2
    d_o = rel_err(seg.o[:spec.N].cpu().numpy(), ser.o[:spec.N].cpu().numpy())
    d_h = rel_err(seg.h.cpu().numpy(), ser.h.cpu().numpy())
    print("%s S=%d seg err(o)=%.3g err(h)=%.3g serial err(o)=%.3g err(h)=%.3g |seg-serial| "
          "o %.3g h %.3g" % (spec.name, S, *e_seg, *e_ser, d_o, d_h), flush=True)
    assert d_o <= tol and d_h <= tol
    assert d_o > 0, "the two scans should differ in rounding: is the state carried?"


def test_refused_calls_leave_buffers_unchanged():
    """A refused call (too many tokens for the workspace, a bad stride, an unsupported
    chunk) launches nothing: the state, conv window and o keep their bytes."""
    import ctypes
    from gated_delta_rule_depthwise_amd import binding as B
    from gated_delta_rule_depthwise_amd.runner import Prefill
    # (float32 rows: the front end runs as a kernel of its own and needs its activations in
    # the workspace)
    spec = spec_small(2, lengths=[200], H=2, dk=64, dv=64, dtype="f32", seed=61)
    inp = inputs.make(spec)
    call = Prefill(inp, "cuda", o_fill=SENTINEL)
    torch.cuda.synchronize()
    before = [t.clone() for t in (call.o, call.h, call.conv_state)]
    s = torch.cuda.current_stream().cuda_stream
    p = call.params
    bad_chunk = B.gdn_params.from_buffer_copy(p)
    bad_chunk.chunk = 16
    bad_ld = B.gdn_params.from_buffer_copy(p)
    bad_ld.ld_qkv = p.ld_qkv + 1
    # the front end's activations alone need N * cd float values
    front = spec.N * spec.cd * 4
    cases = [(p, spec.N, front - 1, B.GDN_E_WORKSPACE),
             (bad_chunk, spec.N, call.ws_bytes, B.GDN_E_UNSUPPORTED),
             (bad_ld, spec.N, call.ws_bytes, B.GDN_E_ARG), (p, 0, call.ws_bytes, B.GDN_E_ARG)]
    for prm, t, nbytes, want in cases:
        rc = B.gdn_prefill(prm, call.q_ptr, call.k_ptr, call.v_ptr, call.g, call.beta, call.h,
                           call.conv_state, call.conv_w, call.o, t, call.ws, nbytes, s)
        assert rc == want, (rc, want)
    rc = B.gdn_decode(bad_chunk, call.q_ptr, call.k_ptr, call.v_ptr, call.g, call.beta,
                      call.h_ptrs, call.cs_ptrs, call.conv_w, call.o, 1, s)
    assert rc == B.GDN_E_UNSUPPORTED
    torch.cuda.synchronize()
    for a, b in zip((call.o, call.h, call.conv_state), before):
        assert torch.equal(a, b)
    assert ctypes.sizeof(p) == 72


@pytest.mark.parametrize("case", ["gdn-front-T4096-H4", "gdn-bf16-T3000-H2",
                                  "batched-2x2048-H2", "f32-front-d64-T2048-H2"])
def test_segmented_scan_fast_decay(case):
    """Fast decay (log-gates -softplus(N(0,1))): each inner segment's transition underflows
    within its first chunks, so the transition jobs stop early and write zeros. The call
    still matches the oracle and the serial scan."""
    from gated_delta_rule_depthwise_amd import binding as B
    spec = {"gdn-front-T4096-H4": lambda: spec_small(2, lengths=[4096], H=4, seed=56),
            "gdn-bf16-T3000-H2": lambda: spec_small(3, lengths=[3000], H=2, seed=57),
            "batched-2x2048-H2": lambda: spec_small(3, lengths=[2048, 2048], H=2, seed=59),
            # float32 rows: the front kernel first, then the segmented scan
            "f32-front-d64-T2048-H2": lambda: spec_small(1, lengths=[2048], H=2,
                                                         front_end=True, h0_std=0.1,
                                                         gate_dist="softplus", seed=60),
            }[case]()
    inp = inputs.make(spec)
    seg = run_gpu(inp)
    ser = run_gpu(inp, segmented=False)
    assert B.gdn_segments(seg.params, seg.plan_kind, spec.B, spec.N // spec.B, seg.ws_bytes) >= 3
    ref = run_oracle(inp)
    e_seg = compare(seg, ref)
    compare(ser, ref)
    assert rel_err(seg.o[:spec.N].cpu().numpy(), ser.o[:spec.N].cpu().numpy()) <= 2e-2
    assert rel_err(seg.h.cpu().numpy(), ser.h.cpu().numpy()) <= 2e-2
    print("%s seg err(o)=%.3g err(h)=%.3g" % (spec.name, *e_seg), flush=True)


def warm_flags(call, S):
    """Whether each head of a single-stream segmented call ran warm: the library's
    warm-start plan leaves, per boundary s = 1..S-1 and head, the chunks of warm-up it found
    (0 for none) in the workspace's segment area, after 3S - 5 state slots and S x H
    transition flags; a head runs warm when every boundary found some."""
    spec = call.spec
    H = spec.H
    base = (3 * S - 5) * spec.H * spec.dk * spec.dv + S * H
    f = call.ws[:(base + S * H) * 4].view(torch.float32).cpu()
    return [float(all(f[base + s * H + h] > 0 for s in range(1, S))) for h in range(H)]


@pytest.mark.parametrize("gate", ["gdn", "kda"])
def test_segmented_scan_mixed_warm_and_chain(gate):
    """Heads 0-1 decay slowly (their segments start from the chain of segment maps), heads
    2-3 fast (their segments start warm, from h = 0 a few chunks early): one call holds both
    modes, and every head matches the oracle and the serial scan. The per-key-channel gate
    bounds a token's decay by its largest channel log-gate; its log-gates are scaled by 4 so
    that the warm windows fit in segments of a 8192-token stream."""
    import dataclasses
    from gated_delta_rule_depthwise_amd import binding as B
    fast = spec_small(2 if gate == "gdn" else 5, lengths=[4096 if gate == "gdn" else 8192],
                      H=4, seed=58)
    slow = dataclasses.replace(fast, gate_dist="slow")
    inp = inputs.make(fast)
    if gate == "kda":
        inp["g"] *= 4.0
    inp["g"][:, :2] = inputs.make(slow)["g"][:, :2]
    seg = run_gpu(inp)
    ser = run_gpu(inp, segmented=False)
    S = B.gdn_segments(seg.params, seg.plan_kind, 1, fast.N, seg.ws_bytes)
    assert S >= 3
    assert warm_flags(seg, S) == [0.0, 0.0, 1.0, 1.0]
    ref = run_oracle(inp)
    compare(seg, ref)
    compare(ser, ref)
    assert rel_err(seg.o[:fast.N].cpu().numpy(), ser.o[:fast.N].cpu().numpy()) <= 2e-2
    assert rel_err(seg.h.cpu().numpy(), ser.h.cpu().numpy()) <= 2e-2


@pytest.mark.parametrize("case", ["gdn-front-T4096-H4", "gdn-front-batched-2x2048-H2",
                                  "kda-front-T8192-H2"])
def test_segmented_warm_fallback_copy(case):
    """The last warm-started segment writes the caller's state and windows once job 0 of the
    same launch has flagged that it read them. With the flag waits bounded at 0 polls
    (gdn_debug_flag_polls) that wait gives up at once: the segment leaves its end state and
    windows in the workspace, flags it, and the second launch copies them over. o, the final
    states and the windows equal the default path's bit for bit (single stream, equal-length
    streams with per-stream states and windows, and the per-key-channel gate, whose
    log-gates are scaled by 4 so that the warm windows fit in a segment)."""
    from gated_delta_rule_depthwise_amd import binding as B
    spec = {"gdn-front-T4096-H4": lambda: spec_small(2, lengths=[4096], H=4, seed=56),
            "gdn-front-batched-2x2048-H2": lambda: spec_small(2, lengths=[2048, 2048], H=2,
                                                              seed=61),
            "kda-front-T8192-H2": lambda: spec_small(5, lengths=[8192], H=2, seed=62)}[case]()
    inp = inputs.make(spec)
    if spec.gate == "kda":
        inp["g"] *= 4.0
    direct = run_gpu(inp)
    S = B.gdn_segments(direct.params, direct.plan_kind, spec.B, spec.N // spec.B,
                       direct.ws_bytes)
    assert S >= 3
    if spec.B == 1:
        assert warm_flags(direct, S) == [1.0] * spec.H
    assert B.gdn_debug_flag_polls(0) == 0
    try:
        fallback = run_gpu(inp)
    finally:
        assert B.gdn_debug_flag_polls(-1) == 0
    # the fallback flags (one per dv slice, after the plan's counts) of every stream and head
    BH = spec.B * spec.H
    base = (3 * S - 5) * spec.B * spec.H * spec.dk * spec.dv + spec.B * 2 * S * spec.H
    f = fallback.ws[:(base + BH * 16) * 4].view(torch.int32).cpu()
    assert [int(f[base + bh * 16 + 10]) for bh in range(BH)] == [1] * BH
    assert torch.equal(fallback.o[:spec.N], direct.o[:spec.N])
    assert torch.equal(fallback.h, direct.h)
    assert torch.equal(fallback.conv_state, direct.conv_state)
    compare(fallback, run_oracle(inp))
