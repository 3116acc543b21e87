"""The C-ABI library on the host: it loads, exports every symbol include/gdn.h declares,
sizes workspaces, and refuses bad calls before any launch (CPU only: the refusals return
before any HIP call, so fake device pointers are never touched)."""
import ctypes
import os
import re

import pytest

from gated_delta_rule_depthwise_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")
FAKE = 1 << 20  # never dereferenced: every call below is refused on the host
FAKE2 = FAKE + 4096


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(gdn_\w+|kda_\w+)\s*\(", src,
                                 flags=re.M)))


def test_header_and_binding_agree():
    assert _declared() == sorted(B.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(B.SO)
    for name in _declared():
        assert hasattr(lib, name), name


def test_debug_flag_polls_setting():
    """The flag-wait bound is a host-side setting: polls >= 0 or -1 (default) are taken,
    anything below -1 is refused."""
    assert B.gdn_debug_flag_polls(-2) == B.GDN_E_ARG
    assert B.gdn_debug_flag_polls(5) == B.GDN_OK
    assert B.gdn_debug_flag_polls(-1) == B.GDN_OK


def test_status_strings():
    for code in (B.GDN_OK, B.GDN_E_ARG, B.GDN_E_UNSUPPORTED, B.GDN_E_WORKSPACE, B.GDN_E_HIP):
        assert B.gdn_status_string(code) not in ("", "unknown status")
    assert B.gdn_status_string(12345) == "unknown status"


def test_workspace_bytes():
    p = B.params(32, 128, 128, conv_k=4)
    cd = 3 * 32 * 128
    # bf16 rows: the front end is fused into the scan, for either gate, so there is no
    # activation buffer, only the segment states and the staged windows of a segmented call
    for kd in (0, B.GDN_PLAN_KDA):
        wg = B.gdn_workspace_bytes(p, 1, 4096, B.GDN_KIND_SINGLE | kd)
        assert 0 < wg < 4096 * cd * 2 and wg % 256 == 0
        assert B.gdn_workspace_bytes(p, 1, 4096, B.GDN_KIND_VARLEN | kd) == 256  # ranking
        assert B.gdn_workspace_bytes(p, 1, 10, B.GDN_KIND_SINGLE | kd) == 0
    # shared q/k heads: several workgroups read a window, so the new windows are staged,
    # [B][cd][conv_k - 1] bf16, even for a short call
    pq = B.params(32, 128, 128, conv_k=3, Hqk=16)
    cdq = 2 * 16 * 128 + 32 * 128
    assert B.gdn_workspace_bytes(pq, 2, 10, B.GDN_KIND_BATCHED | B.GDN_PLAN_KDA) == 2 * cdq * 2 * 2
    # float32 rows: the front kernel and its fp32 activations
    pf = B.params(32, 64, 64, conv_k=4, dtype=B.GDN_F32)
    ws = B.gdn_workspace_bytes(pf, 1, 4096, B.GDN_KIND_SINGLE | B.GDN_PLAN_KDA)
    assert ws >= 4096 * 3 * 32 * 64 * 4 and ws % 256 == 0
    assert B.gdn_workspace_bytes(pf, 1, 10, B.GDN_KIND_VARLEN) == 10 * 3 * 32 * 64 * 4 + 256
    assert B.gdn_workspace_bytes(B.params(32, 128, 128), 8, 16384, B.GDN_KIND_BATCHED) == 0
    assert B.gdn_workspace_bytes(p, 0, 4096, B.GDN_KIND_SINGLE) == 0
    assert B.gdn_workspace_bytes(p, 1, 0, B.GDN_KIND_SINGLE) == 0
    assert B.gdn_workspace_bytes(B.params(32, 96, 128), 1, 10, B.GDN_KIND_SINGLE) == 0


def test_chunk_32():
    """32-row chunks run where a 32-row instance exists (the register path: bf16 rows at
    dk = dv = 128, fp32 rows at 64, either gate) and never segment; the fused bf16 front end
    and other chunk lengths are refused."""
    for kd in (0, B.GDN_PLAN_KDA):
        for p in (B.params(32, 128, 128, chunk=32),
                  B.params(2, 64, 64, chunk=32, dtype=B.GDN_F32),
                  B.params(2, 64, 64, chunk=32, dtype=B.GDN_F32, conv_k=4)):
            assert B.gdn_segments(p, B.GDN_KIND_SINGLE | kd, 1, 1 << 16, 1 << 40) == 0
        assert B.gdn_segments(B.params(32, 128, 128, chunk=32, conv_k=4),
                              B.GDN_KIND_SINGLE | kd, 1, 4096, 1 << 40) == B.GDN_E_UNSUPPORTED
        assert B.gdn_segments(B.params(32, 128, 128, chunk=16),
                              B.GDN_KIND_SINGLE | kd, 1, 4096, 1 << 40) == B.GDN_E_UNSUPPORTED


def test_segment_plan():
    """Few (stream, head) units and long streams: the scan is segmented, and the workspace
    has room for the segment states; a workspace without that room, varlen calls and calls
    that already fill the device run unsegmented."""
    p = B.params(32, 128, 128, conv_k=4)           # one stream, 32 heads
    kd = B.GDN_PLAN_KDA
    full = B.gdn_workspace_bytes(p, 1, 4096, B.GDN_KIND_SINGLE)
    front = B.gdn_workspace_bytes(p, 1, 4096, B.GDN_KIND_VARLEN)
    assert front == 256                              # the varlen stream ranking only
    pf = B.params(32, 64, 64, conv_k=4, dtype=B.GDN_F32)   # float32 rows: front kernel
    assert B.gdn_workspace_bytes(pf, 1, 4096, B.GDN_KIND_VARLEN | kd) == 4096 * 3 * 32 * 64 * 4 + 256
    S = B.gdn_segments(p, B.GDN_KIND_SINGLE, 1, 4096, full)
    assert 3 <= S <= 12
    # the states: per slot [H][dk][dv] fp32, 3S-5 slots
    assert full - front >= (3 * S - 5) * 32 * 128 * 128 * 4
    assert B.gdn_segments(p, B.GDN_KIND_SINGLE, 1, 4096, front) == 0
    assert B.gdn_segments(p, B.GDN_KIND_VARLEN, 1, 4096, full) == 0
    assert B.gdn_segments(p, B.GDN_KIND_SINGLE, 1, 100, full) == 0   # two chunks
    pb = B.params(32, 128, 128)                    # 8 streams x 32 heads fill 256 CUs
    assert B.gdn_workspace_bytes(pb, 8, 16384, B.GDN_KIND_BATCHED) == 0
    assert B.gdn_segments(pb, B.GDN_KIND_BATCHED, 8, 2048, 1 << 40) == 0
    pk = B.params(32, 128, 128, conv_k=4)          # long KDA stream
    kda = B.GDN_KIND_SINGLE | B.GDN_PLAN_KDA
    wk = B.gdn_workspace_bytes(pk, 1, 16384, kda)
    assert B.gdn_segments(pk, kda, 1, 16384, wk) >= 3
    # A call with unit keys (L2 in the call) may start every segment warm, so its plan
    # keeps segment 0 and the warm jobs of all (stream, head) pairs in one round: S <= CUs
    # / (streams * heads) = 8 on 256 CUs, in equal segments (each warm job runs its
    # segment plus its warm-up beside segment 0). Without L2 the segments always chain,
    # with no such cap: the KDA plan is then 9 segments of 40, 27 x 7 and 27 chunks.
    S_g, _, _ = B.gdn_segment_plan(pk, B.GDN_KIND_SINGLE, 1, 16384, wk)
    assert 3 <= S_g <= 8
    assert B.gdn_segment_plan(pk, kda, 1, 16384, wk) == (8, 32 * 64, 32 * 64)
    pn = B.params(32, 128, 128, conv_k=4, eps=-1.0)
    wn = B.gdn_workspace_bytes(pn, 1, 16384, kda)
    assert B.gdn_segment_plan(pn, kda, 1, 16384, wn) == (9, 40 * 64, 27 * 64)
    # the warm-start plan needs no workspace beyond its per-boundary counts
    assert wk == wn
    assert B.gdn_segments(pk, B.GDN_KIND_VARLEN | B.GDN_PLAN_KDA, 1, 16384, wk) == 0
    # no compiled instance: the status of the refused call
    pr = B.params(4, 64, 128, dtype=B.GDN_BF16)
    assert B.gdn_segments(pr, B.GDN_KIND_SINGLE, 1, 4096, 1 << 40) == B.GDN_E_UNSUPPORTED
    assert B.gdn_segments(p, B.GDN_KIND_SINGLE, 2, 4096, full) == B.GDN_E_ARG
    assert B.gdn_segments(p, B.GDN_KIND_BATCHED, 0, 4096, full) == B.GDN_E_ARG
    assert B.gdn_segments(p, 7, 1, 4096, full) == B.GDN_E_ARG


@pytest.mark.parametrize("kda", [0, B.GDN_PLAN_KDA])
@pytest.mark.parametrize("H,T", [(32, 4096), (32, 16384), (4, 4096), (2, 700), (16, 1000),
                                 (32, 1 << 20)])
def test_segment_plan_lengths(H, T, kda):
    """A segmented plan cuts each stream into whole chunks: segment 0 and the S-2 inner
    segments leave at least one chunk for the last segment, and the plan agrees with
    gdn_segments."""
    p = B.params(H, 128, 128, conv_k=4)
    ws = B.gdn_workspace_bytes(p, 1, T, B.GDN_KIND_SINGLE | kda)
    S, l0, l1 = B.gdn_segment_plan(p, B.GDN_KIND_SINGLE | kda, 1, T, ws)
    assert S == B.gdn_segments(p, B.GDN_KIND_SINGLE | kda, 1, T, ws)
    if S == 0:
        assert l0 == 0 and l1 == 0
        return
    assert 3 <= S <= 12
    assert l0 > 0 and l1 > 0 and l0 % 64 == 0 and l1 % 64 == 0
    assert l0 + (S - 2) * l1 < T, "the last segment would be empty"
    # no room for the states: unsegmented, lengths cleared
    front = B.gdn_workspace_bytes(p, 1, T, B.GDN_KIND_VARLEN | kda)
    assert B.gdn_segment_plan(p, B.GDN_KIND_SINGLE | kda, 1, T, front) == (0, 0, 0)


def _single(p, t=10, ws=None, ws_bytes=0, h=FAKE, g=FAKE, cs=None, cw=None, q=FAKE):
    return B.gdn_prefill(p, q, FAKE, FAKE, g, FAKE, h, cs, cw, FAKE, t, ws, ws_bytes, None)


def test_refusals_before_launch():
    p = B.params(2, 64, 64, dtype=B.GDN_F32)
    assert _single(p, t=0) == B.GDN_E_ARG                   # zero tokens
    assert _single(p, t=-5) == B.GDN_E_ARG
    assert _single(p, h=None) == B.GDN_E_ARG                 # null state
    assert _single(p, g=None) == B.GDN_E_ARG
    assert _single(p, q=FAKE + 2) == B.GDN_E_ARG             # misaligned rows
    assert _single(B.params(2, 64, 64, chunk=32)) == B.GDN_E_UNSUPPORTED    # no bf16 d=64 at 32
    assert _single(B.params(2, 64, 64, chunk=16, dtype=B.GDN_F32)) == B.GDN_E_UNSUPPORTED
    assert _single(B.params(2, 96, 96)) == B.GDN_E_UNSUPPORTED
    assert _single(B.params(2, 64, 128)) == B.GDN_E_UNSUPPORTED     # bf16 has 128 x 256
    assert _single(B.params(2, 128, 64, dtype=B.GDN_F32)) == B.GDN_E_UNSUPPORTED
    assert _single(B.params(2, 64, 64, dtype=7)) == B.GDN_E_UNSUPPORTED
    assert _single(B.params(2, 64, 64, conv_k=5)) == B.GDN_E_UNSUPPORTED
    assert _single(B.params(2, 64, 64, ld_qkv=100)) == B.GDN_E_ARG    # ld < H*dk
    assert _single(B.params(2, 64, 64, ld_qkv=388)) == B.GDN_E_ARG    # ld not 16-byte rows
    assert _single(B.params(0, 64, 64)) == B.GDN_E_ARG
    nan = B.params(2, 64, 64, scale=float("nan"))
    assert _single(nan) == B.GDN_E_ARG
    # front end: conv pointers required, and (front kernel: float32 rows) a workspace large
    # enough for t tokens
    pf = B.params(2, 64, 64, conv_k=4, dtype=B.GDN_F32)
    assert _single(pf) == B.GDN_E_ARG
    need = B.gdn_workspace_bytes(pf, 1, 10, B.GDN_KIND_SINGLE)
    assert _single(pf, cs=FAKE, cw=FAKE, ws=FAKE, ws_bytes=need - 1) == B.GDN_E_WORKSPACE
    assert _single(pf, t=11, cs=FAKE, cw=FAKE, ws=FAKE, ws_bytes=need) == B.GDN_E_WORKSPACE
    assert _single(pf, cs=FAKE, cw=None, ws=FAKE, ws_bytes=need) == B.GDN_E_ARG


def test_batched_and_varlen_refusals():
    p = B.params(2, 64, 64)
    assert B.gdn_prefill_batched(p, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, 0,
                                 10, None, 0, None) == B.GDN_E_ARG
    assert B.gdn_prefill_batched(p, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, 2,
                                 0, None, 0, None) == B.GDN_E_ARG
    assert B.gdn_prefill_batched(p, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, FAKE, 2,
                                 5, None, 0, None) == B.GDN_E_ARG
    args = [p, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE]
    assert B.gdn_prefill_varlen(*args, None, 2, 10, 5, None, 0, None) == B.GDN_E_ARG
    assert B.gdn_prefill_varlen(*args, FAKE2, 0, 10, 5, None, 0, None) == B.GDN_E_ARG
    assert B.gdn_prefill_varlen(*args, FAKE2, 2, 0, 1, None, 0, None) == B.GDN_E_ARG
    assert B.gdn_prefill_varlen(*args, FAKE2, 2, 10, 11, None, 0, None) == B.GDN_E_ARG
    assert B.gdn_prefill_varlen(*args, FAKE2, 2, 10, 0, None, 0, None) == B.GDN_E_ARG
    assert B.gdn_chunk_table(None, 2, 64, FAKE, 10, FAKE, None) == B.GDN_E_ARG
    assert B.gdn_chunk_table(FAKE, 0, 64, FAKE, 10, FAKE, None) == B.GDN_E_ARG
    assert B.gdn_chunk_table(FAKE, 2, 0, FAKE, 10, FAKE, None) == B.GDN_E_ARG


def test_decode_refusals():
    p = B.params(2, 64, 64)
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE]
    assert B.gdn_decode(p, *args, 0, None) == B.GDN_E_ARG                 # no streams
    assert B.kda_decode(p, *args, -1, None) == B.GDN_E_ARG
    assert B.gdn_decode(p, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, None, FAKE, 2,
                        None) == B.GDN_E_ARG                               # null h_ptrs
    assert B.gdn_decode(p, *args[:-1], FAKE + 4, 2, None) == B.GDN_E_ARG   # misaligned o
    assert B.gdn_decode(B.params(2, 64, 128), *args, 2, None) == B.GDN_E_UNSUPPORTED
    assert B.gdn_decode(B.params(2, 96, 96), *args, 2, None) == B.GDN_E_UNSUPPORTED
    assert B.gdn_decode(B.params(2, 64, 64, dtype=7), *args, 2, None) == B.GDN_E_UNSUPPORTED
    pf = B.params(2, 64, 64, conv_k=4)                                     # conv pointers
    assert B.gdn_decode(pf, *args, 2, None) == B.GDN_E_ARG
    assert B.gdn_decode(pf, *args[:6], FAKE, None, FAKE, 2, None) == B.GDN_E_ARG


def test_output_gate_refusals():
    ok = dict(z=FAKE, norm_w=FAKE2)
    p = B.params(2, 64, 64, dtype=B.GDN_F32, **ok)
    assert _single(p, t=0) == B.GDN_E_ARG   # the usual checks still come first
    for kw in (dict(norm_w=None), dict(z=FAKE + 4), dict(norm_w=FAKE2 + 4),
               dict(ld_z=2 * 64 - 4), dict(ld_z=2 * 64 + 1), dict(norm_eps=-1.0),
               dict(norm_eps=float("nan")), dict(norm_eps=float("inf"))):
        args = dict(ok, **kw)
        assert _single(B.params(2, 64, 64, dtype=B.GDN_F32, **args)) == B.GDN_E_ARG, kw
        pd = B.params(2, 64, 64, dtype=B.GDN_F32, **args)
        assert B.gdn_decode(pd, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, 2,
                            None) == B.GDN_E_ARG, kw


def test_shared_qk_head_refusals():
    for H, Hqk in ((4, -1), (4, 5), (6, 4)):
        p = B.params(H, 64, 64, dtype=B.GDN_F32, Hqk=Hqk, ld_qkv=2 * H * 64 + H * 64)
        assert _single(p) == B.GDN_E_ARG, (H, Hqk)
        assert B.gdn_decode(p, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, 2,
                            None) == B.GDN_E_ARG
    # the packed row of 2 q/k heads and 4 value heads is 2*2*64 + 4*64 wide
    p = B.params(4, 64, 64, dtype=B.GDN_F32, Hqk=2)
    assert p.ld_qkv == 2 * 2 * 64 + 4 * 64
    # (a fused front end with shared q/k heads stages its new windows: 512 channels x 3)
    assert B.gdn_workspace_bytes(B.params(4, 64, 64, conv_k=4, Hqk=2), 1, 10,
                                 B.GDN_KIND_SINGLE) == (512 * 3 * 2 + 255) // 256 * 256


def test_params_struct_layout():
    """The ctypes struct matches include/gdn.h as a C compiler lays it out."""
    import subprocess
    import tempfile
    fields = [f[0] for f in B.gdn_params._fields_]
    prog = "#include <stddef.h>\n#include <stdio.h>\n#include \"gdn.h\"\nint main(void) {\n"
    prog += '  printf("%zu\\n", sizeof(gdn_params));\n'
    for f in fields:
        prog += '  printf("%%zu\\n", offsetof(gdn_params, %s));\n' % f
    prog += "  return 0;\n}\n"
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "l.c"), os.path.join(d, "l")
        open(src, "w").write(prog)
        subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), src, "-o", exe], check=True)
        out = [int(x) for x in subprocess.run([exe], capture_output=True, text=True,
                                              check=True).stdout.split()]
    assert out[0] == ctypes.sizeof(B.gdn_params) == 72
    assert out[1:] == [getattr(B.gdn_params, f).offset for f in fields]


def test_noalloc_refusals_before_launch():
    """gdn_prefill_noalloc checks its arguments before it touches the device, and refuses a
    call whose activations (float32 rows with the front end) would not fit its array."""
    p = B.params(2, 64, 64, dtype=B.GDN_F32)
    args = [FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE]
    assert B.gdn_prefill_noalloc(p, *args, 0, None) == B.GDN_E_ARG
    assert B.gdn_prefill_noalloc(B.params(2, 64, 64, chunk=32), *args, 10, None) == B.GDN_E_UNSUPPORTED
    cap = B.gdn_noalloc_scratch_bytes()
    assert cap == 64 << 20
    pf = B.params(32, 64, 64, conv_k=4, dtype=B.GDN_F32)    # 6144 fp32 activations per row
    t = cap // (3 * 32 * 64 * 4) + 1
    assert B.gdn_prefill_noalloc(pf, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, t,
                                 None) == B.GDN_E_WORKSPACE
