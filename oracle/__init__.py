"""Plain fp64 CPU oracle for the chunked gated-delta-rule prefill.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. It shares no code with the
HIP path and never imports it.

The arithmetic lives in ``gdn_oracle.c`` (plain C, double precision, OpenMP over the
independent (stream, head) pairs). This module only builds/loads that library, gathers
the channels a caller asks for (indexing, no arithmetic) and converts arrays to float64.

What each function computes, and the passages it follows:

* :func:`conv_silu` -- causal depthwise conv1d (no bias) + SiLU with a carried window of
  raw inputs; page "metrale_model_arch/glm5next_kda/prefill.rs", the conv_prefill launch
  and the "conv + SiLU only" comment; page "split_prefill.rs",
  ``prefill_phase1_conv1d_one`` (the conv advances the request's conv state).
* :func:`recurrence` -- the gated delta rule, token by token (Gated DeltaNet; the KDA
  variant gates each key channel); page "split_prefill.rs", ``prefill_gdn_full`` ("the
  GDN recurrence"), ``prefill_gdn_full_batched`` (equal-length streams back to back, one
  state per stream) and ``prefill_gdn_full_batched_fla_varlen`` (``cu_seqlens``).
  Optional in-call L2 of q and k with eps and the q scale: page
  "metrale_model_arch/glm5next_kda/prefill.rs", the l2 launch and the 1/sqrt(hd) argument of
  the chunk_scan launch.
* :func:`prefill` -- the whole path for packed ``[q | k | v]`` rows: front end, split,
  L2, recurrence; page "metrale_model_arch/glm5next_kda/prefill.rs", the launch sequence of
  ``prefill_with_pad_fill`` from conv_prefill to chunk_scan. Rows at or past a stream's end
  are never read.

* :func:`gated_rmsnorm` -- the output gate that opens phase 3 (page "split_prefill.rs",
  ``prefill_phase3``: gated RMSNorm of the GDN output with Z): per token and head,
  y = o / sqrt(mean(o^2) + eps) * w * silu(z) over the dv values, one weight per value
  channel. The pages name the operation only; normalising before gating, eps inside the
  root and a [dv] weight shared by the heads are the reading taken.

Parity of the conv tap orientation is unpinned by the pages: it follows the convention of
``torch.nn.functional.conv1d`` (tap K-1 multiplies the current token).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_SO = os.path.join(_HERE, "liboracle.so")
_lock = threading.Lock()
_lib = None

_dp = ctypes.POINTER(ctypes.c_double)
_i64p = ctypes.POINTER(ctypes.c_int64)


def build() -> str:
    """Compile ``gdn_oracle.c`` into ``liboracle.so`` (gcc, -O2, OpenMP)."""
    tmp = _SO + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           _SRC, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _SO)
    return _SO


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
            build()
        lib = ctypes.CDLL(_SO)
        lib.gdn_oracle_conv_silu.argtypes = [
            ctypes.c_int64, ctypes.c_int32, ctypes.c_int32, _dp, _dp, _dp, _dp, _dp]
        lib.gdn_oracle_conv_silu.restype = ctypes.c_int
        lib.gdn_oracle_recurrence.argtypes = [
            ctypes.c_int32, _i64p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
            _dp, _dp, _dp, _dp, ctypes.c_int32, _dp, ctypes.c_int32, ctypes.c_double,
            ctypes.c_double, _dp, _dp]
        lib.gdn_oracle_recurrence.restype = ctypes.c_int
        lib.gdn_oracle_gated_rmsnorm.argtypes = [
            ctypes.c_int64, ctypes.c_int32, _dp, _dp, _dp, ctypes.c_double, _dp]
        lib.gdn_oracle_gated_rmsnorm.restype = ctypes.c_int
        lib.gdn_oracle_num_threads.argtypes = []
        lib.gdn_oracle_num_threads.restype = ctypes.c_int
        _lib = lib
        return lib


def num_threads() -> int:
    """OpenMP threads the oracle's loops run on."""
    return int(_load().gdn_oracle_num_threads())


def _f64(a) -> np.ndarray:
    """Contiguous float64 copy of a numpy array or a CPU torch tensor."""
    if hasattr(a, "detach"):  # torch tensor: exact upcast (bf16/f32 -> f64)
        a = a.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(_dp)


def conv_silu(x, w, state=None):
    """Causal depthwise conv1d + SiLU over one stream.

    x: [T, C] raw inputs; w: [C, K] taps (w[:, K-1] multiplies the current token);
    state: [C, K-1] carried raw inputs, oldest first (None = zeros).
    Returns (y [T, C] float64, new_state [C, K-1] float64).
    """
    x = _f64(x)
    w = _f64(w)
    T, C = x.shape
    K = w.shape[1]
    assert w.shape[0] == C
    st = None if state is None else _f64(state)
    if st is not None:
        assert st.shape == (C, K - 1)
    y = np.empty((T, C), np.float64)
    st_out = np.empty((C, K - 1), np.float64)
    rc = _load().gdn_oracle_conv_silu(
        T, C, K, _ptr(x), _ptr(w), None if st is None else _ptr(st), _ptr(y), _ptr(st_out))
    if rc != 0:
        raise RuntimeError("gdn_oracle_conv_silu failed: %d" % rc)
    return y, st_out


def recurrence(q, k, v, g, beta, h0, cu_seqlens=None, l2=True, eps=1e-6, scale=None):
    """Token-by-token gated delta rule for streams lying back to back.

    q, k: [N, H, dk]; v: [N, H, dv]; g: [N, H] (one log-gate per head) or [N, H, dk]
    (one per key channel); beta: [N, H]; h0: [B, H, dk, dv] (B = len(cu_seqlens) - 1).
    cu_seqlens: [B+1] prefix sums (None: one stream of all N rows).
    l2: normalise q and k in the call (eps). scale multiplies q either way (default
    1/sqrt(dk) with l2, 1 without).
    Returns (o [N, H, dv], h [B, H, dk, dv]) in float64; rows past cu_seqlens[-1] of o are 0.
    """
    q, k, v, g, beta = (_f64(a) for a in (q, k, v, g, beta))
    N, H, dk = q.shape
    dv = v.shape[2]
    cu = np.asarray([0, N] if cu_seqlens is None else cu_seqlens, dtype=np.int64)
    B = cu.size - 1
    h = _f64(h0).reshape(B, H, dk, dv).copy()
    per_channel = 1 if g.ndim == 3 else 0
    if scale is None:
        scale = 1.0 / np.sqrt(dk) if l2 else 1.0
    o = np.zeros((N, H, dv), np.float64)
    rc = _load().gdn_oracle_recurrence(
        B, cu.ctypes.data_as(_i64p), H, dk, dv, _ptr(q), _ptr(k), _ptr(v), _ptr(g),
        per_channel, _ptr(beta), 1 if l2 else 0, float(eps), float(scale), _ptr(h), _ptr(o))
    if rc != 0:
        raise RuntimeError("gdn_oracle_recurrence failed: %d" % rc)
    return o, h


def gated_rmsnorm(o, z, w, eps=1e-6):
    """Gated RMSNorm over the last axis: o / sqrt(mean(o^2) + eps) * w * silu(z).

    o, z: [..., dv] (same shape); w: [dv]. Returns float64 of o's shape.
    """
    o = _f64(o)
    z = _f64(z)
    w = _f64(w)
    dv = o.shape[-1]
    assert z.shape == o.shape and w.shape == (dv,)
    y = np.empty_like(o)
    rows = o.size // dv
    rc = _load().gdn_oracle_gated_rmsnorm(rows, dv, _ptr(o), _ptr(z), _ptr(w), float(eps),
                                           _ptr(y))
    if rc != 0:
        raise RuntimeError("gdn_oracle_gated_rmsnorm failed: %d" % rc)
    return y


def prefill(x, g, beta, h0, *, H, dk, dv, cu_seqlens=None, conv_w=None, conv_state=None,
            l2=True, eps=1e-6, scale=None, heads=None, Hqk=None):
    """The whole path over packed rows ``x = [q (Hqk*dk) | k (Hqk*dk) | v (H*dv)]``.

    Hqk (default H) q/k heads; value head h reads q/k head h // (H // Hqk) (each q/k head
    serves H // Hqk consecutive value heads). g, beta, h0 and the outputs have H heads.

    x: [>=N, 2*H*dk + H*dv] (rows at or past cu_seqlens[-1] are never read);
    g: [>=N, H] or [>=N, H, dk]; beta: [>=N, H]; h0: [B, H, dk, dv].
    conv_w: [cd, K] and conv_state: [B, cd, K-1] enable the front end (conv + SiLU).
    heads: optional list of heads to evaluate (each head is independent of the others;
    the conv is depthwise, so only that head's channels are read).
    Returns dict(o [N, Hs, dv], h [B, Hs, dk, dv], conv_state [B, Hs*(2dk+dv) channels in
    q|k|v order, K-1] or None, channels) for the selected heads Hs (a q/k head shared by
    several selected value heads appears once per value head).
    """
    cu = np.asarray([0, x.shape[0]] if cu_seqlens is None else cu_seqlens, dtype=np.int64)
    N = int(cu[-1])
    B = cu.size - 1
    heads = list(range(H)) if heads is None else [int(hh) for hh in heads]
    Hs = len(heads)
    Hqk = H if Hqk is None else int(Hqk)
    assert 1 <= Hqk <= H and H % Hqk == 0
    grp = H // Hqk
    cols = np.concatenate(
        [np.arange((hh // grp) * dk, (hh // grp + 1) * dk) for hh in heads]
        + [Hqk * dk + np.arange((hh // grp) * dk, (hh // grp + 1) * dk) for hh in heads]
        + [2 * Hqk * dk + np.arange(hh * dv, (hh + 1) * dv) for hh in heads]).astype(np.int64)
    if hasattr(x, "detach"):
        import torch
        xs = _f64(x[:N].index_select(1, torch.as_tensor(cols)))
    else:
        xs = _f64(np.asarray(x)[:N][:, cols])
    new_state = None
    if conv_w is not None:
        w = _f64(conv_w)[cols]
        K = w.shape[1]
        new_state = np.empty((B, cols.size, K - 1), np.float64)
        ys = np.empty_like(xs)
        for b in range(B):
            st = None if conv_state is None else _f64(conv_state[b])[cols]
            y, ns = conv_silu(xs[cu[b]:cu[b + 1]], w, st) if cu[b + 1] > cu[b] else (
                xs[0:0], st if st is not None else np.zeros((cols.size, K - 1)))
            ys[cu[b]:cu[b + 1]] = y
            new_state[b] = ns
        xs = ys
    q = xs[:, :Hs * dk].reshape(N, Hs, dk)
    k = xs[:, Hs * dk:2 * Hs * dk].reshape(N, Hs, dk)
    v = xs[:, 2 * Hs * dk:].reshape(N, Hs, dv)
    gg = _f64(g[:N])
    gg = gg[:, heads] if gg.ndim == 2 else gg[:, heads, :]
    bb = _f64(beta[:N])[:, heads]
    hh0 = _f64(h0)[:, heads]
    o, h = recurrence(q, k, v, gg, bb, hh0, cu, l2=l2, eps=eps, scale=scale)
    return {"o": o, "h": h, "conv_state": new_state, "channels": cols}
