"""Thin ctypes binding of libgdn (include/gdn.h): same names, argument marshalling only.

Every function takes device pointers as Python ints (``tensor.data_ptr()``) or torch
tensors, and a HIP stream handle (``torch.cuda.current_stream().cuda_stream``); it returns
the library's status code. Nothing here computes any step of the path, and there is no
fallback: if ``libgdn.so`` is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os
import threading

PKG = os.path.dirname(os.path.abspath(__file__))
SO = os.path.join(PKG, "libgdn.so")

GDN_OK = 0
GDN_E_ARG = -1
GDN_E_UNSUPPORTED = -2
GDN_E_WORKSPACE = -3
GDN_E_HIP = -4
GDN_F32 = 0
GDN_BF16 = 1
GDN_KIND_SINGLE = 0
GDN_KIND_BATCHED = 1
GDN_KIND_VARLEN = 2
GDN_PLAN_KDA = 0x100  # or-ed into the kind of gdn_segments / gdn_segment_plan

# every symbol include/gdn.h declares
EXPORTS = ("gdn_prefill", "gdn_prefill_noalloc", "gdn_noalloc_scratch_bytes", "kda_prefill",
           "gdn_prefill_batched", "gdn_prefill_varlen",
           "kda_prefill_batched", "kda_prefill_varlen", "gdn_decode", "kda_decode",
           "gdn_chunk_table", "gdn_profile_enable", "gdn_profile_read", "gdn_workspace_bytes",
           "gdn_segments", "gdn_segment_plan", "gdn_status_string", "gdn_debug_validate",
           "gdn_debug_flag_polls")
GDN_BAD_CU_START, GDN_BAD_CU_ORDER, GDN_BAD_CU_TOTAL, GDN_BAD_CU_MAXLEN = 1, 2, 4, 8
GDN_BAD_KDA_GATE = 16
GDN_PROF_FRONT = 0
GDN_PROF_RECUR = 1
GDN_PROF_STATE = 2
GDN_PROF_GATE = 3
GDN_PROF_BUCKETS = 4


class gdn_params(ctypes.Structure):
    _fields_ = [("H", ctypes.c_int32), ("dk", ctypes.c_int32), ("dv", ctypes.c_int32),
                ("chunk", ctypes.c_int32), ("eps", ctypes.c_float), ("scale", ctypes.c_float),
                ("dtype", ctypes.c_int32), ("conv_k", ctypes.c_int32),
                ("ld_qkv", ctypes.c_int64), ("z", ctypes.c_void_p),
                ("norm_w", ctypes.c_void_p), ("ld_z", ctypes.c_int64),
                ("norm_eps", ctypes.c_float), ("Hqk", ctypes.c_int32)]


_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t
_pp = ctypes.POINTER(gdn_params)
_lock = threading.Lock()
_lib = None


def load(path: str = SO):
    """Load libgdn.so (raises if it is missing: there is no other implementation)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(path):
            raise RuntimeError("libgdn.so is not built (%s); run __graft_entry__.build()" % path)
        lib = ctypes.CDLL(path)
        single = [_pp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i64, _vp, _sz, _vp]
        lib.gdn_prefill.argtypes = single
        lib.kda_prefill.argtypes = single
        lib.gdn_prefill_noalloc.argtypes = single[:11] + [_vp]
        lib.gdn_prefill_noalloc.restype = ctypes.c_int
        lib.gdn_noalloc_scratch_bytes.argtypes = []
        lib.gdn_noalloc_scratch_bytes.restype = _sz
        batched = [_pp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i64, _vp, _sz, _vp]
        varlen = [_pp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i64, _i32, _vp,
                  _sz, _vp]
        lib.gdn_prefill_batched.argtypes = batched
        lib.kda_prefill_batched.argtypes = batched
        lib.gdn_prefill_varlen.argtypes = varlen
        lib.kda_prefill_varlen.argtypes = varlen
        decode = [_pp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _vp]
        lib.gdn_decode.argtypes = decode
        lib.kda_decode.argtypes = decode
        lib.gdn_chunk_table.argtypes = [_vp, _i32, _i32, _vp, _i64, _vp, _vp]
        lib.gdn_profile_enable.argtypes = [ctypes.c_int]
        lib.gdn_profile_enable.restype = ctypes.c_int
        lib.gdn_profile_read.argtypes = [_vp, _vp, _i32]
        lib.gdn_profile_read.restype = ctypes.c_int
        lib.gdn_workspace_bytes.argtypes = [_pp, _i32, _i64, _i32]
        lib.gdn_workspace_bytes.restype = _sz
        lib.gdn_segments.argtypes = [_pp, _i32, _i32, _i64, _sz]
        lib.gdn_segments.restype = ctypes.c_int
        lib.gdn_segment_plan.argtypes = [_pp, _i32, _i32, _i64, _sz, _vp, _vp]
        lib.gdn_segment_plan.restype = ctypes.c_int
        lib.gdn_debug_validate.argtypes = [_vp]
        lib.gdn_debug_validate.restype = ctypes.c_int
        lib.gdn_debug_flag_polls.argtypes = [ctypes.c_int32]
        lib.gdn_debug_flag_polls.restype = ctypes.c_int
        lib.gdn_status_string.argtypes = [ctypes.c_int]
        lib.gdn_status_string.restype = ctypes.c_char_p
        for name in ("gdn_prefill", "kda_prefill", "gdn_prefill_batched",
                     "gdn_prefill_varlen", "kda_prefill_batched", "kda_prefill_varlen",
                     "gdn_decode", "kda_decode", "gdn_chunk_table"):
            getattr(lib, name).restype = ctypes.c_int
        _lib = lib
        return lib


def _p(x):
    """Device pointer of a tensor (or an int / None passed through)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def params(H, dk, dv, chunk=64, eps=1e-6, scale=None, dtype=GDN_BF16, conv_k=0, ld_qkv=None,
           z=None, norm_w=None, ld_z=None, norm_eps=1e-6, Hqk=0):
    """A gdn_params struct (ld_qkv defaults to the packed row 2*Hqk*dk + H*dv; ld_z to
    H*dv). ``z`` and ``norm_w`` (device tensors or pointers) turn the output gate on;
    ``Hqk`` (0 = H) is the q/k head count."""
    if scale is None:
        scale = dk ** -0.5
    if ld_qkv is None:
        ld_qkv = 2 * (Hqk or H) * dk + H * dv
    if ld_z is None:
        ld_z = H * dv
    return gdn_params(H, dk, dv, chunk, eps, scale, dtype, conv_k, ld_qkv, _p(z), _p(norm_w),
                      ld_z, norm_eps, Hqk)


def gdn_prefill(p, q, k, v, g, beta, h, conv_state, conv_w, o, t, ws, ws_bytes, stream):
    return load().gdn_prefill(ctypes.byref(p), _p(q), _p(k), _p(v), _p(g), _p(beta), _p(h),
                              _p(conv_state), _p(conv_w), _p(o), t, _p(ws), ws_bytes, stream)


def gdn_prefill_noalloc(p, q, k, v, g, beta, h, conv_state, conv_w, o, t, stream):
    return load().gdn_prefill_noalloc(ctypes.byref(p), _p(q), _p(k), _p(v), _p(g), _p(beta),
                                      _p(h), _p(conv_state), _p(conv_w), _p(o), t, stream)


def gdn_noalloc_scratch_bytes():
    return int(load().gdn_noalloc_scratch_bytes())


def kda_prefill(p, q, k, v, g, beta, h, conv_state, conv_w, o, t, ws, ws_bytes, stream):
    return load().kda_prefill(ctypes.byref(p), _p(q), _p(k), _p(v), _p(g), _p(beta), _p(h),
                              _p(conv_state), _p(conv_w), _p(o), t, _p(ws), ws_bytes, stream)


def gdn_prefill_batched(p, q, k, v, g, beta, h_ptrs, conv_state_ptrs, conv_w, o, B,
                        t_per_stream, ws, ws_bytes, stream):
    return load().gdn_prefill_batched(ctypes.byref(p), _p(q), _p(k), _p(v), _p(g), _p(beta),
                                      _p(h_ptrs), _p(conv_state_ptrs), _p(conv_w), _p(o), B,
                                      t_per_stream, _p(ws), ws_bytes, stream)


def gdn_prefill_varlen(p, q, k, v, g, beta, h_ptrs, conv_state_ptrs, conv_w, o, cu_seqlens,
                       B, total_tokens, max_seqlen, ws, ws_bytes, stream):
    return load().gdn_prefill_varlen(ctypes.byref(p), _p(q), _p(k), _p(v), _p(g), _p(beta),
                                     _p(h_ptrs), _p(conv_state_ptrs), _p(conv_w), _p(o),
                                     _p(cu_seqlens), B, total_tokens, max_seqlen, _p(ws),
                                     ws_bytes, stream)


def kda_prefill_batched(p, q, k, v, g, beta, h_ptrs, conv_state_ptrs, conv_w, o, B,
                        t_per_stream, ws, ws_bytes, stream):
    return load().kda_prefill_batched(ctypes.byref(p), _p(q), _p(k), _p(v), _p(g), _p(beta),
                                      _p(h_ptrs), _p(conv_state_ptrs), _p(conv_w), _p(o), B,
                                      t_per_stream, _p(ws), ws_bytes, stream)


def kda_prefill_varlen(p, q, k, v, g, beta, h_ptrs, conv_state_ptrs, conv_w, o, cu_seqlens,
                       B, total_tokens, max_seqlen, ws, ws_bytes, stream):
    return load().kda_prefill_varlen(ctypes.byref(p), _p(q), _p(k), _p(v), _p(g), _p(beta),
                                     _p(h_ptrs), _p(conv_state_ptrs), _p(conv_w), _p(o),
                                     _p(cu_seqlens), B, total_tokens, max_seqlen, _p(ws),
                                     ws_bytes, stream)


def gdn_decode(p, q, k, v, g, beta, h_ptrs, conv_state_ptrs, conv_w, o, B, stream):
    return load().gdn_decode(ctypes.byref(p), _p(q), _p(k), _p(v), _p(g), _p(beta),
                             _p(h_ptrs), _p(conv_state_ptrs), _p(conv_w), _p(o), B, stream)


def kda_decode(p, q, k, v, g, beta, h_ptrs, conv_state_ptrs, conv_w, o, B, stream):
    return load().kda_decode(ctypes.byref(p), _p(q), _p(k), _p(v), _p(g), _p(beta),
                             _p(h_ptrs), _p(conv_state_ptrs), _p(conv_w), _p(o), B, stream)


def gdn_chunk_table(cu_seqlens, B, chunk, table, max_entries, count, stream):
    return load().gdn_chunk_table(_p(cu_seqlens), B, chunk, _p(table), max_entries, _p(count),
                                  stream)


def gdn_profile_enable(on):
    return load().gdn_profile_enable(1 if on else 0)


def gdn_profile_read(nbuckets=GDN_PROF_BUCKETS):
    """Returns (status, [ms per bucket], [launches per bucket])."""
    ms = (ctypes.c_double * nbuckets)()
    n = (ctypes.c_int64 * nbuckets)()
    rc = load().gdn_profile_read(ctypes.addressof(ms), ctypes.addressof(n), nbuckets)
    return rc, list(ms), list(n)


def gdn_workspace_bytes(p, B, max_tokens, kind):
    return int(load().gdn_workspace_bytes(ctypes.byref(p), B, max_tokens, kind))


def gdn_segments(p, kind, B, t_per_stream, ws_bytes):
    return int(load().gdn_segments(ctypes.byref(p), kind, B, t_per_stream, ws_bytes))


def gdn_segment_plan(p, kind, B, t_per_stream, ws_bytes):
    """(S, tokens of segment 0, tokens of each inner segment); S = 0 when unsegmented."""
    s0 = ctypes.c_int64(0)
    s1 = ctypes.c_int64(0)
    S = int(load().gdn_segment_plan(ctypes.byref(p), kind, B, t_per_stream, ws_bytes,
                                    ctypes.byref(s0), ctypes.byref(s1)))
    return S, s0.value, s1.value


def gdn_status_string(status):
    return load().gdn_status_string(status).decode()


def gdn_debug_validate(status):
    """Turn the device-side input checks on (status: a device int32 tensor or pointer) or
    off (None)."""
    return load().gdn_debug_validate(_p(status))


def gdn_debug_flag_polls(polls):
    """Bound the segmented scan's flag waits (polls >= 0) or restore the default (-1)."""
    return load().gdn_debug_flag_polls(int(polls))
