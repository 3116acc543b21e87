"""Device buffers for one workload and the C-ABI call that processes them.

Plumbing only: torch allocates device memory and provides the stream; every step of the
path runs inside libgdn's kernels (binding.py). Used by the tests and by bench.py.
"""
from __future__ import annotations

import torch

from . import binding as B


class Prefill:
    """One call of gdn_prefill / kda_prefill / gdn_prefill_batched / gdn_prefill_varlen.

    ``inp`` is a dict from :func:`inputs.make`. ``mode`` is "single", "batched" or
    "varlen" (default: single for one stream, batched for equal lengths, else varlen).
    ``o_fill`` pre-fills the output so rows the call must not write can be checked.
    ``segmented=False`` gives the call a workspace without room for segment states.
    """

    def __init__(self, inp: dict, device="cuda", mode=None, o_fill=0.0, eps=None,
                 scale=None, segmented=True):
        spec = inp["spec"]
        self.spec = spec
        self.device = device
        lens = list(spec.lengths)
        if mode is None:
            mode = "single" if len(lens) == 1 else (
                "batched" if len(set(lens)) == 1 else "varlen")
        self.mode = mode
        self.x = inp["x"].to(device)
        self.g = inp["g"].to(device)
        self.beta = inp["beta"].to(device)
        self.h0 = inp["h0"].to(device)
        self.h = self.h0.clone()
        self.cu = inp["cu_seqlens"].to(device)
        self.conv_w = None if inp["conv_w"] is None else inp["conv_w"].to(device)
        self.conv_state0 = None if inp["conv_state"] is None else inp["conv_state"].to(device)
        self.conv_state = None if self.conv_state0 is None else self.conv_state0.clone()
        self.o = torch.full((spec.alloc, spec.H, spec.dv), o_fill, dtype=torch.float32,
                            device=device)
        self.h_ptrs = torch.tensor([self.h[b].data_ptr() for b in range(spec.B)],
                                   dtype=torch.int64, device=device)
        self.cs_ptrs = None if self.conv_state is None else torch.tensor(
            [self.conv_state[b].data_ptr() for b in range(spec.B)], dtype=torch.int64,
            device=device)
        self.z = None if inp.get("z") is None else inp["z"].to(device)
        self.norm_w = None if inp.get("norm_w") is None else inp["norm_w"].to(device)
        self.params = B.params(
            spec.H, spec.dk, spec.dv, chunk=spec.chunk,
            eps=spec.eps if eps is None else eps,
            scale=spec.scale if scale is None else scale,
            dtype=B.GDN_BF16 if spec.dtype == "bf16" else B.GDN_F32,
            conv_k=spec.conv_k if spec.front_end else 0, ld_qkv=spec.cd,
            z=self.z, norm_w=self.norm_w, norm_eps=spec.norm_eps, Hqk=spec.Hqk)
        kind = {"single": B.GDN_KIND_SINGLE, "batched": B.GDN_KIND_BATCHED,
                "varlen": B.GDN_KIND_VARLEN}[mode]
        self.kind = kind
        # the kind to ask gdn_segments / gdn_segment_plan with: the plan of this call's gate
        self.plan_kind = kind | (B.GDN_PLAN_KDA if spec.gate == "kda" else 0)
        # segmented=False sizes the workspace for the front end only, which makes a single
        # or batched call run its scan unsegmented
        self.ws_bytes = B.gdn_workspace_bytes(
            self.params, spec.B, spec.N,
            (kind if segmented else B.GDN_KIND_VARLEN) | (self.plan_kind & B.GDN_PLAN_KDA))
        self.ws = torch.empty(max(self.ws_bytes, 1), dtype=torch.uint8, device=device)
        es = self.x.element_size()
        base = self.x.data_ptr()
        self.q_ptr = base
        self.k_ptr = base + spec.qk_heads * spec.dk * es
        self.v_ptr = base + 2 * spec.qk_heads * spec.dk * es

    def reset(self):
        """Restore the initial states (h, conv window)."""
        self.h.copy_(self.h0)
        if self.conv_state is not None:
            self.conv_state.copy_(self.conv_state0)

    def __call__(self, stream=None) -> int:
        s = torch.cuda.current_stream(self.device).cuda_stream if stream is None else stream
        sp = self.spec
        cs = None if self.conv_state is None else self.conv_state
        if self.mode == "single":
            fn = B.kda_prefill if sp.gate == "kda" else B.gdn_prefill
            return fn(self.params, self.q_ptr, self.k_ptr, self.v_ptr, self.g, self.beta,
                      self.h, cs, self.conv_w, self.o, sp.N, self.ws, self.ws_bytes, s)
        kda = sp.gate == "kda"
        if self.mode == "batched":
            fn = B.kda_prefill_batched if kda else B.gdn_prefill_batched
            return fn(self.params, self.q_ptr, self.k_ptr, self.v_ptr, self.g, self.beta,
                      self.h_ptrs, self.cs_ptrs, self.conv_w, self.o, sp.B, sp.lengths[0],
                      self.ws, self.ws_bytes, s)
        fn = B.kda_prefill_varlen if kda else B.gdn_prefill_varlen
        return fn(self.params, self.q_ptr, self.k_ptr, self.v_ptr, self.g, self.beta,
                  self.h_ptrs, self.cs_ptrs, self.conv_w, self.o, self.cu, sp.B, sp.N,
                  max(sp.lengths), self.ws, self.ws_bytes, s)


class Decode:
    """One call of gdn_decode / kda_decode: row b of ``inp`` is stream b's new token.

    ``inp`` is a dict from :func:`inputs.make` whose streams all have length 1. The states
    h (``[B, H, dk, dv]``) and the conv windows are updated in place by every call; ``o`` is
    ``[B, H, dv]``. ``step(t, ...)`` points the call at other token rows (see there).
    """

    def __init__(self, inp: dict, device="cuda", o_fill=0.0, eps=None, scale=None):
        spec = inp["spec"]
        self.spec = spec
        self.device = device
        self.x = inp["x"].to(device)
        self.g = inp["g"].to(device)
        self.beta = inp["beta"].to(device)
        self.h0 = inp["h0"].to(device)
        self.h = self.h0.clone()
        self.conv_w = None if inp["conv_w"] is None else inp["conv_w"].to(device)
        self.conv_state0 = None if inp["conv_state"] is None else inp["conv_state"].to(device)
        self.conv_state = None if self.conv_state0 is None else self.conv_state0.clone()
        self.o = torch.full((spec.B, spec.H, spec.dv), o_fill, dtype=torch.float32,
                            device=device)
        self.h_ptrs = torch.tensor([self.h[b].data_ptr() for b in range(spec.B)],
                                   dtype=torch.int64, device=device)
        self.cs_ptrs = None if self.conv_state is None else torch.tensor(
            [self.conv_state[b].data_ptr() for b in range(spec.B)], dtype=torch.int64,
            device=device)
        self.eps = spec.eps if eps is None else eps
        self.scale = spec.scale if scale is None else scale
        self.z = None if inp.get("z") is None else inp["z"].to(device)
        self.norm_w = None if inp.get("norm_w") is None else inp["norm_w"].to(device)
        self.params = self._params(spec.cd)
        es = self.x.element_size()
        base = self.x.data_ptr()
        self.q_ptr = base
        self.k_ptr = base + spec.qk_heads * spec.dk * es
        self.v_ptr = base + 2 * spec.qk_heads * spec.dk * es

    def _params(self, ld, z=None, ld_z=None):
        sp = self.spec
        return B.params(sp.H, sp.dk, sp.dv, chunk=sp.chunk, eps=self.eps, scale=self.scale,
                        dtype=B.GDN_BF16 if sp.dtype == "bf16" else B.GDN_F32,
                        conv_k=sp.conv_k if sp.front_end else 0, ld_qkv=ld,
                        z=self.z if z is None else z, norm_w=self.norm_w, ld_z=ld_z,
                        norm_eps=sp.norm_eps, Hqk=sp.Hqk)

    def reset(self):
        """Restore the initial states (h, conv window)."""
        self.h.copy_(self.h0)
        if self.conv_state is not None:
            self.conv_state.copy_(self.conv_state0)

    def _call(self, p, q, k, v, g, beta, stream):
        s = torch.cuda.current_stream(self.device).cuda_stream if stream is None else stream
        fn = B.kda_decode if self.spec.gate == "kda" else B.gdn_decode
        return fn(p, q, k, v, g, beta, self.h_ptrs, self.cs_ptrs, self.conv_w, self.o,
                  self.spec.B, s)

    def __call__(self, stream=None) -> int:
        return self._call(self.params, self.q_ptr, self.k_ptr, self.v_ptr, self.g,
                          self.beta, stream)

    def step(self, x, t, T, g, beta, stream=None) -> int:
        """Decode token t of T per stream from prefill-layout rows: stream b's token is row
        b*T + t of ``x`` (a device tensor of packed rows; the row stride between streams
        is T rows); ``g`` and ``beta`` hold this step's [B, H(, dk)] values. With the
        output gate, ``self.z`` must hold the T rows per stream in the same layout."""
        sp = self.spec
        es = x.element_size()
        base = x.data_ptr() + t * sp.cd * es
        # the output gate's z in the same prefill layout: stream b's row b*T + t
        zp = None if self.z is None else self.z.data_ptr() + t * sp.H * sp.dv * es
        p = self._params(T * sp.cd, zp, T * sp.H * sp.dv)
        return self._call(p, base, base + sp.qk_heads * sp.dk * es,
                          base + 2 * sp.qk_heads * sp.dk * es, g, beta, stream)
