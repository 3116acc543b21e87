"""Pins of the fp64 oracle to things other than itself (CPU only).

Each test fixes the oracle against a hand-worked example, a brute-force unrolling, a
different algorithm (the chunked form), a closed form, a library routine or an invariant.
Together they are chosen so that a dropped term, a wrong sign, a wrong index or a
transposed operand anywhere in the oracle fails at least one of them (the planted-mistake
test in test_oracle_mutants.py checks exactly that).
"""
import json
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from tests.chunked_ref import chunked, dense_unroll

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "tiny_hand_examples.json")


def _rand_case(rng, T, H, dk, dv, kda=False, unit_k=False):
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    gshape = (T, H, dk) if kda else (T, H)
    g = -np.logaddexp(0.0, rng.standard_normal(gshape))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    h0 = 0.3 * rng.standard_normal((1, H, dk, dv))
    return q, k, v, g, beta, h0


def _l2(x, eps, scale=1.0):
    return scale * x / np.sqrt((x * x).sum(-1, keepdims=True) + eps)


# ---------------------------------------------------------------------------------------
# hand-worked examples


@pytest.mark.parametrize("variant", ["gdn_scalar_gate", "kda_channel_gate"])
def test_hand_worked_recurrence(variant):
    gold = json.load(open(GOLDEN))
    base = gold["gdn_scalar_gate"]
    case = gold[variant]
    q = np.array(base["q"])[:, None, :]
    k = np.array(base["k"])[:, None, :]
    v = np.array(base["v"])[:, None, :]
    beta = np.array(base["beta"])[:, None]
    alpha = np.array(case["alpha"])
    g = np.log(alpha)[:, None] if alpha.ndim == 1 else np.log(alpha)[:, None, :]
    h0 = np.array(base["h0"])[None, None]
    o, h = oracle.recurrence(q, k, v, g, beta, h0, l2=False)
    np.testing.assert_allclose(o[:, 0], np.array(case["o"]), rtol=0, atol=1e-13)
    np.testing.assert_allclose(h[0, 0], np.array(case["hT"]), rtol=0, atol=1e-13)


def test_hand_worked_conv():
    c = json.load(open(GOLDEN))["conv"]
    x = np.array(c["x"])[:, None]
    w = np.array(c["w"])[None, :]
    st = np.array(c["window"])[None, :]
    y, st_out = oracle.conv_silu(x, w, st)
    z = np.array(c["z"])
    np.testing.assert_allclose(y[:, 0], F.silu(torch.tensor(z)).numpy(), rtol=1e-14, atol=0)
    np.testing.assert_array_equal(st_out[0], np.array(c["window_out"]))
    _, st1 = oracle.conv_silu(x[:1], w, st)
    np.testing.assert_array_equal(st1[0], np.array(c["window_out_T1"]))


# ---------------------------------------------------------------------------------------
# brute force and the chunked algorithm


@pytest.mark.parametrize("kda", [False, True])
@pytest.mark.parametrize("T,dk,dv", [(1, 3, 2), (5, 4, 3), (7, 3, 5)])
def test_dense_unrolling(kda, T, dk, dv):
    rng = np.random.default_rng(100 + T * 10 + dk + int(kda))
    q, k, v, g, beta, h0 = _rand_case(rng, T, 2, dk, dv, kda=kda)
    o, h = oracle.recurrence(q, k, v, g, beta, h0, l2=False)
    for hd in range(2):
        o_ref, h_ref = dense_unroll(q[:, hd], k[:, hd], v[:, hd], g[:, hd], beta[:, hd],
                                    h0[0, hd])
        np.testing.assert_allclose(o[:, hd], o_ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(h[0, hd], h_ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("kda", [False, True])
@pytest.mark.parametrize("C", [1, 2, 3, 7, 16, 64, 128, 150])
def test_chunk_size_invariance(kda, C):
    rng = np.random.default_rng(7 + C + 1000 * int(kda))
    T, H, dk, dv = 150, 2, 16, 12
    q, k, v, g, beta, h0 = _rand_case(rng, T, H, dk, dv, kda=kda)
    eps, scale = 1e-6, 0.25
    o, h = oracle.recurrence(q, k, v, g, beta, h0, l2=True, eps=eps, scale=scale)
    qn, kn = _l2(q, eps, scale), _l2(k, eps)
    for hd in range(H):
        o_c, h_c = chunked(qn[:, hd], kn[:, hd], v[:, hd], g[:, hd], beta[:, hd],
                           h0[0, hd], C)
        ref = max(1.0, np.abs(o_c).max())
        np.testing.assert_allclose(o[:, hd], o_c, rtol=0, atol=1e-11 * ref)
        np.testing.assert_allclose(h[0, hd], h_c, rtol=0, atol=1e-11 * ref)


# ---------------------------------------------------------------------------------------
# closed forms


def test_beta_zero_is_pure_decay():
    rng = np.random.default_rng(11)
    for kda in (False, True):
        q, k, v, g, beta, h0 = _rand_case(rng, 9, 2, 5, 4, kda=kda)
        beta[:] = 0.0
        o, h = oracle.recurrence(q, k, v, g, beta, h0, l2=False)
        G = np.cumsum(g, axis=0)
        Gk = G if kda else G[..., None] * np.ones(5)
        np.testing.assert_allclose(h[0], np.exp(Gk[-1])[..., None] * h0[0], rtol=1e-13)
        for t in range(9):
            for hd in range(2):
                ref = h0[0, hd].T @ (np.exp(Gk[t, hd]) * q[t, hd])
                np.testing.assert_allclose(o[t, hd], ref, rtol=1e-12, atol=1e-14)


def test_beta_zero_gate_zero_is_a_matmul():
    rng = np.random.default_rng(12)
    q, k, v, g, beta, h0 = _rand_case(rng, 6, 3, 4, 7)
    beta[:] = 0.0
    g[:] = 0.0
    o, h = oracle.recurrence(q, k, v, g, beta, h0, l2=False)
    np.testing.assert_allclose(o, np.einsum("thi,hij->thj", q, h0[0]), rtol=1e-13)
    np.testing.assert_array_equal(h, h0)


def test_full_forgetting():
    """g = -1e4 gives alpha = 0 exactly: only the current token survives."""
    rng = np.random.default_rng(13)
    q, k, v, g, beta, h0 = _rand_case(rng, 8, 2, 6, 5)
    g[:] = -1e4
    o, h = oracle.recurrence(q, k, v, g, beta, h0, l2=False)
    ref = beta[..., None] * np.einsum("thi,thi->th", k, q)[..., None] * v
    np.testing.assert_allclose(o, ref, rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(h[0], beta[-1][:, None, None] * np.einsum(
        "hi,hj->hij", k[-1], v[-1]), rtol=1e-13)


def test_orthonormal_keys_give_causal_linear_attention():
    rng = np.random.default_rng(14)
    T, dk, dv = 6, 8, 5
    basis, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = basis[:, :T].T[:, None, :]                      # T orthonormal keys
    q = rng.standard_normal((T, 1, dk))
    v = rng.standard_normal((T, 1, dv))
    g = np.zeros((T, 1))
    beta = np.ones((T, 1))
    h0 = np.zeros((1, 1, dk, dv))
    o, h = oracle.recurrence(q, k, v, g, beta, h0, l2=False)
    np.testing.assert_allclose(h[0, 0], k[:, 0].T @ v[:, 0], atol=1e-13)
    att = np.tril(q[:, 0] @ k[:, 0].T)
    np.testing.assert_allclose(o[:, 0], att @ v[:, 0], atol=1e-13)


def test_retrieval_identity_with_in_call_l2():
    """beta = 1 and a unit key make S_t k_t = v_t; with q = k the output is scale * v."""
    rng = np.random.default_rng(15)
    T, H, dk, dv = 20, 2, 16, 8
    q, k, v, g, beta, h0 = _rand_case(rng, T, H, dk, dv, kda=True)
    beta[:] = 1.0
    scale = 0.37
    o, _ = oracle.recurrence(k, k, v, g, beta, h0, l2=True, eps=0.0, scale=scale)
    np.testing.assert_allclose(o, scale * v, rtol=0, atol=1e-12)


# ---------------------------------------------------------------------------------------
# L2 and front end


def test_l2_properties():
    rng = np.random.default_rng(16)
    T, H, dk, dv = 5, 2, 8, 3
    q, k, v, g, beta, h0 = _rand_case(rng, T, H, dk, dv)
    g[:] = -1e4                                    # o_t = beta (k_n . q_n) v
    beta[:] = 1.0
    eps, scale = 1e-3, 0.5
    o1, _ = oracle.recurrence(q, k, v, g, beta, h0, l2=True, eps=eps, scale=scale)
    cos = o1[..., 0] / v[..., 0]                      # = scale * <q,k> / norms
    qn = np.sqrt((q * q).sum(-1) + eps)
    kn = np.sqrt((k * k).sum(-1) + eps)
    np.testing.assert_allclose(cos * qn * kn / scale, (q * k).sum(-1), rtol=1e-12)
    # scale invariance when eps = 0, and |cos| <= scale
    o2, _ = oracle.recurrence(3.0 * q, 0.5 * k, v, g, beta, h0, l2=True, eps=0.0,
                              scale=scale)
    o3, _ = oracle.recurrence(q, k, v, g, beta, h0, l2=True, eps=0.0, scale=scale)
    np.testing.assert_allclose(o2, o3, rtol=1e-12)
    assert np.all(np.abs(o3[..., 0] / v[..., 0]) <= scale * (1 + 1e-12))


@pytest.mark.parametrize("T", [1, 2, 3, 4, 37])
def test_conv_matches_torch_conv1d(T):
    rng = np.random.default_rng(17 + T)
    C, K = 6, 4
    x = rng.standard_normal((T, C))
    w = 0.5 * rng.standard_normal((C, K))
    st = rng.standard_normal((C, K - 1))
    y, st_out = oracle.conv_silu(x, w, st)
    ext = torch.tensor(np.concatenate([st.T, x], 0).T[None])      # [1, C, K-1+T]
    ref = F.silu(F.conv1d(ext, torch.tensor(w)[:, None, :], groups=C))[0].T.numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-14)
    full = np.concatenate([st, x.T], axis=1)
    np.testing.assert_array_equal(st_out, full[:, -(K - 1):])


def test_conv_split_equals_one_shot():
    rng = np.random.default_rng(18)
    C, K, T = 5, 4, 11
    x = rng.standard_normal((T, C))
    w = rng.standard_normal((C, K))
    st = rng.standard_normal((C, K - 1))
    y, s = oracle.conv_silu(x, w, st)
    parts, cur = [], st
    for a, b in [(0, 1), (1, 3), (3, 4), (4, 11)]:
        yp, cur = oracle.conv_silu(x[a:b], w, cur)
        parts.append(yp)
    np.testing.assert_array_equal(np.concatenate(parts), y)
    np.testing.assert_array_equal(cur, s)


# ---------------------------------------------------------------------------------------
# shared q/k heads


@pytest.mark.parametrize("front", [False, True])
def test_shared_qk_heads_equal_repeated_heads(front):
    """Hqk q/k heads serving H value heads (value head h reads q/k head h // (H/Hqk)) give
    exactly the results of H heads whose q/k columns, conv taps and windows are the
    q/k head's, repeated in place for each value head it serves."""
    rng = np.random.default_rng(41)
    T, H, Hqk, dk, dv, K = 9, 6, 2, 4, 3, 4
    grp = H // Hqk
    cd_s, cd_f = 2 * Hqk * dk + H * dv, 2 * H * dk + H * dv
    x = rng.standard_normal((T, cd_s))
    g = -np.logaddexp(0.0, rng.standard_normal((T, H)))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    h0 = 0.3 * rng.standard_normal((1, H, dk, dv))
    # full layout: channel list of the shared layout for every channel of the full one
    src = np.concatenate(
        [np.arange((h // grp) * dk, (h // grp + 1) * dk) for h in range(H)]
        + [Hqk * dk + np.arange((h // grp) * dk, (h // grp + 1) * dk) for h in range(H)]
        + [2 * Hqk * dk + np.arange(h * dv, (h + 1) * dv) for h in range(H)])
    assert src.size == cd_f
    kw, kf = {}, {}
    if front:
        w = rng.standard_normal((cd_s, K))
        st = rng.standard_normal((1, cd_s, K - 1))
        kw = dict(conv_w=w, conv_state=st)
        kf = dict(conv_w=w[src], conv_state=st[:, src])
    shared = oracle.prefill(x, g, beta, h0, H=H, dk=dk, dv=dv, Hqk=Hqk, **kw)
    full = oracle.prefill(x[:, src], g, beta, h0, H=H, dk=dk, dv=dv, **kf)
    np.testing.assert_array_equal(shared["o"], full["o"])
    np.testing.assert_array_equal(shared["h"], full["h"])
    if front:
        np.testing.assert_array_equal(shared["conv_state"], full["conv_state"])
    # the grouping is seen: value heads that read q/k head h % Hqk instead differ
    alt = np.concatenate(
        [np.arange((h % Hqk) * dk, (h % Hqk + 1) * dk) for h in range(H)]
        + [Hqk * dk + np.arange((h % Hqk) * dk, (h % Hqk + 1) * dk) for h in range(H)]
        + [2 * Hqk * dk + np.arange(h * dv, (h + 1) * dv) for h in range(H)])
    ka = dict(conv_w=kw["conv_w"][alt], conv_state=kw["conv_state"][:, alt]) if front else {}
    other = oracle.prefill(x[:, alt], g, beta, h0, H=H, dk=dk, dv=dv, **ka)
    assert np.abs(other["o"] - shared["o"]).max() > 1e-3


# ---------------------------------------------------------------------------------------
# output gate (gated RMSNorm)


def test_gated_rmsnorm_hand_worked():
    # o = (3, 4): mean square 12.5, root 5 / sqrt(2); w = (1, 2); z = (0, ln 3):
    # sigmoid(ln 3) = 3/4, so silu = (0, 0.75 ln 3); y = (0, 2 * 4 sqrt(2) / 5 * 0.75 ln 3)
    # = (0, 1.2 sqrt(2) ln 3), worked by hand
    y = oracle.gated_rmsnorm(np.array([[3.0, 4.0]]), np.array([[0.0, np.log(3.0)]]),
                             np.array([1.0, 2.0]), eps=0.0)
    assert y[0, 0] == 0.0
    assert abs(y[0, 1] - 1.2 * np.sqrt(2.0) * np.log(3.0)) < 1e-14
    # eps enters beside the mean square: o = (1, 1), eps = 3 -> 1 / sqrt(1 + 3) = 0.5;
    # z = 40: silu(40) = 40 to double precision
    y = oracle.gated_rmsnorm(np.ones((1, 2)), np.full((1, 2), 40.0), np.ones(2), eps=3.0)
    np.testing.assert_allclose(y, [[20.0, 20.0]], rtol=1e-15)


def test_gated_rmsnorm_matches_torch():
    """torch's rms_norm (weight over the last axis) times torch's silu, in float64; a large
    eps so its place in the formula matters."""
    rng = np.random.default_rng(31)
    o = rng.standard_normal((5, 3, 64))
    z = 2.0 * rng.standard_normal((5, 3, 64))
    w = 1.0 + 0.3 * rng.standard_normal(64)
    for eps in (1e-6, 0.5):
        y = oracle.gated_rmsnorm(o, z, w, eps)
        ref = F.rms_norm(torch.tensor(o), (64,), weight=torch.tensor(w), eps=eps) * \
            F.silu(torch.tensor(z))
        np.testing.assert_allclose(y, ref.numpy(), rtol=1e-12, atol=1e-14)


def test_gated_rmsnorm_invariants():
    rng = np.random.default_rng(32)
    o = rng.standard_normal((4, 16))
    z = rng.standard_normal((4, 16))
    w = rng.standard_normal(16)
    # scale invariance with eps = 0; a constant row normalises to its sign
    np.testing.assert_allclose(oracle.gated_rmsnorm(7.5 * o, z, w, 0.0),
                               oracle.gated_rmsnorm(o, z, w, 0.0), rtol=1e-12)
    c = np.full((1, 16), -2.5)
    np.testing.assert_allclose(oracle.gated_rmsnorm(c, z[:1], w, 0.0),
                               -w * z[:1] / (1.0 + np.exp(-z[:1])), rtol=1e-12)


# ---------------------------------------------------------------------------------------
# invariants of the whole path


def test_linearity_in_state_and_values():
    rng = np.random.default_rng(19)
    q, k, v, g, beta, h0 = _rand_case(rng, 12, 2, 6, 5, kda=True)
    f = lambda hh, vv: oracle.recurrence(q, k, vv, g, beta, hh, l2=True)
    o, h = f(h0, v)
    o1, h1 = f(h0, 0 * v)
    o2, h2 = f(0 * h0, v)
    np.testing.assert_allclose(o, o1 + o2, atol=1e-12)
    np.testing.assert_allclose(h, h1 + h2, atol=1e-12)
    o3, h3 = f(2.5 * h0, 2.5 * v)
    np.testing.assert_allclose(o3, 2.5 * o, rtol=1e-12, atol=1e-13)


def test_value_column_and_head_permutation():
    rng = np.random.default_rng(20)
    q, k, v, g, beta, h0 = _rand_case(rng, 10, 3, 6, 5, kda=True)
    o, h = oracle.recurrence(q, k, v, g, beta, h0, l2=True)
    pc = rng.permutation(5)
    o_c, h_c = oracle.recurrence(q, k, v[..., pc], g, beta, h0[..., pc], l2=True)
    np.testing.assert_array_equal(o_c, o[..., pc])
    np.testing.assert_array_equal(h_c, h[..., pc])
    ph = rng.permutation(3)
    o_h, h_h = oracle.recurrence(q[:, ph], k[:, ph], v[:, ph], g[:, ph], beta[:, ph],
                                 h0[:, ph], l2=True)
    np.testing.assert_array_equal(o_h, o[:, ph])
    np.testing.assert_array_equal(h_h, h[:, ph])


def test_split_equals_one_shot_bitwise():
    rng = np.random.default_rng(21)
    q, k, v, g, beta, h0 = _rand_case(rng, 40, 2, 8, 6, kda=True)
    o, h = oracle.recurrence(q, k, v, g, beta, h0)
    parts, cur = [], h0
    for a, b in [(0, 13), (13, 14), (14, 40)]:
        op, cur = oracle.recurrence(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b], cur)
        parts.append(op)
    np.testing.assert_array_equal(np.concatenate(parts), o)
    np.testing.assert_array_equal(cur, h)


def test_varlen_equals_per_stream_and_ignores_tails():
    rng = np.random.default_rng(22)
    lens = [5, 1, 17, 9]
    N = sum(lens)
    pad = 7
    q, k, v, g, beta, _ = _rand_case(rng, N + pad, 2, 8, 6)
    h0 = 0.3 * rng.standard_normal((len(lens), 2, 8, 6))
    cu = np.concatenate([[0], np.cumsum(lens)])
    outs = []
    for fill in (0.0, np.nan, 1e30):
        arrs = [a.copy() for a in (q, k, v, g, beta)]
        for a in arrs:
            a[N:] = fill
        outs.append(oracle.recurrence(*arrs, h0, cu))
    for o_, h_ in outs[1:]:
        np.testing.assert_array_equal(o_[:N], outs[0][0][:N])
        np.testing.assert_array_equal(h_, outs[0][1])
    o, h = outs[0]
    for b in range(len(lens)):
        s = slice(cu[b], cu[b + 1])
        ob, hb = oracle.recurrence(q[s], k[s], v[s], g[s], beta[s], h0[b:b + 1])
        np.testing.assert_array_equal(o[s], ob)
        np.testing.assert_array_equal(h[b], hb[0])
    # a zero-length stream leaves its state unchanged
    o_e, h_e = oracle.recurrence(q[:5], k[:5], v[:5], g[:5], beta[:5], h0[:2],
                                 np.array([0, 5, 5]))
    np.testing.assert_array_equal(h_e[1], h0[1])


def test_prefill_front_end_composition():
    """prefill() = conv+SiLU per stream, then split q|k|v, then the recurrence."""
    rng = np.random.default_rng(23)
    H, dk, dv, K = 2, 4, 3, 4
    cd = 2 * H * dk + H * dv
    lens = [6, 2]
    N = sum(lens)
    x = rng.standard_normal((N + 3, cd))
    g = -np.logaddexp(0, rng.standard_normal((N + 3, H)))
    beta = 1 / (1 + np.exp(-rng.standard_normal((N + 3, H))))
    h0 = rng.standard_normal((2, H, dk, dv))
    w = rng.standard_normal((cd, K))
    st = rng.standard_normal((2, cd, K - 1))
    cu = [0, 6, 8]
    r = oracle.prefill(x, g, beta, h0, H=H, dk=dk, dv=dv, cu_seqlens=cu, conv_w=w,
                       conv_state=st)
    r1 = oracle.prefill(x, g, beta, h0, H=H, dk=dk, dv=dv, cu_seqlens=cu, conv_w=w,
                        conv_state=st, heads=[1])
    np.testing.assert_array_equal(r1["o"][:, 0], r["o"][:, 1])
    np.testing.assert_array_equal(r1["h"][:, 0], r["h"][:, 1])
    for b in range(2):
        s = slice(cu[b], cu[b + 1])
        y, ns = oracle.conv_silu(x[s], w, st[b])
        np.testing.assert_array_equal(ns, r["conv_state"][b])
        q = y[:, :H * dk].reshape(-1, H, dk)
        k = y[:, H * dk:2 * H * dk].reshape(-1, H, dk)
        v = y[:, 2 * H * dk:].reshape(-1, H, dv)
        ob, hb = oracle.recurrence(q, k, v, g[s], beta[s], h0[b:b + 1])
        np.testing.assert_array_equal(ob, r["o"][s])
        np.testing.assert_array_equal(hb[0], r["h"][b])


def test_oracle_reports_allocation_failure():
    """A channel buffer the oracle cannot allocate makes the call fail (ORACLE_ENOMEM = -2)
    instead of skipping the channel: a stream of 2^58 tokens asks for 2^61 bytes per
    channel, which malloc refuses before anything is read or written."""
    import ctypes
    lib = oracle._load()
    dp = ctypes.POINTER(ctypes.c_double)
    x = np.zeros(8)
    w = np.zeros(4)
    y = np.zeros(8)
    rc = lib.gdn_oracle_conv_silu(2 ** 58, 1, 4, x.ctypes.data_as(dp), w.ctypes.data_as(dp),
                                  None, y.ctypes.data_as(dp), None)
    assert rc == -2
    # and a call that can allocate still succeeds
    assert lib.gdn_oracle_conv_silu(2, 1, 4, x.ctypes.data_as(dp), w.ctypes.data_as(dp),
                                    None, y.ctypes.data_as(dp), None) == 0
