"""Independent fp64 checkers used to pin the oracle (test code, NumPy only).

* :func:`dense_unroll` -- brute force: builds the transition matrices of every token and
  multiplies them out. With h = S^T (dk x dv) one token of the gated delta rule is the
  affine map h_t = Phi_t h_{t-1} + beta_t k_t v_t^T with
  Phi_t = (I - beta_t k_t k_t^T) diag(alpha_t), so
  h_t = Phi_t...Phi_1 h_0 + sum_{s<=t} Phi_t...Phi_{s+1} beta_s k_s v_s^T and o_t = h_t^T q_t.
* :func:`chunked` -- the chunk-parallel form (cumulative log-gates, then the beta-weighted
  WY/UT transform w, u and the inter-chunk scan): per chunk of L tokens with entering
  state h0, Gamma = cumsum(g), a = exp(Gamma),
  M = strict_tril(diag(beta) (K.a)(K/a)^T), T = (I + M)^-1, W = T diag(beta) (K.a),
  U~ = T diag(beta) V, U = U~ - W h0, P = tril_incl((Q.a)(K/a)^T),
  O = (Q.a) h0 + P U, h_L = diag(a_L) h0 + (K.(a_L/a))^T U.
  It equals the token recurrence for every chunk size; with chunk 1 it is the recurrence.

Both take q and k as used by the recurrence (already normalised when the call
normalises), one head at a time.
"""
import numpy as np


def _alpha(g_t, dk):
    g_t = np.asarray(g_t, dtype=np.float64)
    return np.exp(g_t) * np.ones(dk) if g_t.ndim == 0 else np.exp(g_t)


def dense_unroll(q, k, v, g, beta, h0):
    """q, k [T, dk]; v [T, dv]; g [T] or [T, dk]; beta [T]; h0 [dk, dv] -> (o, hT)."""
    T, dk = k.shape
    eye = np.eye(dk)
    phis = []
    for t in range(T):
        kt = k[t][:, None]
        phis.append((eye - beta[t] * kt @ kt.T) @ np.diag(_alpha(g[t], dk)))

    def chain(t_hi, s_lo):
        """Phi_{t_hi} ... Phi_{s_lo} (identity when empty); 1-based token indices."""
        m = np.eye(dk)
        for tau in range(s_lo, t_hi + 1):
            m = phis[tau - 1] @ m
        return m

    o = np.zeros((T, v.shape[1]))
    h_t = h0
    for t in range(1, T + 1):
        h_t = chain(t, 1) @ h0
        for s in range(1, t + 1):
            h_t = h_t + chain(t, s + 1) @ (beta[s - 1] * np.outer(k[s - 1], v[s - 1]))
        o[t - 1] = h_t.T @ q[t - 1]
    return o, h_t


def chunked(q, k, v, g, beta, h0, C):
    """Chunk-size-C evaluation of one head; same arguments as :func:`dense_unroll`."""
    T, dk = k.shape
    g = np.asarray(g, dtype=np.float64)
    per_channel = g.ndim == 2
    h = np.array(h0, dtype=np.float64, copy=True)
    o = np.zeros((T, v.shape[1]))
    for s0 in range(0, T, C):
        sl = slice(s0, min(T, s0 + C))
        Q, K, V, b = q[sl], k[sl], v[sl], beta[sl]
        L = K.shape[0]
        G = np.cumsum(g[sl], axis=0)
        G = G if per_channel else np.repeat(G[:, None], dk, axis=1)
        a = np.exp(G)
        Kd, Ki = K * a, K * np.exp(-G)
        M = np.tril(b[:, None] * (Kd @ Ki.T), -1)
        Tm = np.linalg.inv(np.eye(L) + M)
        W = Tm @ (b[:, None] * Kd)
        Ut = Tm @ (b[:, None] * V)
        U = Ut - W @ h
        P = np.tril((Q * a) @ Ki.T)
        o[sl] = (Q * a) @ h + P @ U
        h = a[-1][:, None] * h + (K * np.exp(G[-1][None, :] - G)).T @ U
    return o, h
