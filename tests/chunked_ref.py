"""Test-only f64 chunked (WY / UT-transform) form of the gated delta rule.

It exists to pin two things against each other before any kernel uses the
chunked form: the derivation below and the token-by-token oracle.  It is
written in numpy and shares nothing with either the oracle's C code or the HIP
kernels.

Within one chunk of n tokens of one (sequence, value head), entering state S0
[Dv, Dk], with G_i = sum_{j<=i} g_j and gamma_i = exp(G_i):

    A[j, m] = beta_j exp(G_j - G_m) (k_j . k_m)        for m < j, else 0
    T       = (I + A)^-1                                 (unit lower triangular)
    W       = T diag(beta * gamma) K          [n, Dk]
    U       = T diag(beta) V                  [n, Dv]
    Delta   = U - W S0^T                      [n, Dv]   (rows are the deltas)
    O       = diag(gamma) (s Q) S0^T + (mask_incl * exp(G_i - G_j) * (s Q) K^T) Delta
    S_n     = gamma_n S0 + Delta^T diag(exp(G_n - G_j)) K

Unrolling S_i = exp(g_i) S_{i-1} + delta_i k_i^T gives
S_i = gamma_i S0 + sum_{j<=i} (gamma_i / gamma_j) delta_j k_j^T; substituting
it into delta_j = beta_j (v_j - exp(g_j) S_{j-1} k_j) gives (I + A) Delta =
diag(beta) V - diag(beta gamma) K S0^T, and o_i = S_i (s q_i) gives O.
"""
import numpy as np


def chunked_recurrence(q, k, v, g, beta, cu, state_in, has_init, scale, chunk):
    q, k, v = (np.asarray(a, np.float64) for a in (q, k, v))
    g, beta = np.asarray(g, np.float64), np.asarray(beta, np.float64)
    T, Hk, Dk = q.shape
    Hv, Dv = v.shape[1:]
    r = Hv // Hk
    N = len(cu) - 1
    out = np.zeros((T, Hv, Dv))
    state_out = np.zeros((N, Hv, Dv, Dk))
    for s in range(N):
        for h in range(Hv):
            kh = h // r
            S = np.array(state_in[s, h], np.float64) if has_init[s] else np.zeros((Dv, Dk))
            for c0 in range(int(cu[s]), int(cu[s + 1]), chunk):
                c1 = min(c0 + chunk, int(cu[s + 1]))
                n = c1 - c0
                K = k[c0:c1, kh]
                Q = q[c0:c1, kh] * scale
                V = v[c0:c1, h]
                bb = beta[c0:c1, h]
                G = np.cumsum(g[c0:c1, h])
                gam = np.exp(G)
                diff = G[:, None] - G[None, :]
                lower_incl = np.tril(np.ones((n, n), bool))
                lower_strict = np.tril(np.ones((n, n), bool), -1)
                D_incl = np.where(lower_incl, np.exp(np.where(lower_incl, diff, 0.0)), 0.0)
                A = np.where(lower_strict, bb[:, None] * D_incl * (K @ K.T), 0.0)
                Tm = np.linalg.inv(np.eye(n) + A)
                W = Tm @ ((bb * gam)[:, None] * K)
                U = Tm @ (bb[:, None] * V)
                Delta = U - W @ S.T
                O = gam[:, None] * (Q @ S.T) + (D_incl * (Q @ K.T)) @ Delta
                S = gam[-1] * S + Delta.T @ (np.exp(G[-1] - G)[:, None] * K)
                out[c0:c1, h] = O
            state_out[s, h] = S
    return out, state_out
