"""Test-only f64 chunked (WY / UT-transform) form of KDA, the gated delta
rule with one log-decay per key channel.

It pins the chunked derivation against the token-by-token oracle before any
kernel uses it; it is numpy and shares nothing with the oracle's C code or the
HIP kernels.

Within one chunk of n tokens of one (sequence, value head), entering state S0
[Dv, Dk], with G_t[d] = sum_{m<=t} g_m[d] (the channel's log-decay summed
from the chunk start):

    E_ti[d] = exp(G_t[d] - G_i[d])                         (i <= t; <= 1)
    A[t, i] = beta_t sum_d k_t[d] k_i[d] E_ti[d]           for i < t
    T       = (I + A)^-1
    W       = T diag(beta) (K * exp(G))         [n, Dk]
    U       = T diag(beta) V                    [n, Dv]
    Delta   = U - W S0^T
    O       = ((s Q) * exp(G)) S0^T + P Delta,  P[t, i] = s sum_d q_t[d] k_i[d] E_ti[d], i <= t
    S_n     = S0 diag(exp(G_n)) + Delta^T (K * exp(G_n - G))

Unrolling S_t = S_{t-1} diag(exp(g_t)) + delta_t k_t^T gives
S_t = S0 diag(exp(G_t)) + sum_{i<=t} delta_i (k_i * E_ti)^T, and substituting
it into delta_t = beta_t (v_t - S_{t-1} diag(exp(g_t)) k_t) and o_t = S_t (s q_t)
gives the lines above.

E is never formed as exp(G_t) * exp(-G_i), which overflows once a channel's
decay summed over the chunk is large.  Blocks of B tokens are used instead:
with rho_I = G at the last token before block I (rho_0 = 0), for t in block I
and i in an earlier block J,
    E_ti = exp(G_t - rho_I) exp(rho_I - rho_{J+1}) exp(rho_{J+1} - G_i),
a product of three factors that are each at most 1 (G only decreases), so
the off-diagonal blocks are plain matrix products of scaled rows; inside a
diagonal block E is taken exactly per pair.
"""
import numpy as np


def pair_decay(G, B):
    """E[t, i, :] for i <= t (zero above the diagonal), by the block factoring."""
    n, Dk = G.shape
    E = np.zeros((n, n, Dk))
    nb = (n + B - 1) // B
    rho = [np.zeros(Dk)] + [G[I * B - 1] for I in range(1, nb)]
    for I in range(nb):
        t0, t1 = I * B, min(I * B + B, n)
        for t in range(t0, t1):
            for i in range(t0, t + 1):       # diagonal block: exact
                E[t, i] = np.exp(G[t] - G[i])
            for J in range(I):
                i0, i1 = J * B, J * B + B
                left = np.exp(G[t] - rho[I])                  # <= 1
                mid = np.exp(rho[I] - rho[J + 1])             # <= 1
                right = np.exp(rho[J + 1] - G[i0:i1])         # <= 1, [B, Dk]
                E[t, i0:i1] = left * mid * right
    return E


def chunked_kda(q, k, v, g, beta, cu, state_in, has_init, scale, chunk, block=16):
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
                G = np.cumsum(g[c0:c1, h], axis=0)            # [n, Dk]
                E = pair_decay(G, block)
                KK = np.einsum("td,id,tid->ti", K, K, E)
                QK = np.einsum("td,id,tid->ti", Q, K, E)
                A = np.tril(bb[:, None] * KK, -1)
                Tm = np.linalg.inv(np.eye(n) + A)
                W = Tm @ (bb[:, None] * (K * np.exp(G)))
                U = Tm @ (bb[:, None] * V)
                Delta = U - W @ S.T
                O = (Q * np.exp(G)) @ S.T + np.tril(QK) @ Delta
                S = S * np.exp(G[-1])[None, :] + Delta.T @ (K * np.exp(G[-1][None, :] - G))
                out[c0:c1, h] = O
            state_out[s, h] = S
    return out, state_out
