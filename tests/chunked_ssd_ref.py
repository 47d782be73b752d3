"""Test-only f64 chunked form of Mamba2 / SSD (the state space dual form), to
pin it against the token-by-token oracle before a kernel uses it.  numpy
only; shares nothing with the oracle's C code or the HIP kernels.

Within a chunk of n tokens of one (sequence, head), entering state S0 [P, N],
with a_i = A dt_i, L_i = sum_{j<=i} a_j (the chunk's running log-decay), and
X~ the rows dt_j x_j:
    Y_intra = (M * (C B^T)) X~,   M[i][j] = exp(L_i - L_j) for j <= i, else 0
    Y_inter[i] = exp(L_i) S0 C_i
    S_n = exp(L_n) S0 + sum_j exp(L_n - L_j) dt_j x_j B_j^T
    y = Y_intra + Y_inter (+ D x, then * silu(z))
which is the recurrence S_i = exp(a_i) S_{i-1} + dt_i x_i B_i^T, y_i = S_i C_i
unrolled over the chunk ([P1] Mamba2ChunkScanKernel, stages 1-5).
"""
import numpy as np


def chunked_ssd(x, dt, A, B, C, cu, state_in, has_init, chunk, D=None, z=None):
    x, dt, B, C = (np.asarray(a, np.float64) for a in (x, dt, B, C))
    A = np.asarray(A, np.float64)
    T, H, P = x.shape
    G, N = B.shape[1:]
    hpg = H // G
    Ns = len(cu) - 1
    out = np.zeros((T, H, P))
    st_out = np.zeros((Ns, H, P, N))
    for s in range(Ns):
        for h in range(H):
            g = h // hpg
            S = np.array(state_in[s, h], np.float64) if has_init[s] else np.zeros((P, N))
            for c0 in range(int(cu[s]), int(cu[s + 1]), chunk):
                c1 = min(c0 + chunk, int(cu[s + 1]))
                X, Bc, Cc, d = x[c0:c1, h], B[c0:c1, g], C[c0:c1, g], dt[c0:c1, h]
                L = np.cumsum(A[h] * d)
                n = c1 - c0
                M = np.where(np.tril(np.ones((n, n), bool)), np.exp(np.minimum(L[:, None] - L[None, :], 0.0)), 0.0)
                Xt = d[:, None] * X
                Y = (M * (Cc @ Bc.T)) @ Xt + np.exp(L)[:, None] * (Cc @ S.T)
                S = np.exp(L[-1]) * S + (np.exp(L[-1] - L)[:, None] * Xt).T @ Bc
                if D is not None:
                    Dh = np.asarray(D, np.float64)
                    Y = Y + (Dh[h] if Dh.ndim == 2 else Dh[h]) * X
                if z is not None:
                    zz = np.asarray(z, np.float64)[c0:c1, h]
                    Y = Y * (zz / (1.0 + np.exp(-zz)))
                out[c0:c1, h] = Y
            st_out[s, h] = S
    return out, st_out
