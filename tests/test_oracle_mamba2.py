"""Pins for the Mamba2 / SSD part of the oracle (vllm.cpp cpu_ops.cpp,
Mamba2ChunkScanKernel, Mamba2StateUpdateKernel): brute-force matrix algebra,
closed forms at the two ends of the decay, the step-size processing against
numpy, an independent chunked (dual) form, split calls, and the slot-pool
composition.  G > 1 and P != N throughout, so a wrong group map or a
transposed state fails."""
import numpy as np
import pytest
from scipy.special import expit

import oracle
from tests.chunked_ssd_ref import chunked_ssd


def _problem(T=11, H=4, P=5, G=2, N=3, Ns=1, seed=0, Dper="h"):
    rng = np.random.default_rng(seed)
    x = rng.normal(size=(T, H, P))
    dt = rng.uniform(0.01, 0.5, size=(T, H))
    A = -rng.uniform(0.5, 4.0, size=H)
    B = rng.normal(size=(T, G, N))
    C = rng.normal(size=(T, G, N))
    D = rng.normal(size=H) if Dper == "h" else (rng.normal(size=(H, P)) if Dper == "hp" else None)
    z = rng.normal(size=(T, H, P))
    S0 = rng.normal(size=(Ns, H, P, N)) * 0.3
    return x, dt, A, B, C, D, z, S0


@pytest.mark.parametrize("Dper", ["h", "hp", None])
def test_brute_force(Dper):
    x, dt, A, B, C, D, z, S0 = _problem(seed=1, Dper=Dper)
    out, st = oracle.mamba2_recurrence(x, dt, A, B, C, [0, 11], S0, [1], D=D, z=z)
    T, H, P = x.shape
    for h in range(H):
        g = h // 2
        S = S0[0, h].copy()
        for t in range(T):
            S = np.exp(A[h] * dt[t, h]) * S + dt[t, h] * np.outer(x[t, h], B[t, g])
            y = S @ C[t, g]
            if D is not None:
                y = y + (D[h] if D.ndim == 1 else D[h]) * x[t, h]
            y = y * z[t, h] * expit(z[t, h])
            np.testing.assert_allclose(out[t, h], y, rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(st[0, h], S, rtol=1e-12, atol=1e-13)


def test_closed_forms():
    x, dt, A, B, C, D, z, S0 = _problem(seed=2)
    # no decay left (exp(A dt) = 0 in double): the state is the last token's outer product
    o, s = oracle.mamba2_recurrence(x, dt, np.full(4, -1e5), B, C, [0, 11], S0, [1])
    g = np.arange(4) // 2
    want = dt[:, :, None] * x * np.einsum("tgn,tgn->tg", B, C)[:, g][:, :, None]
    np.testing.assert_allclose(o, want, rtol=1e-13, atol=1e-14)
    # dt = 0: the state never changes
    o, s = oracle.mamba2_recurrence(x, np.zeros_like(dt), A, B, C, [0, 11], S0, [1], D=D)
    want = np.stack([np.stack([S0[0, h] @ C[t, h // 2] for h in range(4)]) for t in range(11)]) + D[None, :, None] * x
    np.testing.assert_allclose(o, want, rtol=1e-13, atol=1e-14)
    np.testing.assert_array_equal(s, S0)


def test_dt_processing():
    rng = np.random.default_rng(3)
    raw = rng.normal(size=(6, 4)) * 8
    bias = rng.uniform(-1, 1, 4)
    got = oracle.mamba2_dt(raw, bias, True, 0.001, 3.0)
    sp = np.where(raw + bias <= 20.0, np.logaddexp(0.0, raw + bias), raw + bias)
    np.testing.assert_allclose(got, np.clip(sp, 0.001, 3.0), rtol=1e-15)
    np.testing.assert_array_equal(oracle.mamba2_dt(raw, None, False, -np.inf, np.inf), raw)
    # the default limits (0, inf) clamp a negative step to 0
    np.testing.assert_array_equal(oracle.mamba2_dt(raw, None, False), np.maximum(raw, 0.0))


@pytest.mark.parametrize("chunk", [4, 16, 64])
def test_chunked_form_equals_recurrence(chunk):
    x, dt, A, B, C, D, z, S0 = _problem(T=70, Ns=3, seed=4)
    cu = np.array([0, 5, 40, 70], np.int32)
    has = np.array([1, 0, 1], np.uint8)
    o1, s1 = oracle.mamba2_recurrence(x, dt, A, B, C, cu, S0, has, D=D, z=z)
    o2, s2 = chunked_ssd(x, dt, A, B, C, cu, S0, has, chunk, D=D, z=z)
    np.testing.assert_allclose(o2, o1, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(s2, s1, rtol=1e-10, atol=1e-12)


def test_split_calls_and_pool():
    x, dt, A, B, C, D, z, S0 = _problem(T=20, seed=5)
    o, s = oracle.mamba2_recurrence(x, dt, A, B, C, [0, 20], S0, [1], D=D, z=z)
    oa, sa = oracle.mamba2_recurrence(x[:7], dt[:7], A, B[:7], C[:7], [0, 7], S0, [1], D=D, z=z[:7])
    ob, sb = oracle.mamba2_recurrence(x[7:], dt[7:], A, B[7:], C[7:], [0, 13], sa, [1], D=D, z=z[7:])
    np.testing.assert_allclose(np.concatenate([oa, ob]), o, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(sb, s, rtol=1e-13, atol=1e-14)
    # pool composition: dt processed, slots gathered and scattered, -1 rows inert, state rounded once
    rng = np.random.default_rng(6)
    pool = rng.normal(size=(6, 4, 5, 3))
    raw = rng.normal(size=(20, 4))
    cu = np.array([0, 1, 2, 3], np.int32)
    out, newp = oracle.mamba2(cu, x[:3], raw[:3], A, B[:3], C[:3], pool, [4, -1, 0], [1, 1, 1], D=D,
                              dt_bias=np.zeros(4), state_dtype="bf16")
    assert np.all(out[1] == 0)
    dtp = oracle.mamba2_dt(raw[[0, 2]], np.zeros(4))
    o2, s2 = oracle.mamba2_recurrence(x[[0, 2]], dtp, A, B[[0, 2]], C[[0, 2]], [0, 1, 2], pool[[4, 0]], [1, 1], D=D)
    np.testing.assert_array_equal(out[[0, 2]], oracle.round_to(o2, "f32"))
    np.testing.assert_array_equal(newp[[4, 0]], oracle.round_to(s2, "bf16"))
    for sl in (1, 2, 3, 5):
        np.testing.assert_array_equal(newp[sl], pool[sl])
