"""Pins for the KDA part of the oracle (vllm.cpp cpu_ops.cpp,
KdaHeadTokenStep, KdaGatedDeltaRuleKernel, KdaChunkPrefillKernel): the
per-key-channel decay against the pinned GDN recurrence, brute-force matrix
algebra, channel-wise invariants, the gate's closed form, and an independent
chunked form.  Dk != Dv and Hv != Hk throughout, so that decaying the state's
rows instead of its columns, or a wrong GQA map, cannot pass."""
import numpy as np
import pytest
from scipy.special import expit

import oracle
from tests.chunked_kda_ref import chunked_kda


def _rand(shape, seed, std=1.0):
    return np.random.default_rng(seed).normal(0.0, std, size=shape)


def _problem(T=9, Hk=2, Hv=4, Dk=6, Dv=5, N=1, seed=0, gscale=0.3):
    rng = np.random.default_rng(seed)
    q = rng.normal(size=(T, Hk, Dk)) * 0.5
    k = rng.normal(size=(T, Hk, Dk)) * 0.5
    v = rng.normal(size=(T, Hv, Dv))
    g = -np.abs(rng.normal(size=(T, Hv, Dk))) * gscale
    beta = rng.uniform(0.1, 0.9, size=(T, Hv))
    S0 = rng.normal(size=(N, Hv, Dv, Dk)) * 0.1
    return q, k, v, g, beta, S0


def test_equal_channel_decays_reduce_to_gdn():
    q, k, v, g, beta, S0 = _problem(seed=1)
    gh = g[:, :, 0]
    g_all = np.repeat(gh[:, :, None], g.shape[2], axis=2)
    o1, s1 = oracle.kda_recurrence(q, k, v, g_all, beta, [0, 9], S0, [1], 0.7)
    o2, s2 = oracle.recurrence(q, k, v, gh, beta, [0, 9], S0, [1], 0.7)
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(s1, s2, rtol=1e-13, atol=1e-14)


def test_brute_force_matrix_algebra():
    """S_t = S_{t-1} diag(exp(g_t)) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
    o_t = S_t (scale q_t), for every value head with its key head h // r."""
    q, k, v, g, beta, S0 = _problem(T=7, seed=2)
    scale = 0.45
    out, st = oracle.kda_recurrence(q, k, v, g, beta, [0, 7], S0, [1], scale)
    Hk, Hv, Dk = q.shape[1], v.shape[1], q.shape[2]
    for h in range(Hv):
        kh = h // (Hv // Hk)
        S = S0[0, h].copy()
        for t in range(7):
            kt = k[t, kh]
            S = S @ np.diag(np.exp(g[t, h])) @ (np.eye(Dk) - beta[t, h] * np.outer(kt, kt)) \
                + beta[t, h] * np.outer(v[t, h], kt)
            np.testing.assert_allclose(out[t, h], S @ (scale * q[t, kh]), rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(st[0, h], S, rtol=1e-12, atol=1e-13)


def test_beta_zero_decays_columns_only():
    """With beta = 0 each state column d is multiplied by exp(g[t, h, d]); a
    channel whose decay is exp(-inf) = 0 has its column reset."""
    q, k, v, g, beta, S0 = _problem(T=3, seed=3)
    beta[:] = 0.0
    g[1, :, 2] = -np.inf
    _, st = oracle.kda_recurrence(q, k, v, g, beta, [0, 3], S0, [1], 1.0)
    total = np.exp(g.sum(axis=0))                    # [Hv, Dk]
    np.testing.assert_allclose(st[0], S0[0] * total[:, None, :], rtol=1e-13, atol=0)
    assert np.all(st[0][:, :, 2] == 0)


def test_gate_closed_form():
    rng = np.random.default_rng(4)
    T, Hv, Dk = 5, 3, 4
    g_raw = rng.normal(size=(T, Hv, Dk)) * 4
    A_log = rng.uniform(0, np.log(16), Hv)
    dt_bias = rng.uniform(-1, 1, (Hv, Dk))
    want = -np.exp(A_log)[None, :, None] * np.logaddexp(0.0, g_raw + dt_bias[None])
    np.testing.assert_allclose(oracle.kda_gate(g_raw, A_log, dt_bias), want, rtol=1e-14)
    want0 = -np.exp(A_log)[None, :, None] * np.logaddexp(0.0, g_raw)
    np.testing.assert_allclose(oracle.kda_gate(g_raw, A_log, None), want0, rtol=1e-14)
    # softplus(0) = ln 2
    assert oracle.kda_gate(np.zeros((1, 1, 1)), [0.0])[0, 0, 0] == pytest.approx(-np.log(2.0), rel=1e-15)


@pytest.mark.parametrize("T,chunk,block,gscale", [(37, 16, 4, 0.3), (64, 64, 16, 0.2), (100, 32, 8, 60.0)])
def test_chunked_form_equals_recurrence(T, chunk, block, gscale):
    """The independent chunked (WY/UT) form with block-factored decays equals
    the token recurrence, including decays large enough that exp(-G) alone
    would overflow."""
    q, k, v, g, beta, S0 = _problem(T=T, N=2, seed=5, gscale=gscale)
    cu = np.array([0, T // 3, T], np.int32)
    has_init = np.array([1, 0], np.uint8)
    o1, s1 = oracle.kda_recurrence(q, k, v, g, beta, cu, S0, has_init, 0.6)
    o2, s2 = chunked_kda(q, k, v, g, beta, cu, S0, has_init, 0.6, chunk, block)
    assert np.all(np.isfinite(o2)) and np.all(np.isfinite(s2))
    np.testing.assert_allclose(o2, o1, rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(s2, s1, rtol=1e-9, atol=1e-11)


def test_split_calls_and_empty_sequences():
    q, k, v, g, beta, S0 = _problem(T=12, seed=6)
    o_all, s_all = oracle.kda_recurrence(q, k, v, g, beta, [0, 12], S0, [1], 0.5)
    o_a, s_a = oracle.kda_recurrence(q[:5], k[:5], v[:5], g[:5], beta[:5], [0, 5], S0, [1], 0.5)
    o_b, s_b = oracle.kda_recurrence(q[5:], k[5:], v[5:], g[5:], beta[5:], [0, 7], s_a, [1], 0.5)
    np.testing.assert_allclose(np.concatenate([o_a, o_b]), o_all, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(s_b, s_all, rtol=1e-13, atol=1e-14)
    # an empty sequence keeps its initial state (zero without one)
    S2 = np.concatenate([S0, S0 * 2])
    _, s_e = oracle.kda_recurrence(q, k, v, g, beta, [0, 12, 12], S2, [1, 1], 0.5)
    np.testing.assert_array_equal(s_e[1], S2[1])
    _, s_z = oracle.kda_recurrence(q, k, v, g, beta, [0, 12, 12], S2, [1, 0], 0.5)
    assert np.all(s_z[1] == 0)


def test_pool_composition_with_gate():
    """oracle.kda applies the gate when A_log is given, gathers and scatters
    slots, and rounds the stored state once."""
    q, k, v, g_raw, beta, _ = _problem(T=10, seed=7)
    rng = np.random.default_rng(8)
    pool = rng.normal(size=(5, 4, 5, 6)) * 0.1
    A_log = rng.uniform(0, 2, 4)
    dtb = rng.uniform(-1, 1, (4, 6))
    cu = np.array([0, 4, 10], np.int32)
    slots = np.array([3, 1])
    out, newp = oracle.kda(None, cu, q, k, v, g_raw, beta, pool, slots, [1, 1], 0.5, A_log=A_log, dt_bias=dtb,
                           state_dtype="bf16")
    g = oracle.kda_gate(g_raw, A_log, dtb)
    o2, s2 = oracle.kda_recurrence(q, k, v, g, beta, cu, pool[slots], [1, 1], 0.5)
    np.testing.assert_array_equal(out, oracle.round_to(o2, "f32"))
    np.testing.assert_array_equal(newp[slots], oracle.round_to(s2, "bf16"))
    for sl in (0, 2, 4):
        np.testing.assert_array_equal(newp[sl], pool[sl])


def _l2n(x):
    """q / sqrt(sum q^2 + 1e-6) per (token, key head): the plain sum, eps
    inside the root (ferrum-kernels cpu.rs, recurrent_gated_delta_rule_f32's
    in-loop normalisation; the same form as the GDN prepare's L2 norm)."""
    return x / np.sqrt((x ** 2).sum(-1, keepdims=True) + 1e-6)


def test_l2norm_inside_equals_prenormalised():
    """kda_recurrence(l2norm=True) equals kda_recurrence on q and k
    normalised beforehand in numpy, with per-channel decays and Hv != Hk."""
    q, k, v, g, beta, S0 = _problem(T=11, N=2, seed=9)
    cu = np.array([0, 4, 11], np.int32)
    has = np.array([1, 0], np.uint8)
    o1, s1 = oracle.kda_recurrence(q, k, v, g, beta, cu, S0, has, 0.55, l2norm=True)
    o2, s2 = oracle.kda_recurrence(_l2n(q), _l2n(k), v, g, beta, cu, S0, has, 0.55, l2norm=False)
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(s1, s2, rtol=1e-13, atol=1e-14)


def test_l2norm_brute_force_matrix_algebra():
    """With the in-loop norm, S_t = S_{t-1} diag(exp(g_t)) (I - beta_t kh kh^T)
    + beta_t v_t kh^T and o_t = S_t (scale qh), kh and qh the normalised key
    and query, written out with explicit Dk x Dk matrices."""
    q, k, v, g, beta, S0 = _problem(T=6, seed=10)
    k *= 3.0  # norms well away from 1, so a skipped normalisation shows
    scale = 0.8
    out, st = oracle.kda_recurrence(q, k, v, g, beta, [0, 6], S0, [1], scale, l2norm=True)
    Hk, Hv, Dk = q.shape[1], v.shape[1], q.shape[2]
    for h in range(Hv):
        kh = h // (Hv // Hk)
        S = S0[0, h].copy()
        for t in range(6):
            kt = k[t, kh] / np.linalg.norm(np.append(k[t, kh], 1e-3))   # sqrt(|k|^2 + 1e-6)
            qt = q[t, kh] / np.linalg.norm(np.append(q[t, kh], 1e-3))
            S = S @ np.diag(np.exp(g[t, h])) @ (np.eye(Dk) - beta[t, h] * np.outer(kt, kt)) \
                + beta[t, h] * np.outer(v[t, h], kt)
            np.testing.assert_allclose(out[t, h], S @ (scale * qt), rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(st[0, h], S, rtol=1e-12, atol=1e-13)


def test_l2norm_eps_inside_the_root_small_vectors():
    """One token from a zero state with q = k = c e_0, beta = 1, scale = 1:
    o = v (kh . qh) with kh . qh = c^2 / (c^2 + 1e-6).  At c = 1e-3 that is
    exactly 1/2; eps outside the root (c / (|c| + 1e-6)) would give 0.998."""
    Dk, Dv = 4, 3
    c = 1e-3
    q = np.zeros((1, 1, Dk)); q[0, 0, 0] = c
    k = q.copy()
    v = np.array([[[1.0, -2.0, 0.5]]])
    g = np.zeros((1, 1, Dk))
    beta = np.ones((1, 1))
    out, st = oracle.kda_recurrence(q, k, v, g, beta, [0, 1], np.zeros((1, 1, Dv, Dk)), [0], 1.0, l2norm=True)
    np.testing.assert_allclose(out[0, 0], v[0, 0] * 0.5, rtol=1e-12)
    # S = beta v kh^T with kh = e_0 / sqrt(2)
    want = np.zeros((Dv, Dk)); want[:, 0] = v[0, 0] / np.sqrt(2.0)
    np.testing.assert_allclose(st[0, 0], want, rtol=1e-12)
