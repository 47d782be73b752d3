"""Pins for the f64 oracle, against things other than itself: hand-worked
fixtures, closed forms, library routines, brute-force matrix algebra,
invariants of the method and an independent chunked (WY/UT) formulation.

Several cases use Dk != Dv and Hv != Hk so that a transposed state, a swapped
operand or a wrong GQA mapping cannot pass.
"""
import json
import math
import os

import numpy as np
import pytest
from scipy.special import expit

import oracle
from gdn_inputs import Config, Dims, make_inputs
from tests.chunked_ref import chunked_recurrence

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _silu(z):
    return z * expit(z)


def _rand(shape, seed, std=1.0):
    return np.random.default_rng(seed).normal(0.0, std, size=shape)


# ---------------------------------------------------------------------------
# Hand-worked fixtures.
# ---------------------------------------------------------------------------
def test_golden_delta_rule_2x2():
    fx = json.load(open(os.path.join(GOLDEN, "worked_delta_rule_2x2.json")))
    T = len(fx["k"])
    k = np.array(fx["k"], float).reshape(T, 1, 2)
    q = np.array(fx["q"], float).reshape(T, 1, 2)
    v = np.array(fx["v"], float).reshape(T, 1, 2)
    g = np.array(fx["g"], float).reshape(T, 1)
    beta = np.array(fx["beta"], float).reshape(T, 1)
    out, st = oracle.recurrence(q, k, v, g, beta, [0, T], np.zeros((1, 1, 2, 2)), [0], scale=1.0)
    np.testing.assert_allclose(out[:, 0], fx["expected_out"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(st[0, 0], fx["expected_final_state"], rtol=0, atol=1e-15)


def test_golden_conv_and_gates():
    fx = json.load(open(os.path.join(GOLDEN, "worked_conv_gates.json")))
    x = np.array(fx["x"], float).reshape(-1, 1)
    w = np.array(fx["w"], float).reshape(1, -1)
    hist = np.array(fx["history"], float).reshape(1, 1, -1)
    y, hout = oracle.conv_silu(x, w, [0, 3], hist, [1])
    z = np.array(fx["expected_preact"])
    np.testing.assert_allclose(y[:, 0], z / (1.0 + np.exp(-z)), rtol=1e-15, atol=0)
    np.testing.assert_array_equal(hout[0, 0], fx["expected_history_out"])
    for case in fx["gate_cases"]:
        g, beta = oracle.gates([[case["a"]]], [[case["b"]]], [case["A_log"]], [case["dt_bias"]])
        assert g[0, 0] == pytest.approx(case["g"], rel=1e-15)
        assert beta[0, 0] == pytest.approx(case["beta"], rel=1e-15)


# ---------------------------------------------------------------------------
# a1: conv, against numpy.convolve and one-hot taps.
# ---------------------------------------------------------------------------
@pytest.mark.parametrize("K", [1, 2, 3, 4])
def test_conv_matches_numpy_convolve(K):
    lens = [1, 2, 5, 9]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, C = cu[-1], 6
    x = _rand((T, C), 1)
    w = _rand((C, K), 2, 0.5)
    hist = _rand((len(lens), C, K - 1), 3)
    has_init = np.array([1, 0, 1, 1], np.uint8)
    y, hout = oracle.conv_silu(x, w, cu, hist, has_init)
    for s in range(len(lens)):
        for c in range(C):
            h = hist[s, c] if has_init[s] else np.zeros(K - 1)
            seq = np.concatenate([h, x[cu[s]:cu[s + 1], c]])
            z = np.convolve(seq, w[c, ::-1], mode="valid")
            np.testing.assert_allclose(y[cu[s]:cu[s + 1], c], _silu(z), rtol=1e-13, atol=1e-15)
            np.testing.assert_array_equal(hout[s, c], seq[len(seq) - (K - 1):])


def test_conv_one_hot_taps_pin_tap_and_history_order():
    K, C = 4, 3
    lens = [2, 7]
    cu = np.array([0, 2, 9], np.int32)
    x = _rand((9, C), 4)
    hist = _rand((2, C, K - 1), 5)
    ones = np.ones(2, np.uint8)
    # last tap alone: identity conv
    w = np.zeros((C, K)); w[:, K - 1] = 1.0
    y, _ = oracle.conv_silu(x, w, cu, hist, ones)
    np.testing.assert_allclose(y, _silu(x), rtol=1e-15)
    # first tap alone: a delay of K-1 tokens, reaching into the history
    w = np.zeros((C, K)); w[:, 0] = 1.0
    y, hout = oracle.conv_silu(x, w, cu, hist, ones)
    for s, L in enumerate(lens):
        seq = np.concatenate([hist[s], x[cu[s]:cu[s + 1]].T], axis=1)  # [C, K-1+L]
        np.testing.assert_allclose(y[cu[s]:cu[s + 1]], _silu(seq[:, :L].T), rtol=1e-15)
        # short sequence (L < K-1): the old history shifts left, then the inputs
        np.testing.assert_array_equal(hout[s], seq[:, L:])


# ---------------------------------------------------------------------------
# a2 + a3: split and L2 norm.
# ---------------------------------------------------------------------------
def test_split_and_l2_norm():
    Hk, Hv, Dk, Dv = 2, 4, 8, 6
    Cc = 2 * Hk * Dk + Hv * Dv
    y = _rand((5, Cc), 6)
    q, k, v = oracle.split_l2(y, Hk, Hv, Dk, Dv, l2norm=True)
    for t in range(5):
        for h in range(Hk):
            qr = y[t, h * Dk:(h + 1) * Dk]
            kr = y[t, Hk * Dk + h * Dk: Hk * Dk + (h + 1) * Dk]
            np.testing.assert_allclose(q[t, h], qr / math.sqrt(np.linalg.norm(qr) ** 2 + 1e-6), rtol=1e-14)
            np.testing.assert_allclose(k[t, h], kr / math.sqrt(np.linalg.norm(kr) ** 2 + 1e-6), rtol=1e-14)
        np.testing.assert_array_equal(v[t].reshape(-1), y[t, 2 * Hk * Dk:])
    q2, k2, _ = oracle.split_l2(y, Hk, Hv, Dk, Dv, l2norm=False)
    np.testing.assert_array_equal(q2.reshape(5, -1), y[:, :Hk * Dk])
    # one-hot: c e_i -> c / sqrt(c^2 + eps)
    y1 = np.zeros((1, Cc)); y1[0, 3] = 0.01
    q1, _, _ = oracle.split_l2(y1, Hk, Hv, Dk, Dv)
    assert q1[0, 0, 3] == pytest.approx(0.01 / math.sqrt(1e-4 + 1e-6), rel=1e-15)


# ---------------------------------------------------------------------------
# a4: gates against library routines.
# ---------------------------------------------------------------------------
def test_gates_against_library():
    a = _rand((7, 5), 7, 5.0)
    a[0, :] = [-40.0, -20.0, 0.0, 20.0, 40.0]
    b = _rand((7, 5), 8, 5.0)
    A_log = np.random.default_rng(9).uniform(0, math.log(16), 5)
    dt = np.random.default_rng(10).uniform(-1, 1, 5)
    g, beta = oracle.gates(a, b, A_log, dt)
    np.testing.assert_allclose(g, -np.exp(A_log) * np.logaddexp(0.0, a + dt), rtol=1e-14)
    np.testing.assert_allclose(beta, expit(b), rtol=1e-14)
    assert np.all(g < 0)


# ---------------------------------------------------------------------------
# a5/a6 definition: the recurrence.
# ---------------------------------------------------------------------------
def _brute_force(q, k, v, g, beta, S0, scale, r):
    """S_t = S_{t-1} exp(g_t) (I - beta_t k_t k_t^T) + beta_t v_t k_t^T,
    o_t = S_t (scale q_t), with explicit Dk x Dk matrices."""
    T, Hk, Dk = q.shape
    Hv = v.shape[1]
    out = np.zeros(v.shape)
    S_all = np.array(S0, float)
    for h in range(Hv):
        S = S_all[h]
        kh = h // r
        for t in range(T):
            kt = k[t, kh][:, None]
            M = math.exp(g[t, h]) * (np.eye(Dk) - beta[t, h] * (kt @ kt.T))
            S = S @ M + beta[t, h] * (v[t, h][:, None] @ kt.T)
            out[t, h] = S @ (scale * q[t, kh])
        S_all[h] = S
    return out, S_all


@pytest.mark.parametrize("Hk,Hv,Dk,Dv", [(1, 1, 4, 3), (2, 4, 8, 6), (2, 6, 5, 7)])
def test_recurrence_brute_force(Hk, Hv, Dk, Dv):
    T = 8
    q = _rand((T, Hk, Dk), 11)
    k = _rand((T, Hk, Dk), 12) / math.sqrt(Dk)
    v = _rand((T, Hv, Dv), 13)
    g = -np.abs(_rand((T, Hv), 14))
    beta = expit(_rand((T, Hv), 15))
    S0 = _rand((1, Hv, Dv, Dk), 16, 0.3)
    out, st = oracle.recurrence(q, k, v, g, beta, [0, T], S0, [1], scale=0.37)
    ref_o, ref_s = _brute_force(q, k, v, g, beta, S0[0], 0.37, Hv // Hk)
    np.testing.assert_allclose(out, ref_o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(st[0], ref_s, rtol=1e-12, atol=1e-13)


def test_recurrence_gqa_maps_value_head_to_key_head_by_division():
    # Hk=2, Hv=4: value heads 0,1 read key head 0; 2,3 read key head 1
    Hk, Hv, Dk, Dv = 2, 4, 4, 4
    T = 1
    q = np.zeros((T, Hk, Dk)); q[0, 0, 0] = 1.0; q[0, 1, 1] = 1.0
    k = q.copy()
    v = np.ones((T, Hv, Dv))
    g = np.zeros((T, Hv)); beta = np.ones((T, Hv))
    _, st = oracle.recurrence(q, k, v, g, beta, [0, 1], np.zeros((1, Hv, Dv, Dk)), [0], scale=1.0)
    for h in range(Hv):
        kh = h // 2
        assert np.all(st[0, h][:, kh] == 1.0) and np.count_nonzero(st[0, h]) == Dv


def test_recurrence_one_token_closed_form():
    Dk, Dv = 6, 5
    q = _rand((1, 1, Dk), 20); k = _rand((1, 1, Dk), 21); v = _rand((1, 1, Dv), 22)
    g = np.array([[-0.3]]); beta = np.array([[0.8]])
    out, st = oracle.recurrence(q, k, v, g, beta, [0, 1], np.zeros((1, 1, Dv, Dk)), [0], scale=0.5)
    np.testing.assert_allclose(st[0, 0], 0.8 * np.outer(v[0, 0], k[0, 0]), rtol=1e-14)
    np.testing.assert_allclose(out[0, 0], 0.8 * v[0, 0] * (k[0, 0] @ (0.5 * q[0, 0])), rtol=1e-14)


def test_invariant_beta0_decay1_keeps_state():
    Dk, Dv, T = 8, 6, 5
    S0 = _rand((1, 1, Dv, Dk), 30)
    q = _rand((T, 1, Dk), 31); k = _rand((T, 1, Dk), 32); v = _rand((T, 1, Dv), 33)
    out, st = oracle.recurrence(q, k, v, np.zeros((T, 1)), np.zeros((T, 1)), [0, T], S0, [1], 0.7)
    np.testing.assert_array_equal(st, S0)
    np.testing.assert_allclose(out[:, 0], (S0[0, 0] @ (0.7 * q[:, 0].T)).T, rtol=1e-14)


def test_invariant_orthonormal_keys_exact_retrieval():
    # Hadamard rows / 4: orthonormal keys in Dk = 16, all entries +-1/4 (exact)
    H = np.array([[1.0]])
    for _ in range(4):
        H = np.block([[H, H], [H, -H]])
    keys = H / 4.0
    Dk, Dv, T = 16, 5, 6
    k = keys[:T].reshape(T, 1, Dk)
    v = _rand((T, 1, Dv), 40)
    S0 = _rand((1, 1, Dv, Dk), 41)
    out, st = oracle.recurrence(k, k, v, np.zeros((T, 1)), np.ones((T, 1)), [0, T], S0, [1], scale=1.0)
    for i in range(T):
        np.testing.assert_allclose(st[0, 0] @ keys[i], v[i, 0], rtol=0, atol=1e-14)
    np.testing.assert_allclose(out[:, 0], v[:, 0], rtol=0, atol=1e-14)  # q = k, scale 1


@pytest.mark.parametrize("gval", [-1e4, -np.inf])
def test_invariant_zero_decay_resets_state(gval):
    Dk, Dv = 8, 4
    q = _rand((1, 1, Dk), 50); k = _rand((1, 1, Dk), 51); v = _rand((1, 1, Dv), 52)
    S0 = _rand((1, 1, Dv, Dk), 53)
    out, st = oracle.recurrence(q, k, v, np.array([[gval]]), np.array([[0.6]]), [0, 1], S0, [1], 0.5)
    np.testing.assert_allclose(st[0, 0], 0.6 * np.outer(v[0, 0], k[0, 0]), rtol=1e-14)
    np.testing.assert_allclose(out[0, 0], 0.6 * v[0, 0] * (k[0, 0] @ (0.5 * q[0, 0])), rtol=1e-14)


@pytest.mark.parametrize("chunk", [1, 4, 16, 64])
def test_chunked_form_equals_sequential(chunk):
    Hk, Hv, Dk, Dv = 2, 4, 16, 8
    lens = [1, 37, 130]
    cu = np.concatenate([[0], np.cumsum(lens)])
    T = cu[-1]
    q = _rand((T, Hk, Dk), 60)
    k = _rand((T, Hk, Dk), 61)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = _rand((T, Hv, Dv), 62)
    g = -np.random.default_rng(63).uniform(0.01, 3.0, (T, Hv))
    beta = expit(_rand((T, Hv), 64))
    S0 = _rand((3, Hv, Dv, Dk), 65, 0.1)
    hi = np.array([1, 0, 1], np.uint8)
    o1, s1 = oracle.recurrence(q, k, v, g, beta, cu, S0, hi, 0.25)
    o2, s2 = chunked_recurrence(q, k, v, g, beta, cu, S0, hi, 0.25, chunk)
    np.testing.assert_allclose(o2, o1, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(s2, s1, rtol=1e-10, atol=1e-11)


def test_split_calls_equal_one_call():
    d = Dims(2, 4, 16, 8, 4)
    cfg = Config(name="t", mode="prefill", dims=d, seqlens=(50,), num_slots=3, act_dtype="f32",
                 state_dtype="f32", qkv_dtype="f32", init_state_std=0.1, conv_state_std=1.0, seed=5)
    inp = make_inputs(cfg)
    full = oracle.prepare(d, [0, 50], inp["x"], inp["w"], inp["a"], inp["b"], inp["A_log"], inp["dt_bias"],
                          inp["conv_pool"], inp["slots"], inp["has_init"], qkv_dtype="f32")
    o_full, s_full = oracle.recurrence(full["q"], full["k"], full["v"], full["g"], full["beta"], [0, 50],
                                       np.asarray(inp["ssm_pool"])[inp["slots"]], inp["has_init"], 0.25)
    pool_c, S = inp["conv_pool"], np.asarray(inp["ssm_pool"], float)[inp["slots"]]
    outs = []
    for t0, t1 in [(0, 2), (2, 19), (19, 50)]:
        part = oracle.prepare(d, [0, t1 - t0], inp["x"][t0:t1], inp["w"], inp["a"][t0:t1], inp["b"][t0:t1],
                              inp["A_log"], inp["dt_bias"], pool_c, inp["slots"], inp["has_init"], qkv_dtype="f32")
        pool_c = part["conv_pool"]
        o, S = oracle.recurrence(part["q"], part["k"], part["v"], part["g"], part["beta"], [0, t1 - t0],
                                 S, [1], 0.25)
        outs.append(o)
    np.testing.assert_array_equal(np.concatenate(outs), o_full)
    np.testing.assert_array_equal(S, s_full)
    np.testing.assert_array_equal(pool_c, full["conv_pool"])


def test_decode_equals_prefill_with_one_token_rows_and_null_rows_are_inert():
    d = Dims(2, 4, 16, 8, 4)
    cfg = Config(name="t", mode="decode", dims=d, batch=6, num_slots=10, act_dtype="f32", state_dtype="f32",
                 qkv_dtype="f32", init_state_std=0.1, conv_state_std=1.0, seed=6, null_rows=2)
    inp = make_inputs(cfg)
    out, cpool, spool = oracle.decode(d, inp["x"], inp["w"], inp["a"], inp["b"], inp["A_log"], inp["dt_bias"],
                                      inp["conv_pool"], inp["ssm_pool"], inp["slots"], 0.25)
    live = inp["slots"] >= 0
    assert np.all(out[~live] == 0)
    untouched = np.setdiff1d(np.arange(10), inp["slots"][live])
    np.testing.assert_array_equal(cpool[untouched], inp["conv_pool"][untouched])
    np.testing.assert_array_equal(spool[untouched], inp["ssm_pool"][untouched])
    # same rows through prepare + prefill, one sequence of length 1 per row
    ls = inp["slots"][live]
    n = int(live.sum())
    cu = np.arange(n + 1, dtype=np.int32)
    pre = oracle.prepare(d, cu, inp["x"][live], inp["w"], inp["a"][live], inp["b"][live], inp["A_log"],
                         inp["dt_bias"], inp["conv_pool"], ls, np.ones(n, np.uint8), qkv_dtype="f32")
    o2, sp2 = oracle.prefill(d, cu, pre["q"], pre["k"], pre["v"], pre["g"], pre["beta"], inp["ssm_pool"], ls,
                             np.ones(n, np.uint8), 0.25)
    # prepare rounds q/k/v/g/beta to f32 where decode keeps them in f64
    np.testing.assert_allclose(out[live], o2, rtol=1e-6, atol=1e-6)
    np.testing.assert_allclose(spool[ls], sp2[ls], rtol=1e-6, atol=1e-6)
    np.testing.assert_array_equal(cpool[ls], pre["conv_pool"][ls])


def test_thread_count_does_not_change_bits():
    q = _rand((40, 2, 16), 70); k = _rand((40, 2, 16), 71) / 4; v = _rand((40, 4, 8), 72)
    g = -np.abs(_rand((40, 4), 73)); beta = expit(_rand((40, 4), 74))
    cu = [0, 7, 40]
    S0 = _rand((2, 4, 8, 16), 75)
    a = oracle.recurrence(q, k, v, g, beta, cu, S0, [1, 1], 0.3, nthreads=1)
    b = oracle.recurrence(q, k, v, g, beta, cu, S0, [1, 1], 0.3, nthreads=5)
    np.testing.assert_array_equal(a[0], b[0])
    np.testing.assert_array_equal(a[1], b[1])


def test_recurrence_l2norm_inside_equals_prenormalised():
    q = _rand((9, 1, 8), 80); k = _rand((9, 1, 8), 81); v = _rand((9, 2, 4), 82)
    g = -np.abs(_rand((9, 2), 83)); beta = expit(_rand((9, 2), 84))
    S0 = np.zeros((1, 2, 4, 8))
    o1, s1 = oracle.recurrence(q, k, v, g, beta, [0, 9], S0, [0], 0.3, l2norm=True)
    qn = q / np.sqrt((q ** 2).sum(-1, keepdims=True) + 1e-6)
    kn = k / np.sqrt((k ** 2).sum(-1, keepdims=True) + 1e-6)
    o2, s2 = oracle.recurrence(qn, kn, v, g, beta, [0, 9], S0, [0], 0.3, l2norm=False)
    np.testing.assert_allclose(o1, o2, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(s1, s2, rtol=1e-13, atol=1e-14)


# ---------------------------------------------------------------------------
# Rounding to storage dtypes.
# ---------------------------------------------------------------------------
def test_round_f16_and_f32_match_numpy():
    rng = np.random.default_rng(90)
    x = np.concatenate([rng.normal(0, 1, 5000), rng.normal(0, 1e-5, 2000), rng.normal(0, 3e4, 2000),
                        [65504.0, 65519.99, 65520.0, 1e-8, 2.0 ** -25, 3 * 2.0 ** -26, -0.0]])
    np.testing.assert_array_equal(oracle.round_to(x, "f16"), x.astype(np.float16).astype(np.float64))
    np.testing.assert_array_equal(oracle.round_to(x, "f32"), x.astype(np.float32).astype(np.float64))


def test_round_bf16_hand_values():
    u = 2.0 ** -7  # bf16 spacing in [1, 2)
    cases = {
        1.0 + u / 2: 1.0,                 # tie -> even (1.0)
        1.0 + 3 * u / 2: 1.0 + 2 * u,     # tie -> even (1 + 2u)
        1.0 + u / 2 + 2.0 ** -30: 1.0 + u,  # just above the tie -> up
        -(1.0 + 0.75 * u): -(1.0 + u),
        255.5 * 2.0 ** 120: float("inf"),       # tie above the largest finite -> overflow
        255.25 * 2.0 ** 120: 255 * 2.0 ** 120,  # largest finite bf16
        2.0 ** -130 + 2.0 ** -140: 2.0 ** -130,  # subnormal spacing 2^-133
    }
    for x, want in cases.items():
        assert oracle.round_to([x], "bf16")[0] == want, x
    # agrees with the float32 bit trick wherever float32 holds the value exactly
    x32 = np.random.default_rng(91).normal(0, 10, 20000).astype(np.float32)
    bits = x32.view(np.uint32).astype(np.uint64)
    ref = (((bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFF0000).astype(np.uint32)).view(np.float32)
    np.testing.assert_array_equal(oracle.round_to(x32, "bf16"), ref.astype(np.float64))


# ---------------------------------------------------------------------------
# Gated RMS norm of the output (vllm.cpp cpu_ops.cpp, RmsNormGatedKernel;
# ferrum-kernels cpu.rs, gated_rms_norm_f32)
# ---------------------------------------------------------------------------
def _zval(s):
    return {"0": 0.0, "ln3": np.log(3.0)}[s]


def test_golden_gated_rmsnorm():
    fx = json.load(open(os.path.join(GOLDEN, "worked_gated_rmsnorm.json")))
    for c in fx["cases"]:
        x = np.array([c["x"]], np.float64)
        z = np.array([[_zval(v) for v in c["z"]]])
        out = oracle.gated_rmsnorm(x, z, np.array(c["w"], np.float64), c["eps"], c["sigmoid_gate"])
        np.testing.assert_allclose(out[0], c["expected"], rtol=1e-14, atol=1e-15)


def test_gated_rmsnorm_rows_have_unit_rms_before_gate():
    # with eps = 0 the normalised row x / rms(x) has mean square exactly 1:
    # fixes the mean (not the sum) and the square root
    rng = np.random.default_rng(7)
    x = rng.normal(size=(5, 3, 48)) * rng.uniform(0.1, 10.0, size=(5, 3, 1))
    z = rng.normal(size=x.shape)
    w = rng.uniform(0.5, 2.0, size=48)
    out = oracle.gated_rmsnorm(x, z, w, 0.0)
    unit = out / (w * z / (1.0 + np.exp(-z)))
    np.testing.assert_allclose(np.mean(unit * unit, axis=-1), 1.0, rtol=1e-12)
    np.testing.assert_allclose(unit * np.sqrt(np.mean(x * x, axis=-1, keepdims=True)), x, rtol=1e-12)


def test_gated_rmsnorm_eps_inside_the_root_is_homogeneous():
    # x / sqrt(mean(x^2) + eps) is unchanged by x -> c x, eps -> c^2 eps only
    # when eps sits inside the root next to the mean
    rng = np.random.default_rng(8)
    x = rng.normal(size=(4, 2, 32))
    z = rng.normal(size=x.shape)
    w = rng.normal(size=32)
    a = oracle.gated_rmsnorm(x, z, w, 0.3)
    b = oracle.gated_rmsnorm(5.0 * x, z, w, 0.3 * 25.0)
    np.testing.assert_allclose(a, b, rtol=1e-12, atol=1e-15)
    c = oracle.gated_rmsnorm(5.0 * x, z, w, 0.3)
    assert np.max(np.abs(c - a)) > 1e-3  # the eps term is not scale-free on its own


def test_gated_rmsnorm_gate_and_weight_act_per_column():
    rng = np.random.default_rng(9)
    x = rng.normal(size=(3, 16))
    z = rng.normal(size=x.shape)
    # a zero gate gives zero under silu and half the normalised value under sigmoid
    w = rng.normal(size=16)
    assert np.all(oracle.gated_rmsnorm(x, np.zeros_like(x), w, 1e-6) == 0.0)
    half = oracle.gated_rmsnorm(x, np.zeros_like(x), w, 0.0, sigmoid_gate=True)
    np.testing.assert_allclose(half, 0.5 * w * x / np.sqrt(np.mean(x * x, -1, keepdims=True)), rtol=1e-12)
    # a one-hot weight keeps exactly one column
    e = np.zeros(16)
    e[5] = 1.0
    out = oracle.gated_rmsnorm(x, z, e, 1e-6)
    assert np.all(out[:, np.arange(16) != 5] == 0.0) and np.all(out[:, 5] != 0.0)
