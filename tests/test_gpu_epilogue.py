"""Parity of the output epilogue (gated RMS norm, vllm.cpp cpu_ops.cpp
RmsNormGatedKernel; ferrum-kernels cpu.rs gated_rms_norm_f32) with the f64
oracle, through the C ABI: the standalone gdn_gated_rmsnorm, the fused
gdn_decode_gated, and the packed input layout of the layer ([q|k|v|z]
projection rows, [b|a] gate rows) end to end through prepare, prefill and the
epilogue.

Tolerances: f32 allclose(atol=1e-4, rtol=1e-4); bf16 outputs max-abs
2e-2 * max(1, |ref|): the epilogue's outputs reach magnitudes near 10, where
one bf16 unit in the last place alone exceeds 2e-2, so the bf16 bound scales
with the value as a bf16 ulp does.  The oracle composes decode (or prefill),
rounds the output to its dtype as the library stores it, and applies the
norm to that.
"""
import sys
import zlib

import numpy as np
import pytest

import oracle
from gdn_inputs import Config, Dims, epilogue_inputs, make_inputs

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def assert_close(got, want, dtype, what):
    got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = np.abs(got - want)
    if dtype == "f32":
        lim = 1e-4 + 1e-4 * np.abs(want)
    else:
        lim = 2e-2 * np.maximum(1.0, np.abs(want))
    worst = float((err / lim).max()) if err.size else 0.0
    assert worst <= 1.0, f"{what}: {dtype} mismatch, max abs err {float(err.max()):.3e}, worst err/bound {worst:.3f}"


def _torch():
    import torch
    from tests import gpu_runner as R
    return torch, R


NORM_CASES = [
    # name, T, Hv, Dv, dtype, eps, sigmoid gate, z offset inside a packed row (elements)
    ("bf16_d128_packed_z", 37, 32, 128, "bf16", 1e-6, False, 8192),
    ("f32_d64_sigmoid", 5, 4, 64, "f32", 1e-5, True, 0),
    ("bf16_d256", 9, 2, 256, "bf16", 1e-6, False, 0),
    ("f32_d16_eps0", 3, 3, 16, "f32", 0.0, False, 16),
    ("bf16_d32_ragged_rows", 11, 5, 32, "bf16", 1e-6, False, 64),
]


@pytest.mark.parametrize("name,T,Hv,Dv,io,eps,sig,zoff", NORM_CASES, ids=[c[0] for c in NORM_CASES])
def test_gated_rmsnorm_parity(name, T, Hv, Dv, io, eps, sig, zoff):
    torch, R = _torch()
    import gated_delta_rule_prepare_amd as gdn
    rng = np.random.default_rng(zlib.crc32(name.encode()))
    # rows of different magnitudes, as the core outputs are
    x = (rng.standard_normal((T, Hv, Dv)) * rng.uniform(0.05, 3.0, size=(T, Hv, 1))).astype(np.float32)
    from gdn_inputs import round_to_dtype
    x = round_to_dtype(x, io)
    ep = epilogue_inputs(T, Hv, Dv, io, seed=77)
    packed = np.concatenate([round_to_dtype(rng.standard_normal((T, zoff)).astype(np.float32), io), ep["z"]],
                            axis=1)
    _say(f"[gated_rmsnorm] {name} T={T} Hv={Hv} Dv={Dv} {io}")
    xt = R.dev(x, io)
    pt = R.dev(packed, io)
    out = torch.empty_like(xt)
    gdn.gdn_gated_rmsnorm(xt, pt[:, zoff:], R.dev(ep["norm_w"], io), out, eps, sigmoid_gate=sig)
    torch.cuda.synchronize()
    want = oracle.round_to(oracle.gated_rmsnorm(x, ep["z"].reshape(T, Hv, Dv), ep["norm_w"], eps, sig), io)
    assert_close(R.host(out), want, io, name)


def test_gated_rmsnorm_in_place():
    torch, R = _torch()
    import gated_delta_rule_prepare_amd as gdn
    T, Hv, Dv = 6, 4, 128
    rng = np.random.default_rng(5)
    from gdn_inputs import round_to_dtype
    x = round_to_dtype(rng.standard_normal((T, Hv, Dv)).astype(np.float32), "bf16")
    ep = epilogue_inputs(T, Hv, Dv, "bf16", seed=78)
    _say("[gated_rmsnorm] in place")
    xt = R.dev(x, "bf16")
    gdn.gdn_gated_rmsnorm(xt, R.dev(ep["z"], "bf16"), R.dev(ep["norm_w"], "bf16"), xt, 1e-6)
    torch.cuda.synchronize()
    want = oracle.round_to(oracle.gated_rmsnorm(x, ep["z"].reshape(T, Hv, Dv), ep["norm_w"], 1e-6), "bf16")
    assert_close(R.host(xt), want, "bf16", "in place")


GATED_DEC_CASES = [
    ("bf16_packed_nulls", Config("g1", "decode", Dims(2, 4, 128, 128, 4), batch=12, num_slots=20, act_dtype="bf16",
                                 init_state_std=0.05, conv_state_std=1.0, seed=41, null_rows=3), "f32", False, 1e-6),
    ("f32_sigmoid_d64_k3", Config("g2", "decode", Dims(2, 2, 64, 64, 3), batch=5, num_slots=6, act_dtype="f32",
                                  init_state_std=0.05, conv_state_std=1.0, seed=42), "f32", True, 1e-5),
    ("bf16_state_bf16_r4_dv32", Config("g3", "decode", Dims(1, 4, 64, 32, 4), batch=7, num_slots=9,
                                       act_dtype="bf16", state_dtype="bf16", init_state_std=0.05,
                                       conv_state_std=1.0, seed=43, null_rows=1), "bf16", False, 1e-6),
]


def _packed_rows(R, inp, ep, act):
    """Device [B, Cc + Hv*Dv] packed [q|k|v|z] rows and [B, 2*Hv] [b|a] rows."""
    packed = np.concatenate([inp["x"], ep["z"]], axis=1)
    ba = np.concatenate([inp["b"], inp["a"]], axis=1)
    return R.dev(packed, act), R.dev(ba, act)


@pytest.mark.parametrize("name,cfg,sdt,sig,eps", GATED_DEC_CASES, ids=[c[0] for c in GATED_DEC_CASES])
def test_decode_gated_parity(name, cfg, sdt, sig, eps):
    torch, R = _torch()
    import gated_delta_rule_prepare_amd as gdn
    d = cfg.dims
    inp = make_inputs(cfg)
    B, Cc, Hv, Dv = cfg.batch, d.Cc, d.Hv, d.Dv
    ep = epilogue_inputs(B, Hv, Dv, cfg.act_dtype, seed=cfg.seed + 100)
    _say(f"[decode_gated] {name} B={B}")
    packed, ba = _packed_rows(R, inp, ep, cfg.act_dtype)
    cp = R.dev(inp["conv_pool"], cfg.act_dtype)
    sp = R.dev(inp["ssm_pool"], sdt)
    out = torch.empty(B, Hv, Dv, device=R.DEV, dtype=R.TORCH_DTYPE[cfg.act_dtype])
    gdn.gdn_decode_gated(R.gdims(d), packed[:, :Cc], ba[:, Hv:], ba[:, :Hv], R.dev(inp["w"], cfg.act_dtype),
                         R.dev(inp["A_log"]), R.dev(inp["dt_bias"]), cp, sp, R.dev(inp["slots"]), packed[:, Cc:],
                         R.dev(ep["norm_w"], cfg.act_dtype), out, cfg.scale, eps, sigmoid_gate=sig)
    torch.cuda.synchronize()
    o_ref, c_ref, s_ref = oracle.decode(d, inp["x"], inp["w"], inp["a"], inp["b"], inp["A_log"], inp["dt_bias"],
                                        inp["conv_pool"], inp["ssm_pool"], inp["slots"], cfg.scale, sdt,
                                        cfg.act_dtype)
    nulls = inp["slots"] < 0
    want = oracle.gated_rmsnorm(o_ref.reshape(B, Hv, Dv), ep["z"].reshape(B, Hv, Dv), ep["norm_w"], eps, sig)
    want = oracle.round_to(want, cfg.act_dtype)
    want[nulls] = 0.0  # inert rows: zero output, as gdn_decode
    got = R.host(out)
    assert_close(got, want, cfg.act_dtype, f"{name} out")
    assert np.all(got[nulls] == 0)
    assert_close(R.host(sp), s_ref, sdt, f"{name} state")
    np.testing.assert_array_equal(R.host(cp), c_ref)


def test_packed_layout_prepare_prefill_epilogue():
    """The layer's own input layout end to end: [q|k|v|z] projection rows
    (the conv reads the first Cc columns through the row stride, the z
    columns feed the epilogue) and [b|a] gate rows, through gdn_prepare,
    gdn_prefill_varlen and gdn_gated_rmsnorm."""
    torch, R = _torch()
    import gated_delta_rule_prepare_amd as gdn
    cfg = Config("g4", "prefill", Dims(2, 4, 128, 128, 4), seqlens=(70, 5, 129), num_slots=4, act_dtype="bf16",
                 qkv_dtype="bf16", init_state_std=0.05, conv_state_std=1.0, seed=44)
    d = cfg.dims
    inp = make_inputs(cfg)
    T, Cc, Hv, Dv = cfg.T, d.Cc, d.Hv, d.Dv
    ep = epilogue_inputs(T, Hv, Dv, "bf16", seed=144)
    _say("[packed layout] prepare + prefill + epilogue")
    packed, ba = _packed_rows(R, inp, ep, "bf16")
    cu = R.dev(inp["cu"])
    pool = R.dev(inp["conv_pool"], "bf16")
    q = torch.empty(T, d.Hk, d.Dk, device=R.DEV, dtype=torch.bfloat16)
    k = torch.empty_like(q)
    v = torch.empty(T, Hv, Dv, device=R.DEV, dtype=torch.bfloat16)
    g = torch.empty(T, Hv, device=R.DEV)
    beta = torch.empty_like(g)
    sl, hi = R.dev(inp["slots"]), R.dev(inp["has_init"])
    gdn.gdn_prepare(R.gdims(d), cu, packed[:, :Cc], ba[:, Hv:], ba[:, :Hv], R.dev(inp["w"], "bf16"),
                    R.dev(inp["A_log"]), R.dev(inp["dt_bias"]), pool, q, k, v, g, beta, slot_idx=sl,
                    has_initial_state=hi, apply_qk_l2norm=True)
    sp = R.dev(inp["ssm_pool"], "f32")
    core = torch.empty(T, Hv, Dv, device=R.DEV, dtype=torch.bfloat16)
    gdn.gdn_prefill_varlen(R.gdims(d), cu, q, k, v, g, beta, sp, core, cfg.scale, slot_idx=sl, has_initial_state=hi)
    out = torch.empty_like(core)
    gdn.gdn_gated_rmsnorm(core, packed[:, Cc:], R.dev(ep["norm_w"], "bf16"), out, 1e-6)
    torch.cuda.synchronize()
    pr = oracle.prepare(d, inp["cu"], inp["x"], inp["w"], inp["a"], inp["b"], inp["A_log"], inp["dt_bias"],
                        inp["conv_pool"], inp["slots"], inp["has_init"], True, "bf16")
    core_ref, pool_ref = oracle.prefill(d, inp["cu"], pr["q"], pr["k"], pr["v"], pr["g"], pr["beta"],
                                        inp["ssm_pool"], inp["slots"], inp["has_init"], cfg.scale, False, "f32",
                                        "bf16")
    want = oracle.round_to(oracle.gated_rmsnorm(core_ref, ep["z"].reshape(T, Hv, Dv), ep["norm_w"], 1e-6), "bf16")
    # both sides ran their own prepare step, so the bound is the chained one (bf16 q/k/v into the recurrence)
    assert_close(R.host(core), core_ref, "bf16", "core output")
    assert_close(R.host(out), want, "bf16", "gated output")
    np.testing.assert_allclose(R.host(sp), pool_ref, atol=2e-3, rtol=0)
