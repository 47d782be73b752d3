"""Parity of the speculative multi-token decode (gdn_decode_spec; vllm.cpp
cpu_ops.cpp CausalConv1dSpecUpdateKernel and GdnSpecDecodeKernel) and of the
widened conv pools it shares with the other entry points, through the C ABI,
against the f64 oracle.

Tolerances as for decode: f32 allclose(atol=1e-4, rtol=1e-4); bf16 max-abs
2e-2; f16 max-abs 2e-3.  The conv rows are raw inputs moved around, so they
must match exactly.
"""
import sys

import numpy as np
import pytest

import oracle
from gdn_inputs import Config, Dims, make_inputs, spec_inputs
from tests.test_gpu_parity import assert_close

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _runner():
    from tests import gpu_runner
    return gpu_runner


def _oracle(d, inp, scale, sdt, act, conv_pool=None, ssm_pool=None):
    return oracle.decode_spec(d, inp["cu"], inp["x"], inp["w"], inp["a"], inp["b"], inp["A_log"], inp["dt_bias"],
                              inp["conv_pool"] if conv_pool is None else conv_pool,
                              inp["ssm_pool"] if ssm_pool is None else ssm_pool, inp["state_idx"],
                              inp["num_accepted"], scale, sdt, act)


SPEC_CASES = [
    # name, dims, requests, cols, act, state, slots, extra: lens / conv_len / nulls
    ("hk2_hv4_d128_c4_bf16_f32", Dims(2, 4, 128, 128, 4), 6, 4, "bf16", "f32", 30, {}),
    ("bf16_state_nulls", Dims(2, 4, 128, 128, 4), 7, 4, "bf16", "bf16", 40, dict(null_reqs=2, null_cols=5)),
    ("f16_state_d256_dv128_c2", Dims(1, 4, 256, 128, 4), 5, 2, "bf16", "f16", 12, {}),
    ("f32_k2_d32_dv64_c8", Dims(2, 2, 32, 64, 2), 4, 8, "f32", "f32", 40, {}),
    ("varlen_k3_d64_dv16_c5", Dims(4, 8, 64, 16, 3), 6, 5, "bf16", "bf16", 36, dict(lens=[5, 1, 3, 5, 2, 4])),
    ("wide_row_d16_c3", Dims(1, 1, 16, 16, 4), 5, 3, "f32", "f32", 20, dict(conv_len=9)),
    ("one_column", Dims(2, 4, 64, 64, 4), 8, 1, "bf16", "f32", 10, {}),
]


@pytest.mark.parametrize("name,d,N,cols,act,sdt,S,extra", SPEC_CASES, ids=[c[0] for c in SPEC_CASES])
def test_decode_spec_parity(name, d, N, cols, act, sdt, S, extra):
    R = _runner()
    seed = 300 + [c[0] for c in SPEC_CASES].index(name)
    inp = spec_inputs(d, N, cols, S, act, sdt, seed=seed, **extra)
    scale = 1.0 / np.sqrt(d.Dk)
    _say(f"[spec] {name} N={N} cols={cols} W={inp['conv_pool'].shape[2]}")
    out, cp, sp = R.decode_spec(d, inp, act, sdt, scale)
    o_ref, c_ref, s_ref = _oracle(d, inp, scale, sdt, act)
    assert_close(out, o_ref, act, f"{name} out")
    assert_close(sp, s_ref, sdt, f"{name} state pool")
    np.testing.assert_array_equal(cp, c_ref)
    sidx, nat = inp["state_idx"], inp["num_accepted"]
    inert = sidx[np.arange(N), nat - 1] < 0
    tok_inert = np.repeat(inert, np.diff(inp["cu"]))
    assert np.all(out[tok_inert] == 0)


def test_decode_spec_two_steps_roll_back():
    """Step two resumes from column num_accepted-1 of step one's snapshots,
    on the GPU's own pools."""
    R = _runner()
    d = Dims(2, 4, 128, 128, 4)
    N, cols, S = 6, 4, 30
    scale = 1.0 / np.sqrt(d.Dk)
    one = spec_inputs(d, N, cols, S, "bf16", "f32", seed=401)
    one["num_accepted"][:] = 1
    two = spec_inputs(d, N, cols, S, "bf16", "f32", seed=402)
    two["state_idx"] = one["state_idx"]
    two["num_accepted"] = np.array([1, 2, 3, 4, 4, 2], np.int32)
    _say("[spec] two steps")
    _, cp, sp = R.decode_spec(d, one, "bf16", "f32", scale)
    out2, cp2, sp2 = R.decode_spec(d, two, "bf16", "f32", scale, conv_pool=cp, ssm_pool=sp)
    _, c1, s1 = _oracle(d, one, scale, "f32", "bf16")
    o2, c2, s2 = _oracle(d, two, scale, "f32", "bf16", conv_pool=c1, ssm_pool=s1)
    assert_close(out2, o2, "bf16", "step two out")
    assert_close(sp2, s2, "f32", "step two state pool")
    np.testing.assert_array_equal(cp2, c2)


def test_decode_spec_unvalidated_bad_rows_are_inert():
    """Without the host copies, a request whose num_accepted or initial slot
    is out of range is treated as padding, and an out-of-range snapshot
    column is skipped (documented kernel behaviour, no device fault)."""
    R = _runner()
    d = Dims(2, 4, 64, 64, 4)
    N, cols, S = 5, 4, 24
    scale = 1.0 / np.sqrt(d.Dk)
    inp = spec_inputs(d, N, cols, S, "bf16", "f32", seed=411)
    inp["num_accepted"][0] = 0                 # out of range -> padding
    inp["num_accepted"][1] = cols + 3          # out of range -> padding
    inp["state_idx"][2, inp["num_accepted"][2] - 1] = S + 5   # initial slot out of range -> padding
    c3 = 1 if inp["num_accepted"][3] != 2 else 2
    inp["state_idx"][3, c3] = S + 100          # snapshot column out of range -> store skipped
    _say("[spec] unvalidated bad rows")
    out, cp, sp = R.decode_spec(d, inp, "bf16", "f32", scale, validate=False)
    ref = dict(inp)
    sidx = inp["state_idx"].copy()
    sidx[0] = -1
    sidx[1] = -1
    sidx[2] = -1
    sidx[3, c3] = -1
    ref["state_idx"] = sidx
    ref["num_accepted"] = np.clip(inp["num_accepted"], 1, cols)
    o_ref, c_ref, s_ref = _oracle(d, ref, scale, "f32", "bf16")
    assert_close(out, o_ref, "bf16", "out")
    assert_close(sp, s_ref, "f32", "state pool")
    np.testing.assert_array_equal(cp, c_ref)


@pytest.mark.parametrize("extra", [3, 7])
def test_decode_and_prepare_on_widened_pool(extra):
    """gdn_decode and gdn_prepare on a pool whose rows carry (K-1)+extra
    taps use the leading K-1 and leave the rest untouched."""
    R = _runner()
    cfg = Config("w1", "decode", Dims(2, 4, 128, 128, 4), batch=6, num_slots=10, act_dtype="bf16",
                 init_state_std=0.05, conv_state_std=1.0, seed=421)
    d = cfg.dims
    inp = make_inputs(cfg)
    rng = np.random.default_rng(422)
    wide = np.concatenate([inp["conv_pool"], rng.standard_normal((10, d.Cc, extra)).astype(np.float32)], axis=2)
    wide = wide.astype(np.float32)
    from gdn_inputs import round_to_dtype
    wide = round_to_dtype(wide, "bf16")
    _say(f"[widened] decode extra={extra}")
    out, cp, sp = R.decode(d, inp, "bf16", "f32", cfg.scale, conv_pool=wide)
    o_ref, c_ref, s_ref = oracle.decode(d, inp["x"], inp["w"], inp["a"], inp["b"], inp["A_log"], inp["dt_bias"],
                                        wide, inp["ssm_pool"], inp["slots"], cfg.scale, "f32", "bf16")
    assert_close(out, o_ref, "bf16", "decode out")
    assert_close(sp, s_ref, "f32", "decode state")
    np.testing.assert_array_equal(cp, c_ref)

    pcfg = Config("w2", "prefill", Dims(2, 4, 128, 128, 4), seqlens=(1, 2, 40, 3), num_slots=10, act_dtype="bf16",
                  qkv_dtype="bf16", init_state_std=0.05, conv_state_std=1.0, seed=423)
    pin = make_inputs(pcfg)
    _say(f"[widened] prepare extra={extra}")
    got = R.prepare(d, pin, "bf16", "bf16", conv_pool=wide)
    want = oracle.prepare(d, pin["cu"], pin["x"], pin["w"], pin["a"], pin["b"], pin["A_log"], pin["dt_bias"],
                          wide, pin["slots"], pin["has_init"], True, "bf16")
    for key in ("q", "k", "v"):
        assert_close(got[key], want[key], "bf16", f"prepare {key}")
    assert_close(got["g"], want["g"], "f32", "prepare g")
    assert_close(got["beta"], want["beta"], "f32", "prepare beta")
    np.testing.assert_array_equal(got["conv_pool"], want["conv_pool"])


def test_prefill_then_speculative_steps():
    """A request's life on one widened pool: prepare + prefill of its prompt,
    then two speculative steps, against the oracle's chain."""
    R = _runner()
    import torch
    d = Dims(2, 4, 128, 128, 4)
    N, cols, S = 3, 4, 16
    scale = 1.0 / np.sqrt(d.Dk)
    W = (d.K - 1) + (cols - 1)
    pcfg = Config("l1", "prefill", d, seqlens=(7, 64, 130), num_slots=S, act_dtype="bf16", qkv_dtype="bf16",
                  seed=431)
    pin = make_inputs(pcfg)
    step1 = spec_inputs(d, N, cols, S, "bf16", "f32", seed=432)
    # column 0 of each request's row is the slot its prompt was prefilled into
    sidx = step1["state_idx"].copy()
    prompt_slots = sidx[:, 0].copy()
    pin["slots"] = prompt_slots
    pin["has_init"] = np.zeros(N, np.uint8)
    wide = np.zeros((S, d.Cc, W), np.float32)
    ssm = np.zeros((S, d.Hv, d.Dv, d.Dk), np.float32)
    _say("[life] prepare + prefill")
    pre = R.prepare(d, pin, "bf16", "bf16", conv_pool=wide)
    o_p, sp = R.prefill(d, pin["cu"], pre["q"], pre["k"], pre["v"], pre["g"], pre["beta"], ssm, prompt_slots,
                        np.ones(N, np.uint8), "bf16", "f32", scale)
    opre = oracle.prepare(d, pin["cu"], pin["x"], pin["w"], pin["a"], pin["b"], pin["A_log"], pin["dt_bias"], wide,
                          prompt_slots, pin["has_init"], True, "bf16")
    np.testing.assert_array_equal(pre["conv_pool"], opre["conv_pool"])
    _, s_ref = oracle.prefill(d, pin["cu"], opre["q"], opre["k"], opre["v"], opre["g"], opre["beta"], ssm,
                              prompt_slots, np.ones(N, np.uint8), scale, False, "f32", "bf16")
    assert_close(sp, s_ref, "f32", "prefill state")
    # the spec steps use the same layer weights as the prompt
    for key in ("w", "A_log", "dt_bias"):
        step1[key] = pin[key]
    step1["num_accepted"][:] = 1
    step2 = spec_inputs(d, N, cols, S, "bf16", "f32", seed=433)
    for key in ("w", "A_log", "dt_bias"):
        step2[key] = pin[key]
    step2["state_idx"] = sidx
    step2["num_accepted"] = np.array([2, 4, 1], np.int32)
    _say("[life] two spec steps")
    _, cp, sp = R.decode_spec(d, step1, "bf16", "f32", scale, conv_pool=pre["conv_pool"], ssm_pool=sp)
    out2, cp, sp = R.decode_spec(d, step2, "bf16", "f32", scale, conv_pool=cp, ssm_pool=sp)
    _, c1, s1 = _oracle(d, step1, scale, "f32", "bf16", conv_pool=opre["conv_pool"], ssm_pool=s_ref)
    o2, c2, s2 = _oracle(d, step2, scale, "f32", "bf16", conv_pool=c1, ssm_pool=s1)
    assert_close(out2, o2, "bf16", "step two out")
    assert_close(sp, s2, "f32", "step two state")
    np.testing.assert_array_equal(cp, c2)
    torch.cuda.synchronize()


@pytest.mark.slow
def test_decode_spec_full_size_sampled_heads():
    """The benchmarked workload (256 requests x 4 tokens, Hk=16 Hv=32
    Dk=Dv=128, 1024-slot f32 pool), in the launch configuration the bench
    times; the oracle checks three sampled key-head groups (heads are
    independent: a key head's channels, value heads and state rows form a
    complete smaller problem)."""
    import torch
    from gdn_inputs import spec_batch
    from tests import gpu_runner as R
    from tests.test_gpu_parity import slice_key_head
    sb = spec_batch()
    d = sb["dims"]
    N, C = sb["num_reqs"], sb["cols"]
    inp = spec_inputs(d, N, C, sb["num_slots"], sb["act_dtype"], sb["state_dtype"], sb["seed"])
    scale = 1.0 / np.sqrt(d.Dk)
    _say(f"[spec full] {sb['name']}")
    cp = R.dev(inp["conv_pool"], "bf16")
    sp = R.dev(inp["ssm_pool"])
    out = torch.empty(N * C, d.Hv, d.Dv, device=R.DEV, dtype=torch.bfloat16)
    import gated_delta_rule_prepare_amd as gdn
    gdn.gdn_decode_spec(R.gdims(d), R.dev(inp["cu"]), R.dev(inp["x"], "bf16"), R.dev(inp["a"], "bf16"),
                        R.dev(inp["b"], "bf16"), R.dev(inp["w"], "bf16"), R.dev(inp["A_log"]), R.dev(inp["dt_bias"]),
                        cp, sp, R.dev(inp["state_idx"]), R.dev(inp["num_accepted"]), out, scale)
    torch.cuda.synchronize()
    for kh in (0, 7, 15):
        ch, hs, sd = slice_key_head(d, kh)
        sub = dict(inp)
        sub["x"], sub["w"] = inp["x"][:, ch], inp["w"][ch]
        sub["a"], sub["b"] = inp["a"][:, hs], inp["b"][:, hs]
        sub["A_log"], sub["dt_bias"] = inp["A_log"][hs], inp["dt_bias"][hs]
        o_ref, c_ref, s_ref = _oracle(sd, sub, scale, "f32", "bf16", conv_pool=inp["conv_pool"][:, ch],
                                      ssm_pool=inp["ssm_pool"][:, hs])
        assert_close(R.host(out[:, hs]), o_ref, "bf16", f"key head {kh} out")
        assert_close(R.host(sp[:, hs]), s_ref, "f32", f"key head {kh} state pool")
        np.testing.assert_array_equal(R.host(cp[:, torch.from_numpy(ch).to(R.DEV)]), c_ref)
