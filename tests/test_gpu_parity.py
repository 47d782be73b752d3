"""Parity of the HIP path (called through the C ABI) with the f64 oracle.

Tolerances: f32 results allclose(atol=1e-4, rtol=1e-4); bf16 results max-abs
2e-2; f16 results max-abs 2e-3.  Both sides read the same seeded inputs; the
recurrence tests feed both sides the q/k/v/g/beta the oracle's prepare step
produced (rounded to the dtype the library stores them in), so a one-ulp
difference in a rounding decision between the two prepare steps cannot leak
into the recurrence comparison.  Full-size workloads are checked on every
key head; where a check runs the oracle on one key head's slice (heads are
independent), the slice holds that key head's channels and value heads.
"""
import dataclasses
import sys

import numpy as np
import pytest

import oracle
from gdn_inputs import Config, Dims, make_inputs, named_configs, prefill_long, prefill_single, prefill_varlen, \
    decode_batch, tiny, tiny_decode

pytestmark = pytest.mark.gpu


def _runner():
    from tests import gpu_runner
    return gpu_runner


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _where(err, lim):
    """Where a mismatch lies: the index of the worst element and how many
    elements exceed the bound (for the failure message)."""
    over = err > lim
    worst = np.unravel_index(int(np.argmax(err)), err.shape) if err.size else ()
    return f"worst at index {tuple(int(i) for i in worst)} of shape {err.shape}, {int(over.sum())} elements over"


def assert_close(got, want, dtype, what):
    got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    err = np.abs(got - want)
    mx = float(err.max()) if err.size else 0.0
    if dtype == "f32":
        lim = 1e-4 + 1e-4 * np.abs(want)
        ok = np.all(err <= lim)
        bad = float((err - 1e-4 * np.abs(want)).max()) if err.size else 0.0
        assert ok, f"{what}: f32 mismatch, max abs err {mx:.3e}, worst excess {bad:.3e}; {_where(err - lim + 1e-4, 1e-4)}"
    else:
        lim = 2e-2 if dtype == "bf16" else 2e-3
        assert mx <= lim, f"{what}: {dtype} max abs err {mx:.3e} > {lim}; {_where(err, lim)}"
    return mx


def slice_key_head(d: Dims, kh: int):
    """Channel indices and value-head range of key head kh."""
    r = d.Hv // d.Hk
    q = np.arange(kh * d.Dk, (kh + 1) * d.Dk)
    k = d.Hk * d.Dk + q
    v = 2 * d.Hk * d.Dk + np.arange(kh * r * d.Dv, (kh + 1) * r * d.Dv)
    return np.concatenate([q, k, v]), slice(kh * r, (kh + 1) * r), Dims(1, r, d.Dk, d.Dv, d.K)


def sliced_inputs(d: Dims, inp, kh: int):
    ch, hs, sd = slice_key_head(d, kh)
    out = dict(inp)
    out["x"] = inp["x"][:, ch]
    out["w"] = inp["w"][ch]
    out["conv_pool"] = inp["conv_pool"][:, ch]
    out["a"] = inp["a"][:, hs]
    out["b"] = inp["b"][:, hs]
    out["A_log"] = inp["A_log"][hs]
    out["dt_bias"] = inp["dt_bias"][hs]
    out["ssm_pool"] = inp["ssm_pool"][:, hs]
    return out, ch, hs, sd


# ---------------------------------------------------------------------------
# prepare
# ---------------------------------------------------------------------------
PREP_CASES = [
    ("tiny_f32", tiny()),
    ("varlen_bf16_to_bf16", Config("p1", "prefill", Dims(2, 4, 128, 128, 4), seqlens=(1, 2, 3, 31, 32, 33, 100),
                                   num_slots=9, act_dtype="bf16", qkv_dtype="bf16", init_state_std=0.05,
                                   conv_state_std=1.0, seed=11)),
    ("varlen_bf16_to_f32", Config("p2", "prefill", Dims(2, 4, 128, 128, 4), seqlens=(5, 77, 1),
                                  num_slots=4, act_dtype="bf16", qkv_dtype="f32", conv_state_std=1.0,
                                  init_state_std=0.05, seed=12)),
    ("d16_dv32_f32", Config("p3", "prefill", Dims(1, 2, 16, 32, 4), seqlens=(40, 3), num_slots=2, act_dtype="f32",
                            qkv_dtype="f32", conv_state_std=1.0, init_state_std=0.1, seed=13)),
    ("d64_dv16_k3_bf16", Config("p4", "prefill", Dims(2, 2, 64, 16, 3), seqlens=(2, 50), num_slots=3,
                                act_dtype="bf16", qkv_dtype="bf16", conv_state_std=1.0, init_state_std=0.1,
                                seed=14)),
    ("d256_dv64_k2_bf16", Config("p5", "prefill", Dims(4, 4, 256, 64, 2), seqlens=(70,), num_slots=1,
                                 act_dtype="bf16", qkv_dtype="bf16", seed=15)),
    ("d32_k1_f32", Config("p6", "prefill", Dims(2, 4, 32, 32, 1), seqlens=(9, 9), num_slots=2, act_dtype="f32",
                          qkv_dtype="f32", seed=16)),
    ("f32_act_to_bf16", Config("p7", "prefill", Dims(2, 4, 64, 64, 4), seqlens=(33, 1, 2), num_slots=5,
                               act_dtype="f32", qkv_dtype="bf16", conv_state_std=1.0, init_state_std=0.1,
                               seed=17)),
    # sequences that start in the last K-2 tokens of a 32-token strip: their
    # first tokens read the old history from two strips, so the history rows
    # are written by a second kernel
    ("starts_at_strip_end", Config("p8", "prefill", Dims(2, 4, 128, 128, 4), seqlens=(30, 1, 33, 2, 40),
                                   num_slots=6, act_dtype="bf16", qkv_dtype="bf16", conv_state_std=1.0,
                                   init_state_std=0.05, seed=18)),
    # every sequence's first K-1 tokens in one strip, one of them ending it
    ("starts_before_strip_end", Config("p9", "prefill", Dims(2, 4, 128, 128, 4), seqlens=(29, 3, 27, 1, 2),
                                       num_slots=6, act_dtype="bf16", qkv_dtype="bf16", conv_state_std=1.0,
                                       init_state_std=0.05, seed=19)),
]


def _check_prepare(d, inp, cfg, got, want, label):
    for key in ("q", "k", "v"):
        assert_close(got[key], want[key], cfg.qkv_dtype, f"{label} {key}")
    assert_close(got["g"], want["g"], "f32", f"{label} g")
    assert_close(got["beta"], want["beta"], "f32", f"{label} beta")
    np.testing.assert_array_equal(got["conv_pool"], want["conv_pool"], err_msg=f"{label} conv history")


@pytest.mark.parametrize("name,cfg", PREP_CASES, ids=[c[0] for c in PREP_CASES])
@pytest.mark.parametrize("l2norm", [True, False], ids=["l2", "nol2"])
def test_prepare_parity(name, cfg, l2norm):
    R = _runner()
    d = cfg.dims
    inp = make_inputs(cfg)
    _say(f"[prepare] {name} l2norm={l2norm} T={cfg.T} N={cfg.N}")
    got = R.prepare(d, inp, cfg.act_dtype, cfg.qkv_dtype, l2norm)
    want = oracle.prepare(d, inp["cu"], inp["x"], inp["w"], inp["a"], inp["b"], inp["A_log"], inp["dt_bias"],
                          inp["conv_pool"], inp["slots"], inp["has_init"], l2norm, cfg.qkv_dtype)
    _check_prepare(d, inp, cfg, got, want, name)


@pytest.mark.parametrize("seqlens", [(1, 2, 40, 1, 3, 20), (30, 1, 2, 33, 1)],
                         ids=["history_in_conv", "history_kernel"])
def test_prepare_mixed_initial_history(seqlens):
    """Sequences with and without a conv history in one call, short ones
    among them (new rows mixing old taps, zeros and inputs), for both ways
    the new history rows are written: by the conv kernel (every sequence's
    first K-1 tokens in one 32-token strip) and by the second kernel."""
    cfg = Config("pmix", "prefill", Dims(2, 4, 128, 128, 4), seqlens=seqlens, num_slots=len(seqlens) + 2,
                 act_dtype="bf16", qkv_dtype="bf16", conv_state_std=1.0, seed=20)
    R = _runner()
    d = cfg.dims
    inp = make_inputs(cfg)
    inp["has_init"] = np.array([i % 2 for i in range(len(seqlens))], np.uint8)
    _say(f"[prepare] mixed initial history {seqlens}")
    got = R.prepare(d, inp, cfg.act_dtype, cfg.qkv_dtype, True)
    want = oracle.prepare(d, inp["cu"], inp["x"], inp["w"], inp["a"], inp["b"], inp["A_log"], inp["dt_bias"],
                          inp["conv_pool"], inp["slots"], inp["has_init"], True, cfg.qkv_dtype)
    _check_prepare(d, inp, cfg, got, want, "mixed initial history")


def test_prepare_bf16_outputs_are_rne_of_f32_outputs():
    """The bf16 q/k/v of the prepare are the f32 results rounded to nearest
    even, bit for bit: the same inputs through the f32-output and the
    bf16-output kernels (the bf16 store uses the hardware conversion).
    Several sequences, so that blocks inside a sequence and blocks that
    straddle a sequence start both run."""
    cfg = Config("p_rne", "prefill", Dims(4, 8, 128, 128, 4), seqlens=(300, 5, 77, 130), num_slots=6,
                 act_dtype="bf16", qkv_dtype="bf16", conv_state_std=1.0, init_state_std=0.05, seed=18)
    R = _runner()
    d = cfg.dims
    inp = make_inputs(cfg)
    _say(f"[prepare rne] T={cfg.T}")
    got32 = R.prepare(d, inp, "bf16", "f32", True)
    got16 = R.prepare(d, inp, "bf16", "bf16", True)
    for key in ("q", "k", "v"):
        np.testing.assert_array_equal(got16[key], oracle.round_to(got32[key], "bf16"), err_msg=key)


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------
DEC_CASES = [
    ("tiny_f32", tiny_decode(), "f32"),
    ("bf16_state_f32_nulls", Config("d1", "decode", Dims(2, 4, 128, 128, 4), batch=12, num_slots=20,
                                    act_dtype="bf16", init_state_std=0.05, conv_state_std=1.0, seed=21,
                                    null_rows=3), "f32"),
    ("bf16_state_bf16", Config("d2", "decode", Dims(2, 4, 128, 128, 4), batch=9, num_slots=9, act_dtype="bf16",
                               state_dtype="bf16", init_state_std=0.05, conv_state_std=1.0, seed=22), "bf16"),
    ("bf16_state_f16", Config("d3", "decode", Dims(2, 4, 128, 128, 4), batch=9, num_slots=30, act_dtype="bf16",
                              state_dtype="f16", init_state_std=0.05, conv_state_std=1.0, seed=23), "f16"),
    ("d256_dv128_r4", Config("d4", "decode", Dims(1, 4, 256, 128, 4), batch=5, num_slots=7, act_dtype="bf16",
                             init_state_std=0.05, conv_state_std=1.0, seed=24), "f32"),
    ("d32_dv64_k2_f32", Config("d5", "decode", Dims(2, 2, 32, 64, 2), batch=6, num_slots=6, act_dtype="f32",
                               state_dtype="f16", init_state_std=0.05, conv_state_std=1.0, seed=25), "f16"),
    ("d64_dv16_k1", Config("d6", "decode", Dims(4, 8, 64, 16, 1), batch=7, num_slots=8, act_dtype="bf16",
                           state_dtype="bf16", init_state_std=0.05, seed=26, null_rows=1), "bf16"),
    ("d16_k3_f32", Config("d7", "decode", Dims(1, 1, 16, 16, 3), batch=4, num_slots=4, act_dtype="f32",
                          init_state_std=0.1, conv_state_std=1.0, seed=27), "f32"),
]


@pytest.mark.parametrize("name,cfg,sdt", DEC_CASES, ids=[c[0] for c in DEC_CASES])
def test_decode_parity(name, cfg, sdt):
    R = _runner()
    d = cfg.dims
    inp = make_inputs(cfg)
    _say(f"[decode] {name} B={cfg.batch}")
    out, cp, sp = R.decode(d, inp, cfg.act_dtype, sdt, cfg.scale)
    o_ref, c_ref, s_ref = oracle.decode(d, inp["x"], inp["w"], inp["a"], inp["b"], inp["A_log"], inp["dt_bias"],
                                        inp["conv_pool"], inp["ssm_pool"], inp["slots"], cfg.scale, sdt,
                                        cfg.act_dtype)
    assert_close(out, o_ref, cfg.act_dtype, f"{name} out")
    assert_close(sp, s_ref, sdt, f"{name} state")
    np.testing.assert_array_equal(cp, c_ref)
    nulls = inp["slots"] < 0
    assert np.all(out[nulls] == 0)


def test_decode_two_steps_carry_state():
    cfg = Config("d8", "decode", Dims(2, 4, 128, 128, 4), batch=6, num_slots=10, act_dtype="bf16",
                 init_state_std=0.05, conv_state_std=1.0, seed=28)
    R = _runner()
    d = cfg.dims
    inp = make_inputs(cfg)
    inp2 = make_inputs(dataclasses.replace(cfg, seed=29))
    _say("[decode] two steps")
    o1, cp, sp = R.decode(d, inp, "bf16", "f32", cfg.scale)
    o2, cp, sp = R.decode(d, {**inp2, "slots": inp["slots"]}, "bf16", "f32", cfg.scale, conv_pool=cp, ssm_pool=sp)
    r1, c1, s1 = oracle.decode(d, inp["x"], inp["w"], inp["a"], inp["b"], inp["A_log"], inp["dt_bias"],
                               inp["conv_pool"], inp["ssm_pool"], inp["slots"], cfg.scale, "f32", "bf16")
    r2, c2, s2 = oracle.decode(d, inp2["x"], inp2["w"], inp2["a"], inp2["b"], inp2["A_log"], inp2["dt_bias"], c1, s1,
                               inp["slots"], cfg.scale, "f32", "bf16")
    assert_close(o2, r2, "bf16", "second step out")
    assert_close(sp, s2, "f32", "second step state")
    np.testing.assert_array_equal(cp, c2)


@pytest.mark.slow
@pytest.mark.parametrize("sdt", ["f32", "bf16"])
def test_decode_full_size(sdt):
    cfg = decode_batch(sdt)
    R = _runner()
    d = cfg.dims
    inp = make_inputs(cfg)
    _say(f"[decode full] {cfg.name} state={sdt}")
    out, cp, sp = R.decode(d, inp, "bf16", sdt, cfg.scale)
    o_ref, c_ref, s_ref = oracle.decode(d, inp["x"], inp["w"], inp["a"], inp["b"], inp["A_log"], inp["dt_bias"],
                                        inp["conv_pool"], inp["ssm_pool"], inp["slots"], cfg.scale, sdt, "bf16")
    assert_close(out, o_ref, "bf16", "out")
    assert_close(sp, s_ref, sdt, "state pool")
    np.testing.assert_array_equal(cp, c_ref)


def test_tiny_as_eight_decode_steps_equals_prefill():
    """The tiny workload (T=8, f32) run as 8 single-token decode calls on one
    slot equals the oracle's 8-token prefill."""
    cfg = tiny()
    d = cfg.dims
    inp = make_inputs(cfg)
    R = _runner()
    _say("[decode] tiny as 8 steps")
    cp, sp = inp["conv_pool"], inp["ssm_pool"]
    outs = []
    for t in range(cfg.T):
        row = dict(x=inp["x"][t:t + 1], a=inp["a"][t:t + 1], b=inp["b"][t:t + 1], w=inp["w"], A_log=inp["A_log"],
                   dt_bias=inp["dt_bias"], slots=np.array([0], np.int32))
        o, cp, sp = R.decode(d, row, "f32", "f32", cfg.scale, conv_pool=cp, ssm_pool=sp)
        outs.append(o[0])
    pre = oracle.prepare(d, inp["cu"], inp["x"], inp["w"], inp["a"], inp["b"], inp["A_log"], inp["dt_bias"],
                         inp["conv_pool"], inp["slots"], inp["has_init"], True, "f32")
    o_ref, s_ref = oracle.prefill(d, inp["cu"], pre["q"], pre["k"], pre["v"], pre["g"], pre["beta"],
                                  inp["ssm_pool"], inp["slots"], inp["has_init"], cfg.scale)
    assert_close(np.stack(outs), o_ref, "f32", "outputs")
    assert_close(sp, s_ref, "f32", "final state")
    np.testing.assert_array_equal(cp, pre["conv_pool"])


# ---------------------------------------------------------------------------
# prefill (recurrence); inputs from the oracle's prepare
# ---------------------------------------------------------------------------
def _oracle_prepared(cfg, inp, l2norm=True):
    d = cfg.dims
    return oracle.prepare(d, inp["cu"], inp["x"], inp["w"], inp["a"], inp["b"], inp["A_log"], inp["dt_bias"],
                          inp["conv_pool"], inp["slots"], inp["has_init"], l2norm, cfg.qkv_dtype)


PF_LENS = (1, 63, 64, 65, 130, 257)
PF_CASES = []
for qkv in ("f32", "bf16"):
    for sdt in ("f32", "bf16", "f16"):
        PF_CASES.append((f"ragged_qkv{qkv}_state{sdt}",
                         Config(f"pf_{qkv}_{sdt}", "prefill", Dims(2, 4, 128, 128, 4), seqlens=PF_LENS, num_slots=8,
                                act_dtype="bf16", qkv_dtype=qkv, state_dtype=sdt, init_state_std=0.05,
                                conv_state_std=1.0, seed=31)))
PF_CASES += [
    ("d16", Config("pf_d16", "prefill", Dims(1, 2, 16, 16, 4), seqlens=(8, 100), num_slots=2, act_dtype="f32",
                   qkv_dtype="f32", init_state_std=0.1, seed=32)),
    ("d64_dv32", Config("pf_d64", "prefill", Dims(2, 2, 64, 32, 4), seqlens=(70, 3, 129), num_slots=5,
                        act_dtype="bf16", qkv_dtype="bf16", init_state_std=0.1, conv_state_std=1.0, seed=33)),
    ("d256_dv128", Config("pf_d256", "prefill", Dims(1, 2, 256, 128, 4), seqlens=(90,), num_slots=1,
                          act_dtype="bf16", qkv_dtype="f32", seed=34)),
    ("d32_dv256_r4", Config("pf_d32", "prefill", Dims(1, 4, 32, 256, 4), seqlens=(65, 2), num_slots=2,
                            act_dtype="bf16", qkv_dtype="bf16", state_dtype="bf16", init_state_std=0.1, seed=35)),
    ("d32_r2", Config("pf_d32b", "prefill", Dims(2, 4, 32, 32, 4), seqlens=(200, 1, 64), num_slots=3,
                      act_dtype="bf16", qkv_dtype="f32", init_state_std=0.1, conv_state_std=1.0, seed=37)),
    ("d32_r2_bf16", Config("pf_d32c", "prefill", Dims(2, 4, 32, 32, 4), seqlens=(200, 1, 64), num_slots=3,
                           act_dtype="bf16", qkv_dtype="bf16", init_state_std=0.1, conv_state_std=1.0, seed=41)),
    # one sequence (no chunk table) continuing from a nonzero state, both block forms
    ("single_seq_init_bf16", Config("pf_1b", "prefill", Dims(2, 4, 128, 128, 4), seqlens=(150,), num_slots=2,
                                    act_dtype="bf16", qkv_dtype="bf16", init_state_std=0.05, conv_state_std=1.0,
                                    seed=42)),
    ("single_seq_init_f32", Config("pf_1f", "prefill", Dims(2, 4, 64, 64, 4), seqlens=(97,), num_slots=2,
                                   act_dtype="bf16", qkv_dtype="f32", init_state_std=0.05, conv_state_std=1.0,
                                   seed=43)),
    ("d64_r3_f16", Config("pf_d64b", "prefill", Dims(1, 3, 64, 64, 2), seqlens=(129, 300), num_slots=4,
                          act_dtype="bf16", qkv_dtype="bf16", state_dtype="f16", init_state_std=0.1, seed=38)),
    # more sequences than the chunk-table wave has lanes: each lane takes two
    ("over_64_seqs", Config("pf_70", "prefill", Dims(1, 2, 64, 64, 4),
                            seqlens=tuple(1 + (i * 37) % 150 for i in range(70)), num_slots=72, act_dtype="bf16",
                            qkv_dtype="bf16", state_dtype="f32", init_state_std=0.05, conv_state_std=1.0, seed=40)),
    ("many_short_seqs", Config("pf_many", "prefill", Dims(2, 4, 128, 128, 4),
                               seqlens=tuple([1, 2, 3, 5, 8, 13, 21, 34, 55, 89, 144, 63, 64, 65, 127, 128]),
                               num_slots=20, act_dtype="bf16", qkv_dtype="bf16", state_dtype="f32",
                               init_state_std=0.05, conv_state_std=1.0, seed=39)),
]


@pytest.mark.parametrize("name,cfg", PF_CASES, ids=[c[0] for c in PF_CASES])
def test_prefill_parity(name, cfg):
    R = _runner()
    d = cfg.dims
    inp = make_inputs(cfg)
    has = inp["has_init"].copy()
    if has.size > 1:
        has[::2] = 0  # mix continuing and fresh sequences
    pre = _oracle_prepared(cfg, {**inp, "has_init": has})
    _say(f"[prefill] {name} T={cfg.T}")
    out, sp = R.prefill(d, inp["cu"], pre["q"], pre["k"], pre["v"], pre["g"], pre["beta"], inp["ssm_pool"],
                        inp["slots"], has, cfg.qkv_dtype, cfg.state_dtype, cfg.scale)
    o_ref, s_ref = oracle.prefill(d, inp["cu"], pre["q"], pre["k"], pre["v"], pre["g"], pre["beta"], inp["ssm_pool"],
                                  inp["slots"], has, cfg.scale, False, cfg.state_dtype, cfg.qkv_dtype)
    assert_close(out, o_ref, cfg.qkv_dtype, f"{name} out")
    assert_close(sp, s_ref, cfg.state_dtype, f"{name} state")


def test_prefill_on_a_side_stream():
    """The prefill enqueued on a stream other than torch's current one (the
    binding then allocates its workspace on that stream) gives the same bits
    as on the current stream, and the oracle's result."""
    import torch
    cfg = Config("pf_side", "prefill", Dims(2, 4, 128, 128, 4), seqlens=(70, 1, 200), num_slots=4, act_dtype="bf16",
                 qkv_dtype="bf16", state_dtype="f32", init_state_std=0.05, conv_state_std=1.0, seed=44)
    R = _runner()
    d = cfg.dims
    inp = make_inputs(cfg)
    pre = _oracle_prepared(cfg, inp)
    args = (d, inp["cu"], pre["q"], pre["k"], pre["v"], pre["g"], pre["beta"], inp["ssm_pool"], inp["slots"],
            inp["has_init"], "bf16", "f32", cfg.scale)
    _say("[prefill] side stream")
    out0, sp0 = R.prefill(*args)
    out1, sp1 = R.prefill(*args, stream=torch.cuda.Stream())
    np.testing.assert_array_equal(out1, out0)
    np.testing.assert_array_equal(sp1, sp0)
    o_ref, s_ref = oracle.prefill(d, inp["cu"], pre["q"], pre["k"], pre["v"], pre["g"], pre["beta"], inp["ssm_pool"],
                                  inp["slots"], inp["has_init"], cfg.scale, False, "f32", "bf16")
    assert_close(out1, o_ref, "bf16", "side stream out")
    assert_close(sp1, s_ref, "f32", "side stream state")


@pytest.mark.parametrize("qkv,D", [("f32", 128), ("bf16", 128), ("bf16", 32)])
def test_prefill_l2norm_inside(qkv, D):
    cfg = Config("pf_l2", "prefill", Dims(2, 4, D, D, 4), seqlens=(20, 90), num_slots=2, act_dtype="bf16",
                 qkv_dtype=qkv, init_state_std=0.05, seed=36)
    R = _runner()
    d = cfg.dims
    inp = make_inputs(cfg)
    pre = _oracle_prepared(cfg, inp, l2norm=False)
    _say(f"[prefill] l2norm inside, {qkv} q/k/v, D={D}")
    out, sp = R.prefill(d, inp["cu"], pre["q"], pre["k"], pre["v"], pre["g"], pre["beta"], inp["ssm_pool"],
                        inp["slots"], inp["has_init"], qkv, "f32", cfg.scale, l2norm=True)
    o_ref, s_ref = oracle.prefill(d, inp["cu"], pre["q"], pre["k"], pre["v"], pre["g"], pre["beta"], inp["ssm_pool"],
                                  inp["slots"], inp["has_init"], cfg.scale, True, "f32", qkv)
    assert_close(out, o_ref, qkv, "out")
    assert_close(sp, s_ref, "f32", "state")


@pytest.mark.slow
@pytest.mark.parametrize("which", ["prefill_single", "varlen"])
def test_full_size_prepare_and_prefill_all_heads(which):
    """The 4096-token single sequence (f32 state from zero, no chunk table)
    and the 16-sequence varlen batch (bf16 state and conv histories carried
    in, through the chunk table), at full size in the launch configuration
    the benchmark times, every key head checked: the prepare against the
    oracle's prepare, then the prefill (fed the oracle's prepared q/k/v/g/beta
    on both sides) against the oracle's recurrence."""
    cfg = {"prefill_single": prefill_single(), "varlen": prefill_varlen()}[which]
    R = _runner()
    d = cfg.dims
    inp = make_inputs(cfg)
    _say(f"[full] {cfg.name} T={cfg.T} N={cfg.N}: prepare")
    got = R.prepare(d, inp, cfg.act_dtype, cfg.qkv_dtype, True)
    pre = _oracle_prepared(cfg, inp)
    _check_prepare(d, inp, cfg, got, pre, f"{which} prepare")
    del got
    _say(f"[full] {cfg.name}: prefill")
    out, sp = R.prefill(d, inp["cu"], pre["q"], pre["k"], pre["v"], pre["g"], pre["beta"], inp["ssm_pool"],
                        inp["slots"], inp["has_init"], cfg.qkv_dtype, cfg.state_dtype, cfg.scale)
    o_ref, s_ref = oracle.prefill(d, inp["cu"], pre["q"], pre["k"], pre["v"], pre["g"], pre["beta"], inp["ssm_pool"],
                                  inp["slots"], inp["has_init"], cfg.scale, False, cfg.state_dtype, cfg.qkv_dtype)
    assert_close(out, o_ref, cfg.qkv_dtype, f"{which} out")
    assert_close(sp, s_ref, cfg.state_dtype, f"{which} state pool")


def f16_ulp_distance(got, ref):
    """|got - ref| in f16 ulps of max(|ref|, rms(ref)): an element's own ulp,
    floored at the ulp of the state's root mean square so that elements near
    zero (whose ulp is tiny) are measured on the scale of the state."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    rms = float(np.sqrt(np.mean(ref ** 2)))
    mag = np.maximum(np.abs(ref), rms).astype(np.float16)
    return np.abs(got - ref) / np.spacing(mag).astype(np.float64)


@pytest.mark.slow
def test_long_prefill_one_call_equals_eight_calls():
    """T=32768, Hv=48, f16 state from zero.  One call against the oracle on
    every key head (prepare, then the recurrence on the oracle's prepared
    inputs); one call against 8 chained 4096-token calls on the same inputs
    (f16 state carried, so it is rounded at 7 more call boundaries), within
    4 f16 ulps elementwise (floored at one ulp of the state's RMS) with the
    measured distance printed; the chained prepare (conv history carried)
    against the one-call prepare; and the chain against the oracle run the
    same way, rounding for rounding, on two key heads."""
    cfg = prefill_long()
    d = cfg.dims
    R = _runner()
    inp = make_inputs(cfg)
    _say("[long] one call: prepare")
    got1 = R.prepare(d, inp, "bf16", "bf16")
    pre = _oracle_prepared(cfg, inp)
    _check_prepare(d, inp, cfg, got1, pre, "long prepare")
    _say("[long] one call: prefill")
    out1, sp1 = R.prefill(d, inp["cu"], pre["q"], pre["k"], pre["v"], pre["g"], pre["beta"], inp["ssm_pool"],
                          inp["slots"], inp["has_init"], "bf16", "f16", cfg.scale)
    o_ref, s_ref = oracle.prefill(d, inp["cu"], pre["q"], pre["k"], pre["v"], pre["g"], pre["beta"], inp["ssm_pool"],
                                  inp["slots"], inp["has_init"], cfg.scale, False, "f16", "bf16")
    assert_close(out1, o_ref, "bf16", "one call out vs oracle")
    assert_close(sp1, s_ref, "f16", "one call final state vs oracle")
    del o_ref
    _say("[long] eight calls")
    cp, sp = inp["conv_pool"], inp["ssm_pool"]
    outs = []
    for i in range(8):
        t0, t1 = 4096 * i, 4096 * (i + 1)
        cu = np.array([0, 4096], np.int32)
        has = np.array([1 if i else 0], np.uint8)
        part = dict(inp, x=inp["x"][t0:t1], a=inp["a"][t0:t1], b=inp["b"][t0:t1], cu=cu, has_init=has)
        gp = R.prepare(d, part, "bf16", "bf16", conv_pool=cp)
        cp = gp["conv_pool"]
        for key in ("q", "k", "v", "g", "beta"):
            assert_close(gp[key], got1[key][t0:t1], "f32" if key in ("g", "beta") else "bf16",
                         f"chained prepare {key}, call {i}")
        o, sp = R.prefill(d, cu, pre["q"][t0:t1], pre["k"][t0:t1], pre["v"][t0:t1], pre["g"][t0:t1],
                          pre["beta"][t0:t1], sp, inp["slots"], has, "bf16", "f16", cfg.scale)
        outs.append(o)
    np.testing.assert_array_equal(cp, got1["conv_pool"], err_msg="conv history, 8 calls vs 1 call")
    out8 = np.concatenate(outs)
    ulps = f16_ulp_distance(sp, sp1)
    _say(f"[long] final state, 8 calls vs 1 call: max {ulps.max():.2f} f16 ulps "
         f"(99.99th pct {np.percentile(ulps, 99.99):.2f}), max abs {np.abs(sp - sp1).max():.3e}")
    assert ulps.max() <= 4.0, f"final state: 8 calls vs 1 call differ by {ulps.max():.2f} f16 ulps"
    assert_close(out8, out1, "bf16", "outputs, 8 calls vs 1 call")
    # the chain against the oracle chained the same way (state rounded to f16 per call)
    for kh in (5, d.Hk - 1):
        _, hs, sd = slice_key_head(d, kh)
        osp = inp["ssm_pool"][:, hs]
        for i in range(8):
            t0, t1 = 4096 * i, 4096 * (i + 1)
            has = np.array([1 if i else 0], np.uint8)
            o_ref, osp = oracle.prefill(sd, [0, 4096], pre["q"][t0:t1, kh:kh + 1], pre["k"][t0:t1, kh:kh + 1],
                                        pre["v"][t0:t1, hs], pre["g"][t0:t1, hs], pre["beta"][t0:t1, hs], osp,
                                        inp["slots"], has, cfg.scale, False, "f16", "bf16")
            assert_close(outs[i][:, hs], o_ref, "bf16", f"call {i} out vs chained oracle, kh={kh}")
        assert_close(sp[:, hs], osp, "f16", f"final state (8 calls) vs chained oracle, kh={kh}")
