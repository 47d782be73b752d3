"""Parity of the KDA entry points (one log-decay per key channel; vllm.cpp
cpu_ops.cpp KdaHeadTokenStep, KdaGatedDeltaRuleKernel, KdaChunkPrefillKernel)
with the f64 oracle, through the C ABI.

Tolerances as for the GDN path: f32 allclose(atol=1e-4, rtol=1e-4); bf16
max-abs 2e-2; f16 max-abs 2e-3.
"""
import sys

import numpy as np
import pytest

import oracle
from gdn_inputs import Dims, kda_inputs
from tests.test_gpu_parity import assert_close

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _runner():
    from tests import gpu_runner
    return gpu_runner


def _oracle(d, inp, scale, l2norm, qkv, sdt, ssm_pool=None):
    return oracle.kda(d, inp["cu"], inp["q"], inp["k"], inp["v"], inp["g"], inp["beta"],
                      inp["ssm_pool"] if ssm_pool is None else ssm_pool, inp["slots"], inp["has_init"], scale,
                      A_log=inp["A_log"], dt_bias=inp["dt_bias"], state_dtype=sdt, out_dtype=qkv, l2norm=l2norm)


REC_CASES = [
    # name, dims, seqlens, qkv, state, options
    ("bf16_f32_gate_bias_l2", Dims(2, 4, 128, 128, 4), (1, 2, 17, 64, 100), "bf16", "f32",
     dict(gate=True, dt_bias=True, l2=True)),
    ("f32_bf16_nogate_small_qk", Dims(1, 2, 64, 64, 4), (5, 33), "f32", "bf16",
     dict(gate=False, l2=False, qk_std=0.125)),
    ("f32_f16_gate_nobias_dk64_dv32", Dims(2, 2, 64, 32, 4), (9, 0, 40), "f32", "f16",
     dict(gate=True, dt_bias=False, l2=True, has_init=(1, 0, 0))),
    ("bf16_f32_mild_decay_d16", Dims(2, 8, 16, 16, 4), (3, 70), "bf16", "f32",
     dict(gate=True, dt_bias=True, l2=True, A_log_range=(-3.0, 0.0))),
    ("f32_f32_d256_dv128", Dims(1, 2, 256, 128, 4), (12,), "f32", "f32", dict(gate=True, dt_bias=True, l2=True)),
    ("decode_like_256x1", Dims(4, 8, 128, 128, 4), (1,) * 64, "bf16", "f32", dict(gate=True, dt_bias=True, l2=True)),
]


@pytest.mark.parametrize("name,d,lens,qkv,sdt,opts", REC_CASES, ids=[c[0] for c in REC_CASES])
def test_kda_recurrent_parity(name, d, lens, qkv, sdt, opts):
    R = _runner()
    opts = dict(opts)
    l2 = opts.pop("l2")
    seed = 500 + [c[0] for c in REC_CASES].index(name)
    inp = kda_inputs(d, lens, len(lens) + 3, qkv, sdt, seed, **opts)
    scale = 1.0 / np.sqrt(d.Dk)
    _say(f"[kda recurrent] {name} T={inp['cu'][-1]}")
    out, sp = R.kda_recurrent(d, inp, qkv, sdt, scale, l2)
    o_ref, s_ref = _oracle(d, inp, scale, l2, qkv, sdt)
    assert_close(out, o_ref, qkv, f"{name} out")
    assert_close(sp, s_ref, sdt, f"{name} state pool")


CHUNK_CASES = [
    # name, dims, seqlens, qkv, state, options
    ("bf16_f32_ragged_d128", Dims(2, 4, 128, 128, 4), (1, 63, 64, 65, 200, 0, 130), "bf16", "f32",
     dict(gate=True, dt_bias=True, l2=True, has_init=(1, 0, 1, 1, 0, 0, 1))),
    ("f32_f16_d64_nobias", Dims(2, 2, 64, 64, 4), (100, 7), "f32", "f16", dict(gate=True, dt_bias=False, l2=True)),
    ("bf16_bf16_d32_nogate", Dims(1, 4, 32, 32, 4), (129, 3), "bf16", "bf16",
     dict(gate=False, l2=False, qk_std=0.17)),
    ("f32_f32_strong_decay", Dims(1, 2, 128, 128, 4), (150,), "f32", "f32",
     dict(gate=True, dt_bias=True, l2=True, A_log_range=(2.5, 3.5))),
    ("bf16_f32_mild_decay_long", Dims(2, 4, 128, 128, 4), (700,), "bf16", "f32",
     dict(gate=True, dt_bias=True, l2=True, A_log_range=(-4.0, -1.0))),
    ("f32_f32_mild_decay_d64", Dims(1, 1, 64, 64, 4), (257,), "f32", "f32",
     dict(gate=True, dt_bias=True, l2=True, A_log_range=(-4.0, -1.0))),
    ("fallback_dk64_dv32", Dims(2, 2, 64, 32, 4), (70, 0), "bf16", "f32", dict(gate=True, dt_bias=True, l2=True)),
    ("all_empty", Dims(1, 2, 64, 64, 4), (0, 0), "bf16", "f32", dict(gate=True, has_init=(0, 1), l2=True)),
    # more (chunk, value head) items than the prep has persistent workgroups
    # (one per CU), over several sequences: each workgroup walks several items
    ("many_items_varlen", Dims(2, 8, 128, 128, 4), (2000, 1500, 700), "bf16", "f32",
     dict(gate=True, dt_bias=True, l2=True, has_init=(1, 0, 1))),
    # more sequences than the chunk-table wave has lanes, empty ones among them
    ("over_64_seqs", Dims(1, 2, 64, 64, 4), tuple((i * 37) % 150 for i in range(70)), "bf16", "f32",
     dict(gate=True, dt_bias=True, l2=True)),
]


@pytest.mark.parametrize("name,d,lens,qkv,sdt,opts", CHUNK_CASES, ids=[c[0] for c in CHUNK_CASES])
def test_kda_prefill_parity(name, d, lens, qkv, sdt, opts):
    R = _runner()
    opts = dict(opts)
    l2 = opts.pop("l2")
    seed = 600 + [c[0] for c in CHUNK_CASES].index(name)
    inp = kda_inputs(d, lens, len(lens) + 2, qkv, sdt, seed, **opts)
    scale = 1.0 / np.sqrt(d.Dk)
    _say(f"[kda prefill] {name} T={inp['cu'][-1]}")
    out, sp = R.kda_prefill(d, inp, qkv, sdt, scale, l2)
    o_ref, s_ref = _oracle(d, inp, scale, l2, qkv, sdt)
    if o_ref.size:
        assert_close(out, o_ref, qkv, f"{name} out")
    assert_close(sp, s_ref, sdt, f"{name} state pool")


def test_kda_prefill_repeated_runs():
    """The ragged KDA case run eight times, every run against the oracle.
    Regression test: the scan's state waves once read the per-column chunk
    decays exp(G_C) from a buffer the output waves could already be filling
    with a later chunk's, so a run now and then gave a wrong final state."""
    R = _runner()
    name, d, lens, qkv, sdt, opts = next(c for c in CHUNK_CASES if c[0] == "bf16_f32_ragged_d128")
    opts = dict(opts)
    l2 = opts.pop("l2")
    inp = kda_inputs(d, lens, len(lens) + 2, qkv, sdt, 777, **opts)
    scale = 1.0 / np.sqrt(d.Dk)
    o_ref, s_ref = _oracle(d, inp, scale, l2, qkv, sdt)
    for run in range(8):
        _say(f"[kda prefill repeated] run {run}")
        out, sp = R.kda_prefill(d, inp, qkv, sdt, scale, l2)
        assert_close(out, o_ref, qkv, f"run {run} out")
        assert_close(sp, s_ref, sdt, f"run {run} state pool")


@pytest.mark.slow
@pytest.mark.parametrize("which", ["prefill", "decode"])
def test_kda_full_size(which):
    """The benchmarked KDA workloads in the launch configuration the bench
    times, every head checked against the oracle."""
    from gdn_inputs import kda_decode_workload, kda_prefill_workload
    from tests import gpu_runner as R
    wl = kda_prefill_workload() if which == "prefill" else kda_decode_workload()
    d = wl["dims"]
    inp = kda_inputs(d, wl["seqlens"], wl["num_slots"], wl["qkv_dtype"], wl["state_dtype"], wl["seed"],
                     has_init=wl["has_init"])
    scale = 1.0 / np.sqrt(d.Dk)
    _say(f"[kda full] {wl['name']}")
    run = R.kda_prefill if which == "prefill" else R.kda_recurrent
    out, sp = run(d, inp, "bf16", "f32", scale, True)
    o_ref, s_ref = _oracle(d, inp, scale, True, "bf16", "f32")
    assert_close(out, o_ref, "bf16", "out, every head")
    assert_close(sp, s_ref, "f32", "state pool, every head")
