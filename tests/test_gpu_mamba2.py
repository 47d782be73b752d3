"""Parity of the Mamba2 / SSD entry points (vllm.cpp cpu_ops.cpp,
Mamba2ChunkScanKernel, Mamba2StateUpdateKernel) with the f64 oracle, through
the C ABI.  Tolerances as for the GDN path: f32 allclose(atol=1e-4,
rtol=1e-4); bf16 max-abs 2e-2 * max(1, |ref|) (the gated outputs reach
magnitudes where a bf16 unit in the last place exceeds 2e-2); f16 state
max-abs 2e-3."""
import sys

import numpy as np
import pytest

import oracle
from gdn_inputs import mamba2_decode_workload, mamba2_inputs, mamba2_prefill_workload

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
    elif dtype == "f16":
        lim = np.full_like(want, 2e-3) * np.maximum(1.0, np.abs(want))
    else:
        lim = 2e-2 * np.maximum(1.0, np.abs(want))
    worst = float((err / lim).max()) if err.size else 0.0
    assert worst <= 1.0, f"{what}: {dtype} mismatch, max abs err {float(err.max()):.3e}, worst err/bound {worst:.3f}"


def _oracle(inp, act, sdt, dt_min=0.0, dt_max=float("inf")):
    return oracle.mamba2(inp["cu"], inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["ssm_pool"], inp["slots"],
                         inp["has_init"], D=inp["D"], z=inp["z"], dt_bias=inp["dt_bias"], softplus=True,
                         dt_min=dt_min, dt_max=dt_max, state_dtype=sdt, out_dtype=act)


DEC_CASES = [
    # name, H, P, G, N, rows, act, state, opts
    ("bf16_f32_h8_p64_n128", 8, 64, 2, 128, 9, "bf16", "f32", dict(null_rows=2)),
    ("f32_bf16_h4_p32_n64_Dhp", 4, 32, 4, 64, 5, "f32", "bf16", dict(D_mode="hp")),
    ("f32_f16_h6_p48_n16_noz", 6, 48, 3, 16, 4, "f32", "f16", dict(with_z=False, D_mode="none")),
    ("bf16_f32_h2_p128_n256", 2, 128, 1, 256, 3, "bf16", "f32", {}),
]


@pytest.mark.parametrize("name,H,P,G,N,rows,act,sdt,opts", DEC_CASES, ids=[c[0] for c in DEC_CASES])
def test_mamba2_state_update_parity(name, H, P, G, N, rows, act, sdt, opts):
    from tests import gpu_runner as R
    seed = 700 + [c[0] for c in DEC_CASES].index(name)
    inp = mamba2_inputs(H, P, G, N, (1,) * rows, rows + 4, act, sdt, seed, **opts)
    _say(f"[mamba2 update] {name}")
    out, sp = R.mamba2(inp, act, sdt, decode=True)
    o_ref, s_ref = _oracle(inp, act, sdt)
    assert_close(out, o_ref, act, f"{name} out")
    assert_close(sp, s_ref, sdt, f"{name} state pool")
    nulls = inp["slots"] < 0
    assert np.all(out[nulls] == 0)


SCAN_CASES = [
    ("bf16_f32_h4_p64_n128_ragged", 4, 64, 2, 128, (1, 63, 64, 65, 200, 130), "bf16", "f32",
     dict(has_init=(1, 0, 1, 1, 0, 1))),
    ("f32_f32_h2_p32_n32_Dhp", 2, 32, 1, 32, (100, 7), "f32", "f32", dict(D_mode="hp")),
    ("f32_bf16_h3_p128_n64_noz", 3, 128, 3, 64, (129,), "f32", "bf16", dict(with_z=False)),
    ("bf16_f16_h8_p64_n64_long", 8, 64, 4, 64, (700,), "bf16", "f16", dict(init_std=0.05)),
    # the largest instantiation (f32 activations, P = N = 128)
    ("f32_f32_h2_p128_n128_Dhp", 2, 128, 2, 128, (150, 70), "f32", "f32", dict(D_mode="hp")),
    ("bf16_f32_h2_p32_n128", 2, 32, 1, 128, (90, 64), "bf16", "f32", {}),
    # more sequences than the chunk-table wave has lanes
    ("bf16_f32_h2_p64_n64_70seqs", 2, 64, 1, 64, tuple(1 + (i * 37) % 150 for i in range(70)), "bf16", "f32", {}),
    # three heads per group (the output kernel's heads taken two at a time,
    # with a last one alone) and one head per group; chunk counts 1 to 5
    ("bf16_f32_h6_p64_n64_3pergroup", 6, 64, 2, 64, (300, 65, 129, 1, 192), "bf16", "f32", dict(has_init=(1, 1, 0, 1, 0))),
    ("bf16_f16_h2_p32_n128_1pergroup", 2, 32, 2, 128, (257, 64), "bf16", "f16", {}),
]


@pytest.mark.parametrize("name,H,P,G,N,lens,act,sdt,opts", SCAN_CASES, ids=[c[0] for c in SCAN_CASES])
def test_mamba2_chunk_scan_parity(name, H, P, G, N, lens, act, sdt, opts):
    from tests import gpu_runner as R
    seed = 750 + [c[0] for c in SCAN_CASES].index(name)
    inp = mamba2_inputs(H, P, G, N, lens, len(lens) + 2, act, sdt, seed, **opts)
    _say(f"[mamba2 scan] {name} T={inp['cu'][-1]}")
    out, sp = R.mamba2(inp, act, sdt, decode=False)
    o_ref, s_ref = _oracle(inp, act, sdt)
    assert_close(out, o_ref, act, f"{name} out")
    assert_close(sp, s_ref, sdt, f"{name} state pool")


def test_mamba2_dt_limits_and_chunk_equals_steps():
    """dt clamped to [dt_min, dt_max]; a sequence run as chunked prefill
    equals the same tokens run one decode step at a time."""
    from tests import gpu_runner as R
    H, P, G, N = 4, 64, 2, 64
    inp = mamba2_inputs(H, P, G, N, (20,), 2, "f32", "f32", 790)
    _say("[mamba2] dt limits, chunk vs steps")
    out, sp = R.mamba2(inp, "f32", "f32", decode=False, dt_min=0.01, dt_max=0.05)
    o_ref, s_ref = _oracle(inp, "f32", "f32", dt_min=0.01, dt_max=0.05)
    assert_close(out, o_ref, "f32", "clamped out")
    assert_close(sp, s_ref, "f32", "clamped state")
    pool = inp["ssm_pool"]
    slot = inp["slots"][0]
    outs = []
    for t in range(20):
        row = {k: (v[t:t + 1] if k in ("x", "z", "B", "C", "dt") else v) for k, v in inp.items()}
        row["slots"] = np.array([slot], np.int32)
        o, pool = R.mamba2({**row, "ssm_pool": pool}, "f32", "f32", decode=True)
        outs.append(o[0])
    o_full, s_full = R.mamba2(inp, "f32", "f32", decode=False)
    assert_close(np.stack(outs), o_full, "f32", "steps vs chunked out")
    assert_close(pool, s_full, "f32", "steps vs chunked state")


@pytest.mark.slow
@pytest.mark.parametrize("which", ["prefill", "decode"])
def test_mamba2_full_size(which):
    """The benchmarked Mamba2 workloads in the launch configuration the bench
    times, checked on every head."""
    from tests import gpu_runner as R
    wl = mamba2_prefill_workload() if which == "prefill" else mamba2_decode_workload()
    inp = mamba2_inputs(wl["H"], wl["P"], wl["G"], wl["N"], wl["seqlens"], wl["num_slots"], wl["act"], wl["state"],
                        wl["seed"], has_init=wl["has_init"])
    _say(f"[mamba2 full] {wl['name']}")
    out, sp = R.mamba2(inp, wl["act"], wl["state"], decode=(which == "decode"))
    o_ref, s_ref = _oracle(inp, wl["act"], wl["state"])
    assert_close(out, o_ref, wl["act"], "out")
    live = inp["slots"][inp["slots"] >= 0]
    assert_close(sp[live], s_ref[live], wl["state"], "state pool")
