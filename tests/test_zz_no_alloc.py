"""gdn_prefill_varlen_noalloc (the prefill on the library's static device
scratch, for callers that cannot allocate) against gdn_prefill_varlen on the
same inputs, through the C ABI: two calls in a row, the second smaller.  The
first needs more scratch than the static array holds (the 4096-token layer
shape with 32 value heads needs about 240 MB), so its value heads run in two
groups; each head is computed exactly as the one-launch path computes it, so
outputs and final states must agree bit for bit."""
import numpy as np
import pytest
import torch

import gated_delta_rule_prepare_amd as gdn
from gdn_inputs import Config, Dims, make_inputs, prefill_single
from tests.gpu_runner import DEV, TORCH_DTYPE, dev, gdims

pytestmark = pytest.mark.gpu


def _prepared(cfg):
    """q/k/v/g/beta from the library's prepare step, on the device."""
    d = cfg.dims
    inp = make_inputs(cfg)
    T = cfg.T
    act, qkv = cfg.act_dtype, cfg.qkv_dtype
    q = torch.empty(T, d.Hk, d.Dk, device=DEV, dtype=TORCH_DTYPE[qkv])
    k = torch.empty_like(q)
    v = torch.empty(T, d.Hv, d.Dv, device=DEV, dtype=TORCH_DTYPE[qkv])
    g = torch.empty(T, d.Hv, device=DEV)
    beta = torch.empty_like(g)
    gdn.gdn_prepare(gdims(d), dev(inp["cu"]), dev(inp["x"], act), dev(inp["a"], act), dev(inp["b"], act),
                    dev(inp["w"], act), dev(inp["A_log"]), dev(inp["dt_bias"]), dev(inp["conv_pool"], act), q, k, v, g,
                    beta, slot_idx=dev(inp["slots"]), has_initial_state=dev(inp["has_init"]), apply_qk_l2norm=True)
    return inp, q, k, v, g, beta


def _both(cfg, has_init=None):
    d = cfg.dims
    inp, q, k, v, g, beta = _prepared(cfg)
    has = inp["has_init"] if has_init is None else has_init
    res = []
    for noalloc in (False, True):
        sp = dev(inp["ssm_pool"], cfg.state_dtype)
        out = torch.full((cfg.T, d.Hv, d.Dv), float("nan"), device=DEV, dtype=TORCH_DTYPE[cfg.qkv_dtype])
        args = (gdims(d), dev(inp["cu"]), q, k, v, g, beta, sp, out, cfg.scale)
        kw = dict(slot_idx=dev(inp["slots"]), has_initial_state=dev(has), cu_seqlens_host=inp["cu"],
                  slot_idx_host=inp["slots"])
        if noalloc:
            gdn.gdn_prefill_varlen_noalloc(*args, **kw)
        else:
            gdn.gdn_prefill_varlen(*args, **kw)
        torch.cuda.synchronize()
        res.append((out.float().cpu().numpy(), sp.float().cpu().numpy()))
    (o0, s0), (o1, s1) = res
    assert np.all(np.isfinite(o1))
    np.testing.assert_array_equal(o1, o0, err_msg=f"{cfg.name}: outputs")
    np.testing.assert_array_equal(s1, s0, err_msg=f"{cfg.name}: final states")


def test_noalloc_prefill_equals_workspace_prefill_two_calls():
    # call 1: 4096 tokens, Hk=16, Hv=32, Dk=Dv=128, bf16 q/k/v, f32 state:
    # about 240 MB of scratch, so two groups of 16 value heads
    big = prefill_single()
    per_head = gdn.gdn_prefill_workspace_size(gdn.Dims(1, 1, 128, 128, 4), 1, big.T)
    assert per_head * big.dims.Hv > (128 << 20) >= per_head
    print(f"[noalloc] call 1: {big.name}", flush=True)
    _both(big)
    # call 2, smaller: 5 sequences, bf16 state, some continuing their slot
    small = Config("noalloc_small", "prefill", Dims(2, 4, 128, 128, 4), seqlens=(1, 63, 64, 65, 200), num_slots=7,
                   act_dtype="bf16", qkv_dtype="bf16", state_dtype="bf16", init_state_std=0.05, conv_state_std=1.0,
                   seed=51)
    print(f"[noalloc] call 2: {small.name}", flush=True)
    _both(small, has_init=np.array([1, 0, 1, 0, 1], np.uint8))


def test_noalloc_prefill_f32_qkv_and_sequential_shapes():
    # f32 q/k/v (the W form of the chunked kernels), then a head shape the
    # chunked kernels do not cover (the token-sequential kernel, no scratch)
    f32 = Config("noalloc_f32", "prefill", Dims(2, 4, 64, 64, 4), seqlens=(97, 3, 130), num_slots=4, act_dtype="bf16",
                 qkv_dtype="f32", state_dtype="f32", init_state_std=0.05, conv_state_std=1.0, seed=52)
    print(f"[noalloc] {f32.name}", flush=True)
    _both(f32)
    seq = Config("noalloc_seq", "prefill", Dims(1, 2, 256, 128, 4), seqlens=(40,), num_slots=1, act_dtype="bf16",
                 qkv_dtype="bf16", state_dtype="f32", seed=53)
    print(f"[noalloc] {seq.name}", flush=True)
    _both(seq)
