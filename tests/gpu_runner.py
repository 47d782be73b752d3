"""Runs the HIP path through the Python binding (and so through the C ABI) on
numpy inputs, returning numpy results.  Used by the GPU tests only."""
import numpy as np
import torch

import gated_delta_rule_prepare_amd as gdn

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
DEV = "cuda:0"


def dev(a, dtype: str = "f32"):
    """numpy values (exactly representable in ``dtype``) -> device tensor."""
    a = np.ascontiguousarray(a)
    if a.dtype in (np.int32, np.uint8, np.int64):
        return torch.from_numpy(a).to(DEV)
    return torch.from_numpy(a.astype(np.float32, copy=False)).to(DEV, TORCH_DTYPE[dtype])


def host(t) -> np.ndarray:
    return t.detach().float().cpu().numpy().astype(np.float64)


def gdims(d) -> gdn.Dims:
    return gdn.Dims(d.Hk, d.Hv, d.Dk, d.Dv, d.K)


def prepare(d, inp, act: str, qkv: str, l2norm: bool = True, conv_pool=None):
    T = int(inp["cu"][-1])
    pool = dev(inp["conv_pool"] if conv_pool is None else conv_pool, act)
    q = torch.empty(T, d.Hk, d.Dk, device=DEV, dtype=TORCH_DTYPE[qkv])
    k = torch.empty_like(q)
    v = torch.empty(T, d.Hv, d.Dv, device=DEV, dtype=TORCH_DTYPE[qkv])
    g = torch.empty(T, d.Hv, device=DEV)
    beta = torch.empty_like(g)
    gdn.gdn_prepare(gdims(d), dev(inp["cu"]), dev(inp["x"], act), dev(inp["a"], act), dev(inp["b"], act),
                    dev(inp["w"], act), dev(inp["A_log"]), dev(inp["dt_bias"]), pool, q, k, v, g, beta,
                    slot_idx=dev(inp["slots"]), has_initial_state=dev(inp["has_init"]), apply_qk_l2norm=l2norm)
    torch.cuda.synchronize()
    return dict(q=host(q), k=host(k), v=host(v), g=host(g), beta=host(beta), conv_pool=host(pool))


def decode(d, inp, act: str, state: str, scale: float, conv_pool=None, ssm_pool=None, slots=None):
    B = inp["x"].shape[0]
    cp = dev(inp["conv_pool"] if conv_pool is None else conv_pool, act)
    sp = dev(inp["ssm_pool"] if ssm_pool is None else ssm_pool, state)
    out = torch.empty(B, d.Hv, d.Dv, device=DEV, dtype=TORCH_DTYPE[act])
    sl = inp["slots"] if slots is None else slots
    gdn.gdn_decode(gdims(d), dev(inp["x"], act), dev(inp["a"], act), dev(inp["b"], act), dev(inp["w"], act),
                   dev(inp["A_log"]), dev(inp["dt_bias"]), cp, sp, dev(sl), out, scale)
    torch.cuda.synchronize()
    return host(out), host(cp), host(sp)


def prefill(d, cu, q, k, v, g, beta, ssm_pool, slots, has_init, qkv: str, state: str, scale: float,
            l2norm: bool = False, stream=None):
    """The prefill through the binding; with ``stream`` (a torch.cuda.Stream)
    the inputs are made on the current stream, which the side stream then
    waits for, and the binding allocates its workspace itself."""
    T = int(cu[-1])
    sp = dev(ssm_pool, state)
    out = torch.empty(T, d.Hv, d.Dv, device=DEV, dtype=TORCH_DTYPE[qkv])
    args = (gdims(d), dev(np.asarray(cu, np.int32)), dev(q, qkv), dev(k, qkv), dev(v, qkv), dev(g), dev(beta), sp,
            out, scale)
    kw = dict(slot_idx=dev(np.asarray(slots, np.int32)), has_initial_state=dev(np.asarray(has_init, np.uint8)),
              use_qk_l2norm=l2norm)
    if stream is not None:
        stream.wait_stream(torch.cuda.current_stream())
    gdn.gdn_prefill_varlen(*args, **kw, stream=stream)
    torch.cuda.synchronize()
    return host(out), host(sp)


def decode_spec(d, inp, act: str, state: str, scale: float, conv_pool=None, ssm_pool=None, validate: bool = True):
    T = int(inp["cu"][-1])
    cp = dev(inp["conv_pool"] if conv_pool is None else conv_pool, act)
    sp = dev(inp["ssm_pool"] if ssm_pool is None else ssm_pool, state)
    out = torch.empty(T, d.Hv, d.Dv, device=DEV, dtype=TORCH_DTYPE[act])
    gdn.gdn_decode_spec(gdims(d), dev(inp["cu"]), dev(inp["x"], act), dev(inp["a"], act), dev(inp["b"], act),
                        dev(inp["w"], act), dev(inp["A_log"]), dev(inp["dt_bias"]), cp, sp,
                        dev(np.ascontiguousarray(inp["state_idx"], np.int32)),
                        dev(np.ascontiguousarray(inp["num_accepted"], np.int32)), out, scale, validate=validate)
    torch.cuda.synchronize()
    return host(out), host(cp), host(sp)


def kda_recurrent(d, inp, qkv: str, state: str, scale: float, l2norm: bool, ssm_pool=None):
    T = int(inp["cu"][-1])
    sp = dev(inp["ssm_pool"] if ssm_pool is None else ssm_pool, state)
    out = torch.empty(max(T, 1), d.Hv, d.Dv, device=DEV, dtype=TORCH_DTYPE[qkv])
    opt = lambda a: None if a is None else dev(a)
    gdn.gdn_kda_recurrent(gdims(d), dev(inp["cu"]), dev(inp["q"], qkv), dev(inp["k"], qkv), dev(inp["v"], qkv),
                          dev(inp["g"]), dev(inp["beta"]), sp, out, scale, A_log=opt(inp["A_log"]),
                          dt_bias=opt(inp["dt_bias"]), slot_idx=dev(inp["slots"]),
                          has_initial_state=dev(inp["has_init"]), use_qk_l2norm=l2norm)
    torch.cuda.synchronize()
    return host(out[:T]), host(sp)


def kda_prefill(d, inp, qkv: str, state: str, scale: float, l2norm: bool, ssm_pool=None):
    T = int(inp["cu"][-1])
    sp = dev(inp["ssm_pool"] if ssm_pool is None else ssm_pool, state)
    out = torch.empty(max(T, 1), d.Hv, d.Dv, device=DEV, dtype=TORCH_DTYPE[qkv])
    opt = lambda a: None if a is None else dev(a)
    gdn.gdn_kda_prefill_varlen(gdims(d), dev(inp["cu"]), dev(inp["q"], qkv), dev(inp["k"], qkv), dev(inp["v"], qkv),
                               dev(inp["g"]), dev(inp["beta"]), sp, out, scale, A_log=opt(inp["A_log"]),
                               dt_bias=opt(inp["dt_bias"]), slot_idx=dev(inp["slots"]),
                               has_initial_state=dev(inp["has_init"]), use_qk_l2norm=l2norm)
    torch.cuda.synchronize()
    return host(out[:T]), host(sp)


def mamba2(inp, act: str, state: str, decode: bool, ssm_pool=None, dt_min=0.0, dt_max=float("inf")):
    T, H, P = inp["x"].shape
    sp = dev(inp["ssm_pool"] if ssm_pool is None else ssm_pool, state)
    out = torch.empty(T, H, P, device=DEV, dtype=TORCH_DTYPE[act])
    opt = lambda a, dt="f32": None if a is None else dev(a, dt)
    args = (dev(inp["x"], act), dev(inp["dt"], act), dev(inp["A"]), dev(inp["B"], act), dev(inp["C"], act))
    kw = dict(D=opt(inp["D"]), z=opt(inp["z"], act), dt_bias=opt(inp["dt_bias"]), dt_min=dt_min, dt_max=dt_max)
    if decode:
        gdn.gdn_mamba2_state_update(*args, sp, dev(inp["slots"]), out, **kw)
    else:
        gdn.gdn_mamba2_chunk_scan(dev(inp["cu"]), *args, sp, out, slot_idx=dev(inp["slots"]),
                                  has_initial_state=dev(inp["has_init"]), **kw)
    torch.cuda.synchronize()
    return host(out), host(sp)
