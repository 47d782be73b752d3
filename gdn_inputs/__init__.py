"""Seeded synthetic inputs for the gated-delta-rule (GDN) prepare / decode /
prefill workloads.

This module is shared by the GPU path's tests and benchmark and by the CPU
oracle's tests.  It holds *no* arithmetic of the method itself: it only draws
random numbers, rounds them to their storage format (so that both sides see
exactly the same values) and lays them out.  Every array is returned as
float32 (or int32 / uint8 for indices and flags); the values of an array whose
storage dtype is bf16 or f16 are exactly representable in that dtype.

Shapes follow the GDN layer's layout (vllm.cpp qwen3_5.cpp, GDN state-cache
layout checks; ferrum-kernels cpu.rs, linear_attention_prepare_varlen_f32):

* ``x``        [T, Cc] mixed q|k|v projection rows, Cc = 2*Hk*Dk + Hv*Dv
* ``w``        [Cc, K] depthwise conv taps, tap j multiplies token t-(K-1)+j
* ``a``, ``b`` [T, Hv] raw gate projections
* ``A_log``, ``dt_bias`` [Hv]
* ``conv_pool`` [S, Cc, K-1] raw-input history per slot, oldest column first
* ``ssm_pool``  [S, Hv, Dv, Dk] recurrent state per slot
* ``cu``       [N+1] int32 sequence offsets, ``slots`` [N] int32, ``has_init`` [N] uint8
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence

import numpy as np

DTYPES = ("f32", "bf16", "f16")


@dataclasses.dataclass(frozen=True)
class Dims:
    Hk: int
    Hv: int
    Dk: int
    Dv: int
    K: int

    @property
    def Cc(self) -> int:
        return 2 * self.Hk * self.Dk + self.Hv * self.Dv


@dataclasses.dataclass(frozen=True)
class Config:
    """One synthetic workload.

    mode is "decode" (one token per row, state pools indexed by ``slots``) or
    "prefill" (varlen sequences given by ``seqlens``).
    """
    name: str
    mode: str
    dims: Dims
    seqlens: Sequence[int] = ()      # prefill: token count per sequence
    batch: int = 0                   # decode: rows
    num_slots: int = 1
    act_dtype: str = "bf16"          # raw activations, conv weight, conv pool
    state_dtype: str = "f32"         # ssm pool
    qkv_dtype: str = "bf16"          # prepare outputs / prefill inputs
    init_state_std: float = 0.0      # 0 => zero initial state (has_init = 0)
    conv_state_std: float = 0.0      # 0 => zero conv history
    conv_weight_std: float = 0.5
    chunk: int = 64
    seed: int = 0
    null_rows: int = 0               # decode: rows whose slot is -1

    @property
    def T(self) -> int:
        return int(sum(self.seqlens)) if self.mode == "prefill" else self.batch

    @property
    def N(self) -> int:
        return len(self.seqlens) if self.mode == "prefill" else self.batch

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.dims.Dk)


def round_to_dtype(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float values to the storage dtype (round-to-nearest-even) and
    return them as float32.  Used only to define input values."""
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == "f32":
        return x32
    if dtype == "f16":
        return x32.astype(np.float16).astype(np.float32)
    if dtype == "bf16":
        bits = x32.view(np.uint32).astype(np.uint64)
        lsb = (bits >> 16) & 1
        bits = (bits + 0x7FFF + lsb) & 0xFFFF0000
        return bits.astype(np.uint32).view(np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def _normal(rng: np.random.Generator, shape, std: float, dtype: str) -> np.ndarray:
    # float32 draws keep the multi-GiB pools affordable
    v = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        v *= np.float32(std)
    return round_to_dtype(v, dtype)


def varlen_lengths(n: int, lo: int, hi: int, seed: int) -> List[int]:
    """Sequence lengths ~ U[lo, hi] (inclusive), seeded."""
    rng = np.random.default_rng(seed)
    return [int(v) for v in rng.integers(lo, hi + 1, size=n)]


def make_inputs(cfg: Config, slot_seed: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Draw every input of ``cfg`` from numpy's PCG64 seeded with cfg.seed."""
    d = cfg.dims
    rng = np.random.default_rng(cfg.seed)
    T, N, S = cfg.T, cfg.N, cfg.num_slots
    out: Dict[str, np.ndarray] = {}
    out["x"] = _normal(rng, (T, d.Cc), 1.0, cfg.act_dtype)
    out["w"] = _normal(rng, (d.Cc, d.K), cfg.conv_weight_std, cfg.act_dtype)
    out["a"] = _normal(rng, (T, d.Hv), 1.0, cfg.act_dtype)
    out["b"] = _normal(rng, (T, d.Hv), 1.0, cfg.act_dtype)
    out["A_log"] = rng.uniform(0.0, math.log(16.0), size=d.Hv).astype(np.float32)
    out["dt_bias"] = rng.uniform(-1.0, 1.0, size=d.Hv).astype(np.float32)
    if cfg.conv_state_std > 0:
        out["conv_pool"] = _normal(rng, (S, d.Cc, d.K - 1), cfg.conv_state_std, cfg.act_dtype)
    else:
        out["conv_pool"] = np.zeros((S, d.Cc, d.K - 1), np.float32)
    if cfg.init_state_std > 0:
        out["ssm_pool"] = _normal(rng, (S, d.Hv, d.Dv, d.Dk), cfg.init_state_std, cfg.state_dtype)
    else:
        out["ssm_pool"] = np.zeros((S, d.Hv, d.Dv, d.Dk), np.float32)
    srng = np.random.default_rng(cfg.seed + 7 if slot_seed is None else slot_seed)
    if cfg.mode == "decode":
        slots = srng.permutation(S)[:N].astype(np.int32)
        if cfg.null_rows:
            where = srng.choice(N, size=cfg.null_rows, replace=False)
            slots[where] = -1
        out["slots"] = slots
        out["cu"] = np.arange(N + 1, dtype=np.int32)
        out["has_init"] = np.ones(N, np.uint8)
    else:
        out["cu"] = np.concatenate([[0], np.cumsum(cfg.seqlens)]).astype(np.int32)
        out["slots"] = srng.permutation(S)[:N].astype(np.int32)
        flag = 1 if (cfg.init_state_std > 0 or cfg.conv_state_std > 0) else 0
        out["has_init"] = np.full(N, flag, np.uint8)
    return out


def epilogue_inputs(T: int, Hv: int, Dv: int, dtype: str, seed: int) -> Dict[str, np.ndarray]:
    """Inputs of the output epilogue (gated RMS norm): the gate ``z`` [T, Hv*Dv]
    ~ N(0, 1) (the z columns of a packed [q|k|v|z] projection row) and the
    norm weight [Dv] ~ U(0.5, 1.5), both rounded to ``dtype``."""
    rng = np.random.default_rng(seed)
    z = _normal(rng, (T, Hv * Dv), 1.0, dtype)
    w = round_to_dtype(rng.uniform(0.5, 1.5, size=Dv).astype(np.float32), dtype)
    return {"z": z, "norm_w": w}


def spec_inputs(dims: Dims, num_reqs: int, cols: int, num_slots: int, act_dtype: str, state_dtype: str,
                seed: int, lens: Optional[Sequence[int]] = None, conv_len: Optional[int] = None,
                null_reqs: int = 0, null_cols: int = 0) -> Dict[str, np.ndarray]:
    """Inputs of one speculative decode step.

    ``num_reqs`` requests of ``cols`` tokens each (or ``lens[i]`` tokens,
    1 <= lens[i] <= cols); x, a, b ~ N(0, 1), conv weight ~ N(0, 0.5), A_log ~
    U(0, log 16), dt_bias ~ U(-1, 1); the conv pool [num_slots, Cc, W] ~ N(0, 1)
    with W = (K-1) + (cols-1) unless ``conv_len`` is given; the state pool
    ~ N(0, 0.05).  ``state_idx`` [num_reqs, cols] holds distinct slots drawn
    from one permutation; ``num_accepted`` ~ U[1, cols].  ``null_reqs``
    requests have every column -1 (padding rows); ``null_cols`` further
    columns of live requests, never column 0 nor the initial column
    num_accepted-1, are set to -1."""
    rng = np.random.default_rng(seed)
    lens = [cols] * num_reqs if lens is None else [int(v) for v in lens]
    assert len(lens) == num_reqs and all(1 <= v <= cols for v in lens)
    W = (dims.K - 1) + (cols - 1) if conv_len is None else conv_len
    T = int(sum(lens))
    out: Dict[str, np.ndarray] = {}
    out["x"] = _normal(rng, (T, dims.Cc), 1.0, act_dtype)
    out["w"] = _normal(rng, (dims.Cc, dims.K), 0.5, act_dtype)
    out["a"] = _normal(rng, (T, dims.Hv), 1.0, act_dtype)
    out["b"] = _normal(rng, (T, dims.Hv), 1.0, act_dtype)
    out["A_log"] = rng.uniform(0.0, math.log(16.0), size=dims.Hv).astype(np.float32)
    out["dt_bias"] = rng.uniform(-1.0, 1.0, size=dims.Hv).astype(np.float32)
    out["conv_pool"] = _normal(rng, (num_slots, dims.Cc, W), 1.0, act_dtype)
    out["ssm_pool"] = _normal(rng, (num_slots, dims.Hv, dims.Dv, dims.Dk), 0.05, state_dtype)
    out["cu"] = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    assert num_reqs * cols <= num_slots
    sidx = rng.permutation(num_slots)[: num_reqs * cols].astype(np.int32).reshape(num_reqs, cols)
    nat = rng.integers(1, cols + 1, size=num_reqs).astype(np.int32)
    if null_reqs:
        sidx[rng.choice(num_reqs, size=null_reqs, replace=False)] = -1
    if null_cols:
        cand = [(i, c) for i in range(num_reqs) for c in range(1, cols)
                if c != nat[i] - 1 and sidx[i, 0] >= 0]
        for j in rng.choice(len(cand), size=min(null_cols, len(cand)), replace=False):
            sidx[cand[j]] = -1
    out["state_idx"] = sidx
    out["num_accepted"] = nat
    return out


def decode_slot_sets(cfg: Config, count: int, seed: int) -> np.ndarray:
    """``count`` independent draws of the decode slot subset (distinct slots
    within each draw), so that repeated timed calls touch different slots."""
    rng = np.random.default_rng(seed)
    return np.stack([rng.permutation(cfg.num_slots)[: cfg.batch] for _ in range(count)]).astype(np.int32)


# ---------------------------------------------------------------------------
# The named workloads.
# ---------------------------------------------------------------------------
QWEN_DIMS = Dims(Hk=16, Hv=32, Dk=128, Dv=128, K=4)


def tiny() -> Config:
    """1 sequence of 8 tokens, Hk=1, Hv=2, Dk=Dv=16, K=4, f32 throughout."""
    return Config(name="tiny_f32_T8", mode="prefill", dims=Dims(1, 2, 16, 16, 4), seqlens=(8,),
                  num_slots=1, act_dtype="f32", state_dtype="f32", qkv_dtype="f32", seed=1001)


def tiny_decode() -> Config:
    """The tiny workload's shapes as a decode batch of 8 rows."""
    return Config(name="tiny_f32_decode", mode="decode", dims=Dims(1, 2, 16, 16, 4), batch=8,
                  num_slots=16, act_dtype="f32", state_dtype="f32", qkv_dtype="f32",
                  init_state_std=0.05, conv_state_std=1.0, seed=1001)


def decode_batch(state_dtype: str = "f32") -> Config:
    """256 rows x 1 token, Hk=16, Hv=32, Dk=Dv=128, K=4; bf16 activations;
    512-slot state pool ~N(0, 0.05); bf16 conv pool [512, Cc, 3]."""
    return Config(name="decode_b256_hk16_hv32_d128", mode="decode", dims=QWEN_DIMS, batch=256,
                  num_slots=512, act_dtype="bf16", state_dtype=state_dtype, qkv_dtype="bf16",
                  init_state_std=0.05, conv_state_std=1.0, seed=1002)


def prefill_single(qkv_dtype: str = "bf16") -> Config:
    """1 sequence of 4096 tokens, Hk=16, Hv=32, Dk=Dv=128, K=4; bf16 raw
    activations; f32 state from zero; chunk 64."""
    return Config(name="prefill_T4096_hk16_hv32_d128", mode="prefill", dims=QWEN_DIMS, seqlens=(4096,),
                  num_slots=1, act_dtype="bf16", state_dtype="f32", qkv_dtype=qkv_dtype, seed=1003)


def prefill_varlen() -> Config:
    """16 sequences, lengths ~U[128, 8192] (seeded), bf16 activations, bf16
    state cache with nonzero initial states ~N(0, 0.05)."""
    return Config(name="varlen_16seq_hk16_hv32_d128", mode="prefill", dims=QWEN_DIMS,
                  seqlens=tuple(varlen_lengths(16, 128, 8192, 2004)), num_slots=32, act_dtype="bf16",
                  state_dtype="bf16", qkv_dtype="bf16", init_state_std=0.05, conv_state_std=1.0, seed=1004)


def prefill_long(tokens: int = 32768) -> Config:
    """1 sequence of 32768 tokens, Hk=16, Hv=48, Dk=Dv=128, K=4; bf16
    activations; f16 state from zero."""
    return Config(name=f"long_T{tokens}_hk16_hv48_d128", mode="prefill", dims=Dims(16, 48, 128, 128, 4),
                  seqlens=(tokens,), num_slots=1, act_dtype="bf16", state_dtype="f16", qkv_dtype="bf16",
                  seed=1005)


def named_configs() -> Dict[str, Config]:
    cs = [tiny(), decode_batch(), prefill_single(), prefill_varlen(), prefill_long()]
    return {c.name: c for c in cs}


def spec_batch() -> Dict[str, object]:
    """The speculative decode workload at the layer's shapes: 256 requests x
    4 tokens (the last accepted token and 3 drafts), Hk=16, Hv=32,
    Dk=Dv=128, K=4; bf16 activations, a 1024-slot f32 state pool (4 slot
    columns per request), conv rows of (K-1)+3 = 6 taps."""
    return dict(name="spec_decode_n256_c4_hk16_hv32_d128", dims=QWEN_DIMS, num_reqs=256, cols=4, num_slots=1024,
                act_dtype="bf16", state_dtype="f32", seed=1006)


def kda_inputs(dims: Dims, seqlens: Sequence[int], num_slots: int, qkv_dtype: str, state_dtype: str, seed: int,
               gate: bool = True, dt_bias: bool = True, A_log_range=(0.0, math.log(16.0)), qk_std: float = 1.0,
               init_std: float = 0.05, has_init: Optional[Sequence[int]] = None) -> Dict[str, np.ndarray]:
    """Inputs of the KDA variant (one log-decay per key channel).

    q, k [T, Hk, Dk] ~ N(0, qk_std^2) and v [T, Hv, Dv] ~ N(0, 1), rounded to
    ``qkv_dtype``; with ``gate`` the gate input g [T, Hv, Dk] ~ N(0, 1),
    A_log ~ U(A_log_range), dt_bias [Hv, Dk] ~ U(-1, 1) (or none); without,
    g is a log-decay -|N(0, 1)| * 0.5 directly.  beta = logistic(N(0, 1)) as
    f32.  The state pool ~ N(0, init_std^2) in ``state_dtype``; each sequence
    gets a distinct slot from one permutation.  Empty sequences are allowed."""
    rng = np.random.default_rng(seed)
    T = int(sum(seqlens))
    N = len(seqlens)
    out: Dict[str, np.ndarray] = {}
    out["q"] = _normal(rng, (T, dims.Hk, dims.Dk), qk_std, qkv_dtype)
    out["k"] = _normal(rng, (T, dims.Hk, dims.Dk), qk_std, qkv_dtype)
    out["v"] = _normal(rng, (T, dims.Hv, dims.Dv), 1.0, qkv_dtype)
    if gate:
        out["g"] = rng.standard_normal((T, dims.Hv, dims.Dk), dtype=np.float32)
        out["A_log"] = rng.uniform(A_log_range[0], A_log_range[1], size=dims.Hv).astype(np.float32)
        out["dt_bias"] = rng.uniform(-1.0, 1.0, size=(dims.Hv, dims.Dk)).astype(np.float32) if dt_bias else None
    else:
        out["g"] = (-0.5 * np.abs(rng.standard_normal((T, dims.Hv, dims.Dk)))).astype(np.float32)
        out["A_log"] = None
        out["dt_bias"] = None
    z = rng.standard_normal((T, dims.Hv))
    out["beta"] = (1.0 / (1.0 + np.exp(-z))).astype(np.float32)
    out["ssm_pool"] = _normal(rng, (num_slots, dims.Hv, dims.Dv, dims.Dk), init_std, state_dtype)
    out["cu"] = np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int32)
    out["slots"] = rng.permutation(num_slots)[:N].astype(np.int32)
    out["has_init"] = (np.ones(N, np.uint8) if has_init is None else np.asarray(has_init, np.uint8))
    return out


def kda_prefill_workload() -> Dict[str, object]:
    """The KDA prefill workload at the layer's shapes: one 4096-token sequence,
    Hk=16, Hv=32, Dk=Dv=128, bf16 q/k/v, f32 state from zero, the gate applied
    in the kernel (A_log ~ U(0, ln 16), dt_bias [Hv, Dk] ~ U(-1, 1)), q/k L2
    normalised in the kernel."""
    return dict(name="kda_prefill_T4096_hk16_hv32_d128", dims=QWEN_DIMS, seqlens=(4096,), num_slots=1,
                qkv_dtype="bf16", state_dtype="f32", seed=1007, has_init=(0,))


def kda_decode_workload() -> Dict[str, object]:
    """The KDA decode workload: 256 sequences x 1 token, Hk=16, Hv=32,
    Dk=Dv=128, bf16 q/k/v, a 512-slot f32 state pool ~ N(0, 0.05), gate in
    the kernel, q/k L2 normalised."""
    return dict(name="kda_decode_b256_hk16_hv32_d128", dims=QWEN_DIMS, seqlens=(1,) * 256, num_slots=512,
                qkv_dtype="bf16", state_dtype="f32", seed=1008, has_init=None)


def mamba2_inputs(H: int, P: int, G: int, N: int, seqlens: Sequence[int], num_slots: int, act_dtype: str,
                  state_dtype: str, seed: int, D_mode: str = "h", with_z: bool = True, init_std: float = 0.1,
                  has_init: Optional[Sequence[int]] = None, null_rows: int = 0) -> Dict[str, np.ndarray]:
    """Inputs of the Mamba2 / SSD layer (no page gives a workload; these
    follow the layer's usual initialisation).  x, z [T, H, P] and B, C
    [T, G, N] ~ N(0, 1) in ``act_dtype``; the raw step dt [T, H] ~ N(0, 0.5^2)
    in ``act_dtype`` with dt_bias [H] = softplus^-1(u), u log-uniform in
    [0.001, 0.1]; A = -exp(A_log), A_log ~ U(0, ln 16); D [H] (or [H, P]) ~
    N(0, 1); the state pool ~ N(0, init_std^2).  Each sequence (or decode row,
    one token each) gets a distinct slot; ``null_rows`` decode rows get -1."""
    rng = np.random.default_rng(seed)
    T = int(sum(seqlens))
    Ns = len(seqlens)
    out: Dict[str, np.ndarray] = {}
    out["x"] = _normal(rng, (T, H, P), 1.0, act_dtype)
    out["z"] = _normal(rng, (T, H, P), 1.0, act_dtype) if with_z else None
    out["B"] = _normal(rng, (T, G, N), 1.0, act_dtype)
    out["C"] = _normal(rng, (T, G, N), 1.0, act_dtype)
    out["dt"] = _normal(rng, (T, H), 0.5, act_dtype)
    u = np.exp(rng.uniform(math.log(0.001), math.log(0.1), size=H))
    out["dt_bias"] = np.log(np.expm1(u)).astype(np.float32)
    out["A"] = (-np.exp(rng.uniform(0.0, math.log(16.0), size=H))).astype(np.float32)
    if D_mode == "h":
        out["D"] = rng.standard_normal(H).astype(np.float32)
    elif D_mode == "hp":
        out["D"] = rng.standard_normal((H, P)).astype(np.float32)
    else:
        out["D"] = None
    out["ssm_pool"] = _normal(rng, (num_slots, H, P, N), init_std, state_dtype)
    out["cu"] = np.concatenate([[0], np.cumsum(seqlens)]).astype(np.int32)
    slots = rng.permutation(num_slots)[:Ns].astype(np.int32)
    if null_rows:
        slots[rng.choice(Ns, size=null_rows, replace=False)] = -1
    out["slots"] = slots
    out["has_init"] = np.ones(Ns, np.uint8) if has_init is None else np.asarray(has_init, np.uint8)
    return out


def mamba2_prefill_workload() -> Dict[str, object]:
    """The Mamba2 prefill workload: one 4096-token sequence, H=64 heads of
    P=64, G=8 groups, N=128; bf16 activations, f32 state from zero, z gate
    and D per head."""
    return dict(name="mamba2_prefill_T4096_h64_p64_g8_n128", H=64, P=64, G=8, N=128, seqlens=(4096,),
                num_slots=1, act="bf16", state="f32", seed=1009, has_init=(0,))


def mamba2_decode_workload() -> Dict[str, object]:
    """The Mamba2 decode workload: 256 rows x 1 token at the same shapes
    against a 512-slot f32 pool ~ N(0, 0.1^2)."""
    return dict(name="mamba2_decode_b256_h64_p64_g8_n128", H=64, P=64, G=8, N=128, seqlens=(1,) * 256,
                num_slots=512, act="bf16", state="f32", seed=1010, has_init=None)
