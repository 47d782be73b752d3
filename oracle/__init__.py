"""f64 CPU oracle for the gated-delta-rule (GDN) prepare / decode / prefill path.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the CPU-baseline leg of ``bench.py``, never by the library.  It shares
no code with the HIP path; the two meet only in the seeded input generators
(``gdn_inputs``), which hold none of the method's arithmetic.

The arithmetic lives in ``gdn_oracle.c`` (double precision, ``-ffp-contract=off``).
This module only marshals arrays, gathers and scatters pool rows by slot index
and calls the C functions in the order the library's entry points define:

* :func:`prepare`  -- conv + SiLU, split, L2 norm, gates; q/k/v rounded to the
  dtype the library stores them in, g/beta rounded to f32.
* :func:`prefill`  -- the token-by-token recurrence per (sequence, value head);
  out rounded to its dtype, the state rounded once to the pool dtype.
* :func:`decode`   -- prepare + recurrence for one token per row against the
  slot-indexed pools; slot -1 gives a zero output and writes nothing.

Parity pins: every function here is checked in ``tests/test_oracle_pins.py``
against closed forms, invariants, library routines and brute-force algebra.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB_PATH = os.environ.get("GDN_ORACLE_LIB") or os.path.join(_HERE, "libgdn_oracle.so")
_DTYPE_CODE = {"f32": 0, "bf16": 1, "f16": 2}
EPS = 1e-6
_lib = None


def build() -> str:
    """Compile the oracle (gcc, no FMA contraction)."""
    cmd = ["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-std=c11",
           "-o", _LIB_PATH + ".tmp", _SRC, "-lm", "-lpthread"]
    subprocess.run(cmd, check=True)
    os.replace(_LIB_PATH + ".tmp", _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    i64, i32, f64 = ctypes.c_int64, ctypes.c_int, ctypes.c_double
    lib.gdn_oracle_conv_silu.argtypes = [i64, i32, i32, P, P, i64, P, P, P, P, P, i32]
    lib.gdn_oracle_split_l2.argtypes = [i64, i32, i32, i32, i32, P, i32, f64, P, P, P]
    lib.gdn_oracle_gates.argtypes = [i64, i32, P, i64, P, i64, P, P, P, P]
    lib.gdn_oracle_recurrence.argtypes = [i32, i32, i32, i32, i32, P, P, P, P, P, P, f64, i32, f64,
                                          P, P, P, P, i32]
    lib.gdn_oracle_round.argtypes = [P, P, i64, i32]
    lib.gdn_oracle_gated_rmsnorm.argtypes = [i64, i32, P, P, P, f64, i32, P]
    for fn in (lib.gdn_oracle_conv_silu, lib.gdn_oracle_split_l2, lib.gdn_oracle_gates,
               lib.gdn_oracle_recurrence, lib.gdn_oracle_round, lib.gdn_oracle_gated_rmsnorm):
        fn.restype = None
    _lib = lib
    return lib


def default_threads() -> int:
    return int(os.environ.get("GDN_ORACLE_THREADS", os.cpu_count() or 1))


def _f64(x) -> np.ndarray:
    return np.ascontiguousarray(x, dtype=np.float64)


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


# ---------------------------------------------------------------------------
# Thin wrappers over the C functions.
# ---------------------------------------------------------------------------
def round_to(x, dtype: str) -> np.ndarray:
    """Round values to ``dtype`` (RNE, directly from double)."""
    x = _f64(x)
    y = np.empty_like(x)
    _load().gdn_oracle_round(_ptr(x), _ptr(y), x.size, _DTYPE_CODE[dtype])
    return y


def gated_rmsnorm(x, z, w, eps: float, sigmoid_gate: bool = False) -> np.ndarray:
    """Gated RMS norm over the last axis: x / sqrt(mean(x^2) + eps) * w * act(z),
    act = silu (or the logistic function).  x and z have the same shape
    [..., D]; w is [D].  [P1] RmsNormGatedKernel; [P3] gated_rms_norm_f32."""
    x = _f64(x)
    z = _f64(z)
    w = _f64(w)
    D = x.shape[-1]
    assert z.shape == x.shape and w.shape == (D,)
    out = np.empty_like(x)
    _load().gdn_oracle_gated_rmsnorm(x.size // D, D, _ptr(x), _ptr(z), _ptr(w), float(eps), int(sigmoid_gate),
                                     _ptr(out))
    return out


def conv_silu(x, w, cu, hist, has_init, nthreads: Optional[int] = None):
    """Causal depthwise conv + SiLU per sequence.  x [T, Cc], w [Cc, K],
    hist [N, Cc, K-1] (history entering each sequence).  Returns
    (y [T, Cc], hist_out [N, Cc, K-1])."""
    x, w = _f64(x), _f64(w)
    cu = np.ascontiguousarray(cu, dtype=np.int32)
    N = cu.size - 1
    Cc, K = w.shape
    hist = _f64(hist).reshape(N, Cc, K - 1) if K > 1 else np.zeros((N, Cc, 0))
    has_init = np.ascontiguousarray(has_init, dtype=np.uint8)
    y = np.empty((x.shape[0], Cc))
    hist_out = np.empty((N, Cc, K - 1))
    _load().gdn_oracle_conv_silu(Cc, K, N, _ptr(cu), _ptr(x), x.shape[1], _ptr(w), _ptr(hist),
                                 _ptr(has_init), _ptr(y), _ptr(hist_out),
                                 nthreads or default_threads())
    return y, hist_out


def split_l2(y, Hk, Hv, Dk, Dv, l2norm: bool = True):
    """Split conv rows into q, k [T, Hk, Dk] and v [T, Hv, Dv]; L2-normalise q, k."""
    y = _f64(y)
    T = y.shape[0]
    q = np.empty((T, Hk, Dk))
    k = np.empty((T, Hk, Dk))
    v = np.empty((T, Hv, Dv))
    _load().gdn_oracle_split_l2(T, Hk, Hv, Dk, Dv, _ptr(y), int(l2norm), EPS, _ptr(q), _ptr(k), _ptr(v))
    return q, k, v


def gates(a, b, A_log, dt_bias):
    """g = -exp(A_log) softplus(a + dt_bias), beta = sigmoid(b); [T, Hv] each."""
    a, b, A_log, dt_bias = _f64(a), _f64(b), _f64(A_log), _f64(dt_bias)
    T, Hv = a.shape
    g = np.empty((T, Hv))
    beta = np.empty((T, Hv))
    _load().gdn_oracle_gates(T, Hv, _ptr(a), Hv, _ptr(b), Hv, _ptr(A_log), _ptr(dt_bias), _ptr(g), _ptr(beta))
    return g, beta


def recurrence(q, k, v, g, beta, cu, state_in, has_init, scale: float, l2norm: bool = False,
               nthreads: Optional[int] = None):
    """Token-by-token gated delta rule.  q, k [T, Hk, Dk]; v [T, Hv, Dv];
    g, beta [T, Hv]; state_in [N, Hv, Dv, Dk].  Returns (out [T, Hv, Dv],
    state_out [N, Hv, Dv, Dk])."""
    q, k, v, g, beta = _f64(q), _f64(k), _f64(v), _f64(g), _f64(beta)
    T, Hk, Dk = q.shape
    Hv, Dv = v.shape[1], v.shape[2]
    cu = np.ascontiguousarray(cu, dtype=np.int32)
    N = cu.size - 1
    state_in = _f64(state_in).reshape(N, Hv, Dv, Dk)
    has_init = np.ascontiguousarray(has_init, dtype=np.uint8)
    out = np.empty((T, Hv, Dv))
    state_out = np.empty((N, Hv, Dv, Dk))
    _load().gdn_oracle_recurrence(Hk, Hv, Dk, Dv, N, _ptr(cu), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                  _ptr(beta), float(scale), int(l2norm), EPS, _ptr(state_in),
                                  _ptr(has_init), _ptr(out), _ptr(state_out), nthreads or default_threads())
    return out, state_out


# ---------------------------------------------------------------------------
# Compositions matching the library's entry points.
# ---------------------------------------------------------------------------
def prepare(dims, cu, x, w, a, b, A_log, dt_bias, conv_pool, slots, has_init, l2norm: bool = True,
            qkv_dtype: str = "f32", nthreads: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Prepare step for varlen prefill (a1-a4).  Returns q, k, v (rounded to
    ``qkv_dtype``), g, beta (rounded to f32) and the updated conv pool (the
    history rows of ``slots`` replaced by each sequence's last K-1 inputs)."""
    slots = np.asarray(slots, dtype=np.int64)
    conv_pool = _f64(conv_pool)
    hist = conv_pool[slots] if dims.K > 1 else np.zeros((len(slots), dims.Cc, 0))
    y, hist_out = conv_silu(x, w, cu, hist, has_init, nthreads)
    q, k, v = split_l2(y, dims.Hk, dims.Hv, dims.Dk, dims.Dv, l2norm)
    g, beta = gates(a, b, A_log, dt_bias)
    new_pool = conv_pool.copy()
    if dims.K > 1:
        new_pool[slots] = hist_out
    return dict(q=round_to(q, qkv_dtype), k=round_to(k, qkv_dtype), v=round_to(v, qkv_dtype),
                g=round_to(g, "f32"), beta=round_to(beta, "f32"), conv_pool=new_pool)


def prefill(dims, cu, q, k, v, g, beta, ssm_pool, slots, has_init, scale: float, l2norm: bool = False,
            state_dtype: str = "f32", out_dtype: str = "f32", nthreads: Optional[int] = None):
    """Varlen prefill (a6 by its definition, the sequential recurrence).
    The pool slot of each sequence is both its initial and final state.
    Returns (out rounded to ``out_dtype``, updated pool rounded to ``state_dtype``)."""
    slots = np.asarray(slots, dtype=np.int64)
    ssm_pool = _f64(ssm_pool)
    out, st = recurrence(q, k, v, g, beta, cu, ssm_pool[slots], has_init, scale, l2norm, nthreads)
    new_pool = ssm_pool.copy()
    new_pool[slots] = round_to(st, state_dtype)
    return round_to(out, out_dtype), new_pool


def decode(dims, x, w, a, b, A_log, dt_bias, conv_pool, ssm_pool, slots, scale: float,
           state_dtype: str = "f32", out_dtype: str = "f32", nthreads: Optional[int] = None):
    """Fused decode (a1-a5): one token per row, pools indexed by ``slots``.
    q/k/v/g/beta are never stored, so they are not rounded.  Rows with slot
    -1 produce zeros and leave both pools untouched.
    Returns (out [B, Hv, Dv], conv_pool, ssm_pool)."""
    slots = np.asarray(slots, dtype=np.int64)
    B = slots.size
    conv_pool = _f64(conv_pool)
    ssm_pool = _f64(ssm_pool)
    out = np.zeros((B, dims.Hv, dims.Dv))
    live = np.nonzero(slots >= 0)[0]
    new_conv, new_ssm = conv_pool.copy(), ssm_pool.copy()
    if live.size:
        ls = slots[live]
        n = live.size
        cu = np.arange(n + 1, dtype=np.int32)
        ones = np.ones(n, np.uint8)
        hist = conv_pool[ls] if dims.K > 1 else np.zeros((n, dims.Cc, 0))
        y, hist_out = conv_silu(_f64(x)[live], w, cu, hist, ones, nthreads)
        q, k, v = split_l2(y, dims.Hk, dims.Hv, dims.Dk, dims.Dv, True)
        g, beta = gates(_f64(a)[live], _f64(b)[live], A_log, dt_bias)
        o, st = recurrence(q, k, v, g, beta, cu, ssm_pool[ls], ones, scale, False, nthreads)
        out[live] = o
        if dims.K > 1:
            new_conv[ls] = hist_out
        new_ssm[ls] = round_to(st, state_dtype)
    return round_to(out, out_dtype), new_conv, new_ssm
