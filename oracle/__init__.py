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
* :func:`decode_spec` -- speculative multi-token decode: the widened-window
  conv update, prepare, and the recurrence with a state snapshot per token.
* :func:`kda`      -- the KDA variant (one log-decay per key channel), with
  its optional gate, against the slot-indexed pool.
* :func:`mamba2`   -- Mamba2 / SSD (no delta term; a scalar decay per head,
  B and C shared by head groups), prefill or decode, against a slot pool.

Conv history pools are [S, Cc, W] with W >= K-1 taps per channel.  W = K-1 is
the ordinary layout; a wider row (speculative decoding keeps
(K-1) + (max_query_len-1) taps) is used by the non-speculative steps through
its leading K-1 taps only, the rest left as it is (vllm.cpp cpu_ops.cpp,
CausalConv1dUpdateKernel and GdnStateGatherKernel / GdnStateScatterKernel on
widened rows).

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
    lib.gdn_oracle_kda_recurrence.argtypes = [i32, i32, i32, i32, i32, P, P, P, P, P, P, f64, i32, f64,
                                              P, P, P, P, i32]
    lib.gdn_oracle_kda_gate.argtypes = [i64, i32, i32, P, P, P, P]
    lib.gdn_oracle_mamba2.argtypes = [i32, i32, i32, i32, i32, P, P, P, P, P, P, P, i32, P, P, P, P, P, i32]
    lib.gdn_oracle_mamba2_dt.argtypes = [i64, i32, P, P, i32, f64, f64, P]
    for fn in (lib.gdn_oracle_conv_silu, lib.gdn_oracle_split_l2, lib.gdn_oracle_gates,
               lib.gdn_oracle_recurrence, lib.gdn_oracle_round, lib.gdn_oracle_gated_rmsnorm,
               lib.gdn_oracle_kda_recurrence, lib.gdn_oracle_kda_gate, lib.gdn_oracle_mamba2,
               lib.gdn_oracle_mamba2_dt):
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
    """Round values to ``dtype`` (RNE, directly from double); "f64" keeps them."""
    x = _f64(x)
    if dtype == "f64":
        return x.copy()
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


def _silu(z):
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def conv_spec(x, w, cu, rows, num_accepted):
    """Speculative multi-token conv update + SiLU, per request i with tokens
    cu[i] .. cu[i+1]-1 ([P1] CausalConv1dSpecUpdateKernel).

    rows [N, Cc, W] is each request's widened conv row.  With off =
    num_accepted[i] - 1 and L the request's token count, the stream the conv
    reads is the K-1 taps of the row starting at tap off, followed by the L
    inputs; token t's pre-activation is the K-tap product of w with stream
    positions t .. t+K-1.  The row then becomes its taps off+1 .. off+W-L
    followed by the L inputs.  A tap index past the row's end reads as zero.
    Returns (y [T, Cc], rows_out [N, Cc, W])."""
    x, w = _f64(x), _f64(w)
    cu = np.asarray(cu, dtype=np.int64)
    nat = np.asarray(num_accepted, dtype=np.int64)
    N = cu.size - 1
    Cc, K = w.shape
    rows = _f64(rows)
    assert rows.shape[:2] == (N, Cc)
    W = rows.shape[2]
    y = np.zeros((x.shape[0], Cc))
    rows_out = rows.copy()
    zero = np.zeros(Cc)
    for i in range(N):
        lo, hi = int(cu[i]), int(cu[i + 1])
        L = hi - lo
        if L == 0:
            continue
        assert L <= W, "the widened row must hold at least the request's tokens"
        off = int(nat[i]) - 1
        row = rows[i]

        def tap(j):
            return row[:, j] if j < W else zero

        stream = np.stack([tap(off + j) for j in range(K - 1)] + [x[lo + t] for t in range(L)], axis=1)
        for t in range(L):
            y[lo + t] = _silu(np.sum(w * stream[:, t:t + K], axis=1))
        keep = W - L
        rows_out[i] = np.stack([tap(off + 1 + j) for j in range(keep)] + [x[lo + t] for t in range(L)], axis=1)
    return y, rows_out


def _conv_pool(dims, conv_pool) -> np.ndarray:
    """The conv pool as [S, Cc, W] f64 (W >= K-1 taps per channel)."""
    pool = _f64(conv_pool)
    if pool.ndim != 3:
        pool = pool.reshape(pool.shape[0], dims.Cc, -1)
    assert pool.shape[2] >= dims.K - 1
    return pool


def kda_gate(g_raw, A_log, dt_bias=None):
    """KDA gate per (token, value head, key channel):
    g = -exp(A_log[h]) softplus(g_raw + dt_bias[h, d]); g_raw [T, Hv, Dk],
    dt_bias [Hv, Dk] or None.  [P1] KdaChunkPrefillKernel."""
    g_raw, A_log = _f64(g_raw), _f64(A_log)
    T, Hv, Dk = g_raw.shape
    db = None if dt_bias is None else _f64(dt_bias).reshape(Hv, Dk)
    g = np.empty_like(g_raw)
    _load().gdn_oracle_kda_gate(T, Hv, Dk, _ptr(g_raw), _ptr(A_log), None if db is None else _ptr(db), _ptr(g))
    return g


def kda_recurrence(q, k, v, g, beta, cu, state_in, has_init, scale: float, l2norm: bool = False,
                   nthreads: Optional[int] = None):
    """Token-by-token KDA (one log-decay per key channel, g [T, Hv, Dk]).
    q, k [T, Hk, Dk]; v [T, Hv, Dv]; beta [T, Hv]; state_in [N, Hv, Dv, Dk].
    Returns (out [T, Hv, Dv], state_out [N, Hv, Dv, Dk]).  [P1]
    KdaHeadTokenStep, KdaGatedDeltaRuleKernel."""
    q, k, v, g, beta = _f64(q), _f64(k), _f64(v), _f64(g), _f64(beta)
    T, Hk, Dk = q.shape
    Hv, Dv = v.shape[1], v.shape[2]
    assert g.shape == (T, Hv, Dk)
    cu = np.ascontiguousarray(cu, dtype=np.int32)
    N = cu.size - 1
    state_in = _f64(state_in).reshape(N, Hv, Dv, Dk)
    has_init = np.ascontiguousarray(has_init, dtype=np.uint8)
    out = np.empty((T, Hv, Dv))
    state_out = np.empty((N, Hv, Dv, Dk))
    _load().gdn_oracle_kda_recurrence(Hk, Hv, Dk, Dv, N, _ptr(cu), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                      _ptr(beta), float(scale), int(l2norm), EPS, _ptr(state_in),
                                      _ptr(has_init), _ptr(out), _ptr(state_out), nthreads or default_threads())
    return out, state_out


def mamba2_dt(dt_raw, dt_bias=None, softplus: bool = True, dt_min: float = 0.0, dt_max: float = float("inf")):
    """Mamba2 step size dt = clamp(softplus(dt_raw + dt_bias), dt_min, dt_max)
    ([P1] Mamba2ChunkScanKernel stage 1).  dt_raw [T, H]."""
    dt_raw = _f64(dt_raw)
    T, H = dt_raw.shape
    db = None if dt_bias is None else _f64(dt_bias)
    out = np.empty_like(dt_raw)
    _load().gdn_oracle_mamba2_dt(T, H, _ptr(dt_raw), None if db is None else _ptr(db), int(softplus),
                                 float(dt_min), float(dt_max), _ptr(out))
    return out


def mamba2_recurrence(x, dt, A, B, C, cu, state_in, has_init, D=None, z=None, nthreads: Optional[int] = None):
    """Token-by-token Mamba2 / SSD.  x [T, H, P]; dt [T, H] (already processed);
    A [H]; B, C [T, G, N]; D [H] or [H, P] or None; z [T, H, P] or None;
    state_in [N_seq, H, P, N].  Returns (out [T, H, P], state_out)."""
    x, dt, A, B, C = _f64(x), _f64(dt), _f64(A), _f64(B), _f64(C)
    T, H, P = x.shape
    G, N = B.shape[1], B.shape[2]
    cu = np.ascontiguousarray(cu, dtype=np.int32)
    Ns = cu.size - 1
    state_in = _f64(state_in).reshape(Ns, H, P, N)
    has_init = np.ascontiguousarray(has_init, dtype=np.uint8)
    Dv = None if D is None else _f64(D)
    zz = None if z is None else _f64(z)
    out = np.empty((T, H, P))
    state_out = np.empty((Ns, H, P, N))
    _load().gdn_oracle_mamba2(H, P, G, N, Ns, _ptr(cu), _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C),
                              None if Dv is None else _ptr(Dv), int(Dv is not None and Dv.ndim == 2),
                              None if zz is None else _ptr(zz), _ptr(state_in), _ptr(has_init), _ptr(out),
                              _ptr(state_out), nthreads or default_threads())
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
    conv_pool = _conv_pool(dims, conv_pool)
    Km1 = dims.K - 1
    hist = conv_pool[slots, :, :Km1]
    y, hist_out = conv_silu(x, w, cu, hist, has_init, nthreads)
    q, k, v = split_l2(y, dims.Hk, dims.Hv, dims.Dk, dims.Dv, l2norm)
    g, beta = gates(a, b, A_log, dt_bias)
    new_pool = conv_pool.copy()
    if dims.K > 1:
        new_pool[slots, :, :Km1] = hist_out
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
    conv_pool = _conv_pool(dims, conv_pool)
    ssm_pool = _f64(ssm_pool)
    out = np.zeros((B, dims.Hv, dims.Dv))
    live = np.nonzero(slots >= 0)[0]
    new_conv, new_ssm = conv_pool.copy(), ssm_pool.copy()
    if live.size:
        ls = slots[live]
        n = live.size
        cu = np.arange(n + 1, dtype=np.int32)
        ones = np.ones(n, np.uint8)
        hist = conv_pool[ls, :, :dims.K - 1]
        y, hist_out = conv_silu(_f64(x)[live], w, cu, hist, ones, nthreads)
        q, k, v = split_l2(y, dims.Hk, dims.Hv, dims.Dk, dims.Dv, True)
        g, beta = gates(_f64(a)[live], _f64(b)[live], A_log, dt_bias)
        o, st = recurrence(q, k, v, g, beta, cu, ssm_pool[ls], ones, scale, False, nthreads)
        out[live] = o
        if dims.K > 1:
            new_conv[ls, :, :dims.K - 1] = hist_out
        new_ssm[ls] = round_to(st, state_dtype)
    return round_to(out, out_dtype), new_conv, new_ssm


def decode_spec(dims, cu, x, w, a, b, A_log, dt_bias, conv_pool, ssm_pool, state_idx, num_accepted,
                scale: float, state_dtype: str = "f32", out_dtype: str = "f32",
                nthreads: Optional[int] = None):
    """Speculative multi-token decode ([P1] CausalConv1dSpecUpdateKernel,
    GdnSpecDecodeKernel; [P2] the speculative part of
    ValidateGdnAttentionMetadata).

    Request i has tokens cu[i] .. cu[i+1]-1 (L_i of them) and a row of
    C = state_idx.shape[1] state slots.  Its recurrence starts from the state
    in slot state_idx[i, num_accepted[i]-1] (the snapshot taken after the
    last accepted token of the previous step) and, after its token t, the
    state is stored into slot state_idx[i, t] (rounded to ``state_dtype``;
    the running state itself stays unrounded); a -1 column skips that store.
    A request whose initial slot is -1 gets zero outputs and touches neither
    pool.  Its conv row is the widened row of slot state_idx[i, 0] (the pages
    leave the conv slot open; column 0 is the request's fixed slot), updated
    by :func:`conv_spec`.  q/k are L2-normalised as in :func:`decode`.
    Returns (out [T, Hv, Dv], conv_pool, ssm_pool)."""
    cu = np.asarray(cu, dtype=np.int64)
    N = cu.size - 1
    sidx = np.asarray(state_idx, dtype=np.int64).reshape(N, -1)
    nat = np.asarray(num_accepted, dtype=np.int64).reshape(N)
    T = int(cu[-1])
    conv_pool = _conv_pool(dims, conv_pool)
    ssm_pool = _f64(ssm_pool)
    x, a, b = _f64(x), _f64(a), _f64(b)
    out = np.zeros((T, dims.Hv, dims.Dv))
    new_conv, new_ssm = conv_pool.copy(), ssm_pool.copy()
    init = sidx[np.arange(N), nat - 1] if N else np.zeros(0, np.int64)
    live = np.nonzero(init >= 0)[0]
    if live.size == 0:
        return round_to(out, out_dtype), new_conv, new_ssm
    assert np.all(sidx[live, 0] >= 0), "a live request needs its conv slot (column 0)"
    lens = (cu[1:] - cu[:-1])[live]
    toks = np.concatenate([np.arange(cu[i], cu[i + 1]) for i in live])
    cu_l = np.concatenate([[0], np.cumsum(lens)])
    conv_slots = sidx[live, 0]
    y, rows_out = conv_spec(x[toks], w, cu_l, conv_pool[conv_slots], nat[live])
    new_conv[conv_slots] = rows_out
    q, k, v = split_l2(y, dims.Hk, dims.Hv, dims.Dk, dims.Dv, True)
    g, beta = gates(a[toks], b[toks], A_log, dt_bias)
    S = ssm_pool[init[live]]                    # every initial state is read before any store
    o_l = np.zeros((toks.size, dims.Hv, dims.Dv))
    for t in range(int(lens.max())):
        act = np.nonzero(lens > t)[0]           # live requests that have a token t
        tok = cu_l[act] + t
        one = np.arange(act.size + 1, dtype=np.int32)
        o, S_new = recurrence(q[tok], k[tok], v[tok], g[tok], beta[tok], one, S[act],
                              np.ones(act.size, np.uint8), scale, False, nthreads)
        o_l[tok] = o
        S[act] = S_new
        snap = sidx[live[act], t]
        keep = snap >= 0
        new_ssm[snap[keep]] = round_to(S_new[keep], state_dtype)
    out[toks] = o_l
    return round_to(out, out_dtype), new_conv, new_ssm


def kda(dims, cu, q, k, v, g, beta, ssm_pool, slots, has_init, scale: float, A_log=None, dt_bias=None,
        state_dtype: str = "f32", out_dtype: str = "f32", l2norm: bool = False, nthreads: Optional[int] = None):
    """KDA over varlen sequences against the slot-indexed state pool ([P1]
    KdaGatedDeltaRuleKernel; with A_log given, g is the raw gate input and the
    gate of :func:`kda_gate` is applied first, as [P1] KdaChunkPrefillKernel
    does).  Each sequence starts from its slot's state (zero when has_init is
    0) and its final state is written back, rounded to ``state_dtype``; a
    sequence with no tokens writes back its initial state.  With ``l2norm``
    q and k are L2-normalised per (token, key head) first (eps 1e-6).  Returns
    (out rounded to ``out_dtype``, updated pool)."""
    slots = np.asarray(slots, dtype=np.int64)
    ssm_pool = _f64(ssm_pool)
    gg = kda_gate(g, A_log, dt_bias) if A_log is not None else _f64(g)
    out, st = kda_recurrence(q, k, v, gg, beta, cu, ssm_pool[slots], has_init, scale, l2norm, nthreads)
    new_pool = ssm_pool.copy()
    new_pool[slots] = round_to(st, state_dtype)
    return round_to(out, out_dtype), new_pool


def mamba2(cu, x, dt_raw, A, B, C, ssm_pool, slots, has_init, D=None, z=None, dt_bias=None, softplus: bool = True,
           dt_min: float = 0.0, dt_max: float = float("inf"), state_dtype: str = "f32", out_dtype: str = "f32",
           nthreads: Optional[int] = None):
    """Mamba2 / SSD over varlen sequences against a slot-indexed pool [S, H, P, N]
    ([P1] Mamba2ChunkScanKernel, Mamba2StateUpdateKernel): dt processed by
    :func:`mamba2_dt`, then the recurrence; each sequence starts from its
    slot's state (zero when has_init is 0), its final state is written back
    rounded to ``state_dtype``; a slot of -1 (decode rows only) gives zero
    output and touches nothing.  Returns (out rounded to ``out_dtype``, pool)."""
    slots = np.asarray(slots, dtype=np.int64)
    pool = _f64(ssm_pool)
    cu = np.asarray(cu, dtype=np.int64)
    x = _f64(x)
    T, H, P = x.shape
    out = np.zeros((T, H, P))
    new_pool = pool.copy()
    live = np.nonzero(slots >= 0)[0]
    if live.size:
        toks = np.concatenate([np.arange(cu[i], cu[i + 1]) for i in live]).astype(np.int64)
        lens = (cu[1:] - cu[:-1])[live]
        cu_l = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        dt = mamba2_dt(_f64(dt_raw)[toks], dt_bias, softplus, dt_min, dt_max)
        o, st = mamba2_recurrence(x[toks], dt, A, _f64(B)[toks], _f64(C)[toks], cu_l, pool[slots[live]],
                                  np.asarray(has_init, np.uint8)[live], D, None if z is None else _f64(z)[toks],
                                  nthreads)
        out[toks] = o
        new_pool[slots[live]] = round_to(st, state_dtype)
    return round_to(out, out_dtype), new_pool
