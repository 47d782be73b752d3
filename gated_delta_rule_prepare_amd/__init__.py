"""Python binding of the GDN prepare / decode / prefill library (libgdn.so).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in ``include/gdn.h``.  PyTorch supplies
device memory and the current HIP stream.  If the library is not built, the
first call raises; there is no fallback path.

Function names follow the C ABI: :func:`gdn_prepare`, :func:`gdn_decode`, :func:`gdn_decode_gated`,
:func:`gdn_decode_spec`, :func:`gdn_gated_rmsnorm`, :func:`gdn_kda_recurrent`,
:func:`gdn_kda_prefill_varlen`, :func:`gdn_kda_prefill_workspace_size`, :func:`gdn_mamba2_state_update`,
:func:`gdn_mamba2_chunk_scan`, :func:`gdn_mamba2_workspace_size`,
:func:`gdn_prefill_varlen`, :func:`gdn_prefill_workspace_size`, :func:`gdn_prefill_varlen_noalloc`.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

GDN_F32, GDN_BF16, GDN_F16 = 0, 1, 2
_STATUS = {0: "ok", 1: "invalid argument", 2: "shape mismatch", 3: "bad slot index", 4: "unsupported dtype",
           5: "workspace too small", 6: "device error"}


class GdnError(RuntimeError):
    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn} failed ({_STATUS.get(status, status)}): {message}")
        self.status = status
        self.message = message


class _Dims(ctypes.Structure):
    _fields_ = [("num_k_heads", ctypes.c_int32), ("num_v_heads", ctypes.c_int32),
                ("head_k_dim", ctypes.c_int32), ("head_v_dim", ctypes.c_int32),
                ("conv_kernel", ctypes.c_int32), ("conv_state_len", ctypes.c_int32)]


class _SsmDims(ctypes.Structure):
    _fields_ = [("num_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("num_groups", ctypes.c_int32),
                ("state_dim", ctypes.c_int32)]


class _SsmDt(ctypes.Structure):
    _fields_ = [("dt_bias", ctypes.c_void_p), ("softplus", ctypes.c_int32), ("dt_min", ctypes.c_float),
                ("dt_max", ctypes.c_float)]


@dataclass(frozen=True)
class Dims:
    Hk: int
    Hv: int
    Dk: int
    Dv: int
    K: int

    @property
    def Cc(self) -> int:
        return 2 * self.Hk * self.Dk + self.Hv * self.Dv

    def c(self, conv_pool=None) -> _Dims:
        """The C struct; the conv-history row length is taken from a 3-D
        conv pool [S, Cc, W] (0, meaning K-1, otherwise)."""
        W = int(conv_pool.shape[-1]) if conv_pool is not None and conv_pool.dim() == 3 else 0
        return _Dims(self.Hk, self.Hv, self.Dk, self.Dv, self.K, W)


_lib = None
EXPORTS = ("gdn_prepare", "gdn_decode", "gdn_decode_gated", "gdn_decode_spec", "gdn_prefill_varlen",
           "gdn_prefill_workspace_size", "gdn_prefill_varlen_noalloc", "gdn_gated_rmsnorm", "gdn_kda_recurrent",
           "gdn_kda_prefill_varlen", "gdn_kda_prefill_workspace_size", "gdn_mamba2_state_update",
           "gdn_mamba2_chunk_scan", "gdn_mamba2_workspace_size", "gdn_status_string", "gdn_last_error", "gdn_version")


def load_library():
    """Load libgdn.so and declare the C signatures.  Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"libgdn.so is not built ({LIB_PATH}); run __graft_entry__.build() or "
                           "python gated_delta_rule_prepare_amd/build.py")
    lib = ctypes.CDLL(LIB_PATH)
    P, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    D = ctypes.POINTER(_Dims)
    lib.gdn_prepare.argtypes = [D, i32, i64, P, P, P, i64, P, i64, P, i64, i32, P, P, P, P, i32, P, P, P, i32,
                                P, P, P, i32, P, P, P]
    lib.gdn_decode.argtypes = [D, i32, P, i64, P, i64, P, i64, i32, P, P, P, P, P, i32, i32, P, P, f32, P, P]
    lib.gdn_decode_gated.argtypes = [D, i32, P, i64, P, i64, P, i64, i32, P, P, P, P, P, i32, i32, P, P, f32,
                                     P, i64, P, f32, i32, P, P]
    lib.gdn_decode_spec.argtypes = [D, i32, i64, P, P, P, i64, P, i64, P, i64, i32, P, P, P, P, P, i32, i32, i32,
                                    P, P, P, P, f32, P, P]
    lib.gdn_kda_recurrent.argtypes = [D, i32, i64, P, P, P, P, P, i32, P, P, P, P, P, i32, i32, P, P, P, f32, i32,
                                      P, P]
    lib.gdn_kda_prefill_varlen.argtypes = [D, i32, i64, P, P, P, P, P, i32, P, P, P, P, P, i32, i32, P, P, P, f32,
                                           i32, i32, P, P, sz, P]
    lib.gdn_kda_prefill_workspace_size.argtypes = [D, i32, i64, i32, i32]
    lib.gdn_kda_prefill_workspace_size.restype = sz
    SD, ST = ctypes.POINTER(_SsmDims), ctypes.POINTER(_SsmDt)
    lib.gdn_mamba2_state_update.argtypes = [SD, i32, P, P, P, P, P, P, i32, P, ST, i32, P, i32, i32, P, P, P, P]
    lib.gdn_mamba2_chunk_scan.argtypes = [SD, i32, i64, P, P, P, P, P, P, P, P, i32, P, ST, i32, P, i32, i32, P, P,
                                          P, P, P, sz, P]
    lib.gdn_mamba2_workspace_size.argtypes = [SD, i32, i64]
    lib.gdn_mamba2_workspace_size.restype = sz
    lib.gdn_gated_rmsnorm.argtypes = [i32, i32, i32, P, P, i64, P, f32, i32, P, i32, P]
    lib.gdn_prefill_varlen.argtypes = [D, i32, i64, P, P, P, P, P, i32, P, P, P, i32, i32, P, P, P, f32, i32,
                                       i32, P, P, sz, P]
    lib.gdn_prefill_workspace_size.argtypes = [D, i32, i64, i32]
    lib.gdn_prefill_workspace_size.restype = sz
    lib.gdn_prefill_varlen_noalloc.argtypes = [D, i32, i64, P, P, P, P, P, i32, P, P, P, i32, i32, P, P, P, f32,
                                               i32, i32, P, P]
    for fn in ("gdn_prepare", "gdn_decode", "gdn_decode_gated", "gdn_decode_spec", "gdn_prefill_varlen",
               "gdn_prefill_varlen_noalloc",
               "gdn_gated_rmsnorm", "gdn_kda_recurrent", "gdn_kda_prefill_varlen", "gdn_mamba2_state_update",
               "gdn_mamba2_chunk_scan"):
        getattr(lib, fn).restype = ctypes.c_int
    lib.gdn_status_string.argtypes = [ctypes.c_int]
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_last_error.argtypes = []
    lib.gdn_last_error.restype = ctypes.c_char_p
    lib.gdn_version.restype = i32
    _lib = lib
    return lib


def _check(fn: str, status: int):
    if status != 0:
        raise GdnError(fn, status, _lib.gdn_last_error().decode())


def _dtype_code(t) -> int:
    import torch
    return {torch.float32: GDN_F32, torch.bfloat16: GDN_BF16, torch.float16: GDN_F16}[t.dtype]


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _host_i32(a) -> Optional[np.ndarray]:
    if a is None:
        return None
    if hasattr(a, "detach"):
        a = a.detach().cpu().numpy()
    return np.ascontiguousarray(a, dtype=np.int32)


def _hptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _stream(stream) -> Optional[int]:
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _workspace(nbytes: int, device, stream):
    """A uint8 scratch tensor owned by the stream the kernels run on: torch's
    caching allocator hands a freed block back only to later work on the
    stream it was allocated on, so the block is not reused while the kernels
    enqueued on ``stream`` may still read it."""
    import torch
    if stream is None:
        return torch.empty(nbytes, dtype=torch.uint8, device=device)
    with torch.cuda.stream(stream):
        return torch.empty(nbytes, dtype=torch.uint8, device=device)


def gdn_prepare(dims: Dims, cu_seqlens, mixed_qkv, a_raw, b_raw, conv_weight, A_log, dt_bias, conv_state_pool,
                q_out, k_out, v_out, g_out, beta_out, slot_idx=None, has_initial_state=None,
                apply_qk_l2norm: bool = True, cu_seqlens_host=None, slot_idx_host=None, stream=None) -> None:
    """Varlen prepare step; writes q/k/v/g/beta and updates the conv pool in place.

    ``cu_seqlens`` and ``slot_idx`` are int32 device tensors; their host copies
    are taken from ``*_host`` if given, else copied from the device tensors.
    """
    lib = load_library()
    cu_h = _host_i32(cu_seqlens_host if cu_seqlens_host is not None else cu_seqlens)
    sl_h = _host_i32(slot_idx_host if slot_idx_host is not None else slot_idx)
    n = int(cu_h.size - 1)
    T = int(cu_h[-1]) if n > 0 else 0
    st = lib.gdn_prepare(ctypes.byref(dims.c(conv_state_pool)), n, T, _hptr(cu_h), _ptr(cu_seqlens), _ptr(mixed_qkv),
                         mixed_qkv.stride(0), _ptr(a_raw), a_raw.stride(0), _ptr(b_raw), b_raw.stride(0),
                         _dtype_code(mixed_qkv), _ptr(conv_weight), _ptr(A_log), _ptr(dt_bias),
                         _ptr(conv_state_pool), conv_state_pool.shape[0] if conv_state_pool is not None else 0,
                         _hptr(sl_h), _ptr(slot_idx), _ptr(has_initial_state), int(apply_qk_l2norm),
                         _ptr(q_out), _ptr(k_out), _ptr(v_out), _dtype_code(q_out), _ptr(g_out), _ptr(beta_out),
                         _stream(stream))
    _check("gdn_prepare", st)


def gdn_decode(dims: Dims, mixed_qkv, a_raw, b_raw, conv_weight, A_log, dt_bias, conv_state_pool, ssm_state_pool,
               slot_idx, out, scale: float, slot_idx_host=None, validate: bool = True, stream=None) -> None:
    """Fused decode step for ``mixed_qkv.shape[0]`` rows; pools updated in place.

    With ``validate`` the slot indices are checked on the host (a host copy is
    made from ``slot_idx`` unless ``slot_idx_host`` is given)."""
    lib = load_library()
    sl_h = None
    if validate:
        sl_h = _host_i32(slot_idx_host if slot_idx_host is not None else slot_idx)
    st = lib.gdn_decode(ctypes.byref(dims.c(conv_state_pool)), mixed_qkv.shape[0], _ptr(mixed_qkv), mixed_qkv.stride(0),
                        _ptr(a_raw), a_raw.stride(0), _ptr(b_raw), b_raw.stride(0), _dtype_code(mixed_qkv),
                        _ptr(conv_weight), _ptr(A_log), _ptr(dt_bias), _ptr(conv_state_pool),
                        _ptr(ssm_state_pool), _dtype_code(ssm_state_pool), ssm_state_pool.shape[0],
                        _ptr(slot_idx), _hptr(sl_h), float(scale), _ptr(out), _stream(stream))
    _check("gdn_decode", st)


def gdn_decode_gated(dims: Dims, mixed_qkv, a_raw, b_raw, conv_weight, A_log, dt_bias, conv_state_pool,
                     ssm_state_pool, slot_idx, z, norm_weight, out, scale: float, eps: float,
                     sigmoid_gate: bool = False, slot_idx_host=None, validate: bool = True, stream=None) -> None:
    """gdn_decode with the gated RMS norm epilogue fused.  ``z`` is a 2-D
    view [B, >= Hv*Dv] with unit column stride (for example the z columns of
    a packed [q|k|v|z] row); row b head h sits at z[b, h*Dv:(h+1)*Dv]."""
    lib = load_library()
    sl_h = None
    if validate:
        sl_h = _host_i32(slot_idx_host if slot_idx_host is not None else slot_idx)
    if z.stride(-1) != 1:
        raise ValueError("z must have unit column stride")
    st = lib.gdn_decode_gated(ctypes.byref(dims.c(conv_state_pool)), mixed_qkv.shape[0], _ptr(mixed_qkv), mixed_qkv.stride(0),
                              _ptr(a_raw), a_raw.stride(0), _ptr(b_raw), b_raw.stride(0), _dtype_code(mixed_qkv),
                              _ptr(conv_weight), _ptr(A_log), _ptr(dt_bias), _ptr(conv_state_pool),
                              _ptr(ssm_state_pool), _dtype_code(ssm_state_pool), ssm_state_pool.shape[0],
                              _ptr(slot_idx), _hptr(sl_h), float(scale), _ptr(z), z.stride(0), _ptr(norm_weight),
                              float(eps), int(bool(sigmoid_gate)), _ptr(out), _stream(stream))
    _check("gdn_decode_gated", st)


def gdn_decode_spec(dims: Dims, cu_seqlens, mixed_qkv, a_raw, b_raw, conv_weight, A_log, dt_bias, conv_state_pool,
                    ssm_state_pool, state_idx, num_accepted, out, scale: float, cu_seqlens_host=None,
                    state_idx_host=None, num_accepted_host=None, validate: bool = True, stream=None) -> None:
    """Speculative multi-token decode; pools updated in place.

    ``conv_state_pool`` is [S, Cc, W] with W >= (K-1) + (C-1); ``state_idx``
    [N, C] and ``num_accepted`` [N] are int32 device tensors, ``cu_seqlens``
    [N+1] too (its host copy is always taken).  With ``validate`` the slot
    table is checked on the host (copies are made from the device tensors
    unless the ``*_host`` arrays are given)."""
    lib = load_library()
    if conv_state_pool.dim() != 3 or state_idx.dim() != 2:
        raise ValueError("conv_state_pool must be [S, Cc, W] and state_idx [N, C]")
    cu_h = _host_i32(cu_seqlens_host if cu_seqlens_host is not None else cu_seqlens)
    si_h = na_h = None
    if validate:
        si_h = _host_i32(state_idx_host if state_idx_host is not None else state_idx)
        na_h = _host_i32(num_accepted_host if num_accepted_host is not None else num_accepted)
    n = int(cu_h.size - 1)
    T = int(cu_h[-1]) if n > 0 else 0
    st = lib.gdn_decode_spec(ctypes.byref(dims.c(conv_state_pool)), n, T, _hptr(cu_h), _ptr(cu_seqlens),
                             _ptr(mixed_qkv), mixed_qkv.stride(0), _ptr(a_raw), a_raw.stride(0), _ptr(b_raw),
                             b_raw.stride(0), _dtype_code(mixed_qkv), _ptr(conv_weight), _ptr(A_log), _ptr(dt_bias),
                             _ptr(conv_state_pool), _ptr(ssm_state_pool), _dtype_code(ssm_state_pool),
                             ssm_state_pool.shape[0], state_idx.shape[1], _ptr(state_idx), _ptr(num_accepted),
                             _hptr(si_h), _hptr(na_h), float(scale), _ptr(out), _stream(stream))
    _check("gdn_decode_spec", st)


def gdn_gated_rmsnorm(x, z, weight, out, eps: float, sigmoid_gate: bool = False, stream=None) -> None:
    """Gated RMS norm of the output rows: x and out [T, Hv, Dv]; ``z`` a 2-D
    view [T, >= Hv*Dv] with unit column stride; weight [Dv].  out may be x."""
    lib = load_library()
    if z.stride(-1) != 1:
        raise ValueError("z must have unit column stride")
    T, Hv, Dv = x.shape
    st = lib.gdn_gated_rmsnorm(T, Hv, Dv, _ptr(x), _ptr(z), z.stride(0), _ptr(weight), float(eps),
                               int(bool(sigmoid_gate)), _ptr(out), _dtype_code(x), _stream(stream))
    _check("gdn_gated_rmsnorm", st)


def gdn_prefill_workspace_size(dims: Dims, num_seqs: int, total_tokens: int, chunk_size: int = 64) -> int:
    lib = load_library()
    return int(lib.gdn_prefill_workspace_size(ctypes.byref(dims.c()), num_seqs, total_tokens, chunk_size))


def gdn_prefill_varlen(dims: Dims, cu_seqlens, q, k, v, g, beta, ssm_state_pool, out, scale: float,
                       slot_idx=None, has_initial_state=None, use_qk_l2norm: bool = False, chunk_size: int = 64,
                       workspace=None, cu_seqlens_host=None, slot_idx_host=None, stream=None) -> None:
    """Chunked varlen prefill; the pool slot of each sequence is its initial
    and final state.  ``workspace`` (a uint8 device tensor) is allocated here
    with torch if not given."""
    lib = load_library()
    cu_h = _host_i32(cu_seqlens_host if cu_seqlens_host is not None else cu_seqlens)
    sl_h = _host_i32(slot_idx_host if slot_idx_host is not None else slot_idx)
    n = int(cu_h.size - 1)
    T = int(cu_h[-1]) if n > 0 else 0
    need = gdn_prefill_workspace_size(dims, n, T, chunk_size)
    if workspace is None and need > 0:
        workspace = _workspace(need, q.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.gdn_prefill_varlen(ctypes.byref(dims.c()), n, T, _hptr(cu_h), _ptr(cu_seqlens), _ptr(q), _ptr(k),
                                _ptr(v), _dtype_code(q), _ptr(g), _ptr(beta), _ptr(ssm_state_pool),
                                _dtype_code(ssm_state_pool), ssm_state_pool.shape[0], _hptr(sl_h), _ptr(slot_idx),
                                _ptr(has_initial_state), float(scale), int(use_qk_l2norm), int(chunk_size),
                                _ptr(out), _ptr(workspace), ws_bytes, _stream(stream))
    _check("gdn_prefill_varlen", st)


def gdn_prefill_varlen_noalloc(dims: Dims, cu_seqlens, q, k, v, g, beta, ssm_state_pool, out, scale: float,
                               slot_idx=None, has_initial_state=None, use_qk_l2norm: bool = False,
                               chunk_size: int = 64, cu_seqlens_host=None, slot_idx_host=None, stream=None) -> None:
    """:func:`gdn_prefill_varlen` on the library's static device scratch: no
    device memory is allocated, here or in the library.  Pass the host copies
    of ``cu_seqlens`` and ``slot_idx`` to avoid a device-to-host copy."""
    lib = load_library()
    cu_h = _host_i32(cu_seqlens_host if cu_seqlens_host is not None else cu_seqlens)
    sl_h = _host_i32(slot_idx_host if slot_idx_host is not None else slot_idx)
    n = int(cu_h.size - 1)
    T = int(cu_h[-1]) if n > 0 else 0
    st = lib.gdn_prefill_varlen_noalloc(ctypes.byref(dims.c()), n, T, _hptr(cu_h), _ptr(cu_seqlens), _ptr(q),
                                        _ptr(k), _ptr(v), _dtype_code(q), _ptr(g), _ptr(beta), _ptr(ssm_state_pool),
                                        _dtype_code(ssm_state_pool), ssm_state_pool.shape[0], _hptr(sl_h),
                                        _ptr(slot_idx), _ptr(has_initial_state), float(scale), int(use_qk_l2norm),
                                        int(chunk_size), _ptr(out), _stream(stream))
    _check("gdn_prefill_varlen_noalloc", st)


def gdn_kda_recurrent(dims: Dims, cu_seqlens, q, k, v, g, beta, ssm_state_pool, out, scale: float, A_log=None,
                      dt_bias=None, slot_idx=None, has_initial_state=None, use_qk_l2norm: bool = False,
                      cu_seqlens_host=None, slot_idx_host=None, stream=None) -> None:
    """KDA token by token over varlen sequences (empty ones allowed); the
    pool slot of each sequence is its initial and final state.  g [T, Hv, Dk]
    f32 is the log-decay, or the gate's input when ``A_log`` is given."""
    lib = load_library()
    cu_h = _host_i32(cu_seqlens_host if cu_seqlens_host is not None else cu_seqlens)
    sl_h = _host_i32(slot_idx_host if slot_idx_host is not None else slot_idx)
    n = int(cu_h.size - 1)
    T = int(cu_h[-1]) if n > 0 else 0
    st = lib.gdn_kda_recurrent(ctypes.byref(dims.c()), n, T, _hptr(cu_h), _ptr(cu_seqlens), _ptr(q), _ptr(k), _ptr(v),
                               _dtype_code(q), _ptr(g), _ptr(A_log), _ptr(dt_bias), _ptr(beta), _ptr(ssm_state_pool),
                               _dtype_code(ssm_state_pool), ssm_state_pool.shape[0], _hptr(sl_h), _ptr(slot_idx),
                               _ptr(has_initial_state), float(scale), int(bool(use_qk_l2norm)), _ptr(out),
                               _stream(stream))
    _check("gdn_kda_recurrent", st)


def gdn_kda_prefill_workspace_size(dims: Dims, num_seqs: int, total_tokens: int, qkv_dtype: int = GDN_BF16,
                                   chunk_size: int = 64) -> int:
    lib = load_library()
    return int(lib.gdn_kda_prefill_workspace_size(ctypes.byref(dims.c()), num_seqs, total_tokens, chunk_size,
                                                  qkv_dtype))


def gdn_kda_prefill_varlen(dims: Dims, cu_seqlens, q, k, v, g, beta, ssm_state_pool, out, scale: float, A_log=None,
                           dt_bias=None, slot_idx=None, has_initial_state=None, use_qk_l2norm: bool = False,
                           chunk_size: int = 64, workspace=None, cu_seqlens_host=None, slot_idx_host=None,
                           stream=None) -> None:
    """Chunked KDA over varlen sequences (empty ones allowed); arguments as
    :func:`gdn_kda_recurrent`.  ``workspace`` (a uint8 device tensor) is
    allocated here with torch if not given."""
    lib = load_library()
    cu_h = _host_i32(cu_seqlens_host if cu_seqlens_host is not None else cu_seqlens)
    sl_h = _host_i32(slot_idx_host if slot_idx_host is not None else slot_idx)
    n = int(cu_h.size - 1)
    T = int(cu_h[-1]) if n > 0 else 0
    need = gdn_kda_prefill_workspace_size(dims, n, T, _dtype_code(q), chunk_size)
    if workspace is None and need > 0:
        workspace = _workspace(need, q.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.gdn_kda_prefill_varlen(ctypes.byref(dims.c()), n, T, _hptr(cu_h), _ptr(cu_seqlens), _ptr(q), _ptr(k),
                                    _ptr(v), _dtype_code(q), _ptr(g), _ptr(A_log), _ptr(dt_bias), _ptr(beta),
                                    _ptr(ssm_state_pool), _dtype_code(ssm_state_pool), ssm_state_pool.shape[0],
                                    _hptr(sl_h), _ptr(slot_idx), _ptr(has_initial_state), float(scale),
                                    int(bool(use_qk_l2norm)), int(chunk_size), _ptr(out), _ptr(workspace), ws_bytes,
                                    _stream(stream))
    _check("gdn_kda_prefill_varlen", st)


def _ssm(x, B, dt_bias, dt_softplus, dt_min, dt_max):
    H, P = x.shape[1], x.shape[2]
    G, N = B.shape[1], B.shape[2]
    d = _SsmDims(H, P, G, N)
    t = _SsmDt(_ptr(dt_bias), int(bool(dt_softplus)), float(dt_min), float(dt_max))
    return d, t


def gdn_mamba2_state_update(x, dt, A, B, C, state_pool, slot_idx, out, D=None, z=None, dt_bias=None,
                            dt_softplus: bool = True, dt_min: float = 0.0, dt_max: float = float("inf"),
                            slot_idx_host=None, validate: bool = True, stream=None) -> None:
    """One Mamba2 / SSD step per row: x, z, out [B, H, P]; dt [B, H]; A [H];
    B, C [B, G, N]; D [H] or [H, P]; the pool [S, H, P, N] is updated in place."""
    lib = load_library()
    sl_h = _host_i32(slot_idx_host if slot_idx_host is not None else slot_idx) if validate else None
    d, t = _ssm(x, B, dt_bias, dt_softplus, dt_min, dt_max)
    st = lib.gdn_mamba2_state_update(ctypes.byref(d), x.shape[0], _ptr(x), _ptr(dt), _ptr(A), _ptr(B), _ptr(C),
                                     _ptr(D), int(D is not None and D.dim() == 2), _ptr(z), ctypes.byref(t),
                                     _dtype_code(x), _ptr(state_pool), _dtype_code(state_pool), state_pool.shape[0],
                                     _ptr(slot_idx), _hptr(sl_h), _ptr(out), _stream(stream))
    _check("gdn_mamba2_state_update", st)


def gdn_mamba2_workspace_size(num_heads: int, head_dim: int, state_dim: int, num_seqs: int, total_tokens: int,
                              num_groups: int = 1) -> int:
    lib = load_library()
    d = _SsmDims(num_heads, head_dim, num_groups, state_dim)
    return int(lib.gdn_mamba2_workspace_size(ctypes.byref(d), num_seqs, total_tokens))


def gdn_mamba2_chunk_scan(cu_seqlens, x, dt, A, B, C, state_pool, out, D=None, z=None, dt_bias=None,
                          dt_softplus: bool = True, dt_min: float = 0.0, dt_max: float = float("inf"), slot_idx=None,
                          has_initial_state=None, workspace=None, cu_seqlens_host=None, slot_idx_host=None,
                          stream=None) -> None:
    """Chunked Mamba2 / SSD over varlen sequences; the pool slot of each
    sequence is its initial and final state.  ``workspace`` (uint8 device
    tensor) is allocated here with torch if not given."""
    lib = load_library()
    cu_h = _host_i32(cu_seqlens_host if cu_seqlens_host is not None else cu_seqlens)
    sl_h = _host_i32(slot_idx_host if slot_idx_host is not None else slot_idx)
    n = int(cu_h.size - 1)
    T = int(cu_h[-1]) if n > 0 else 0
    d, t = _ssm(x, B, dt_bias, dt_softplus, dt_min, dt_max)
    need = int(lib.gdn_mamba2_workspace_size(ctypes.byref(d), n, T))
    if workspace is None and need > 0:
        workspace = _workspace(need, x.device, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = lib.gdn_mamba2_chunk_scan(ctypes.byref(d), n, T, _hptr(cu_h), _ptr(cu_seqlens), _ptr(x), _ptr(dt), _ptr(A),
                                   _ptr(B), _ptr(C), _ptr(D), int(D is not None and D.dim() == 2), _ptr(z),
                                   ctypes.byref(t), _dtype_code(x), _ptr(state_pool), _dtype_code(state_pool),
                                   state_pool.shape[0], _hptr(sl_h), _ptr(slot_idx), _ptr(has_initial_state),
                                   _ptr(out), _ptr(workspace), ws_bytes, _stream(stream))
    _check("gdn_mamba2_chunk_scan", st)
