"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every entry point include/gdn.h declares, and refuses bad arguments with the
right status before any device work (every call below fails its checks, so
the fake device addresses are never touched)."""
import ctypes
import os
import re

import numpy as np
import pytest

import gated_delta_rule_prepare_amd as gdn

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdn.h")
OK, INVALID, SHAPE, INDEX, DTYPE, WORKSPACE = 0, 1, 2, 3, 4, 5
FAKE = 0x100000  # 16-byte aligned stand-in for a device address; never dereferenced


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(gdn.LIB_PATH):
        import __graft_entry__
        __graft_entry__.build()
    return gdn.load_library()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[\w]+\s*\*?\s*(gdn_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"gdn_prepare", "gdn_decode", "gdn_prefill_varlen", "gdn_prefill_workspace_size"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert set(gdn.EXPORTS) == set(names)


def test_status_strings_and_version(lib):
    assert lib.gdn_status_string(0) == b"ok"
    assert lib.gdn_status_string(3) == b"bad slot index"
    assert lib.gdn_version() >= 100


def _dims(Hk=2, Hv=4, Dk=128, Dv=128, K=4):
    return ctypes.byref(gdn._Dims(Hk, Hv, Dk, Dv, K))


def _arr(a):
    a = np.ascontiguousarray(a, dtype=np.int32)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def _prepare(lib, dims=None, N=2, T=10, cu=(0, 4, 10), stride=None, act=1, qkv=1, slots=(0, 1), num_slots=4,
             x=FAKE, l2=1, ptr_q=FAKE, w=FAKE, pool=FAKE):
    cu_a, cu_p = _arr(cu)
    sl_a, sl_p = _arr(slots) if slots is not None else (None, None)
    d = dims if dims is not None else _dims()
    cc = 2 * 2 * 128 + 4 * 128
    return lib.gdn_prepare(d, N, T, cu_p, FAKE, x, cc if stride is None else stride, FAKE, 4, FAKE, 4, act, w,
                           FAKE, FAKE, pool, num_slots, sl_p, FAKE if slots is not None else None, None, l2, ptr_q,
                           FAKE, FAKE, qkv, FAKE, FAKE, None)


def _err(lib):
    return lib.gdn_last_error().decode()


def test_prepare_rejects_bad_arguments(lib):
    assert lib.gdn_prepare(None, 1, 1, None, None, None, 0, None, 0, None, 0, 0, None, None, None, None, 0, None,
                           None, None, 1, None, None, None, 0, None, None, None) == INVALID
    assert _prepare(lib, dims=_dims(Hk=0)) == SHAPE
    assert _prepare(lib, dims=_dims(Hk=3, Hv=4)) == SHAPE and "multiple" in _err(lib)
    assert _prepare(lib, dims=_dims(Dk=48)) == SHAPE
    assert _prepare(lib, dims=_dims(K=5)) == SHAPE
    assert _prepare(lib, cu=(1, 4, 10)) == SHAPE and "start at 0" in _err(lib)
    assert _prepare(lib, cu=(0, 4, 9)) == SHAPE
    assert _prepare(lib, cu=(0, 0, 10)) == SHAPE and "empty" in _err(lib)
    assert _prepare(lib, cu=(0, 6, 4), T=4) == SHAPE
    assert _prepare(lib, N=1, T=0, cu=(0, 0)) == SHAPE
    assert _prepare(lib, act=2) == DTYPE
    assert _prepare(lib, qkv=2) == DTYPE
    assert _prepare(lib, stride=100) == SHAPE
    assert _prepare(lib, x=FAKE + 4) == INVALID and "aligned" in _err(lib)
    assert _prepare(lib, x=None) == INVALID
    assert _prepare(lib, ptr_q=None) == INVALID
    assert _prepare(lib, slots=(0, 0)) == INDEX and "more than one" in _err(lib)
    assert _prepare(lib, slots=(0, 4)) == INDEX and "out of range" in _err(lib)
    assert _prepare(lib, slots=(0, -1)) == INDEX
    assert _prepare(lib, slots=None, num_slots=1) == INDEX
    assert _prepare(lib, l2=2) == INVALID
    assert _prepare(lib, w=FAKE + 2) == INVALID and "conv weight" in _err(lib)
    assert _prepare(lib, pool=FAKE + 8) == INVALID


def test_prepare_empty_batch_is_a_no_op(lib):
    assert _prepare(lib, N=0, T=0, cu=(0,)) == OK


def _decode(lib, dims=None, B=3, slots=(2, -1, 0), num_slots=4, act=1, state=0, ssm=FAKE, validate=True,
            scale=0.125):
    sl_a, sl_p = _arr(slots)
    d = dims if dims is not None else _dims()
    cc = 2 * 2 * 128 + 4 * 128
    return lib.gdn_decode(d, B, FAKE, cc, FAKE, 4, FAKE, 4, act, FAKE, FAKE, FAKE, FAKE, ssm, state, num_slots,
                          FAKE, sl_p if validate else None, ctypes.c_float(scale), FAKE, None)


def test_decode_rejects_bad_arguments(lib):
    assert _decode(lib, dims=_dims(Hv=6, Hk=4)) == SHAPE
    assert _decode(lib, slots=(2, -2, 0)) == INDEX and "only -1" in _err(lib)
    assert _decode(lib, slots=(2, 2, 0)) == INDEX
    assert _decode(lib, slots=(2, 4, 0)) == INDEX
    assert _decode(lib, act=2) == DTYPE
    assert _decode(lib, state=3) == DTYPE
    assert _decode(lib, ssm=None) == INVALID
    assert _decode(lib, ssm=FAKE + 8) == INVALID
    assert _decode(lib, num_slots=0) == SHAPE
    assert _decode(lib, B=-1) == SHAPE
    assert _decode(lib, scale=float("nan")) == INVALID


def test_decode_empty_batch_is_a_no_op(lib):
    assert _decode(lib, B=0) == OK


def _prefill(lib, dims=None, N=2, T=10, cu=(0, 4, 10), qkv=1, state=0, slots=(1, 0), num_slots=2, chunk=64,
             ws=None, ws_bytes=0, q=FAKE):
    cu_a, cu_p = _arr(cu)
    sl_a, sl_p = _arr(slots) if slots is not None else (None, None)
    d = dims if dims is not None else _dims()
    return lib.gdn_prefill_varlen(d, N, T, cu_p, FAKE, q, FAKE, FAKE, qkv, FAKE, FAKE, FAKE, state, num_slots,
                                  sl_p, FAKE if slots is not None else None, None, ctypes.c_float(0.125), 0, chunk,
                                  FAKE, ws, ws_bytes, None)


def test_prefill_rejects_bad_arguments(lib):
    assert _prefill(lib, cu=(0, 10, 10)) == SHAPE
    assert _prefill(lib, slots=(1, -1)) == INDEX
    assert _prefill(lib, slots=(1, 1)) == INDEX
    assert _prefill(lib, slots=None, num_slots=1) == INDEX
    assert _prefill(lib, qkv=2) == DTYPE
    assert _prefill(lib, state=5) == DTYPE
    assert _prefill(lib, chunk=32) == INVALID
    assert _prefill(lib, q=None) == INVALID
    need = lib.gdn_prefill_workspace_size(_dims(), 2, 10, 64)
    if need > 0:
        assert _prefill(lib, ws=None) == WORKSPACE
        assert _prefill(lib, ws=FAKE, ws_bytes=need - 1) == WORKSPACE


def test_prefill_empty_is_a_no_op(lib):
    assert _prefill(lib, N=0, T=0, cu=(0,), slots=None) == OK


def test_workspace_size_query(lib):
    assert lib.gdn_prefill_workspace_size(_dims(), 2, 100, 32) == 0  # unsupported chunk
    assert lib.gdn_prefill_workspace_size(_dims(Hk=3), 2, 100, 64) == 0  # invalid dims
    a = lib.gdn_prefill_workspace_size(_dims(), 2, 100, 64)
    b = lib.gdn_prefill_workspace_size(_dims(), 2, 1000, 0)
    assert b >= a


def _decode_gated(lib, B=3, slots=(2, -1, 0), z=FAKE, zs=4 * 128, w=FAKE, eps=1e-6, sig=0):
    sl_a, sl_p = _arr(slots)
    cc = 2 * 2 * 128 + 4 * 128
    return lib.gdn_decode_gated(_dims(), B, FAKE, cc, FAKE, 4, FAKE, 4, 1, FAKE, FAKE, FAKE, FAKE, FAKE, 0, 4, FAKE,
                                sl_p, ctypes.c_float(0.125), z, zs, w, ctypes.c_float(eps), sig, FAKE, None)


def test_decode_gated_rejects_bad_arguments(lib):
    assert _decode_gated(lib, z=None) == INVALID
    assert _decode_gated(lib, w=None) == INVALID
    assert _decode_gated(lib, zs=100) == SHAPE and "z_row_stride" in _err(lib)
    assert _decode_gated(lib, eps=-1.0) == INVALID
    assert _decode_gated(lib, eps=float("nan")) == INVALID
    assert _decode_gated(lib, eps=float("inf")) == INVALID
    assert _decode_gated(lib, sig=2) == INVALID
    assert _decode_gated(lib, slots=(2, 2, 0)) == INDEX  # the decode checks still apply
    assert _decode_gated(lib, B=0) == OK


def _norm(lib, T=4, H=4, D=128, x=FAKE, z=FAKE, zs=None, w=FAKE, eps=1e-6, sig=0, out=FAKE, io=1):
    return lib.gdn_gated_rmsnorm(T, H, D, x, z, H * D if zs is None else zs, w, ctypes.c_float(eps), sig, out, io,
                                 None)


def test_gated_rmsnorm_rejects_bad_arguments(lib):
    assert _norm(lib, D=48) == SHAPE
    assert _norm(lib, H=0) == SHAPE
    assert _norm(lib, T=-1) == SHAPE
    assert _norm(lib, io=2) == DTYPE
    assert _norm(lib, x=None) == INVALID
    assert _norm(lib, out=None) == INVALID
    assert _norm(lib, zs=100) == SHAPE
    assert _norm(lib, zs=4 * 128 + 4) == INVALID and "aligned" in _err(lib)
    assert _norm(lib, z=FAKE + 8) == INVALID
    assert _norm(lib, w=FAKE + 2) == INVALID
    assert _norm(lib, eps=-1.0) == INVALID
    assert _norm(lib, eps=float("nan")) == INVALID
    assert _norm(lib, sig=3) == INVALID


def test_gated_rmsnorm_empty_is_a_no_op(lib):
    assert _norm(lib, T=0) == OK


def _wdims(Hk=2, Hv=4, Dk=128, Dv=128, K=4, W=0):
    return ctypes.byref(gdn._Dims(Hk, Hv, Dk, Dv, K, W))


def test_conv_state_len_is_checked(lib):
    # conv rows narrower than K-1 taps, or absurdly wide, are refused by every entry point
    assert _prepare(lib, dims=_wdims(W=2)) == SHAPE and "conv_state_len" in _err(lib)
    assert _prepare(lib, dims=_wdims(W=2000)) == SHAPE
    assert _decode(lib, dims=_wdims(W=1)) == SHAPE and "conv_state_len" in _err(lib)


def _spec(lib, dims=None, N=2, T=8, cu=(0, 4, 8), cols=4, sidx=((0, 1, 2, 3), (4, 5, 6, 7)), nat=(1, 2),
          num_slots=8, act=1, state=0, validate=True, ssm=FAKE, W=6):
    cu_a, cu_p = _arr(cu)
    si_a, si_p = _arr(np.asarray(sidx).ravel())
    na_a, na_p = _arr(nat)
    d = dims if dims is not None else _wdims(W=W)
    return lib.gdn_decode_spec(d, N, T, cu_p, FAKE, FAKE, 1 << 20, FAKE, 64, FAKE, 64, act, FAKE, FAKE, FAKE, FAKE, ssm,
                               state, num_slots, cols, FAKE, FAKE, si_p if validate else None,
                               na_p if validate else None, ctypes.c_float(0.1), FAKE, None)


def test_decode_spec_rejects_bad_arguments(lib):
    assert _spec(lib, dims=_wdims(K=1, W=3)) == SHAPE and "conv_kernel" in _err(lib)
    assert _spec(lib, cols=9, sidx=np.arange(18).reshape(2, 9), num_slots=18, W=12) == SHAPE
    assert _spec(lib, W=5) == SHAPE and "narrower" in _err(lib)          # needs (K-1)+(cols-1) = 6
    assert _spec(lib, dims=_wdims(W=0)) == SHAPE                          # rows of K-1 taps are too narrow
    assert _spec(lib, cu=(0, 5, 8)) == SHAPE and "more than num_cols" in _err(lib)
    assert _spec(lib, cu=(0, 4, 4), T=4) == SHAPE and "empty" in _err(lib)
    assert _spec(lib, nat=(0, 1)) == INDEX and "num_accepted" in _err(lib)
    assert _spec(lib, nat=(5, 1)) == INDEX
    assert _spec(lib, sidx=((0, 1, 2, 3), (4, 5, 6, 8))) == INDEX and "out of range" in _err(lib)
    assert _spec(lib, sidx=((0, 1, 2, 3), (4, 5, 6, 3))) == INDEX and "more than once" in _err(lib)
    assert _spec(lib, sidx=((0, 1, 2, 3), (-1, 5, 6, 7))) == INDEX and "column 0" in _err(lib)
    assert _spec(lib, sidx=((0, 1, 2, 3), (4, -2, 6, 7))) == INDEX
    assert _spec(lib, act=2) == DTYPE
    assert _spec(lib, state=3) == DTYPE
    assert _spec(lib, ssm=FAKE + 4) == INVALID
    assert _spec(lib, num_slots=0) == SHAPE
    # Hv/Hk = 32 value heads per key head of Dv = 256 do not fit one workgroup's LDS at 8 columns
    assert _spec(lib, dims=_wdims(Hk=1, Hv=32, Dv=256, W=10), cols=8, sidx=np.arange(16).reshape(2, 8),
                 num_slots=16, cu=(0, 8, 16), T=16) == SHAPE and "too large" in _err(lib)


def test_decode_spec_empty_is_a_no_op(lib):
    assert _spec(lib, N=0, T=0, cu=(0,), sidx=np.zeros((0, 4)), nat=()) == OK


def _kda(lib, dims=None, N=2, T=10, cu=(0, 4, 10), qkv=1, state=0, slots=(1, 0), num_slots=2, g=FAKE, A=None,
         bias=None, q=FAKE, l2=0, ssm=FAKE):
    cu_a, cu_p = _arr(cu)
    sl_a, sl_p = _arr(slots) if slots is not None else (None, None)
    d = dims if dims is not None else _dims()
    return lib.gdn_kda_recurrent(d, N, T, cu_p, FAKE, q, FAKE, FAKE, qkv, g, A, bias, FAKE, ssm, state, num_slots,
                                 sl_p, FAKE if slots is not None else None, None, ctypes.c_float(0.1), l2, FAKE, None)


def test_kda_recurrent_rejects_bad_arguments(lib):
    assert _kda(lib, dims=_dims(Hk=3, Hv=4)) == SHAPE
    assert _kda(lib, cu=(0, 5, 4), T=4) == SHAPE and "decrease" in _err(lib)
    assert _kda(lib, cu=(1, 4, 10)) == SHAPE
    assert _kda(lib, qkv=2) == DTYPE
    assert _kda(lib, state=5) == DTYPE
    assert _kda(lib, g=None) == INVALID
    assert _kda(lib, g=FAKE + 4) == INVALID and "aligned" in _err(lib)
    assert _kda(lib, bias=FAKE) == INVALID and "A_log" in _err(lib)
    assert _kda(lib, slots=(0, 0)) == INDEX
    assert _kda(lib, slots=(0, 2)) == INDEX
    assert _kda(lib, slots=(-1, 0)) == INDEX
    assert _kda(lib, l2=2) == INVALID
    assert _kda(lib, num_slots=0) == SHAPE


def test_kda_recurrent_empty_is_a_no_op(lib):
    assert _kda(lib, N=0, T=0, cu=(0,), slots=()) == OK


def _sdims(H=4, P=64, G=2, N=128):
    return ctypes.byref(gdn._SsmDims(H, P, G, N))


def _sdt(softplus=1, dt_min=0.0, dt_max=float("inf")):
    return ctypes.byref(gdn._SsmDt(None, softplus, dt_min, dt_max))


def _m2u(lib, sd=None, batch=2, act=1, state=0, dtp=None, slots=(1, 0), num_slots=2, Dp=0, x=FAKE, pool=FAKE,
         A=FAKE):
    sl_a, sl_p = _arr(slots)
    return lib.gdn_mamba2_state_update(sd if sd is not None else _sdims(), batch, x, FAKE, A, FAKE, FAKE, None, Dp,
                                       None, dtp if dtp is not None else _sdt(), act, pool, state, num_slots, FAKE,
                                       sl_p, FAKE, None)


def test_mamba2_state_update_rejects_bad_arguments(lib):
    assert _m2u(lib, sd=_sdims(H=6, G=4)) == SHAPE
    assert _m2u(lib, sd=_sdims(N=24)) == SHAPE and "state_dim" in _err(lib)
    assert _m2u(lib, sd=_sdims(P=2048)) == SHAPE and "1024" in _err(lib)
    assert _m2u(lib, act=2) == DTYPE
    assert _m2u(lib, state=7) == DTYPE
    assert _m2u(lib, x=None) == INVALID
    assert _m2u(lib, A=None) == INVALID
    assert _m2u(lib, x=FAKE + 8) == INVALID and "aligned" in _err(lib)
    assert _m2u(lib, Dp=2) == INVALID
    assert _m2u(lib, dtp=_sdt(softplus=3)) == INVALID
    assert _m2u(lib, dtp=_sdt(dt_min=-1.0)) == INVALID
    assert _m2u(lib, dtp=_sdt(dt_min=0.5, dt_max=0.1)) == INVALID
    assert _m2u(lib, dtp=_sdt(dt_min=float("nan"))) == INVALID
    assert _m2u(lib, slots=(0, 0)) == INDEX
    assert _m2u(lib, slots=(0, 2)) == INDEX
    assert _m2u(lib, num_slots=0) == SHAPE
    assert _m2u(lib, batch=-1) == SHAPE
    assert lib.gdn_mamba2_state_update(None, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None, _sdt(), 1, FAKE, 0, 1,
                                       FAKE, None, FAKE, None) == INVALID


def test_mamba2_state_update_empty_is_a_no_op(lib):
    assert _m2u(lib, batch=0, slots=(), x=None) == OK


def _m2s(lib, sd=None, N=2, T=100, cu=(0, 36, 100), act=1, state=0, slots=(1, 0), num_slots=2, ws=FAKE,
         ws_bytes=None, dtp=None, slots_dev=FAKE):
    cu_a, cu_p = _arr(cu)
    sl_a, sl_p = _arr(slots) if slots is not None else (None, None)
    sd = sd if sd is not None else _sdims()
    if ws_bytes is None:
        ws_bytes = lib.gdn_mamba2_workspace_size(sd, N, T)
    return lib.gdn_mamba2_chunk_scan(sd, N, T, cu_p, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, 0, None,
                                     dtp if dtp is not None else _sdt(), act, FAKE, state, num_slots, sl_p,
                                     slots_dev if slots is not None else None, None, FAKE, ws, ws_bytes, None)


def test_mamba2_workspace_size(lib):
    # two sequences of 36 and 64 tokens: at most 100 / 64 + 2 = 3 chunk blocks per head
    n = lib.gdn_mamba2_workspace_size(_sdims(H=4, P=64, N=128), 2, 100)
    # per (chunk, head): the f32 state contribution, the 1280-byte decay
    # vector, the f16 state entering the chunk
    blk = 64 * 128 * 4 + 1280 + 64 * 128 * 2
    assert n == 256 + 2 * 256 + 3 * 4 * blk
    assert lib.gdn_mamba2_workspace_size(_sdims(P=48), 2, 100) == 0
    assert lib.gdn_mamba2_workspace_size(_sdims(), 0, 0) == 0
    assert lib.gdn_mamba2_workspace_size(None, 1, 10) == 0


def test_mamba2_chunk_scan_rejects_bad_arguments(lib):
    assert _m2s(lib, sd=_sdims(P=48)) == SHAPE and "head_dim" in _err(lib)
    assert _m2s(lib, sd=_sdims(N=256)) == SHAPE
    assert _m2s(lib, sd=_sdims(N=16)) == SHAPE
    assert _m2s(lib, cu=(0, 36, 36), T=36) == SHAPE and "empty" in _err(lib)
    assert _m2s(lib, cu=(0, 36, 99)) == SHAPE
    assert _m2s(lib, act=0, state=9) == DTYPE
    assert _m2s(lib, slots=(0, 0)) == INDEX
    assert _m2s(lib, slots=(-1, 0)) == INDEX
    assert _m2s(lib, slots=(0, 5)) == INDEX
    assert _m2s(lib, slots=None, num_slots=1) == INDEX
    assert _m2s(lib, slots_dev=None) == INVALID and "both" in _err(lib)
    assert _m2s(lib, ws=None) == WORKSPACE
    assert _m2s(lib, ws_bytes=1024) == WORKSPACE
    assert _m2s(lib, ws=FAKE + 16) == WORKSPACE and "aligned" in _err(lib)
    assert _m2s(lib, dtp=_sdt(dt_max=-1.0)) == INVALID


def test_mamba2_chunk_scan_empty_is_a_no_op(lib):
    assert _m2s(lib, N=0, T=0, cu=(0,), slots=()) == OK


def test_prefill_noalloc_refuses_batches_beyond_its_scratch(lib):
    """The allocation-free prefill refuses, before any device work, a batch
    whose one value head needs more scratch than the static array holds."""
    d = _dims(Hk=1, Hv=1)
    T = 80000
    per_head = lib.gdn_prefill_workspace_size(d, 1, T, 64)
    assert per_head > (128 << 20)
    cu_a, cu_p = _arr((0, T))
    st = lib.gdn_prefill_varlen_noalloc(d, 1, T, cu_p, FAKE, FAKE, FAKE, FAKE, 1, FAKE, FAKE, FAKE, 0, 1, None, None,
                                        None, 0.1, 0, 64, FAKE, None)
    assert st == WORKSPACE and "static scratch" in _err(lib)
    # the ordinary checks come first, as in gdn_prefill_varlen
    st = lib.gdn_prefill_varlen_noalloc(d, 1, T, cu_p, FAKE, None, FAKE, FAKE, 1, FAKE, FAKE, FAKE, 0, 1, None, None,
                                        None, 0.1, 0, 64, FAKE, None)
    assert st == INVALID
