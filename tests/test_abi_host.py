"""C ABI checks that need no GPU: libpi.so loads, exports every function include/pi_sparse_ffn.h
declares, and rejects bad arguments on the host with the documented codes before any HIP call."""
import ctypes
import os
import re

import pytest

from activation_sparse_ffn_rank_amd import _abi, build

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "pi_sparse_ffn.h")

A = 0x10000          # fake, 16-byte aligned device addresses: host validation never dereferences them
U = 0x10008          # 8-byte aligned only


@pytest.fixture(scope="module")
def L():
    if build.is_stale():
        build.build()
    return _abi.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pi_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_function(L):
    names = declared_functions()
    assert set(names) == set(_abi.EXPORTS), names
    for n in names:
        assert hasattr(L, n), n
    assert L.pi_version() == 200


def pred(d=1024, f=4096, r=128, p1=A, p2=A, c=A):
    return _abi.pi_predictor(d, f, r, p1, p2, c)


def ffn(d=1024, f=4096, gated=0, wtype=_abi.PI_F16, n_slots=None, slot_of=None, w_in=A, w_dn=A, b_up=None, b_down=None,
        act=0):
    return _abi.pi_ffn(d, f, gated, wtype, f if n_slots is None else n_slots, slot_of, w_in, w_dn, b_up, b_down, act)


def ws_for(L, p, f, B):
    return L.pi_workspace_bytes(ctypes.byref(p) if p else None, ctypes.byref(f) if f else None, B)


def test_workspace_sizes(L):
    p, f = pred(), ffn()
    both, only_p, only_f = ws_for(L, p, f, 1), ws_for(L, p, None, 1), ws_for(L, None, f, 1)
    assert only_p > 0 and only_f > 0 and both >= only_p + only_f
    assert ws_for(L, p, f, 8) > both
    assert ws_for(L, p, f, 0) == 0 and ws_for(L, p, f, 17) == 0 and ws_for(L, None, None, 1) == 0
    assert ws_for(L, pred(d=512), f, 1) == 0                      # d_model mismatch


def test_predict_rejects(L):
    p = pred()
    big = ws_for(L, p, None, 1)
    call = lambda pp, x=A, B=1, mask=A, ws=A, n=big: L.pi_predict(pp, x, B, mask, None, ws, n, None)
    assert call(None) == _abi.PI_ERR_NULL
    assert call(ctypes.byref(pred(p1=0))) == _abi.PI_ERR_NULL
    assert call(ctypes.byref(p), x=0) == _abi.PI_ERR_NULL
    assert call(ctypes.byref(p), mask=0) == _abi.PI_ERR_NULL
    assert call(ctypes.byref(p), B=0) == _abi.PI_ERR_BATCH
    assert call(ctypes.byref(p), B=17) == _abi.PI_ERR_BATCH
    assert call(ctypes.byref(pred(r=100))) == _abi.PI_ERR_SHAPE       # rank % 8
    assert call(ctypes.byref(pred(r=4096))) == _abi.PI_ERR_SHAPE      # rank > 2048
    assert call(ctypes.byref(pred(d=1020))) == _abi.PI_ERR_SHAPE
    assert call(ctypes.byref(pred(d=(1 << 24) + 8))) == _abi.PI_ERR_SHAPE     # d_model > 2^24
    assert call(ctypes.byref(pred(f=(1 << 26) + 1))) == _abi.PI_ERR_SHAPE     # d_ffn > 2^26
    assert call(ctypes.byref(pred(p1=U))) == _abi.PI_ERR_ALIGN
    assert call(ctypes.byref(p), x=U) == _abi.PI_ERR_ALIGN
    assert call(ctypes.byref(p), ws=0) == _abi.PI_ERR_WORKSPACE
    assert call(ctypes.byref(p), n=big - 1) == _abi.PI_ERR_WORKSPACE


def test_sparse_ffn_noalloc_rejects(L):
    """Argument checks of the no-allocation entry point run on the host before any HIP call,
    including the bound on the library-held scratch (a layer that needs more is refused)."""
    call = lambda ff, x=A, B=1, idx=A, cnt=A, y=A: L.pi_sparse_ffn_noalloc(ff, x, B, idx, cnt, y, None)
    f = ffn()
    assert call(None) == _abi.PI_ERR_NULL
    for kw in (dict(x=0), dict(idx=0), dict(cnt=0), dict(y=0)):
        assert call(ctypes.byref(f), **kw) == _abi.PI_ERR_NULL
    assert call(ctypes.byref(f), x=U) == _abi.PI_ERR_ALIGN
    assert call(ctypes.byref(f), B=0) == _abi.PI_ERR_BATCH and call(ctypes.byref(f), B=17) == _abi.PI_ERR_BATCH
    assert call(ctypes.byref(ffn(wtype=3))) == _abi.PI_ERR_DTYPE
    big = ffn(d=16384, f=1 << 20)
    assert ws_for(L, None, big, 1) > _abi.PI_NOALLOC_SCRATCH_BYTES
    assert call(ctypes.byref(big)) == _abi.PI_ERR_WORKSPACE
    # the benchmarked shapes fit: the 175B-shaped Q4_0 layer at batch 1 and 8
    q = ffn(d=12288, f=49152, wtype=_abi.PI_Q4_0)
    assert ws_for(L, None, q, 1) <= _abi.PI_NOALLOC_SCRATCH_BYTES and ws_for(L, None, q, 8) <= _abi.PI_NOALLOC_SCRATCH_BYTES


def test_compact_rejects(L):
    assert L.pi_compact(None, 10, None, A, A, None) == _abi.PI_ERR_NULL
    assert L.pi_compact(A, 10, None, None, A, None) == _abi.PI_ERR_NULL
    assert L.pi_compact(A, 0, None, A, A, None) == _abi.PI_ERR_SHAPE
    assert L.pi_compact(A, (1 << 26) + 1, None, A, A, None) == _abi.PI_ERR_SHAPE


def test_sparse_ffn_rejects(L):
    f = ffn()
    big = ws_for(L, None, f, 1)
    call = lambda ff, x=A, B=1, ws=A, n=big: L.pi_sparse_ffn(ff, x, B, A, A, A, ws, n, None)
    assert call(None) == _abi.PI_ERR_NULL
    assert call(ctypes.byref(ffn(w_in=0))) == _abi.PI_ERR_NULL
    assert call(ctypes.byref(ffn(wtype=3))) == _abi.PI_ERR_DTYPE
    assert call(ctypes.byref(ffn(gated=1, wtype=_abi.PI_Q4_0))) == _abi.PI_ERR_DTYPE
    assert call(ctypes.byref(ffn(gated=1, b_up=A))) == _abi.PI_ERR_DTYPE
    assert call(ctypes.byref(ffn(act=2))) == _abi.PI_ERR_DTYPE                         # no such activation
    assert call(ctypes.byref(ffn(gated=1, act=_abi.PI_ACT_SQUARED_RELU))) == _abi.PI_ERR_DTYPE
    assert call(ctypes.byref(ffn(d=1000, wtype=_abi.PI_Q4_0))) == _abi.PI_ERR_SHAPE   # Q4_0 needs d % 256
    assert call(ctypes.byref(ffn(d=(1 << 24) + 256))) == _abi.PI_ERR_SHAPE             # d_model > 2^24
    assert call(ctypes.byref(ffn(n_slots=100))) == _abi.PI_ERR_SHAPE                  # slot_of NULL: n_slots == f
    assert call(ctypes.byref(ffn(n_slots=5000, slot_of=A))) == _abi.PI_ERR_SHAPE      # n_slots > f
    assert call(ctypes.byref(ffn(w_dn=U))) == _abi.PI_ERR_ALIGN
    assert call(ctypes.byref(f), B=17) == _abi.PI_ERR_BATCH
    assert call(ctypes.byref(f), n=big - 1) == _abi.PI_ERR_WORKSPACE


def test_sparse_ffn_wide_rejects(L):
    f = ffn()
    wsz = lambda ff, B: L.pi_sparse_ffn_wide_workspace_bytes(ff, B)
    big = wsz(ctypes.byref(f), 16)
    assert big > 0 and wsz(ctypes.byref(f), 1) < big                                  # partials scale with batch
    assert wsz(ctypes.byref(f), 17) == 0 and wsz(ctypes.byref(f), 0) == 0
    assert wsz(ctypes.byref(ffn(d=1024, wtype=_abi.PI_Q4_0)), 16) > 0
    assert wsz(ctypes.byref(ffn(d=1000, wtype=_abi.PI_Q4_0)), 16) == 0               # Q4_0 needs d % 256
    call = lambda ff, x=A, B=16, ws=A, n=big: L.pi_sparse_ffn_wide(ff, x, B, A, A, A, ws, n, None)
    assert call(None) == _abi.PI_ERR_NULL
    assert call(ctypes.byref(ffn(w_dn=0))) == _abi.PI_ERR_NULL
    assert call(ctypes.byref(ffn(wtype=3))) == _abi.PI_ERR_DTYPE
    assert call(ctypes.byref(ffn(gated=1, wtype=_abi.PI_Q4_0))) == _abi.PI_ERR_DTYPE
    assert call(ctypes.byref(ffn(gated=1, act=_abi.PI_ACT_SQUARED_RELU))) == _abi.PI_ERR_DTYPE
    assert call(ctypes.byref(ffn(d=1001))) == _abi.PI_ERR_SHAPE
    assert call(ctypes.byref(f), B=17) == _abi.PI_ERR_BATCH and call(ctypes.byref(f), B=0) == _abi.PI_ERR_BATCH
    assert call(ctypes.byref(f), n=big - 1) == _abi.PI_ERR_WORKSPACE
    assert call(ctypes.byref(f), ws=None) == _abi.PI_ERR_WORKSPACE
    assert call(ctypes.byref(f), x=U) == _abi.PI_ERR_ALIGN and call(ctypes.byref(f), ws=U) == _abi.PI_ERR_ALIGN
    assert call(ctypes.byref(f), x=None) == _abi.PI_ERR_NULL


def test_layer_rejects(L):
    p, f = pred(), ffn()
    big = ws_for(L, p, f, 2)
    call = lambda pp, ff, B=2, n=big: L.pi_ffn_layer(pp, ff, A, B, A, None, None, None, A, n, None)
    assert call(ctypes.byref(p), None) == _abi.PI_ERR_NULL
    assert call(ctypes.byref(pred(f=4000)), ctypes.byref(f)) == _abi.PI_ERR_SHAPE
    assert call(ctypes.byref(p), ctypes.byref(f), n=big - 1) == _abi.PI_ERR_WORKSPACE
    assert call(ctypes.byref(p), ctypes.byref(f), B=0) == _abi.PI_ERR_BATCH


def test_status_strings(L):
    for code in range(0, -8, -1):
        s = _abi.pi_status_string(code)
        assert s and s != "unknown status"
    assert _abi.pi_status_string(5) == "unknown status"


def test_two_step_layer_rejects(L):
    p, f = pred(), ffn()
    big = ws_for(L, p, f, 2)
    hid = lambda pp, x=A, B=2, z=A: L.pi_predict_hidden(pp, x, B, z, None)
    assert hid(None) == _abi.PI_ERR_NULL
    assert hid(ctypes.byref(p), z=0) == _abi.PI_ERR_NULL
    assert hid(ctypes.byref(p), x=U) == _abi.PI_ERR_ALIGN
    assert hid(ctypes.byref(p), z=U) == _abi.PI_ERR_ALIGN
    assert hid(ctypes.byref(p), B=17) == _abi.PI_ERR_BATCH
    rest = lambda pp, ff, B=2, z=A, n=big: L.pi_ffn_layer_from_hidden(pp, ff, A, B, z, A, None, None, None, A, n, None)
    assert rest(ctypes.byref(p), ctypes.byref(f), z=0) == _abi.PI_ERR_NULL
    assert rest(ctypes.byref(p), ctypes.byref(f), z=U) == _abi.PI_ERR_ALIGN
    assert rest(ctypes.byref(p), ctypes.byref(f), n=big - 1) == _abi.PI_ERR_WORKSPACE
    assert rest(ctypes.byref(pred(d=512)), ctypes.byref(f)) == _abi.PI_ERR_SHAPE


def test_layer_path(L):
    path = lambda pp, ff, B: L.pi_layer_path(ctypes.byref(pp) if pp else None, ctypes.byref(ff) if ff else None, B)
    # one persistent kernel: d_ffn <= 12288, batch <= 3 and x, z fit LDS
    assert path(pred(d=4096, f=11008, r=1024), ffn(d=4096, f=11008, gated=1), 1) == 1
    assert path(pred(d=1024, f=4096, r=128), ffn(d=1024, f=4096), 3) == 1
    # past 3 tokens separate kernels (faster there)
    assert path(pred(d=4096, f=11008, r=1024), ffn(d=4096, f=11008, gated=1), 4) == 2
    assert path(pred(d=1024, f=4096, r=128), ffn(d=1024, f=4096), 8) == 2
    # separate kernels: more than 12288 neurons (at batch <= 2: k_pred_up and the split kernels, faster
    # there), or x too large for LDS
    assert path(pred(d=8192, f=32768, r=1024), ffn(d=8192, f=32768), 1) == 2
    assert path(pred(d=7168, f=28672, r=1024), ffn(d=7168, f=28672), 1) == 2
    assert path(pred(d=8192, f=32768, r=1024), ffn(d=8192, f=32768), 4) == 2
    assert path(pred(d=12288, f=49152, r=1024), ffn(d=12288, f=49152), 1) == 2
    assert path(pred(d=12288, f=12288, r=1024), ffn(d=12288, f=12288), 8) == 2
    # past 8 tokens too (MFMA second predictor matrix and FFN)
    assert path(pred(d=1024, f=4096, r=128), ffn(d=1024, f=4096), 9) == 2
    assert path(pred(d=1024, f=4096, r=128), ffn(d=1024, f=4096), 16) == 2
    # invalid
    assert path(pred(), ffn(), 0) == 0
    assert path(pred(d=512), ffn(), 1) == 0
    assert path(None, ffn(), 1) == 0


def test_h_offset(L):
    kind = ctypes.c_int32(0)
    small, large = ffn(d=1024, f=4096), ffn(d=12288, f=4096)
    off = L.pi_sparse_ffn_h_offset(ctypes.byref(small), 1, ctypes.byref(kind))
    assert kind.value == 1 and 0 < off < ws_for(L, None, small, 1)
    off = L.pi_sparse_ffn_h_offset(ctypes.byref(large), 4, ctypes.byref(kind))
    assert kind.value == 2 and off >= 512                     # x [4][12288] does not fit LDS: two kernels,
    assert off % 256 == 0 and off < ws_for(L, None, large, 4)  # after the control block
    L.pi_sparse_ffn_h_offset(ctypes.byref(small), 4, ctypes.byref(kind))
    assert kind.value == 2                                    # batch > 2: two kernels
    off = L.pi_sparse_ffn_h_offset(ctypes.byref(large), 8, ctypes.byref(kind))
    assert kind.value == 3 and off >= 512 and off % 256 == 0   # batch >= 6: the MFMA kernels
    assert off + 2 * 16 * 4096 * 2 <= ws_for(L, None, large, 8)  # hi and lo tables inside the workspace
    L.pi_sparse_ffn_h_offset(ctypes.byref(small), 6, ctypes.byref(kind))
    assert kind.value == 3
    for gated_or_q4 in (ffn(d=1024, f=4096, gated=1), ffn(d=1024, f=4096, wtype=_abi.PI_Q4_0)):
        L.pi_sparse_ffn_h_offset(ctypes.byref(gated_or_q4), 3, ctypes.byref(kind))
        assert kind.value == 3                                # gated / Q4_0: MFMA kernels from batch 3
    L.pi_sparse_ffn_h_offset(ctypes.byref(small), 16, ctypes.byref(kind))
    assert kind.value == 3                                    # 9..16 tokens: the MFMA kernels
    assert L.pi_sparse_ffn_h_offset(ctypes.byref(small), 17, ctypes.byref(kind)) == 2**64 - 1
    assert L.pi_sparse_ffn_h_offset(ctypes.byref(small), 1, None) == 2**64 - 1
