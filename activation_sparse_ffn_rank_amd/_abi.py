"""ctypes binding of the C ABI in include/pi_sparse_ffn.h (argument marshalling only).

Every step of the path runs in libpi.so's HIP kernels; this module only turns torch tensors
into device pointers and the caller's current HIP stream into a ``hipStream_t``.  There is no
fallback: if libpi.so is missing the first call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch  # loaded first so libpi.so binds to the HIP runtime torch already uses

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpi.so")

PI_OK, PI_ERR_NULL, PI_ERR_SHAPE, PI_ERR_DTYPE, PI_ERR_BATCH, PI_ERR_WORKSPACE, PI_ERR_ALIGN, PI_ERR_HIP = (
    0, -1, -2, -3, -4, -5, -6, -7)
PI_F16, PI_Q4_0 = 1, 2
PI_ACT_RELU, PI_ACT_SQUARED_RELU = 0, 1
PI_MAX_BATCH = 16
PI_MAX_WIDE_BATCH = 16

# Every function the header declares; the CPU tests check that libpi.so exports them all.
EXPORTS = ("pi_workspace_bytes", "pi_predict", "pi_compact", "pi_sparse_ffn", "pi_sparse_ffn_wide_workspace_bytes", "pi_sparse_ffn_wide",
           "pi_ffn_layer",
           "pi_predict_hidden", "pi_ffn_layer_from_hidden", "pi_layer_path", "pi_sparse_ffn_h_offset",
           "pi_cold_workspace_bytes", "pi_cold_ffn_host", "pi_place", "pi_predictor_ranks", "pi_sparse_ffn_noalloc",
           "pi_status_string",
           "pi_version")
PI_NOALLOC_SCRATCH_BYTES = 32 << 20


class pi_predictor(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("d_ffn", ctypes.c_int32), ("rank", ctypes.c_int32),
                ("p1", ctypes.c_void_p), ("p2", ctypes.c_void_p), ("c", ctypes.c_void_p)]


class pi_ffn(ctypes.Structure):
    _fields_ = [("d_model", ctypes.c_int32), ("d_ffn", ctypes.c_int32), ("gated", ctypes.c_int32),
                ("wtype", ctypes.c_int32), ("n_slots", ctypes.c_int32), ("slot_of", ctypes.c_void_p),
                ("w_in", ctypes.c_void_p), ("w_down_t", ctypes.c_void_p), ("b_up", ctypes.c_void_p),
                ("b_down", ctypes.c_void_p), ("act", ctypes.c_int32)]


class PiError(RuntimeError):
    def __init__(self, fn: str, code: int):
        super().__init__(f"{fn} returned {code}: {pi_status_string(code)}")
        self.code = code


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: the HIP library must be built "
                               "(python -m activation_sparse_ffn_rank_amd.build); there is no fallback")
        L = ctypes.CDLL(LIB_PATH)
        P, vp, i32, sz = ctypes.POINTER, ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        L.pi_workspace_bytes.restype = sz
        L.pi_workspace_bytes.argtypes = [P(pi_predictor), P(pi_ffn), i32]
        L.pi_predict.restype = ctypes.c_int
        L.pi_predict.argtypes = [P(pi_predictor), vp, i32, vp, vp, vp, sz, vp]
        L.pi_compact.restype = ctypes.c_int
        L.pi_compact.argtypes = [vp, i32, vp, vp, vp, vp]
        L.pi_sparse_ffn.restype = ctypes.c_int
        L.pi_sparse_ffn.argtypes = [P(pi_ffn), vp, i32, vp, vp, vp, vp, sz, vp]
        L.pi_sparse_ffn_wide_workspace_bytes.restype = sz
        L.pi_sparse_ffn_wide_workspace_bytes.argtypes = [P(pi_ffn), i32]
        L.pi_sparse_ffn_wide.restype = ctypes.c_int
        L.pi_sparse_ffn_wide.argtypes = [P(pi_ffn), vp, i32, vp, vp, vp, vp, sz, vp]
        L.pi_ffn_layer.restype = ctypes.c_int
        L.pi_ffn_layer.argtypes = [P(pi_predictor), P(pi_ffn), vp, i32, vp, vp, vp, vp, vp, sz, vp]
        L.pi_predict_hidden.restype = ctypes.c_int
        L.pi_predict_hidden.argtypes = [P(pi_predictor), vp, i32, vp, vp]
        L.pi_ffn_layer_from_hidden.restype = ctypes.c_int
        L.pi_ffn_layer_from_hidden.argtypes = [P(pi_predictor), P(pi_ffn), vp, i32, vp, vp, vp, vp, vp, vp, sz, vp]
        L.pi_layer_path.restype = ctypes.c_int
        L.pi_layer_path.argtypes = [P(pi_predictor), P(pi_ffn), i32]
        L.pi_sparse_ffn_h_offset.restype = sz
        L.pi_sparse_ffn_h_offset.argtypes = [P(pi_ffn), i32, P(i32)]
        L.pi_cold_workspace_bytes.restype = sz
        L.pi_cold_workspace_bytes.argtypes = [P(pi_ffn), i32]
        L.pi_cold_ffn_host.restype = ctypes.c_int
        L.pi_cold_ffn_host.argtypes = [P(pi_ffn), vp, i32, vp, vp, P(i32), vp, sz, i32]
        L.pi_place.restype = ctypes.c_int
        L.pi_place.argtypes = [i32, vp, vp, vp, ctypes.c_int64, ctypes.c_double, ctypes.c_double, vp, vp,
                               P(ctypes.c_double)]
        L.pi_predictor_ranks.restype = ctypes.c_int
        L.pi_predictor_ranks.argtypes = [i32, vp, vp, vp, ctypes.c_int64, i32, i32, i32, vp, vp]
        L.pi_sparse_ffn_noalloc.restype = ctypes.c_int
        L.pi_sparse_ffn_noalloc.argtypes = [P(pi_ffn), vp, i32, vp, vp, vp, vp]
        L.pi_status_string.restype = ctypes.c_char_p
        L.pi_status_string.argtypes = [ctypes.c_int]
        L.pi_version.restype = ctypes.c_int
        L.pi_version.argtypes = []
        _lib = L
    return _lib


def _ptr(t) -> int | None:
    """Device pointer of a tensor (None stays NULL; ints pass through as raw addresses)."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _byref(s):
    return None if s is None else ctypes.byref(s)


def _nbytes(t) -> int:
    return t.numel() * t.element_size()


def _check(fn: str, rc: int) -> None:
    if rc != PI_OK:
        raise PiError(fn, rc)


def make_predictor(p1: torch.Tensor, p2: torch.Tensor, c: torch.Tensor) -> pi_predictor:
    """Descriptor of a predictor from device tensors P1 [r][d], P2 [f][r], c [f] (fp16 storage)."""
    r, d = p1.shape
    f = p2.shape[0]
    return pi_predictor(d, f, r, _ptr(p1), _ptr(p2), _ptr(c))


def make_ffn(w_in: torch.Tensor, w_down_t: torch.Tensor, *, d_model: int, d_ffn: int, gated: bool, wtype: int,
             slot_of: torch.Tensor | None = None, b_up: torch.Tensor | None = None,
             b_down: torch.Tensor | None = None, act: int = PI_ACT_RELU) -> pi_ffn:
    """Descriptor of resident FFN weights (neuron-major rows, see the header)."""
    return pi_ffn(d_model, d_ffn, int(gated), wtype, int(w_in.shape[0]), _ptr(slot_of), _ptr(w_in), _ptr(w_down_t),
                  _ptr(b_up), _ptr(b_down), act)


def pi_workspace_bytes(pred: pi_predictor | None, ffn: pi_ffn | None, batch: int) -> int:
    return int(lib().pi_workspace_bytes(_byref(pred), _byref(ffn), batch))


def pi_predict(pred, x, batch, mask, logits, ws, stream=None) -> None:
    _check("pi_predict", lib().pi_predict(_byref(pred), _ptr(x), batch, _ptr(mask), _ptr(logits), _ptr(ws),
                                          _nbytes(ws) if ws is not None and not isinstance(ws, int) else 0,
                                          _stream(stream)))


def pi_compact(mask, d_ffn, slot_of, idx, counts, stream=None) -> None:
    _check("pi_compact", lib().pi_compact(_ptr(mask), d_ffn, _ptr(slot_of), _ptr(idx), _ptr(counts),
                                          _stream(stream)))


def pi_sparse_ffn(ffn, x, batch, idx, counts, y, ws, stream=None) -> None:
    _check("pi_sparse_ffn", lib().pi_sparse_ffn(_byref(ffn), _ptr(x), batch, _ptr(idx), _ptr(counts), _ptr(y),
                                                _ptr(ws), _nbytes(ws) if ws is not None and not isinstance(ws, int) else 0,
                                                _stream(stream)))


def pi_sparse_ffn_noalloc(ffn, x, batch, idx, counts, y, stream=None) -> None:
    """pi_sparse_ffn with the library's own device scratch (no caller workspace, no allocation)."""
    _check("pi_sparse_ffn_noalloc", lib().pi_sparse_ffn_noalloc(_byref(ffn), _ptr(x), batch, _ptr(idx), _ptr(counts),
                                                                _ptr(y), _stream(stream)))


def pi_sparse_ffn_wide_workspace_bytes(ffn, batch: int) -> int:
    return int(lib().pi_sparse_ffn_wide_workspace_bytes(_byref(ffn), batch))


def pi_sparse_ffn_wide(ffn, x, batch, idx, counts, y, ws, stream=None) -> None:
    _check("pi_sparse_ffn_wide", lib().pi_sparse_ffn_wide(
        _byref(ffn), _ptr(x), batch, _ptr(idx), _ptr(counts), _ptr(y), _ptr(ws),
        _nbytes(ws) if ws is not None and not isinstance(ws, int) else 0, _stream(stream)))


def pi_ffn_layer(pred, ffn, x, batch, y, mask_out, idx_out, counts_out, ws, stream=None) -> None:
    _check("pi_ffn_layer", lib().pi_ffn_layer(_byref(pred), _byref(ffn), _ptr(x), batch, _ptr(y), _ptr(mask_out),
                                              _ptr(idx_out), _ptr(counts_out), _ptr(ws),
                                              _nbytes(ws) if ws is not None and not isinstance(ws, int) else 0,
                                              _stream(stream)))


def pi_predict_hidden(pred, x, batch, z, stream=None) -> None:
    _check("pi_predict_hidden", lib().pi_predict_hidden(_byref(pred), _ptr(x), batch, _ptr(z), _stream(stream)))


def pi_ffn_layer_from_hidden(pred, ffn, x, batch, z, y, mask_out, idx_out, counts_out, ws, stream=None) -> None:
    _check("pi_ffn_layer_from_hidden", lib().pi_ffn_layer_from_hidden(
        _byref(pred), _byref(ffn), _ptr(x), batch, _ptr(z), _ptr(y), _ptr(mask_out), _ptr(idx_out),
        _ptr(counts_out), _ptr(ws), _nbytes(ws) if ws is not None and not isinstance(ws, int) else 0,
        _stream(stream)))


def pi_layer_path(pred, ffn, batch) -> int:
    """1: pi_ffn_layer_from_hidden is one persistent kernel; 2: separate kernels; 0: invalid."""
    return int(lib().pi_layer_path(_byref(pred), _byref(ffn), batch))


PI_WS_STATUS_OFFSET = 384      # byte offset of the layer workspace's sticky status word


PI_STATUS_H_RANGE = 64        # status bit: an |h| the MFMA form's fp16 pair cannot carry


def workspace_status(ws) -> int:
    """Sticky status word of a pi_ffn_layer or pi_sparse_ffn workspace (0 = every cross-workgroup
    wait completed and every h was in range)."""
    return int(ws[PI_WS_STATUS_OFFSET:PI_WS_STATUS_OFFSET + 4].view(torch.int32).item())


def wide_workspace_status(ws) -> int:
    """Sticky status word of a pi_sparse_ffn_wide workspace (its first int32)."""
    return int(ws[0:4].view(torch.int32).item())


def pi_sparse_ffn_h_offset(ffn, batch: int) -> tuple[int, int]:
    """(byte offset, kind) of the h table a pi_sparse_ffn call leaves in its workspace."""
    kind = ctypes.c_int32(0)
    off = int(lib().pi_sparse_ffn_h_offset(_byref(ffn), batch, ctypes.byref(kind)))
    if off == (1 << 64) - 1:
        raise PiError("pi_sparse_ffn_h_offset", PI_ERR_SHAPE)
    return off, int(kind.value)


def sparse_ffn_h(ffn, batch: int, ws: torch.Tensor, n: int) -> tuple[torch.Tensor, torch.Tensor]:
    """h [batch][n] (fp32) and the slot-valid flags [n] that the last pi_sparse_ffn call on `ws` left
    for list positions 0..n-1 (a device-side view, for counting the rows that had to be read)."""
    off, kind = pi_sparse_ffn_h_offset(ffn, batch)
    if kind == 1:
        f = int(ffn.d_ffn)
        h = ws[off: off + 4 * batch * f].view(torch.float32).view(batch, f)[:, :n]
        return h, torch.ones(n, dtype=torch.bool, device=ws.device)
    if kind == 3:
        # MFMA form: 16-byte units [hs/4][16 tokens] of (4 fp16 hi, 4 fp16 lo) for 4 positions each,
        # hs = n_slots rounded up to 32
        hs = (max(int(ffn.n_slots), 1) + 31) // 32 * 32
        t = ws[off: off + 64 * hs].view(torch.float16).view(hs // 4, 16, 8)
        h = (t[:, :batch, :4].float() + t[:, :batch, 4:].float())       # [hs/4][batch][4]
        h = h.permute(1, 0, 2).reshape(batch, hs)[:, :n]
        return h, torch.ones(n, dtype=torch.bool, device=ws.device)
    stride = max(int(ffn.n_slots), 1)
    h = ws[off: off + 4 * batch * stride].view(torch.float32).view(batch, stride)[:, :n]
    return h, torch.ones(n, dtype=torch.bool, device=ws.device)


class HostFFN:
    """Descriptor of FFN rows held in HOST memory (numpy arrays, kept alive here) for
    pi_cold_ffn_host: neuron-major rows of the neurons held on the host, slot_of [d_ffn] (-1 = not
    held here) or None (all neurons, identity)."""

    def __init__(self, w_in, w_down_t, *, d_model: int, d_ffn: int, gated: bool, wtype: int, slot_of=None,
                 b_up=None, act: int = PI_ACT_RELU):
        import numpy as np
        self._keep = [np.ascontiguousarray(a) if a is not None else None for a in (w_in, w_down_t, slot_of, b_up)]
        w_in, w_down_t, slot_of, b_up = self._keep
        hp = lambda a: None if a is None else a.ctypes.data
        self.ffn = pi_ffn(d_model, d_ffn, int(gated), wtype, int(w_in.shape[0]), hp(slot_of), hp(w_in),
                          hp(w_down_t), hp(b_up), None, act)


def pi_cold_workspace_bytes(host: HostFFN, batch: int) -> int:
    return int(lib().pi_cold_workspace_bytes(ctypes.byref(host.ffn), batch))


def pi_cold_ffn_host(host: HostFFN, x, batch: int, mask, y, ws, n_threads: int = 0) -> int:
    """Host half of the hybrid split: y [batch][d] (numpy fp32, overwritten) = the contribution of
    the predicted neurons held on the host; returns how many were computed.  x [batch][d] fp16
    bits and mask [d_ffn] u8 are numpy arrays; ws a numpy byte array of pi_cold_workspace_bytes."""
    import numpy as np
    for a in (x, mask, y, ws):
        assert isinstance(a, np.ndarray) and a.flags["C_CONTIGUOUS"], "host arrays must be contiguous numpy arrays"
    assert y.dtype == np.float32 and mask.dtype == np.uint8 and x.dtype.itemsize == 2
    n = ctypes.c_int32(0)
    _check("pi_cold_ffn_host", lib().pi_cold_ffn_host(ctypes.byref(host.ffn), x.ctypes.data, batch, mask.ctypes.data,
                                                       y.ctypes.data, ctypes.byref(n), ws.ctypes.data, ws.nbytes,
                                                       n_threads))
    return int(n.value)


def pi_place(d_ffn, neuron_bytes, freq, budget_bytes: int, gpu_bytes_per_s: float, host_bytes_per_s: float):
    """Offline placement (host): returns (slot_of list of int32 arrays per layer, n_placed array,
    expected seconds per token).  d_ffn, neuron_bytes: per layer; freq: per-layer float arrays."""
    import numpy as np
    d = np.ascontiguousarray(d_ffn, dtype=np.int32)
    nb = np.ascontiguousarray(neuron_bytes, dtype=np.int64)
    fr = np.ascontiguousarray(np.concatenate([np.asarray(p, np.float32) for p in freq]), dtype=np.float32)
    so = np.empty(int(d.sum()), np.int32)
    npl = np.empty(d.size, np.int32)
    t = ctypes.c_double(0.0)
    _check("pi_place", lib().pi_place(d.size, d.ctypes.data, nb.ctypes.data, fr.ctypes.data, int(budget_bytes),
                                      float(gpu_bytes_per_s), float(host_bytes_per_s), so.ctypes.data,
                                      npl.ctypes.data, ctypes.byref(t)))
    return np.split(so, np.cumsum(d)[:-1]), npl, float(t.value)


def pi_predictor_ranks(d_model, d_ffn, freq, budget_bytes: int, r_min: int, r_max: int, r_step: int):
    """Per-layer predictor ranks under a budget for the predictor matrices (host): returns (rank
    array, rounded firing entropy in bits per layer).  d_model, d_ffn: per layer; freq: per-layer
    float arrays."""
    import numpy as np
    dm = np.ascontiguousarray(d_model, dtype=np.int32)
    df = np.ascontiguousarray(d_ffn, dtype=np.int32)
    fr = np.ascontiguousarray(np.concatenate([np.asarray(p, np.float32) for p in freq]), dtype=np.float32)
    rank = np.empty(df.size, np.int32)
    ent = np.empty(df.size, np.float64)
    _check("pi_predictor_ranks", lib().pi_predictor_ranks(df.size, dm.ctypes.data, df.ctypes.data, fr.ctypes.data,
                                                          int(budget_bytes), r_min, r_max, r_step, rank.ctypes.data,
                                                          ent.ctypes.data))
    return rank, ent


def pi_status_string(code: int) -> str:
    return lib().pi_status_string(code).decode()


def pi_version() -> int:
    return int(lib().pi_version())
