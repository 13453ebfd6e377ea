"""Seeded synthetic inputs for the predictor-gated sparse FFN (workload generator only).

This package makes the inputs that both the CPU oracle and the HIP path consume: predictor
weights, FFN weights in neuron-major order (fp16 or Q4_0), token vectors, per-neuron Zipf
firing frequencies and the predictor offsets calibrated to them, and the hot-neuron
placement.  It holds none of the method's arithmetic (no predictor evaluation, masking,
compaction or FFN), so sharing it does not couple the oracle to the kernels.

The workload statistics follow the pages' description of activation skew: a small share of
"hot" neurons fire for most inputs while the rest fire rarely, about 26% of neurons giving
80% of all activations (PowerInfer, arXiv 2312.12456, abstract and key results).  Weight
shapes, densities and the predictor form are the five layer configurations this repository
measures (``CONFIGS``).
"""
from __future__ import annotations

import ctypes
import functools
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libpisynth.so")
_SRC_PATH = os.path.join(_HERE, "pisynth.c")

# Hash stream ids (the `tensor` coordinate of the counter-based hash).
T_P1, T_P2, T_PERM, T_WGATE, T_WUP, T_WDOWN, T_BUP, T_BDOWN, T_X = 1, 2, 3, 4, 5, 6, 7, 8, 9
T_Q4_UP, T_Q4_DOWN = 10, 12          # codes; +1 is the matching scale stream

F16, Q4_0 = 1, 2                     # weight storage kinds (same values as the C ABI)


def build(verbose: bool = False) -> str:
    """Compile libpisynth.so with gcc (OpenMP, -O2)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-o", _LIB_PATH, _SRC_PATH, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is not built; run __graft_entry__.build() first")
        L = ctypes.CDLL(_LIB_PATH)
        u64, u32, i64, dbl, vp = ctypes.c_uint64, ctypes.c_uint32, ctypes.c_int64, ctypes.c_double, ctypes.c_void_p
        L.ps_hash.restype = u64
        L.ps_hash.argtypes = [u64, u32, u32, u64, u64]
        L.ps_f32_to_f16.restype = ctypes.c_uint16
        L.ps_f32_to_f16.argtypes = [ctypes.c_float]
        L.ps_normal_f16.restype = None
        L.ps_normal_f16.argtypes = [u64, u32, u32, vp, i64, i64, i64, dbl, vp, i64]
        L.ps_normal_f32.restype = None
        L.ps_normal_f32.argtypes = [u64, u32, u32, i64, i64, i64, dbl, vp]
        L.ps_q4_0_rows.restype = None
        L.ps_q4_0_rows.argtypes = [u64, u32, u32, vp, i64, i64, i64, vp, i64]
        L.ps_zipf_solve.restype = ctypes.c_int
        L.ps_zipf_solve.argtypes = [i64, dbl, dbl, dbl, dbl, ctypes.POINTER(dbl), ctypes.POINTER(dbl)]
        L.ps_zipf_freq.restype = None
        L.ps_zipf_freq.argtypes = [u64, u32, u32, i64, dbl, dbl, dbl, vp, vp, vp]
        L.ps_offsets.restype = None
        L.ps_offsets.argtypes = [vp, i64, i64, vp, vp]
        L.ps_num_threads.restype = ctypes.c_int
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


# ----------------------------------------------------------------------------- configs

@dataclass(frozen=True)
class Config:
    """One layer-stack shape.  Sizes: d = d_model, f = d_ffn, r = predictor rank."""
    cid: int
    name: str
    layers: int
    d: int
    f: int
    r: int
    gated: bool
    wtype: int
    bias_up: bool
    density: float
    tokens: int
    batches: tuple
    hot_frac: float | None = None     # placement: keep this share of neurons resident
    seed: int = 0
    act: int = 0                      # 1: squared ReLU (non-gated)

    def row_bytes(self) -> int:
        return self.d * 2 if self.wtype == F16 else self.d * 9 // 16

    def n_hot(self) -> int:
        return self.f if self.hot_frac is None else int(round(self.hot_frac * self.f))


CONFIGS = {
    1: Config(1, "relu-ffn-1x1024x4096", 1, 1024, 4096, 128, False, F16, True, 0.10, 64, (1,), seed=1),
    2: Config(2, "relu-llama-7b-reglu", 32, 4096, 11008, 1024, True, F16, False, 0.12, 128, (1,), seed=2),
    3: Config(3, "opt-30b-relu", 48, 7168, 28672, 1024, False, F16, True, 0.06, 128, (1, 4), seed=3),
    4: Config(4, "falcon-40b-relu-hot26", 60, 8192, 32768, 1024, False, F16, False, 0.08, 128, (1,),
              hot_frac=0.26, seed=4),
    5: Config(5, "opt-175b-relu-q4_0", 96, 12288, 49152, 1024, False, Q4_0, True, 0.05, 64, (1, 8), seed=5),
}

TOP_FRAC, TOP_SHARE, P_CAP = 0.26, 0.80, 0.99


def custom_config(d, f, r, *, gated=False, wtype=F16, bias_up=True, density=0.1, hot_frac=None,
                  seed=1234, layers=1, tokens=4, name="custom", act=0) -> Config:
    return Config(0, name, layers, d, f, r, gated, wtype, bias_up, density, tokens, (1,), hot_frac, seed, act)


# ----------------------------------------------------------------------------- primitives

def normal_f16(seed, layer, tensor, nrows, ncols, sigma, rows=None, row0=0) -> np.ndarray:
    """fp16 bit patterns (uint16) of N(0, sigma^2) Irwin-Hall(4) draws, [nrows][ncols]."""
    out = np.empty((nrows, ncols), dtype=np.uint16)
    rows_arr = None if rows is None else np.ascontiguousarray(rows, dtype=np.int32)
    lib().ps_normal_f16(seed, layer, tensor, _ptr(rows_arr), row0, nrows, ncols, float(sigma), _ptr(out), ncols)
    return out


def q4_0_rows(seed, layer, code_tensor, nrows, d, rows=None, row0=0) -> np.ndarray:
    """Q4_0 rows, uint8 [nrows][9d/16]: d/2 nibble-code bytes then d/32 fp16 scales."""
    assert d % 32 == 0
    rb = d * 9 // 16
    out = np.empty((nrows, rb), dtype=np.uint8)
    rows_arr = None if rows is None else np.ascontiguousarray(rows, dtype=np.int32)
    lib().ps_q4_0_rows(seed, layer, code_tensor, _ptr(rows_arr), row0, nrows, d, _ptr(out), rb)
    return out


@functools.lru_cache(maxsize=None)
def zipf_solve(f, density, top_frac=TOP_FRAC, share=TOP_SHARE, cap=P_CAP):
    """(s, A) of p_k = min(cap, A k^-s) with mean `density` and top-`top_frac` share `share`."""
    s, A = ctypes.c_double(), ctypes.c_double()
    rc = lib().ps_zipf_solve(f, density, top_frac, share, cap, ctypes.byref(s), ctypes.byref(A))
    if rc != 0:
        raise ValueError("zipf_solve: bad arguments")
    return s.value, A.value


def zipf_freq(seed, layer, f, s, A, cap=P_CAP):
    perm = np.empty(f, dtype=np.int32)
    p = np.empty(f, dtype=np.float64)
    rank = np.empty(f, dtype=np.int32)
    lib().ps_zipf_freq(seed, layer, T_PERM, f, s, A, cap, _ptr(perm), _ptr(p), _ptr(rank))
    return p, rank


def offsets(p2_bits: np.ndarray, p: np.ndarray) -> np.ndarray:
    f, r = p2_bits.shape
    c = np.empty(f, dtype=np.uint16)
    lib().ps_offsets(_ptr(np.ascontiguousarray(p2_bits)), f, r, _ptr(np.ascontiguousarray(p)), _ptr(c))
    return c


def hot_set(p: np.ndarray, n_hot: int) -> np.ndarray:
    """Ascending ids of the n_hot most frequent neurons (ties broken by lower id)."""
    order = np.lexsort((np.arange(p.size), -p))      # primary key -p, secondary id
    return np.sort(order[:n_hot]).astype(np.int32)


# ----------------------------------------------------------------------------- layers

@dataclass
class Layer:
    cfg: Config
    layer: int
    p1: np.ndarray            # uint16 [r][d]
    p2: np.ndarray            # uint16 [f][r]
    c: np.ndarray             # uint16 [f]
    freq: np.ndarray          # float64 [f]
    slot_of: np.ndarray | None  # int32 [f] (-1 = not resident) or None (identity)
    hot: np.ndarray | None    # int32 ascending resident neuron ids, or None
    w_in: np.ndarray          # uint16 [n_slots][g*d] (fp16) or uint8 [n_slots][g*rowbytes] (Q4_0)
    w_down_t: np.ndarray      # uint16 [n_slots][d] or uint8 [n_slots][rowbytes]
    b_up: np.ndarray | None   # uint16 [n_slots]
    b_down: np.ndarray | None  # uint16 [d]
    extra: dict = field(default_factory=dict)

    @property
    def n_slots(self) -> int:
        return self.w_in.shape[0]


def make_predictor(cfg: Config, layer: int):
    """P1 ~ N(0,1/d) [r][d], P2 ~ N(0,1/r) [f][r], Zipf frequencies and offsets c."""
    s, A = zipf_solve(cfg.f, cfg.density)
    p1 = normal_f16(cfg.seed, layer, T_P1, cfg.r, cfg.d, 1.0 / np.sqrt(cfg.d))
    p2 = normal_f16(cfg.seed, layer, T_P2, cfg.f, cfg.r, 1.0 / np.sqrt(cfg.r))
    freq, _ = zipf_freq(cfg.seed, layer, cfg.f, s, A)
    c = offsets(p2, freq)
    return p1, p2, c, freq


def make_ffn(cfg: Config, layer: int, rows: np.ndarray | None, bias_scale: float | None = None,
             b_down: bool = False):
    """Neuron-major FFN weights for generator rows `rows` (None = all f neurons, in order)."""
    d = cfg.d
    n = cfg.f if rows is None else len(rows)
    sig = 1.0 / np.sqrt(d)
    bsig = sig if bias_scale is None else bias_scale
    if cfg.wtype == F16:
        if cfg.gated:
            w_in = np.empty((n, 2 * d), dtype=np.uint16)
            w_in[:, :d] = normal_f16(cfg.seed, layer, T_WGATE, n, d, sig, rows=rows)
            w_in[:, d:] = normal_f16(cfg.seed, layer, T_WUP, n, d, sig, rows=rows)
        else:
            w_in = normal_f16(cfg.seed, layer, T_WUP, n, d, sig, rows=rows)
        w_down_t = normal_f16(cfg.seed, layer, T_WDOWN, n, d, sig, rows=rows)
    else:
        if cfg.gated:
            raise ValueError("gated Q4_0 layers are not part of any configuration")
        w_in = q4_0_rows(cfg.seed, layer, T_Q4_UP, n, d, rows=rows)
        w_down_t = q4_0_rows(cfg.seed, layer, T_Q4_DOWN, n, d, rows=rows)
    b_up = None
    if cfg.bias_up:
        b_up = normal_f16(cfg.seed, layer, T_BUP, 1, cfg.f, bsig)[0]
        if rows is not None:
            b_up = np.ascontiguousarray(b_up[rows])
    bd = normal_f16(cfg.seed, layer, T_BDOWN, 1, d, bsig)[0] if b_down else None
    return w_in, w_down_t, b_up, bd


def layer_freq(cfg: Config, layer: int) -> np.ndarray:
    """The layer's generated firing frequencies p_i (the law its predictor offsets are calibrated to)."""
    s, A = zipf_solve(cfg.f, cfg.density)
    freq, _ = zipf_freq(cfg.seed, layer, cfg.f, s, A)
    return freq


def make_layer(cfg: Config, layer: int, bias_scale: float | None = None, b_down: bool = False,
               hot: np.ndarray | None = None) -> Layer:
    """One layer's predictor and FFN rows.  With a placement (cfg.hot_frac, or an explicit ascending
    `hot` list of resident neuron ids), only the resident neurons' rows are generated, in ascending
    id order, and slot_of maps ids to them."""
    p1, p2, c, freq = make_predictor(cfg, layer)
    slot_of = None
    if hot is None and cfg.hot_frac is not None:
        hot = hot_set(freq, cfg.n_hot())
    if hot is not None:
        hot = np.ascontiguousarray(hot, dtype=np.int32)
        slot_of = np.full(cfg.f, -1, dtype=np.int32)
        slot_of[hot] = np.arange(hot.size, dtype=np.int32)
    w_in, w_down_t, b_up, bd = make_ffn(cfg, layer, hot, bias_scale, b_down)
    return Layer(cfg, layer, p1, p2, c, freq, slot_of, hot, w_in, w_down_t, b_up, bd)


def make_x(cfg: Config, layer: int, token: int, B: int) -> np.ndarray:
    """Token vectors x ~ N(0,1), fp16 bits [B][d]; independent per (layer, token, b)."""
    return normal_f16(cfg.seed, layer, T_X, B, cfg.d, 1.0, row0=token * B)


def make_x_all(cfg: Config, layers: int, tokens: int, B: int) -> np.ndarray:
    """All token vectors for a decode run, uint16 [tokens][layers][B][d]."""
    out = np.empty((tokens, layers, B, cfg.d), dtype=np.uint16)
    for l in range(layers):
        xs = normal_f16(cfg.seed, l, T_X, tokens * B, cfg.d, 1.0, row0=0)
        out[:, l] = xs.reshape(tokens, B, cfg.d)
    return out


def f16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    return a.view(np.float16).astype(np.float32)


def num_threads() -> int:
    return lib().ps_num_threads()
