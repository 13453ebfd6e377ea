"""CPU oracle of the predictor-gated, neuron-aware sparse FFN -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package.  The product path (the HIP library and its binding) never does.

The arithmetic lives in ``pi_oracle.c`` (plain C, fp64, the method's steps in the order the
pages describe them: predictor, firing mask, placement restriction, compaction, neuron-wise
FFN).  This module only marshals numpy arrays.  fp16 tensors are passed as uint16 bit
patterns (as the workload generator ``synth`` produces them).

Pins: every function here is checked against values fixed independently of it (the IEEE
binary16 definition via numpy, closed forms, hand-worked fixtures in ``tests/golden/``,
brute force on tiny layers, and the dense-equals-sparse invariants) by the ``not gpu`` tests.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libpioracle.so")
_SRC = os.path.join(_HERE, "pi_oracle.c")

F16, Q4_0 = 1, 2


def build(verbose: bool = False) -> str:
    """Compile the oracle with gcc (-O2, OpenMP over independent outputs only)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-o", _LIB_PATH, _SRC, "-lm"]
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
        i64, vp, ci = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        L.pio_half.restype = ctypes.c_double
        L.pio_half.argtypes = [ctypes.c_uint16]
        L.pio_row_bytes.restype = i64
        L.pio_row_bytes.argtypes = [ci, i64]
        L.pio_decode_row.restype = None
        L.pio_decode_row.argtypes = [vp, ci, i64, vp]
        L.pio_predict.restype = ci
        L.pio_predict.argtypes = [i64, i64, i64, vp, vp, vp, vp, i64, vp, vp, vp]
        L.pio_compact.restype = ci
        L.pio_compact.argtypes = [vp, i64, vp, vp, vp]
        L.pio_sparse_ffn.restype = ci
        L.pio_sparse_ffn.argtypes = [i64, i64, ci, ci, i64, vp, vp, vp, vp, vp, vp, i64, vp, i64, vp, vp]
        L.pio_dense_ffn.restype = ci
        L.pio_dense_ffn.argtypes = [i64, i64, ci, ci, vp, vp, vp, vp, vp, i64, vp, vp]
        L.pio_ffn_layer.restype = ci
        L.pio_ffn_layer.argtypes = [i64, i64, i64, vp, vp, vp, ci, ci, i64, vp, vp, vp, vp, vp, vp, i64,
                                    vp, vp, vp, vp, vp]
        L.pio_num_threads.restype = ci
        L.pio_num_threads.argtypes = []
        L.pio_set_num_threads.restype = None
        L.pio_set_num_threads.argtypes = [ci]
        _lib = L
    return _lib


def _p(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} failed with code {rc}")


def half(bits: int) -> float:
    return lib().pio_half(bits)


def row_bytes(wtype: int, d: int) -> int:
    return lib().pio_row_bytes(wtype, d)


def decode_row(row: np.ndarray, wtype: int, d: int) -> np.ndarray:
    row = np.ascontiguousarray(row)
    out = np.empty(d, dtype=np.float64)
    lib().pio_decode_row(_p(row), wtype, d, _p(out))
    return out


def predict(p1, p2, c, x, want_tok_masks=False):
    """Returns (logits [B][f] f64, union mask [f] u8, per-token masks [B][f] u8 or None)."""
    p1, p2, c, x = _c(p1, np.uint16), _c(p2, np.uint16), _c(c, np.uint16), _c(np.atleast_2d(x), np.uint16)
    r, d = p1.shape
    f = p2.shape[0]
    B = x.shape[0]
    assert p2.shape == (f, r) and c.shape == (f,) and x.shape == (B, d)
    logits = np.empty((B, f), dtype=np.float64)
    mask = np.empty(f, dtype=np.uint8)
    tok = np.empty((B, f), dtype=np.uint8) if want_tok_masks else None
    _check(lib().pio_predict(d, f, r, _p(p1), _p(p2), _p(c), _p(x), B, _p(logits), _p(tok), _p(mask)), "predict")
    return logits, mask, tok


def compact(mask, slot_of=None):
    """Returns (idx int32 [n], n, n_pred)."""
    mask = _c(mask, np.uint8)
    f = mask.size
    slot_of = _c(slot_of, np.int32)
    idx = np.empty(max(f, 1), dtype=np.int32)
    counts = np.zeros(2, dtype=np.int32)
    _check(lib().pio_compact(_p(mask), f, _p(slot_of), _p(idx), _p(counts)), "compact")
    return idx[: counts[0]].copy(), int(counts[0]), int(counts[1])


RELU, REGLU, SQUARED_RELU = 0, 1, 2     # FFN kinds of the C oracle (its `gated` argument)


def _kind(gated, act) -> int:
    """ReGLU when gated; otherwise ReLU, or squared ReLU when act == 1 (the C ABI's pi_act)."""
    if gated and act:
        raise ValueError("squared ReLU is a non-gated form")
    return REGLU if gated else (SQUARED_RELU if act else RELU)


def sparse_ffn(d, f, gated, wtype, w_in, w_down_t, x, idx, b_up=None, b_down=None, slot_of=None,
               want_h=False, act=0):
    """y [B][d] float64 (caller rounds to fp32); optionally h [B][n] float64.  act=1: squared ReLU."""
    w_in, w_down_t = np.ascontiguousarray(w_in), np.ascontiguousarray(w_down_t)
    x = _c(np.atleast_2d(x), np.uint16)
    idx = _c(idx, np.int32)
    B = x.shape[0]
    n = idx.size
    n_slots = w_in.shape[0]
    y = np.empty((B, d), dtype=np.float64)
    h = np.empty((B, max(n, 1)), dtype=np.float64) if want_h else None
    rc = lib().pio_sparse_ffn(d, f, _kind(gated, act), wtype, n_slots, _p(_c(slot_of, np.int32)), _p(w_in), _p(w_down_t),
                              _p(_c(b_up, np.uint16)), _p(_c(b_down, np.uint16)), _p(x), B,
                              _p(idx) if n else None, n, _p(h), _p(y))
    _check(rc, "sparse_ffn")
    return (y, h[:, :n]) if want_h else y


def dense_ffn(d, f, gated, wtype, w_in, w_down_t, x, b_up=None, b_down=None, act=0):
    """Dense FFN over all f neurons: (y [B][d] f64, true mask [B][f] u8)."""
    w_in, w_down_t = np.ascontiguousarray(w_in), np.ascontiguousarray(w_down_t)
    x = _c(np.atleast_2d(x), np.uint16)
    B = x.shape[0]
    y = np.empty((B, d), dtype=np.float64)
    tm = np.empty((B, f), dtype=np.uint8)
    rc = lib().pio_dense_ffn(d, f, _kind(gated, act), wtype, _p(w_in), _p(w_down_t), _p(_c(b_up, np.uint16)),
                             _p(_c(b_down, np.uint16)), _p(x), B, _p(tm), _p(y))
    _check(rc, "dense_ffn")
    return y, tm


def ffn_layer(layer, x, want_logits=True, b_down=None):
    """Whole layer for a ``synth.Layer``: dict(logits, mask, idx, n, n_pred, y)."""
    cfg = layer.cfg
    x = _c(np.atleast_2d(x), np.uint16)
    B = x.shape[0]
    f, d, r = cfg.f, cfg.d, cfg.r
    logits = np.empty((B, f), dtype=np.float64) if want_logits else None
    mask = np.empty(f, dtype=np.uint8)
    idx = np.empty(f, dtype=np.int32)
    counts = np.zeros(2, dtype=np.int32)
    y = np.empty((B, d), dtype=np.float64)
    bd = layer.b_down if b_down is None else b_down
    rc = lib().pio_ffn_layer(d, f, r, _p(layer.p1), _p(layer.p2), _p(layer.c), _kind(cfg.gated, getattr(cfg, "act", 0)),
                             cfg.wtype,
                             layer.n_slots, _p(_c(layer.slot_of, np.int32)), _p(layer.w_in), _p(layer.w_down_t),
                             _p(_c(layer.b_up, np.uint16)), _p(_c(bd, np.uint16)), _p(x), B, _p(logits),
                             _p(mask), _p(idx), _p(counts), _p(y))
    _check(rc, "ffn_layer")
    n = int(counts[0])
    return dict(logits=logits, mask=mask, idx=idx[:n].copy(), n=n, n_pred=int(counts[1]), y=y)


def num_threads() -> int:
    return lib().pio_num_threads()


def set_num_threads(n: int) -> None:
    lib().pio_set_num_threads(n)


# ------------------------------------------------------------------ offline placement (tiny cases)
# The model the placement solves (the pages name an integer linear program over activation
# frequency and hardware bandwidth, without a formulation): layer l keeps the set H_l on the
# device; a token streams c_l * sum_{i in H_l} p_{l,i} bytes there and c_l * sum_{i not in H_l}
# p_{l,i} bytes on the host, in parallel, so the layer takes the larger of the two times.

def place_objective(neuron_bytes, freq, placed, bw_gpu, bw_host):
    """Expected seconds per token of a placement: sum over layers of
    max(c * (sum of p over placed) / bw_gpu, c * (sum of p over the rest) / bw_host)."""
    t = 0.0
    for c, p, h in zip(neuron_bytes, freq, placed):
        p = np.asarray(p, np.float64)
        on = float(p[np.asarray(h, bool)].sum())
        t += max(c * on / bw_gpu, c * (float(p.sum()) - on) / bw_host)
    return t


def place_exact(neuron_bytes, freq, budget, bw_gpu, bw_host):
    """The optimum by brute force over every subset of all neurons (pure Python: tiny cases only).
    Returns (objective, placement as per-layer boolean arrays)."""
    import itertools
    sizes = [len(p) for p in freq]
    cost = np.concatenate([np.full(n, c, np.int64) for n, c in zip(sizes, neuron_bytes)])
    best, arg = None, None
    for bits in itertools.product((False, True), repeat=int(sum(sizes))):
        sel = np.array(bits, bool)
        if int(cost[sel].sum()) > budget:
            continue
        placed = np.split(sel, np.cumsum(sizes)[:-1])
        t = place_objective(neuron_bytes, freq, placed, bw_gpu, bw_host)
        if best is None or t < best:
            best, arg = t, placed
    return best, arg


def place_exact_prefix(neuron_bytes, freq, budget, bw_gpu, bw_host):
    """The optimum over placements that keep, in every layer, its n_l most frequent neurons (ties:
    lower id), by enumerating every (n_0, n_1, ...) under the budget.  Returns the objective."""
    import itertools
    orders = [np.argsort(-np.asarray(p, np.float64), kind="stable") for p in freq]
    best = None
    for ns in itertools.product(*[range(len(p) + 1) for p in freq]):
        if sum(n * c for n, c in zip(ns, neuron_bytes)) > budget:
            continue
        placed = []
        for n, order, p in zip(ns, orders, freq):
            h = np.zeros(len(p), bool)
            h[order[:n]] = True
            placed.append(h)
        t = place_objective(neuron_bytes, freq, placed, bw_gpu, bw_host)
        if best is None or t < best:
            best = t
    return best


# ------------------------------------------------------------------ adaptive predictor size
# The pages name adaptive predictors, sized per layer so that they take little GPU memory, without
# a formula.  The reading checked here: a layer's rank follows the entropy of its firing pattern
# (independent neurons: H = sum_i h(p_i) bits, h the binary entropy, rounded to 1/1024 bit); rank
# r_l(lambda) = the largest grid rank (r_min + k step, <= r_max) not above max(r_min, lambda H_l),
# for the largest lambda at which sum_l 2 r_l (d_l + f_l) fits the budget; at that budget's edge,
# the raises that share the next lambda are taken in layer order while they fit.

def binary_entropy_bits(p) -> float:
    """sum_i h(p_i) in bits, h(p) = -p log2 p - (1-p) log2 (1-p), h(0) = h(1) = 0 (exact sum)."""
    import math
    terms = []
    for v in np.asarray(p, np.float64).ravel():
        if 0.0 < v < 1.0:
            terms.append(-(v * math.log2(v) + (1.0 - v) * math.log2(1.0 - v)))
    return math.fsum(terms)


def predictor_ranks(d_model, d_ffn, freq, budget, r_min, r_max, step):
    """Ranks by the definition above, in exact rational arithmetic: evaluate r(lambda) at every
    lambda where some layer's rank changes, keep the largest that fits, then take the next
    lambda's raises in layer order while they fit.  Returns (ranks, rounded entropies)."""
    from fractions import Fraction
    L = len(d_ffn)
    H = [round(binary_entropy_bits(p) * 1024) / 1024 for p in freq]
    per_rank = [2 * (int(d) + int(f)) for d, f in zip(d_model, d_ffn)]
    if sum(r_min * c for c in per_rank) > budget:
        raise ValueError("budget below r_min in every layer")

    def ranks_at(lam):
        out = []
        for h in H:
            r = r_min
            if h > 0:
                t = lam * Fraction(h)                 # the rank lambda H_l asks for
                while r + step <= r_max and r + step <= t:
                    r += step
            out.append(r)
        return out

    def cost(rs):
        return sum(r * c for r, c in zip(rs, per_rank))

    lams = sorted({Fraction(r) / Fraction(h) for h in H if h > 0 for r in range(r_min + step, r_max + 1, step)})
    ranks = [r_min] * L
    nxt = None
    for lam in lams:
        rs = ranks_at(lam)
        if cost(rs) <= budget:
            ranks = rs
        else:
            nxt = lam
            break
    if nxt is not None:
        target = ranks_at(nxt)
        for l in range(L):
            if target[l] > ranks[l]:
                trial = list(ranks)
                trial[l] = target[l]
                if cost(trial) > budget:
                    break
                ranks = trial
    return ranks, H
