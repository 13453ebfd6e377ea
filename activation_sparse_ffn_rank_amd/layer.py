"""Device-resident layer: uploads host arrays once and keeps the ABI descriptors.

Memory is plain torch device memory (HBM); the descriptors point into it.  Weights are kept
neuron-major as the C ABI expects, so every active neuron is one contiguous row read.
"""
from __future__ import annotations

import numpy as np
import torch

from . import _abi


def _dev(a: np.ndarray | None, device) -> torch.Tensor | None:
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    t = torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a)
    return t.to(device, non_blocking=False)


class DeviceLayer:
    """One layer's predictor and resident FFN weights in HBM.

    Host arrays use fp16 bit patterns (uint16) for fp16 tensors and raw bytes (uint8) for
    Q4_0 rows, with shapes p1 [r][d], p2 [f][r], c [f], w_in [n_slots][...], w_down_t
    [n_slots][...], slot_of [f] (or None), b_up [n_slots] (or None), b_down [d] (or None).
    """

    def __init__(self, *, p1, p2, c, w_in, w_down_t, d_model, d_ffn, gated, wtype, slot_of=None, b_up=None,
                 b_down=None, act=0, device="cuda"):
        self.d_model, self.d_ffn, self.gated, self.wtype = d_model, d_ffn, bool(gated), wtype
        self.p1, self.p2, self.c = _dev(p1, device), _dev(p2, device), _dev(c, device)
        self.w_in = _dev(np.ascontiguousarray(w_in).reshape(w_in.shape[0], -1), device)
        self.w_down_t = _dev(np.ascontiguousarray(w_down_t).reshape(w_down_t.shape[0], -1), device)
        self.slot_of = _dev(slot_of, device)
        self.b_up, self.b_down = _dev(b_up, device), _dev(b_down, device)
        self.pred = _abi.make_predictor(self.p1, self.p2, self.c)
        self.ffn = _abi.make_ffn(self.w_in, self.w_down_t, d_model=d_model, d_ffn=d_ffn, gated=self.gated,
                                 wtype=wtype, slot_of=self.slot_of, b_up=self.b_up, b_down=self.b_down, act=act)

    @classmethod
    def from_host(cls, layer, device="cuda", b_down=None):
        """From any object carrying the host arrays (e.g. a generated layer)."""
        cfg = layer.cfg
        return cls(p1=layer.p1, p2=layer.p2, c=layer.c, w_in=layer.w_in, w_down_t=layer.w_down_t, d_model=cfg.d,
                   d_ffn=cfg.f, gated=cfg.gated, wtype=cfg.wtype, slot_of=layer.slot_of, b_up=layer.b_up,
                   b_down=layer.b_down if b_down is None else b_down, act=getattr(cfg, "act", 0), device=device)

    @property
    def n_slots(self) -> int:
        return int(self.w_in.shape[0])

    def workspace(self, batch: int, device="cuda") -> torch.Tensor:
        """Zero-filled workspace for pi_ffn_layer (it must start zeroed; calls leave it ready)."""
        n = _abi.pi_workspace_bytes(self.pred, self.ffn, batch)
        if n == 0:
            raise ValueError("invalid layer for the C ABI")
        return torch.zeros(n, dtype=torch.uint8, device=device)
