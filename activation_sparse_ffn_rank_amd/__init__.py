"""Predictor-gated, neuron-aware sparse FFN for MI355X (gfx950): a C-ABI HIP library plus a thin binding.

PowerInfer (arXiv 2312.12456) observes that a ReLU-family FFN fires only a small,
input-dependent set of neurons per token; a low-rank predictor picks them and a neuron-aware
sparse operator computes only those, with a GPU index naming the neurons resident on the
device.  This package exposes that decode-step hot path:

* ``pi_predict``    predictor GEMVs -> firing mask (batch union)
* ``pi_compact``    placement restriction + ascending active-neuron list
* ``pi_sparse_ffn`` gathered up/gate rows with fused ReLU/ReGLU, then the active rows of W_down^T
* ``pi_ffn_layer``  all three, stream-ordered (also as ``pi_predict_hidden`` + ``pi_ffn_layer_from_hidden``)

All compute runs in ``libpi.so``; torch only provides device memory and streams.
"""
from ._abi import (PI_F16, PI_MAX_BATCH, PI_Q4_0, PiError, make_ffn, make_predictor, pi_compact, pi_ffn_layer,
                   pi_ffn_layer_from_hidden, pi_predict, pi_predict_hidden, pi_sparse_ffn,
                   pi_status_string, pi_version, pi_workspace_bytes)
from .layer import DeviceLayer

__all__ = ["PI_F16", "PI_Q4_0", "PI_MAX_BATCH", "PiError", "make_ffn", "make_predictor", "pi_compact",
           "pi_ffn_layer", "pi_ffn_layer_from_hidden", "pi_predict_hidden", "pi_predict", "pi_sparse_ffn", "pi_status_string", "pi_version", "pi_workspace_bytes",
           "DeviceLayer"]
