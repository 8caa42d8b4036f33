"""Float64 GEMV on dequantized weights (oracle; test infrastructure only).

LazyWeights decodes weights on demand so that the matrix-vector products of
token generation read only coded bytes from DRAM (LazyWeights abstract,
arXiv 2611.17108); EntroLLM notes that token generation is bound by memory
bandwidth (gist.science technical summary, Problem statement).  The product
itself is the plain definition

    y[b][o] = sum_i  w[o][i] * x[b][i]

with ``w`` the bf16 dequantized weight of a ``[rows=out][cols=in]`` matrix and
``x`` bf16 activations, both taken exactly into float64 (numpy matmul).

Error metric (the pages state none): per matrix,
``max_{b,o} |y - y_ref| / max(|y_ref[b][o]|, 1e-3 * max_o |y_ref[b][o]|)``.
"""
from __future__ import annotations

import numpy as np

from .dequant import bf16_to_f64


def gemv_f64(w_bf16: np.ndarray, x_bf16: np.ndarray) -> np.ndarray:
    """``y[batch][rows]`` in float64 from bf16 weights ``[rows][cols]`` and ``x[batch][cols]``."""
    w = bf16_to_f64(w_bf16)
    x = bf16_to_f64(np.atleast_2d(x_bf16))
    return x @ w.T


def rel_err(y: np.ndarray, y_ref: np.ndarray) -> float:
    """Largest floor-guarded relative error of ``y`` against ``y_ref`` (both [batch][rows])."""
    y = np.atleast_2d(np.asarray(y, dtype=np.float64))
    r = np.atleast_2d(np.asarray(y_ref, dtype=np.float64))
    floor = 1e-3 * np.abs(r).max(axis=1, keepdims=True)
    den = np.maximum(np.abs(r), floor)
    den = np.where(den == 0, 1.0, den)
    return float((np.abs(y - r) / den).max()) if r.size else 0.0
