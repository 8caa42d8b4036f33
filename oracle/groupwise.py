"""Group-wise (block-wise) quantization and the entropy study that compares it
with tensor-level quantization (oracle; test infrastructure only).

EntroLLM argues for quantizing each weight tensor as a whole: block-based
quantizers give every small group of weights its own scale, which stretches
each group over the whole code range, flattens the code histogram and raises
its entropy, so a Huffman code gains little; tensor-level quantization keeps
the histogram peaked (gist.science technical summary, Methodology item 1 and
Problem statement; EntroLLM summary on shd-paper.top, abstract).  The pages
state this qualitatively and give no group-wise formulas.  Readings:

* a group is ``group`` consecutive weights of one row (the input dimension of
  an ``[out][in]`` weight), the usual layout of group-wise weight quantizers;
  ``cols`` must be a multiple of ``group``;
* each group is quantized by exactly the per-tensor rules of ``oracle.quant``
  (asymmetric min-max, or unsigned symmetric range with zero point 2^(b-1)),
  applied to the group's weights alone;
* the code histogram, entropy and Huffman code are taken over all codes of the
  tensor (one codebook per tensor, as for tensor-level codes);
* side information: tensor-level 64 bits per tensor (f32 scale + i32 zero
  point); group-wise one fp16 scale per group, plus a ``bits``-bit zero point
  for the asymmetric scheme (the unsigned zero point is fixed).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import huffman, quant


@dataclass
class GroupQuantized:
    q: np.ndarray          # uint8 codes, same shape as the weight
    scales: np.ndarray     # float32 [rows, cols // group]
    zero_points: np.ndarray  # int64 [rows, cols // group]
    scheme: str
    bits: int
    group: int


def quantize_groupwise(w: np.ndarray, bits: int, group: int, scheme: str) -> GroupQuantized:
    """Quantize every ``group`` consecutive weights of each row on their own.

    ``w`` is 2-D ``[rows, cols]``; the per-group rules are those of
    ``quant.quantize_asymmetric`` / ``quant.quantize_unsigned`` (float64 on the
    float32 weights, scale rounded to float32 first, ``rint``).
    """
    w = np.asarray(w, dtype=np.float32)
    if w.ndim != 2 or w.shape[1] % group:
        raise ValueError("weight must be [rows, cols] with cols a multiple of group")
    Q = (1 << bits) - 1
    rows, cols = w.shape
    g = w.astype(np.float64).reshape(rows, cols // group, group)
    if scheme == "asymmetric":
        lo = g.min(axis=2)
        hi = g.max(axis=2)
        s = np.where(hi > lo, ((hi - lo) / Q), 1.0).astype(np.float32)
        s64 = s.astype(np.float64)
        zp = np.where(hi > lo, np.clip(np.rint(-lo / s64), 0, Q), 0).astype(np.int64)
    elif scheme == "unsigned":
        half = 1 << (bits - 1)
        m = np.abs(g).max(axis=2)
        s = np.where(m > 0, m / (half - 1), 1.0).astype(np.float32)
        s64 = s.astype(np.float64)
        zp = np.full(s.shape, half, dtype=np.int64)
    else:
        raise ValueError(f"unknown scheme {scheme!r}")
    q = np.clip(np.rint(g / s64[:, :, None]) + zp[:, :, None], 0, Q).astype(np.uint8)
    return GroupQuantized(q.reshape(rows, cols), s, zp, scheme, bits, group)


def dequant_groupwise_f64(gq: GroupQuantized) -> np.ndarray:
    """``scale_g * (q - zp_g)`` in float64, for round-off checks."""
    rows, cols = gq.q.shape
    q = gq.q.astype(np.float64).reshape(rows, cols // gq.group, gq.group)
    v = gq.scales.astype(np.float64)[:, :, None] * (q - gq.zero_points[:, :, None])
    return v.reshape(rows, cols)


@dataclass
class CodeStats:
    entropy: float          # H of the code histogram, bits per weight
    mean_len: float         # Huffman mean code length under the length cap
    side_bits: float        # side information, bits per weight
    n: int

    @property
    def total(self) -> float:
        return self.mean_len + self.side_bits


def code_stats(counts: np.ndarray, bits: int, n: int, side_bits_total: float) -> CodeStats:
    """Entropy and capped-Huffman mean length of a code histogram."""
    limit = 16 if bits == 8 else 12
    lengths = huffman.code_lengths(counts, limit)
    return CodeStats(quant.entropy_bits(counts), huffman.mean_length(counts, lengths), side_bits_total / n, n)


def tensor_level_stats(w: np.ndarray, bits: int, scheme: str) -> CodeStats:
    """One scale for the whole tensor (``scheme`` asymmetric, unsigned or mixed)."""
    if scheme == "asymmetric":
        qz = quant.quantize_asymmetric(w, bits)
    elif scheme == "unsigned":
        qz = quant.quantize_unsigned(w, bits)
    else:
        qz = quant.quantize_mixed(w, bits)
    return code_stats(quant.histogram(qz.q, bits), bits, qz.q.size, 64.0)


def groupwise_stats(w: np.ndarray, bits: int, group: int, scheme: str) -> CodeStats:
    """Group-wise codes, one Huffman code over the whole tensor's codes."""
    gq = quantize_groupwise(w, bits, group, scheme)
    n_groups = gq.scales.size
    side = n_groups * (16 + (bits if scheme == "asymmetric" else 0))
    return code_stats(quant.histogram(gq.q, bits), bits, gq.q.size, float(side))
