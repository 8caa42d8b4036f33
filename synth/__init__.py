"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This module draws random numbers and nothing else: it holds none of the
method's arithmetic (no quantizer, no code construction, no stream layout, no
dequantization).  Both the CPU oracle and the HIP path receive exactly these
arrays as inputs.

Workloads (weights are float32, stored ``[out][in]`` row-major, the order in
which a PyTorch ``nn.Linear`` keeps its weight):

* ``tensor_2048``   2048 x 2048, N(0, 0.02), ``default_rng(0)``.
* ``tensor_4096``   4096 x 4096, Laplace(0, 0.015).
* ``smollm_stack``  24 layers of {q,k,v,o 2048x2048; gate,up 8192x2048;
  down 2048x8192} plus a 49152 x 2048 embedding; Student-t(4) scaled so the
  tensor's std is sigma_T ~ U(0.01, 0.04).
* ``phi3_stack``    32 layers of {qkv 9216x3072, o 3072x3072,
  gate_up 16384x3072, down 3072x8192}; Student-t(5) with std 0.02.
* ``mistral_stack`` 32 layers of {q 4096x4096, k 1024x4096, v 1024x4096,
  o 4096x4096, gate 14336x4096, up 14336x4096, down 4096x14336};
  Student-t(4) with std 0.02.

Seeds: the 2048 tensor uses ``default_rng(0)``; every other tensor ``t`` of
workload ``k`` uses ``default_rng(SeedSequence(0, spawn_key=(k, t)))`` with
``t`` counted layer-major in the listing order above; activations for GEMV
group ``g`` use ``spawn_key=(k, 10000 + g)``.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np

WORKLOAD_IDS = {
    "tensor_2048": 1,
    "tensor_4096": 2,
    "smollm_stack": 3,
    "phi3_stack": 4,
    "mistral_stack": 5,
}


# Clip factor of the Mistral-shaped workload's unsigned 4-bit codes: each
# tensor's range end is MISTRAL_CLIP_SIGMA * std(w), so that the stack, coded
# in one-row chunks of 64 lanes, takes 3.90 bits per weight (found by
# ``python -m oracle.clip_calibration``; 3.9006 on layer 0, 3.9005 on layer 1).
MISTRAL_CLIP_SIGMA = 1.9219

@dataclass(frozen=True)
class TensorSpec:
    """One weight matrix of a workload: ``rows`` = out features, ``cols`` = in."""

    workload: str
    index: int          # position in the workload's enumeration (seed key)
    layer: int          # -1 for tensors outside the layer stack
    name: str
    rows: int
    cols: int
    group: str          # tensors with the same group share one GEMV input

    @property
    def numel(self) -> int:
        return self.rows * self.cols


def _rng(workload: str, t: int) -> np.random.Generator:
    k = WORKLOAD_IDS[workload]
    if k == 1:
        return np.random.default_rng(0)
    return np.random.default_rng(np.random.SeedSequence(0, spawn_key=(k, t)))


# (name, rows=out, cols=in, GEMV group)
_SMOLLM_LAYER = [
    ("q", 2048, 2048, "qkv"), ("k", 2048, 2048, "qkv"), ("v", 2048, 2048, "qkv"),
    ("o", 2048, 2048, "o"),
    ("gate", 8192, 2048, "gate_up"), ("up", 8192, 2048, "gate_up"),
    ("down", 2048, 8192, "down"),
]
_PHI3_LAYER = [
    ("qkv", 9216, 3072, "qkv"), ("o", 3072, 3072, "o"),
    ("gate_up", 16384, 3072, "gate_up"), ("down", 3072, 8192, "down"),
]
_MISTRAL_LAYER = [
    ("q", 4096, 4096, "qkv"), ("k", 1024, 4096, "qkv"), ("v", 1024, 4096, "qkv"),
    ("o", 4096, 4096, "o"),
    ("gate", 14336, 4096, "gate_up"), ("up", 14336, 4096, "gate_up"),
    ("down", 4096, 14336, "down"),
]


def tensor_specs(workload: str) -> list[TensorSpec]:
    """Every weight matrix of ``workload`` in seed order."""
    if workload == "tensor_2048":
        return [TensorSpec(workload, 0, -1, "w", 2048, 2048, "w")]
    if workload == "tensor_4096":
        return [TensorSpec(workload, 0, -1, "w", 4096, 4096, "w")]
    layer_def, n_layers = {
        "smollm_stack": (_SMOLLM_LAYER, 24),
        "phi3_stack": (_PHI3_LAYER, 32),
        "mistral_stack": (_MISTRAL_LAYER, 32),
    }[workload]
    out = []
    t = 0
    for layer in range(n_layers):
        for name, rows, cols, group in layer_def:
            out.append(TensorSpec(workload, t, layer, f"L{layer}.{name}", rows, cols, group))
            t += 1
    if workload == "smollm_stack":
        out.append(TensorSpec(workload, t, -1, "embed", 49152, 2048, "embed"))
    return out


def _student_t(rng: np.random.Generator, nu: float, std: float, shape) -> np.ndarray:
    # Student-t scaled so that its standard deviation is ``std``.
    t = rng.standard_t(nu, size=shape)
    return (t * (std / math.sqrt(nu / (nu - 2.0)))).astype(np.float32)


def weights(spec: TensorSpec) -> np.ndarray:
    """The float32 ``[rows][cols]`` weight of one tensor (deterministic)."""
    rng = _rng(spec.workload, spec.index)
    shape = (spec.rows, spec.cols)
    if spec.workload == "tensor_2048":
        return rng.normal(0.0, 0.02, size=shape).astype(np.float32)
    if spec.workload == "tensor_4096":
        return rng.laplace(0.0, 0.015, size=shape).astype(np.float32)
    if spec.workload == "smollm_stack":
        sigma = rng.uniform(0.01, 0.04)
        return _student_t(rng, 4.0, sigma, shape)
    if spec.workload == "phi3_stack":
        return _student_t(rng, 5.0, 0.02, shape)
    if spec.workload == "mistral_stack":
        return _student_t(rng, 4.0, 0.02, shape)
    raise KeyError(spec.workload)


def activations_f32(workload: str, group_index: int, cols: int, batch: int) -> np.ndarray:
    """GEMV input ``x`` as float32 N(0, 1), shape ``[batch][cols]``.

    The GEMV consumes these rounded to bf16 (``activations_bf16``).
    """
    k = WORKLOAD_IDS[workload]
    rng = np.random.default_rng(np.random.SeedSequence(0, spawn_key=(k, 10000 + group_index)))
    return rng.standard_normal(size=(batch, cols), dtype=np.float32)


def activations_bf16(workload: str, group_index: int, cols: int, batch: int) -> np.ndarray:
    """``activations_f32`` rounded to bf16 by torch (CPU); returned as uint16 bits."""
    import torch

    x = torch.from_numpy(activations_f32(workload, group_index, cols, batch))
    return x.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


# ---------------------------------------------------------------------------
# Small code arrays for fuzzing the codec directly (no weights involved).
# ---------------------------------------------------------------------------

CODE_KINDS = ("uniform", "skewed", "peaked", "degenerate", "two", "sparse")


def fuzz_codes(seed: int, n: int, bits: int, kind: str) -> np.ndarray:
    """``n`` integer codes in ``[0, 2**bits)`` drawn from a histogram of ``kind``.

    * uniform    - every code equally likely
    * skewed     - geometric decay away from a random centre (ratio 0.7)
    * peaked     - very steep decay (ratio 0.2): long codes, tiny probabilities
    * degenerate - one code only
    * two        - two codes
    * sparse     - a random handful of codes with random weights
    """
    rng = np.random.default_rng(np.random.SeedSequence(seed, spawn_key=(bits, CODE_KINDS.index(kind))))
    a = 1 << bits
    if kind == "uniform":
        return rng.integers(0, a, size=n, dtype=np.int64).astype(np.uint8)
    if kind in ("skewed", "peaked"):
        r = 0.7 if kind == "skewed" else 0.2
        centre = int(rng.integers(0, a))
        p = r ** np.abs(np.arange(a) - centre).astype(np.float64)
        p /= p.sum()
        return rng.choice(a, size=n, p=p).astype(np.uint8)
    if kind == "degenerate":
        v = int(rng.integers(0, a))
        return np.full(n, v, dtype=np.uint8)
    if kind == "two":
        vals = rng.choice(a, size=2, replace=False)
        return vals[rng.integers(0, 2, size=n)].astype(np.uint8)
    if kind == "sparse":
        k = int(rng.integers(3, min(a, 12) + 1))
        vals = rng.choice(a, size=k, replace=False)
        p = rng.random(k) ** 3 + 1e-3
        p /= p.sum()
        return vals[rng.choice(k, size=n, p=p)].astype(np.uint8)
    raise KeyError(kind)
