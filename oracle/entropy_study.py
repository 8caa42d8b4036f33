"""Entropy study: tensor-level versus group-wise quantization on the synthetic
workloads (oracle only; test infrastructure, no GPU).

Tests the method's central premise (gist.science technical summary,
Methodology item 1; EntroLLM summary on shd-paper.top, abstract): codes of a
tensor-level quantizer are more compressible by a Huffman code than codes of a
block-wise one.  For every workload it reports, per quantizer, the code
entropy H, the mean length of the length-capped Huffman code, the side
information (scales and zero points) and their sum, all in bits per weight,
weighted by tensor size.  The readings behind the group-wise quantizer are
listed in ``oracle.groupwise``.

Usage: ``python -m oracle.entropy_study [--sample-layers N] [--out FILE]``.
The layer stacks are sampled: their first ``N`` layers (default 1), all
tensors of each sampled layer; the single tensors are taken whole.
"""
from __future__ import annotations

import argparse
import sys

import numpy as np

from synth import tensor_specs, weights

from . import groupwise

# workload -> (tensor-level scheme the workload uses, include these layers)
WORKLOADS = [
    ("tensor_2048", "asymmetric"),
    ("tensor_4096", "unsigned"),
    ("smollm_stack", "mixed"),
    ("phi3_stack", "mixed"),
    ("mistral_stack", "mixed"),
]

QUANTIZERS = [
    ("tensor-level", None, None),
    ("group 128, asymmetric", 128, "asymmetric"),
    ("group 32, asymmetric", 32, "asymmetric"),
    ("group 128, unsigned", 128, "unsigned"),
    ("group 32, unsigned", 32, "unsigned"),
]


def sample_specs(workload: str, layers: int):
    specs = tensor_specs(workload)
    return [s for s in specs if s.layer < layers and (s.layer >= 0 or workload.startswith("tensor_"))]


def study(layers: int = 1, log=sys.stderr):
    """Rows (workload, bits, quantizer, H, mean length, side bits, total, n)."""
    rows = []
    for workload, scheme in WORKLOADS:
        specs = sample_specs(workload, layers)
        for bits in (4, 8):
            acc = {name: np.zeros(4) for name, _, _ in QUANTIZERS}
            for spec in specs:
                w = weights(spec).reshape(spec.rows, spec.cols)
                for name, group, gscheme in QUANTIZERS:
                    if group is None:
                        st = groupwise.tensor_level_stats(w, bits, scheme)
                    else:
                        st = groupwise.groupwise_stats(w, bits, group, gscheme)
                    acc[name] += np.array([st.entropy * st.n, st.mean_len * st.n, st.side_bits * st.n, st.n])
                print(f"  {workload} {spec.name} layer {spec.layer} {bits}-bit done", file=log, flush=True)
            for name, _, _ in QUANTIZERS:
                h, l, side, n = acc[name]
                rows.append((workload, bits, name, h / n, l / n, side / n, (l + side) / n, int(n)))
    return rows


def table(rows) -> str:
    out = ["| workload | bits | quantizer | H | Huffman mean length | side info | total bits/weight |",
           "|---|---|---|---|---|---|---|"]
    for workload, bits, name, h, l, side, total, n in rows:
        out.append(f"| {workload} | {bits} | {name} | {h:.3f} | {l:.3f} | {side:.3f} | {total:.3f} |")
    return "\n".join(out)


def main(argv=None) -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--sample-layers", type=int, default=1)
    ap.add_argument("--out", default="")
    a = ap.parse_args(argv)
    t = table(study(a.sample_layers))
    print(t)
    if a.out:
        with open(a.out, "w") as f:
            f.write(t + "\n")
    return 0


if __name__ == "__main__":
    raise SystemExit(main())
