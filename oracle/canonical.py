"""Canonical code assignment (oracle; test infrastructure only).

The pages describe a Huffman code built from value frequencies (gist.science
technical summary, Methodology item 2) but never say how codewords are chosen
for given lengths.  Reading: the canonical rule also used by DEFLATE
(RFC 1951, section 3.2.2) - codes of one length are consecutive integers in
increasing symbol order, every shorter code precedes every longer one, and
the first code is all zeros.  Codewords are written most significant bit
first.  The whole codebook is therefore fixed by the per-symbol lengths.
"""
from __future__ import annotations

import numpy as np


def canonical_codes(lengths: np.ndarray) -> np.ndarray:
    """Codeword (as an integer, MSB-first) of every symbol; absent symbols get 0.

    1. ``bl_count[l]`` = number of symbols of length ``l``.
    2. ``code = 0``; for ``l = 1 .. max``: ``code = (code + bl_count[l-1]) << 1``
       and ``next[l] = code`` (``bl_count[0]`` is taken as 0).
    3. Symbols in increasing value with a nonzero length take ``next[l]++``.
    """
    ls = [int(x) for x in np.asarray(lengths).ravel()]
    max_len = max(ls) if ls else 0
    bl_count = [0] * (max_len + 1)
    for l in ls:
        if l > 0:
            bl_count[l] += 1
    nxt = [0] * (max_len + 1)
    code = 0
    for l in range(1, max_len + 1):
        code = (code + bl_count[l - 1]) << 1
        nxt[l] = code
    codes = np.zeros(len(ls), dtype=np.int64)
    for s, l in enumerate(ls):
        if l > 0:
            codes[s] = nxt[l]
            nxt[l] += 1
    return codes


def codeword_str(code: int, length: int) -> str:
    """The codeword as a string of ``'0'``/``'1'``, first bit first."""
    return format(code, f"0{length}b") if length > 0 else ""
