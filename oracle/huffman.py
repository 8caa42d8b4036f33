"""Optimal prefix-code lengths (oracle; test infrastructure only).

EntroLLM builds a Huffman code from the frequencies of the quantized weight
values: frequent values get short codes, rare values long ones, and the
compression is lossless (gist.science technical summary, Methodology item 2;
shd-paper.top summary, key design item 2).  A Huffman code is by definition a
minimum-cost prefix code, so the oracle computes that definition:

* ``huffman_lengths``  - the classic two-smallest merge on a binary heap keyed
  ``(count, node_id)``; leaves have ``node_id = symbol`` and internal nodes
  ``2^b, 2^b + 1, ...`` in creation order (only to make ties deterministic).
* ``package_merge``    - the minimum-cost code among those with every length
  at most ``L`` (Larmore and Hirschberg's package-merge, coin-collector form).
  The pages state no length limit; the decoder tables need one (16 for 8-bit
  codes, 12 for 4-bit codes).
* ``code_lengths``     - Huffman, replaced by package-merge only when the
  Huffman code is longer than the limit.

A tensor whose codes are all one value gets that value a length-1 code; an
empty histogram is an error.
"""
from __future__ import annotations

import heapq

import numpy as np


def huffman_lengths(counts: np.ndarray) -> np.ndarray:
    """Unconstrained Huffman code length of every symbol (0 for absent ones)."""
    counts = np.asarray(counts, dtype=np.int64)
    a = len(counts)
    used = [s for s in range(a) if counts[s] > 0]
    if not used:
        raise ValueError("empty histogram: no code can be built")
    lengths = np.zeros(a, dtype=np.int64)
    if len(used) == 1:
        lengths[used[0]] = 1
        return lengths
    parent: dict[int, int] = {}
    heap = [(int(counts[s]), s) for s in used]
    heapq.heapify(heap)
    next_id = a
    while len(heap) > 1:
        c1, n1 = heapq.heappop(heap)
        c2, n2 = heapq.heappop(heap)
        parent[n1] = next_id
        parent[n2] = next_id
        heapq.heappush(heap, (c1 + c2, next_id))
        next_id += 1
    for s in used:
        d = 0
        node = s
        while node in parent:
            node = parent[node]
            d += 1
        lengths[s] = d
    return lengths


def package_merge(counts: np.ndarray, limit: int) -> np.ndarray:
    """Minimum-cost prefix code with every length ``<= limit`` (coin collector).

    1. The leaf list holds the used symbols sorted by (count, symbol).
    2. ``limit - 1`` times: pair adjacent items of the current list into
       packages (an odd last item is dropped) and merge the packages with a
       fresh copy of the leaves, stably, leaves first on equal weight.
    3. The first ``2(n - 1)`` items of the final list are selected; a symbol's
       length is the number of selected items that contain it.
    """
    counts = np.asarray(counts, dtype=np.int64)
    a = len(counts)
    used = sorted((s for s in range(a) if counts[s] > 0), key=lambda s: (counts[s], s))
    n = len(used)
    if n == 0:
        raise ValueError("empty histogram: no code can be built")
    lengths = np.zeros(a, dtype=np.int64)
    if n == 1:
        lengths[used[0]] = 1
        return lengths
    if (1 << limit) < n:
        raise ValueError(f"{n} symbols cannot have codes of length <= {limit}")

    # An item is (weight, multiplicity of every symbol inside it).
    def leaves():
        out = []
        for s in used:
            m = np.zeros(a, dtype=np.int64)
            m[s] = 1
            out.append((int(counts[s]), m))
        return out

    current = leaves()
    for _ in range(limit - 1):
        packages = []
        for i in range(0, len(current) - 1, 2):
            w1, m1 = current[i]
            w2, m2 = current[i + 1]
            packages.append((w1 + w2, m1 + m2))
        fresh = leaves()
        merged = []
        i = j = 0
        while i < len(fresh) or j < len(packages):
            if j >= len(packages) or (i < len(fresh) and fresh[i][0] <= packages[j][0]):
                merged.append(fresh[i])
                i += 1
            else:
                merged.append(packages[j])
                j += 1
        current = merged
    for _, m in current[: 2 * (n - 1)]:
        lengths += m
    return lengths


def code_lengths(counts: np.ndarray, limit: int) -> np.ndarray:
    """Huffman lengths, or package-merge lengths if Huffman exceeds ``limit``."""
    h = huffman_lengths(counts)
    if h.max() <= limit:
        return h
    return package_merge(counts, limit)


def kraft_sum(lengths: np.ndarray) -> float:
    """``sum 2^-l`` over used symbols (exact in float64 for l <= 52)."""
    ls = np.asarray(lengths, dtype=np.int64)
    return float(sum(2.0 ** (-int(l)) for l in ls if l > 0))


def mean_length(counts: np.ndarray, lengths: np.ndarray) -> float:
    """Average code length ``sum p_s l_s`` in bits per symbol."""
    c = np.asarray(counts, dtype=np.float64)
    return float((c * np.asarray(lengths, dtype=np.float64)).sum() / c.sum())
