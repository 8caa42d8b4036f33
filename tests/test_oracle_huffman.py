"""Pins for oracle.huffman: hand-derived fixture, brute force, closed forms, invariants."""
import itertools
import math

import numpy as np
import pytest

from oracle import huffman
from oracle.quant import entropy_bits
from tests._golden import load


def brute_force_min_cost(counts, max_len):
    """Minimum of sum c*l over all length vectors in {1..max_len}^n with Kraft <= 1."""
    counts = [c for c in counts if c > 0]
    n = len(counts)
    best = None
    for ls in itertools.product(range(1, max_len + 1), repeat=n):
        if sum(2.0 ** -l for l in ls) <= 1.0:
            cost = sum(c * l for c, l in zip(counts, ls))
            best = cost if best is None else min(best, cost)
    return best


def cost(counts, lengths):
    return int((np.asarray(counts) * np.asarray(lengths)).sum())


def test_golden_tiny():
    g, _ = load("huffman_tiny.txt")
    counts = np.array([int(x) for x in g["counts"][0]])
    h = huffman.huffman_lengths(counts)
    assert cost(counts, h) == int(g["unlimited_cost"][0][0])
    assert list(h) == [int(x) for x in g["unlimited_lengths"][0]]
    lim = int(g["limit"][0][0])
    pm = huffman.package_merge(counts, lim)
    assert cost(counts, pm) == int(g["limited_cost"][0][0])
    assert list(pm) == [int(x) for x in g["limited_lengths"][0]]
    assert list(huffman.code_lengths(counts, lim)) == list(pm)


@pytest.mark.parametrize("seed", range(40))
def test_huffman_is_optimal_brute_force(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(2, 8))
    counts = rng.integers(1, 60, size=n) ** int(rng.integers(1, 4))
    h = huffman.huffman_lengths(counts)
    assert cost(counts, h) == brute_force_min_cost(counts, n - 1)


@pytest.mark.parametrize("seed", range(40))
def test_package_merge_is_optimal_under_limit(seed):
    rng = np.random.default_rng(1000 + seed)
    n = int(rng.integers(3, 8))
    # geometric-ish counts make the limit bind
    counts = np.array(sorted((2 ** rng.integers(0, 9, size=n)) + rng.integers(0, 3, size=n)))
    limit = int(rng.integers(max(2, math.ceil(math.log2(n))), n))
    pm = huffman.package_merge(counts, limit)
    assert pm.max() <= limit
    assert huffman.kraft_sum(pm) <= 1.0
    assert cost(counts, pm) == brute_force_min_cost(counts, limit)


def test_package_merge_without_binding_limit_matches_huffman_cost():
    rng = np.random.default_rng(7)
    for _ in range(20):
        counts = rng.integers(1, 1000, size=int(rng.integers(2, 30)))
        h = huffman.huffman_lengths(counts)
        pm = huffman.package_merge(counts, int(h.max()) + 2)
        assert cost(counts, pm) == cost(counts, h)


@pytest.mark.parametrize("bits", [4, 8])
def test_kraft_equality_and_entropy_bounds(bits):
    rng = np.random.default_rng(bits)
    for _ in range(25):
        a = 1 << bits
        k = int(rng.integers(2, a + 1))
        counts = np.zeros(a, dtype=np.int64)
        idx = rng.choice(a, size=k, replace=False)
        counts[idx] = (rng.pareto(1.2, size=k) * 100).astype(np.int64) + 1
        h = huffman.huffman_lengths(counts)
        assert huffman.kraft_sum(h) == 1.0
        H = entropy_bits(counts)
        L = huffman.mean_length(counts, h)
        assert H - 1e-12 <= L < H + 1
        # frequent values never get longer codes than rarer ones
        used = np.flatnonzero(counts)
        for s in used:
            for t in used:
                if counts[s] > counts[t]:
                    assert h[s] <= h[t]
        limit = 16 if bits == 8 else 12
        cl = huffman.code_lengths(counts, min(limit, max(int(h.max()) - 1, int(np.ceil(np.log2(k))))))
        assert huffman.kraft_sum(cl) <= 1.0
        assert huffman.mean_length(counts, cl) >= H - 1e-12


def test_closed_forms():
    for k in range(1, 9):
        counts = np.full(1 << k, 17)
        h = huffman.huffman_lengths(counts)
        assert set(h.tolist()) == {k}
        assert huffman.mean_length(counts, h) == pytest.approx(entropy_bits(counts)) == pytest.approx(k)
    # dyadic probabilities 1/2, 1/4, 1/8, 1/16, 1/32, 1/32
    counts = np.array([16, 8, 4, 2, 1, 1])
    h = huffman.huffman_lengths(counts)
    assert h.tolist() == [1, 2, 3, 4, 5, 5]
    assert huffman.mean_length(counts, h) == pytest.approx(entropy_bits(counts))
    assert huffman.huffman_lengths(np.array([0, 3, 0, 9])).tolist() == [0, 1, 0, 1]
    assert huffman.huffman_lengths(np.array([0, 0, 5, 0])).tolist() == [0, 0, 1, 0]
    assert huffman.package_merge(np.array([0, 0, 5, 0]), 4).tolist() == [0, 0, 1, 0]


def test_empty_histogram_is_an_error():
    with pytest.raises(ValueError):
        huffman.huffman_lengths(np.zeros(16, dtype=np.int64))
    with pytest.raises(ValueError):
        huffman.package_merge(np.zeros(16, dtype=np.int64), 12)


def test_limit_too_small_is_an_error():
    with pytest.raises(ValueError):
        huffman.package_merge(np.ones(9, dtype=np.int64), 3)
