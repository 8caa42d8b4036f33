"""Pins for oracle.canonical: hand-derived fixture and the defining properties."""
import numpy as np
import pytest

from oracle import huffman
from oracle.canonical import canonical_codes, codeword_str
from tests._golden import load


def test_golden_tiny():
    g, _ = load("canonical_tiny.txt")
    lengths = np.array([int(x) for x in g["lengths"][0]])
    codes = canonical_codes(lengths)
    for sym, word in g["code"]:
        s = int(sym)
        assert codeword_str(int(codes[s]), int(lengths[s])) == word


@pytest.mark.parametrize("seed", range(30))
def test_canonical_properties(seed):
    """Prefix-free; ordered by (length, symbol); no gaps; first code zero.

    Together these fix the canonical code uniquely: left-aligned to the
    longest length, the codes in (length, symbol) order start at 0 and each
    next code begins exactly where the previous one's interval ends.
    """
    rng = np.random.default_rng(seed)
    bits = int(rng.choice([4, 8]))
    a = 1 << bits
    counts = np.zeros(a, dtype=np.int64)
    k = int(rng.integers(2, a + 1))
    counts[rng.choice(a, size=k, replace=False)] = rng.integers(1, 10 ** int(rng.integers(1, 6)), size=k)
    lengths = huffman.code_lengths(counts, 16 if bits == 8 else 12)
    codes = canonical_codes(lengths)
    used = [s for s in range(a) if lengths[s] > 0]
    words = {s: codeword_str(int(codes[s]), int(lengths[s])) for s in used}
    for s in used:
        assert len(words[s]) == lengths[s]
        for t in used:
            if s != t:
                assert not words[t].startswith(words[s])
    order = sorted(used, key=lambda s: (lengths[s], s))
    m = int(lengths.max())
    pos = 0
    for s in order:
        assert int(codes[s]) << (m - int(lengths[s])) == pos
        pos += 1 << (m - int(lengths[s]))
    assert pos == 1 << m  # complete (Kraft sum 1)


def test_single_symbol_code_is_zero():
    lengths = np.zeros(16, dtype=np.int64)
    lengths[9] = 1
    assert canonical_codes(lengths)[9] == 0
