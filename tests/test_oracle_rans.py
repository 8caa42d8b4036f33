"""Pins for oracle.rans: hand-derived streams, the frequency quantizer's
invariants and closed forms, lossless round trips over a fuzz grid, the coded
size against the ideal code length, and the degenerate single-code tensor."""
import numpy as np
import pytest

from oracle import huffman, quant, rans
from synth import CODE_KINDS, fuzz_codes
from tests._golden import load


def _units(vals):
    return [int(v, 16) for v in vals]


@pytest.mark.parametrize("case", ["a", "b"])
def test_golden_streams(case):
    g, _ = load("rans_tiny.txt")
    counts = [int(v) for v in g[f"{case}_counts"][0]]
    freqs = rans.quantize_freqs(counts)
    assert freqs.tolist() == [int(v) for v in g[f"{case}_freqs"][0]]
    q = np.array([int(v) for v in g[f"{case}_q"][0]], dtype=np.uint8)
    chunk, lanes = int(g[f"{case}_chunk"][0][0]), int(g[f"{case}_lanes"][0][0])
    units, offs = rans.encode(q, freqs, chunk, lanes)
    assert units.tolist() == _units(g[f"{case}_units"][0])
    assert offs.tolist() == [int(v) for v in g[f"{case}_offs"][0]]
    assert rans.decode(units, offs, freqs, q.size, chunk, lanes).tolist() == q.tolist()


def test_frequency_quantizer_invariants():
    rng = np.random.default_rng(0)
    for trial in range(200):
        a = int(rng.choice([2, 16, 256]))
        counts = np.zeros(a, dtype=np.int64)
        k = int(rng.integers(1, a + 1))
        idx = rng.choice(a, size=k, replace=False)
        counts[idx] = rng.geometric(0.05, size=k) * rng.integers(1, 1000, size=k)
        f = rans.quantize_freqs(counts)
        assert int(f.sum()) == rans.M
        assert ((f > 0) == (counts > 0)).all()
        ideal = rans.M * counts / counts.sum()
        # codes that were not raised to 1 stay within one slot plus the
        # correction that the raised ones force
        raised = int(((counts > 0) & (ideal < 1)).sum())
        assert (np.abs(f - ideal)[counts > 0] <= 1 + raised).all()


def test_frequency_quantizer_closed_forms():
    # dyadic histograms scale exactly
    assert rans.quantize_freqs([8, 4, 2, 2]).tolist() == [2048, 1024, 512, 512]
    assert rans.quantize_freqs([5]).tolist() == [4096]
    assert rans.quantize_freqs([0, 3, 0]).tolist() == [0, 4096, 0]
    # 1/3 each: floors 1365 x 3 = 4095, the remaining slot goes to the lowest code
    assert rans.quantize_freqs([1, 1, 1]).tolist() == [1366, 1365, 1365]
    # a vanishing code keeps one slot; the excess is taken from the largest
    assert rans.quantize_freqs([10 ** 9, 1]).tolist() == [4095, 1]
    with pytest.raises(ValueError):
        rans.quantize_freqs([0, 0])


GRID = [(4, 1, 16), (8, 2, 32), (4, 8, 64), (8, 32, 96), (4, 64, 128), (8, 64, 256), (4, 16, 48)]


@pytest.mark.parametrize("bits,lanes,chunk", GRID)
@pytest.mark.parametrize("kind", CODE_KINDS)
def test_round_trip(bits, lanes, chunk, kind):
    seed = bits * 131 + lanes * 7 + chunk + CODE_KINDS.index(kind)
    q = fuzz_codes(seed, 3 * chunk + 17, bits, kind)
    freqs = rans.quantize_freqs(quant.histogram(q, bits))
    units, offs = rans.encode(q, freqs, chunk, lanes)
    assert rans.decode(units, offs, freqs, q.size, chunk, lanes).tolist() == q.tolist()


def test_corrupted_streams_are_rejected():
    q = fuzz_codes(5, 300, 4, "skewed")
    freqs = rans.quantize_freqs(quant.histogram(q, 4))
    units, offs = rans.encode(q, freqs, 64, 8)
    with pytest.raises(rans.StreamError):
        rans.decode(units[:-1], np.append(offs[:-1], offs[-1] - 1), freqs, q.size, 64, 8)
    bad = units.copy()
    bad[0] ^= 0x5A5A
    with pytest.raises(rans.StreamError):
        rans.decode(bad, offs, freqs, q.size, 64, 8)


@pytest.mark.parametrize("kind", ["skewed", "peaked", "uniform"])
def test_coded_size_tracks_the_ideal_length(kind):
    """Renormalization units carry the information: 16 x units equals the
    ideal length sum -log2(f/M) up to each lane's final state (at most 32
    bits) and the coder's rounding (well under 0.01 bit per code here)."""
    bits, lanes, chunk = 8, 32, 4096
    q = fuzz_codes(11, 4 * chunk, bits, kind)
    freqs = rans.quantize_freqs(quant.histogram(q, bits))
    units, offs = rans.encode(q, freqs, chunk, lanes)
    n_chunks = len(offs) - 1
    renorm_bits = 16 * (len(units) - 2 * lanes * n_chunks)
    ideal = rans.ideal_bits(q, freqs)
    assert renorm_bits <= ideal + 0.01 * q.size
    assert renorm_bits >= ideal - 16 * lanes * n_chunks - 0.01 * q.size


def test_single_code_tensor_costs_only_the_states():
    q = np.full(1000, 7, dtype=np.uint8)
    freqs = rans.quantize_freqs(quant.histogram(q, 4))
    units, offs = rans.encode(q, freqs, 256, 16)
    assert len(units) == 4 * 2 * 16          # four chunks, two units per lane state
    assert set(units.tolist()) == {0, 1}       # every state stays at L = 0x00010000
    assert rans.decode(units, offs, freqs, q.size, 256, 16).tolist() == q.tolist()


def test_rans_beats_huffman_on_peaked_codes_and_follows_entropy():
    """On a histogram where one code dominates, the Huffman code cannot go
    below one bit per code while rANS follows the entropy."""
    q = fuzz_codes(3, 20000, 4, "peaked")
    counts = quant.histogram(q, 4)
    h = quant.entropy_bits(counts)
    lengths = huffman.code_lengths(counts, 12)
    l_huff = huffman.mean_length(counts, lengths)
    freqs = rans.quantize_freqs(counts)
    r = rans.ideal_bits(q, freqs) / q.size
    assert h <= r < h + 0.01
    assert l_huff >= 1.0 and r < l_huff
