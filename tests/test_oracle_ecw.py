"""Pins for the oracle stream codec (oracle.ecw, oracle.ccodec).

* hand-derived fixtures (tests/golden/ecw_tiny.txt, ecw_pairs_tiny.txt,
  ecw_ahead_tiny.txt), both directions;
* lossless round trip over a grid of lanes, chunk sizes, ragged tails and
  histogram shapes (the pages call the coding lossless);
* word count per chunk = sum over lanes of ceil(bits / 32), computed here
  from the code lengths alone;
* for one lane, the chunk is a plain MSB-first bit string, decoded here by a
  greedy prefix match against a codeword dictionary (no canonical tables);
* the C codec is byte-identical to the Python one;
* malformed streams are rejected.
"""
import numpy as np
import pytest

from oracle import ccodec, ecw, huffman
from oracle.canonical import canonical_codes, codeword_str
from oracle.quant import histogram
from synth import fuzz_codes
from tests._golden import load


def golden():
    g, _ = load("ecw_tiny.txt")
    lengths = np.array([int(x) for x in g["lengths"][0]])
    q = np.array([int(x) for x in g["q"][0]], dtype=np.uint8)
    words = np.array([int(x, 16) for x in g["words"][0]], dtype=np.uint32)
    offs = np.array([int(x) for x in g["chunk_bit_off"][0]], dtype=np.uint64)
    return lengths, q, int(g["chunk"][0][0]), int(g["lanes"][0][0]), words, offs


def test_golden_pairs_encode_decode():
    g, _ = load("ecw_pairs_tiny.txt")
    lengths = np.array([int(x) for x in g["lengths"][0]])
    q = np.array([int(x) for x in g["q"][0]], dtype=np.uint8)
    chunk, lanes = int(g["chunk"][0][0]), int(g["lanes"][0][0])
    offs = np.array([int(x) for x in g["chunk_bit_off"][0]], dtype=np.uint64)
    for rs in (1, 2):
        words = np.array([int(x, 16) for x in g[f"words_steps{rs}"][0]], dtype=np.uint32)
        w, o = ecw.encode(q, lengths, chunk, lanes, rs)
        assert w.tolist() == words.tolist() and o.tolist() == offs.tolist()
        assert ecw.decode(words, offs, lengths, len(q), chunk, lanes, rs).tolist() == q.tolist()
        w2, o2 = ccodec.encode(q, lengths, chunk, lanes, refill_steps=rs)
        assert w2.tolist() == words.tolist() and o2.tolist() == offs.tolist()
        assert ccodec.decode(words, offs, lengths, len(q), chunk, lanes, refill_steps=rs).tolist() == q.tolist()
    # the two orders differ here, so each rule rejects the other's stream
    w1 = np.array([int(x, 16) for x in g["words_steps1"][0]], dtype=np.uint32)
    with pytest.raises(ecw.StreamError):
        ecw.decode(w1, offs, lengths, len(q), chunk, lanes, 2)


def test_golden_ahead_encode_decode():
    g, _ = load("ecw_ahead_tiny.txt")
    lengths = np.array([int(x) for x in g["lengths"][0]])
    q = np.array([int(x) for x in g["q"][0]], dtype=np.uint8)
    chunk, lanes = int(g["chunk"][0][0]), int(g["lanes"][0][0])
    offs = np.array([int(x) for x in g["chunk_bit_off"][0]], dtype=np.uint64)
    streams = {}
    for key, ahead in (("words_demand", False), ("words_ahead", True)):
        words = np.array([int(x, 16) for x in g[key][0]], dtype=np.uint32)
        streams[ahead] = words
        w, o = ecw.encode(q, lengths, chunk, lanes, 2, ahead=ahead)
        assert w.tolist() == words.tolist() and o.tolist() == offs.tolist()
        assert ecw.decode(words, offs, lengths, len(q), chunk, lanes, 2, ahead=ahead).tolist() == q.tolist()
        w2, o2 = ccodec.encode(q, lengths, chunk, lanes, refill_steps=2, ahead=ahead)
        assert w2.tolist() == words.tolist() and o2.tolist() == offs.tolist()
        assert ccodec.decode(words, offs, lengths, len(q), chunk, lanes, refill_steps=2,
                             ahead=ahead).tolist() == q.tolist()
    # the orders differ: read under the other rule, a stream fails or decodes wrongly
    for ahead in (False, True):
        try:
            back = ecw.decode(streams[ahead], offs, lengths, len(q), chunk, lanes, 2, ahead=not ahead)
        except ecw.StreamError:
            back = None
        assert back is None or back.tolist() != q.tolist()


AHEAD_GRID = [
    (bits, kind, lanes, steps, n_chunks_, refill_steps)
    for bits in (4, 8)
    for kind in ("uniform", "skewed", "peaked", "two", "sparse")
    for lanes, steps, n_chunks_ in ((1, 200, 2), (2, 81, 3), (8, 40, 2), (32, 64, 2), (64, 33, 3))
    for refill_steps in (1, 2)
]


@pytest.mark.parametrize("bits,kind,lanes,steps,n_chunks_,refill_steps", AHEAD_GRID)
def test_ahead_round_trip_python_and_c(bits, kind, lanes, steps, n_chunks_, refill_steps):
    """Refilling ahead: lossless, Python and C byte-identical, and the same
    word count per chunk as the demand rule (no padding words)."""
    chunk = lanes * steps
    n = chunk * (n_chunks_ - 1) + (7 * lanes + 3) % chunk + 1          # ragged last chunk
    q, lengths = make_case(1000 * lanes + steps + bits, bits, kind, n)
    w, o = ecw.encode(q, lengths, chunk, lanes, refill_steps, ahead=True)
    assert ecw.decode(w, o, lengths, n, chunk, lanes, refill_steps, ahead=True).tolist() == q.tolist()
    wc, oc = ccodec.encode(q, lengths, chunk, lanes, refill_steps=refill_steps, ahead=True)
    assert wc.tolist() == w.tolist() and oc.tolist() == o.tolist()
    assert np.array_equal(ccodec.decode(w, o, lengths, n, chunk, lanes, refill_steps=refill_steps, ahead=True), q)
    for c in range(len(o) - 1):
        sl = q[c * chunk:(c + 1) * chunk]
        expect = sum(-(-int(lengths[sl[j::lanes]].sum()) // 32) for j in range(lanes))
        assert (int(o[c + 1]) - int(o[c])) // 32 == expect


@pytest.mark.parametrize("refill_steps", [1, 2])
def test_ahead_equals_demand_when_no_lane_is_early(refill_steps):
    """With fewer than 32 / l_min steps per lane no decision is an early one,
    so refilling ahead stores exactly the demand rule's words."""
    q, lengths = make_case(5, 4, "skewed", 5000)
    l_min = ecw.min_length(lengths)
    steps = max(1, 32 // l_min - 1)
    while steps * l_min >= 32:
        steps -= 1
    chunk = 16 * steps
    w1, o1 = ccodec.encode(q, lengths, chunk, 16, refill_steps=refill_steps)
    w2, o2 = ccodec.encode(q, lengths, chunk, 16, refill_steps=refill_steps, ahead=True)
    assert np.array_equal(w1, w2) and np.array_equal(o1, o2)
    # and with long chunks the two rules do store the words differently
    w3, _ = ccodec.encode(q, lengths, 16 * 200, 16, refill_steps=refill_steps)
    w4, _ = ccodec.encode(q, lengths, 16 * 200, 16, refill_steps=refill_steps, ahead=True)
    assert w3.size == w4.size and not np.array_equal(w3, w4)


def test_golden_encode_decode():
    lengths, q, chunk, lanes, words, offs = golden()
    w, o = ecw.encode(q, lengths, chunk, lanes)
    assert w.tolist() == words.tolist()
    assert o.tolist() == offs.tolist()
    assert ecw.decode(words, offs, lengths, len(q), chunk, lanes).tolist() == q.tolist()
    w2, o2 = ccodec.encode(q, lengths, chunk, lanes)
    assert w2.tolist() == words.tolist() and o2.tolist() == offs.tolist()
    assert ccodec.decode(words, offs, lengths, len(q), chunk, lanes).tolist() == q.tolist()


def make_case(seed, bits, kind, n):
    q = fuzz_codes(seed, n, bits, kind)
    lengths = huffman.code_lengths(histogram(q, bits), 16 if bits == 8 else 12)
    return q, lengths


GRID = [
    (bits, kind, lanes, chunk_mult, n)
    for bits in (4, 8)
    for kind in ("uniform", "skewed", "peaked", "degenerate", "two", "sparse")
    for lanes, chunk_mult, n in ((1, 16, 70), (2, 8, 100), (4, 3, 61), (8, 2, 200), (16, 2, 97),
                                 (32, 1, 300), (64, 2, 333))
]


@pytest.mark.parametrize("refill_steps", [1, 2])
@pytest.mark.parametrize("bits,kind,lanes,chunk_mult,n", GRID)
def test_round_trip_python_and_c(bits, kind, lanes, chunk_mult, n, refill_steps):
    q, lengths = make_case(lanes * 100 + n, bits, kind, n)
    chunk = lanes * chunk_mult
    w, o = ecw.encode(q, lengths, chunk, lanes, refill_steps)
    assert ecw.decode(w, o, lengths, n, chunk, lanes, refill_steps).tolist() == q.tolist()
    wc, oc = ccodec.encode(q, lengths, chunk, lanes, refill_steps=refill_steps)
    assert wc.tolist() == w.tolist() and oc.tolist() == o.tolist()
    assert ccodec.decode(w, o, lengths, n, chunk, lanes, refill_steps=refill_steps).tolist() == q.tolist()
    # a stream decoded under the other decision period either fails or (when
    # the word orders happen to agree) still gives the codes back
    other = 3 - refill_steps
    try:
        back = ccodec.decode(w, o, lengths, n, chunk, lanes, refill_steps=other)
    except ccodec.CodecError:
        back = None
    if back is not None:
        w2, _ = ccodec.encode(q, lengths, chunk, lanes, refill_steps=other)
        assert np.array_equal(w2, w) and np.array_equal(back, q)
    # word count identity, chunk by chunk
    for c in range(len(o) - 1):
        sl = q[c * chunk:(c + 1) * chunk]
        expect = sum(-(-int(lengths[sl[j::lanes]].sum()) // 32) for j in range(lanes))
        assert (int(o[c + 1]) - int(o[c])) // 32 == expect


@pytest.mark.parametrize("seed", range(6))
def test_single_lane_is_plain_msb_first_bitstream(seed):
    bits = 8 if seed % 2 else 4
    q, lengths = make_case(seed, bits, "skewed", 500)
    chunk = 128
    w, o = ecw.encode(q, lengths, chunk, 1)
    codes = canonical_codes(lengths)
    book = {codeword_str(int(codes[s]), int(lengths[s])): s for s in range(len(lengths)) if lengths[s]}
    out = []
    for c in range(len(o) - 1):
        ws = w[int(o[c]) // 32: int(o[c + 1]) // 32]
        stream = "".join(format(int(x), "032b") for x in ws)
        cur = ""
        got = []
        for b in stream:
            cur += b
            if cur in book:
                got.append(book[cur])
                cur = ""
            if len(got) == min(chunk, len(q) - c * chunk):
                break
        out.extend(got)
        # the rest of the chunk is zero padding, shorter than one word
        rest = stream[sum(int(lengths[s]) for s in got):]
        assert set(rest) <= {"0"} and len(rest) < 32
    assert out == q.tolist()


def test_full_size_tensor_c_codec_round_trip():
    q = fuzz_codes(11, 1 << 20, 8, "skewed")
    lengths = huffman.code_lengths(histogram(q, 8), 16)
    w, o = ccodec.encode(q, lengths, 4096, 32, threads=4)
    w1, o1 = ccodec.encode(q, lengths, 4096, 32, threads=1)
    assert np.array_equal(w, w1) and np.array_equal(o, o1)
    assert np.array_equal(ccodec.decode(w, o, lengths, q.size, 4096, 32, threads=4), q)


def test_empty_tensor():
    lengths = np.zeros(16, dtype=np.int64)
    lengths[3] = 1
    w, o = ecw.encode(np.zeros(0, dtype=np.uint8), lengths, 64, 64)
    assert w.size == 0 and o.tolist() == [0]
    assert ecw.decode(w, o, lengths, 0, 64, 64).size == 0
    w2, o2 = ccodec.encode(np.zeros(0, dtype=np.uint8), lengths, 64, 64)
    assert w2.size == 0 and o2.tolist() == [0]


def test_malformed_streams_are_rejected():
    lengths, q, chunk, lanes, words, offs = golden()
    n = len(q)
    # a word missing from the last chunk
    with pytest.raises(ecw.StreamError):
        ecw.decode(words[:-1], np.array([0, 128, 160], dtype=np.uint64), lengths, n, chunk, lanes)
    with pytest.raises(ccodec.CodecError):
        ccodec.decode(words[:-1], np.array([0, 128, 160], dtype=np.uint64), lengths, n, chunk, lanes)
    # an extra word in chunk 1
    extra = np.concatenate([words, np.zeros(1, dtype=np.uint32)])
    with pytest.raises(ecw.StreamError):
        ecw.decode(extra, np.array([0, 128, 224], dtype=np.uint64), lengths, n, chunk, lanes)
    with pytest.raises(ccodec.CodecError):
        ccodec.decode(extra, np.array([0, 128, 224], dtype=np.uint64), lengths, n, chunk, lanes)
    # a nonzero padding bit (last bit of lane 1's final word in chunk 0)
    bad = words.copy()
    bad[3] |= 1
    with pytest.raises(ecw.StreamError):
        ecw.decode(bad, offs, lengths, n, chunk, lanes)
    with pytest.raises(ccodec.CodecError):
        ccodec.decode(bad, offs, lengths, n, chunk, lanes)
    # a symbol with no codeword cannot be encoded
    with pytest.raises(ValueError):
        ecw.encode(np.array([3], dtype=np.uint8), lengths, chunk, lanes)
    with pytest.raises(ccodec.CodecError):
        ccodec.encode(np.array([3], dtype=np.uint8), lengths, chunk, lanes)
    # lanes must be a power of two dividing the chunk
    with pytest.raises(ValueError):
        ecw.encode(q, lengths, 24, 3)
    with pytest.raises(ValueError):
        ecw.encode(q, lengths, 20, 8)


def test_single_symbol_code_rejects_a_one_bit():
    lengths = np.zeros(16, dtype=np.int64)
    lengths[5] = 1
    q = np.full(40, 5, dtype=np.uint8)
    w, o = ecw.encode(q, lengths, 40, 4)
    assert (w == 0).all()
    assert ecw.decode(w, o, lengths, 40, 40, 4).tolist() == q.tolist()
    bad = w.copy()
    bad[0] = 0x80000000
    with pytest.raises(ecw.StreamError):
        ecw.decode(bad, o, lengths, 40, 40, 4)
    with pytest.raises(ccodec.CodecError):
        ccodec.decode(bad, o, lengths, 40, 40, 4)
