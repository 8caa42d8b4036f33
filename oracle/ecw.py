"""Chunked, lane-interleaved canonical-Huffman stream, "ECW v1"
(oracle; pure Python, small inputs; test infrastructure only).

What the pages fix: EntroLLM splits the encoded weights into independent
chunks that keep the tensor's structure and decodes them concurrently
(gist.science technical summary, Methodology item 3); LazyWeights Huffman-codes
the integer codes in interleaved lanes and decodes them bit-exactly (LazyWeights
abstract, arXiv 2611.17108).  The layout below is the reading of those two
statements; nothing in it is printed on the pages.

Layout
------
1. The tensor is flattened row-major (``N`` symbols).
2. Chunk ``c`` holds symbols ``[c*C, min((c+1)*C, N))``; the last may be short.
3. Inside a chunk of ``C_c`` symbols, symbol ``k`` belongs to lane
   ``j = k mod W`` and is decoded at step ``t = k div W``.
4. Lane ``j``'s bit sequence is its codewords in step order, first bit first,
   cut into 32-bit words whose first bit is bit 31; the last word is padded
   with zero bits.
5. Word order inside a chunk: each lane keeps a count ``n`` of loaded but
   unconsumed bits (0 at the start).  Refill decisions are taken every
   ``refill_steps`` (D, 1 or 2) steps: at a step ``t`` with ``t mod D == 0`` a
   lane takes its next word exactly when its codewords of steps
   ``t .. t+D-1`` (those it has) are together longer than ``n`` (then
   ``n += 32``), and then consumes them.  Since codes are at most 16 bits
   long, one word always suffices.  The chunk's words are stored in the order
   they are taken, lanes of one decision point in increasing lane index.
   D = 1 decides per step; D = 2 decides per pair of steps, which halves the
   decision points a decoder has to synchronize on.
   With ``ahead`` the decision changes while a lane still has many codes to
   go: if R codes of the lane remain from step t on and R * l_min >= 32
   (l_min = the shortest code length of the codebook), the lane takes its
   next word exactly when n < 32, whatever its next codewords are; once
   R * l_min < 32 it decides as above.  Such a word always exists (the R
   codes hold at least 32 > n bits), so no padding words arise and the word
   count is the same; a decoder can issue the fetch before looking at the
   codewords.
6. Chunks are concatenated; ``chunk_bit_off[c]`` = 32 x (words before chunk c),
   with a final entry for the end.  Words are little-endian uint32 in memory.
"""
from __future__ import annotations

import numpy as np

from .canonical import canonical_codes, codeword_str


def n_chunks(n_symbols: int, chunk: int) -> int:
    return -(-n_symbols // chunk)


def min_length(lengths) -> int:
    """Shortest code length of a codebook (lengths of absent values are 0)."""
    ls = [int(x) for x in lengths if int(x) > 0]
    return min(ls) if ls else 1


def _check_params(chunk: int, lanes: int, refill_steps: int = 1) -> None:
    if lanes < 1 or lanes > 64 or (lanes & (lanes - 1)):
        raise ValueError("lanes must be a power of two in [1, 64]")
    if chunk < 1 or chunk % lanes:
        raise ValueError("chunk must be a positive multiple of lanes")
    if refill_steps not in (1, 2):
        raise ValueError("refill_steps must be 1 or 2")


def encode(q: np.ndarray, lengths: np.ndarray, chunk: int, lanes: int, refill_steps: int = 1,
           ahead: bool = False):
    """Encode codes ``q`` (any shape, row-major) -> ``(words uint32, chunk_bit_off uint64)``."""
    _check_params(chunk, lanes, refill_steps)
    q = np.asarray(q, dtype=np.uint8).ravel()
    lengths = np.asarray(lengths, dtype=np.int64)
    codes = canonical_codes(lengths)
    l_min = min_length(lengths)
    if len(q) and (lengths[q] == 0).any():
        raise ValueError("a code value present in the tensor has no codeword")
    words: list[int] = []
    offs = [0]
    for c in range(n_chunks(len(q), chunk)):
        sl = q[c * chunk: min((c + 1) * chunk, len(q))]
        cc = len(sl)
        lane_words = []
        for j in range(lanes):
            bits = "".join(codeword_str(int(codes[s]), int(lengths[s])) for s in sl[j::lanes])
            lane_words.append([int(bits[i:i + 32].ljust(32, "0"), 2) for i in range(0, len(bits), 32)])
        n = [0] * lanes
        taken = [0] * lanes
        for t0 in range(0, -(-cc // lanes), refill_steps):
            for j in range(lanes):
                ks = [t * lanes + j for t in range(t0, t0 + refill_steps) if t * lanes + j < cc]
                if not ks:
                    continue
                l = sum(int(lengths[sl[k]]) for k in ks)
                codes_left = -(-(cc - j) // lanes) - t0
                if ahead and codes_left * l_min >= 32:
                    take = n[j] < 32
                else:
                    take = l > n[j]
                if take:
                    words.append(lane_words[j][taken[j]])
                    taken[j] += 1
                    n[j] += 32
                n[j] -= l
        assert all(taken[j] == len(lane_words[j]) for j in range(lanes))
        offs.append(32 * len(words))
    return np.array(words, dtype=np.uint32), np.array(offs, dtype=np.uint64)


class StreamError(ValueError):
    """The stream does not decode under the given codebook and layout."""


def _canonical_tables(lengths: np.ndarray):
    ls = [int(x) for x in lengths]
    max_len = max(ls)
    count = [0] * (max_len + 1)
    for l in ls:
        if l > 0:
            count[l] += 1
    first = [0] * (max_len + 1)
    code = 0
    for l in range(1, max_len + 1):
        code = (code + count[l - 1]) << 1
        first[l] = code
    offset = [0] * (max_len + 1)
    acc = 0
    for l in range(1, max_len + 1):
        offset[l] = acc
        acc += count[l]
    sorted_syms = [s for l in range(1, max_len + 1) for s in range(len(ls)) if ls[s] == l]
    return max_len, count, first, offset, sorted_syms


def decode(words: np.ndarray, chunk_bit_off: np.ndarray, lengths: np.ndarray,
           n_symbols: int, chunk: int, lanes: int, refill_steps: int = 1, ahead: bool = False) -> np.ndarray:
    """Bit-serial canonical decoder: reads one bit at a time, never a table.

    At each decision point a lane first tries to read its next codewords
    (one, or two for ``refill_steps`` 2) bit by bit from the bits it holds;
    if it runs dry it takes the chunk's next word and reads them again.  This
    finds the encoder's word order by decoding, without computing it from
    code lengths.  With ``ahead``, a lane with R codes left and R * l_min >= 32
    instead takes a word whenever it holds fewer than 32 bits, then reads.
    Raises ``StreamError`` on an undecodable prefix, on running past the
    chunk's words, on unused words, or on nonzero padding bits.
    """
    _check_params(chunk, lanes, refill_steps)
    lengths = np.asarray(lengths, dtype=np.int64)
    max_len, count, first, offset, sorted_syms = _canonical_tables(lengths)
    l_min = min_length(lengths)
    words = [int(w) for w in np.asarray(words, dtype=np.uint32)]
    offs = [int(o) for o in np.asarray(chunk_bit_off, dtype=np.uint64)]
    out = np.zeros(n_symbols, dtype=np.uint8)
    nc = n_chunks(n_symbols, chunk)
    if len(offs) != nc + 1 or offs[0] != 0 or offs[-1] != 32 * len(words):
        raise StreamError("chunk offsets do not span the word array")
    for c in range(nc):
        if offs[c] % 32 or offs[c + 1] < offs[c]:
            raise StreamError("chunk offsets must be ascending multiples of 32")
        pos = offs[c] // 32
        end = offs[c + 1] // 32
        cc = min(chunk, n_symbols - c * chunk)
        pending = [[] for _ in range(lanes)]   # unconsumed bits of each lane, first bit first

        def read_codewords(bits, count_):
            """Symbols of the next ``count_`` codewords of ``bits`` and the bits they
            use, or None if ``bits`` end first."""
            syms, p = [], 0
            for _ in range(count_):
                code = 0
                for l in range(1, max_len + 1):
                    if p >= len(bits):
                        return None
                    code = (code << 1) | bits[p]
                    p += 1
                    d = code - first[l]
                    if 0 <= d < count[l]:
                        syms.append(sorted_syms[offset[l] + d])
                        break
                else:
                    raise StreamError(f"chunk {c}: no codeword matches")
            return syms, p

        for t0 in range(0, -(-cc // lanes), refill_steps):
            for j in range(lanes):
                ks = [t * lanes + j for t in range(t0, t0 + refill_steps) if t * lanes + j < cc]
                if not ks:
                    continue
                codes_left = -(-(cc - j) // lanes) - t0
                if ahead and codes_left * l_min >= 32:
                    if len(pending[j]) < 32:
                        if pos >= end:
                            raise StreamError(f"chunk {c}: lane {j} runs past the chunk's words")
                        w = words[pos]
                        pos += 1
                        pending[j].extend((w >> (31 - i)) & 1 for i in range(32))
                    got = read_codewords(pending[j], len(ks))
                    if got is None:
                        raise StreamError(f"chunk {c}: lane {j}: codewords longer than the loaded bits")
                else:
                    got = read_codewords(pending[j], len(ks))
                if got is None:
                    if pos >= end:
                        raise StreamError(f"chunk {c}: lane {j} runs past the chunk's words")
                    w = words[pos]
                    pos += 1
                    pending[j].extend((w >> (31 - i)) & 1 for i in range(32))
                    got = read_codewords(pending[j], len(ks))
                    if got is None:
                        raise StreamError(f"chunk {c}: lane {j}: codewords longer than a word")
                syms, used = got
                for k, sym in zip(ks, syms):
                    out[c * chunk + k] = sym
                del pending[j][:used]
        if pos != end:
            raise StreamError(f"chunk {c}: {end - pos} words left unused")
        for j in range(lanes):
            if any(pending[j]):
                raise StreamError(f"chunk {c}: lane {j} has nonzero padding bits")
    return out


def stream_bits(words: np.ndarray, n_chunks_: int) -> int:
    """Coded size in bits: stream words plus one 64-bit offset per chunk boundary."""
    return 32 * int(len(words)) + 64 * (n_chunks_ + 1)
