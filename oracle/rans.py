"""Interleaved rANS coding of the same integer codes, "ECR v1" (oracle; pure
Python, small inputs; test infrastructure only).

LazyWeights compares its Huffman decoder with an rANS decoder and finds the
Huffman one better in rate and area at equal throughput (LazyWeights
abstract, arXiv 2611.17108).  The pages give no rANS parameters; everything
below is a reading, chosen to match the Huffman stream's structure so that
the two decoders can be compared on one GPU:

* Frequencies: the code histogram scaled to ``M = 2^12`` (``quantize_freqs``):
  every present code gets ``max(1, floor(M c / N))``; while the sum is below
  ``M`` the code with the largest shortfall ``M c / N - f`` gains one (ties:
  lower code); while above, the largest frequency above 1 loses one (ties:
  lower code).  ``cum[s]`` is the sum of the frequencies of the codes below s.
* Coder: range ANS with a 32-bit state, ``L = 2^16`` and 16-bit renormalization
  units.  Decoding a code from state x: ``slot = x mod M``, s is the code
  with ``cum[s] <= slot < cum[s] + f[s]``, ``x = f[s] (x div M) + slot - cum[s]``,
  then if ``x < L``, ``x = x * 2^16 + (next unit)``; one unit always
  suffices.  The encoder is the exact inverse, run backwards: before coding s
  from x, if ``x >= f[s] * 2^20`` it emits ``x mod 2^16`` and divides x by 2^16;
  then ``x = (x div f) M + (x mod f) + cum[s]``.  States start (encoder) and
  end (decoder) at L.
* Chunks and lanes exactly as in the Huffman stream (``oracle.ecw``): chunk c
  holds codes ``[cC, (c+1)C)``, code k of a chunk belongs to lane ``k mod W``
  at step ``k div W``; every lane has its own state.
* Stream of a chunk, in 16-bit units: first each lane's initial decoder state
  (two units, low half first, lanes in order), then the renormalization units
  in the order a lockstep decoder takes them: step by step, lanes of one step
  in increasing order.  ``chunk_unit_off[c]`` counts the units before chunk c.
"""
from __future__ import annotations

import numpy as np

M_BITS = 12
M = 1 << M_BITS
L = 1 << 16


def quantize_freqs(counts) -> np.ndarray:
    """Frequencies summing to ``M`` (see the module doc); absent codes get 0."""
    c = [int(x) for x in counts]
    n = sum(c)
    if n <= 0:
        raise ValueError("empty histogram")
    present = [s for s in range(len(c)) if c[s] > 0]
    if len(present) > M:
        raise ValueError("more code values than frequency slots")
    f = [0] * len(c)
    for s in present:
        f[s] = max(1, (M * c[s]) // n)
    total = sum(f)
    while total < M:
        # largest shortfall M c / N - f, compared exactly as (M c - f N)
        s = max(present, key=lambda t: (M * c[t] - f[t] * n, -t))
        f[s] += 1
        total += 1
    while total > M:
        s = max((t for t in present if f[t] > 1), key=lambda t: (f[t], -t))
        f[s] -= 1
        total -= 1
    return np.array(f, dtype=np.int64)


def cumulative(freqs) -> np.ndarray:
    f = np.asarray(freqs, dtype=np.int64)
    return np.concatenate([[0], np.cumsum(f)[:-1]]).astype(np.int64)


def _check(chunk: int, lanes: int) -> None:
    if lanes < 1 or lanes > 64 or (lanes & (lanes - 1)):
        raise ValueError("lanes must be a power of two in [1, 64]")
    if chunk < 1 or chunk % lanes:
        raise ValueError("chunk must be a positive multiple of lanes")


def encode(q, freqs, chunk: int, lanes: int):
    """Codes ``q`` -> ``(units uint16, chunk_unit_off uint64)``."""
    _check(chunk, lanes)
    q = [int(v) for v in np.asarray(q, dtype=np.uint8).ravel()]
    f = [int(v) for v in freqs]
    cum = [int(v) for v in cumulative(freqs)]
    if any(f[s] == 0 for s in q):
        raise ValueError("a code value present in the tensor has frequency 0")
    units: list[int] = []
    offs = [0]
    n = len(q)
    for c0 in range(0, n, chunk):
        sl = q[c0: min(c0 + chunk, n)]
        cc = len(sl)
        steps = -(-cc // lanes)
        x = [L] * lanes
        rev: list[int] = []          # renormalization units, last consumed first
        for t in reversed(range(steps)):
            for j in reversed(range(lanes)):
                k = t * lanes + j
                if k >= cc:
                    continue
                s = sl[k]
                if x[j] >= f[s] << 20:
                    rev.append(x[j] & 0xFFFF)
                    x[j] >>= 16
                x[j] = (x[j] // f[s]) * M + (x[j] % f[s]) + cum[s]
        for j in range(lanes):
            units += [x[j] & 0xFFFF, x[j] >> 16]
        units += rev[::-1]
        offs.append(len(units))
    return np.array(units, dtype=np.uint16), np.array(offs, dtype=np.uint64)


class StreamError(ValueError):
    """The stream does not decode under the given frequencies and layout."""


def decode(units, chunk_unit_off, freqs, n_symbols: int, chunk: int, lanes: int) -> np.ndarray:
    """Lockstep decoder; raises ``StreamError`` on a slot of an absent code,
    on running past the chunk's units, on unused units, or on a final state
    other than L."""
    _check(chunk, lanes)
    f = [int(v) for v in freqs]
    cum = [int(v) for v in cumulative(freqs)]
    slot_sym = [0] * M
    for s in range(len(f)):
        for u in range(cum[s], cum[s] + f[s]):
            slot_sym[u] = s
    units = [int(v) for v in np.asarray(units, dtype=np.uint16)]
    offs = [int(v) for v in np.asarray(chunk_unit_off, dtype=np.uint64)]
    nc = -(-n_symbols // chunk)
    if len(offs) != nc + 1 or offs[0] != 0 or offs[-1] != len(units):
        raise StreamError("chunk offsets do not span the units")
    out = np.zeros(n_symbols, dtype=np.uint8)
    for c in range(nc):
        pos, end = offs[c], offs[c + 1]
        cc = min(chunk, n_symbols - c * chunk)
        if end - pos < 2 * lanes:
            raise StreamError(f"chunk {c}: no room for the initial states")
        x = [units[pos + 2 * j] | (units[pos + 2 * j + 1] << 16) for j in range(lanes)]
        pos += 2 * lanes
        for t in range(-(-cc // lanes)):
            for j in range(lanes):
                k = t * lanes + j
                if k >= cc:
                    continue
                slot = x[j] % M
                s = slot_sym[slot]
                if f[s] == 0:
                    raise StreamError(f"chunk {c}: slot of an absent code")
                x[j] = f[s] * (x[j] // M) + slot - cum[s]
                if x[j] < L:
                    if pos >= end:
                        raise StreamError(f"chunk {c}: lane {j} runs past the chunk's units")
                    x[j] = (x[j] << 16) | units[pos]
                    pos += 1
                out[c * chunk + k] = s
        if pos != end:
            raise StreamError(f"chunk {c}: {end - pos} units left unused")
        if any(v != L for v in x):
            raise StreamError(f"chunk {c}: a lane does not end in the initial encoder state")
    return out


def stream_bits(units, n_chunks: int) -> int:
    """Coded size in bits: the units plus one 64-bit offset per chunk boundary."""
    return 16 * int(len(units)) + 64 * (n_chunks + 1)


def ideal_bits(q, freqs) -> float:
    """Sum of -log2(f[s] / M) over the codes: what the coder spends, up to the
    states' bounded slack (at most 32 bits per lane and chunk)."""
    f = np.asarray(freqs, dtype=np.float64)
    qq = np.asarray(q, dtype=np.int64).ravel()
    return float(-np.log2(f[qq] / M).sum())
