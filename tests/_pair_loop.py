"""A host model of the fused GEMV's pair-loop bookkeeping, for streams of
64 lanes with a refill decision every two steps and chunks of whole rows.

The loop decides, pair by pair, whether a lane takes a word by the
refill-ahead rule (while fewer than 32 bits are held) or on demand (when
the next two codewords are longer than the held bits).  The encoder applies
the refill-ahead rule while a lane's codes_left * l_min >= 32, which for
chunks of whole rows (a multiple of 64 codes) holds for the same number of
leading pairs in every lane: ``early_pairs``.  Which pairs the loop treats
so is its bookkeeping; ``decode_chunk`` runs a chunk through the loop with a
given rule (a predicate on the pair's index within the chunk), reading the
real words of the stream, and returns what the kernel would flag: the word
pointer against the chunk's end (overrun / underrun) and nonzero bits left
in a lane (padding).  Bits are read one at a time against the canonical
code, as the oracle's serial decoder does.
"""
from __future__ import annotations

import numpy as np

from oracle.canonical import canonical_codes

OVERRUN, UNDERRUN, PADDING = 0x01, 0x02, 0x08


def early_pairs(ahead: bool, steps: int, l_min: int) -> int:
    """Leading pairs of a chunk whose refill follows the refill-ahead rule:
    a lane with R codes left and R * l_min >= 32 takes a word exactly when it
    holds fewer than 32 bits (steps: codes per lane in the chunk)."""
    if not ahead:
        return 0
    need = -(-32 // l_min)
    return (steps - need) // 2 + 1 if steps >= need else 0


def _code_table(lengths):
    codes = canonical_codes(lengths)
    return {(int(lengths[s]), int(codes[s])): s for s in range(len(lengths)) if lengths[s]}


def _read(bits, count, table, max_len):
    """Lengths of the next ``count`` codewords of ``bits`` (a list of 0/1),
    or None if the bits end first; an unmatched prefix reads as max_len bits."""
    p, used = 0, []
    for _ in range(count):
        code, l = 0, 0
        while True:
            if p >= len(bits):
                return None
            code = (code << 1) | bits[p]
            p += 1
            l += 1
            if (l, code) in table or l == max_len:
                break
        used.append(l)
    return sum(used)


def decode_chunk(words, start: int, end: int, lengths, codes_per_lane: int, rule) -> int:
    """Flags of one chunk (words [start, end) of ``words``) decoded by the
    pair loop; ``rule(k)`` is true if pair k of the chunk takes the
    refill-ahead rule.  Past the chunk's end the loop reads what follows (or
    zeros past the stream), as a kernel reading ahead would."""
    lengths = np.asarray(lengths, dtype=np.int64)
    table = _code_table(lengths)
    max_len = int(lengths.max())
    pend = [[] for _ in range(64)]
    pos = start

    def take(j):
        nonlocal pos
        w = int(words[pos]) if pos < len(words) else 0
        pos += 1
        pend[j].extend((w >> (31 - i)) & 1 for i in range(32))

    for k in range(codes_per_lane // 2):
        ahead = rule(k)
        for j in range(64):
            if ahead:
                if len(pend[j]) < 32:
                    take(j)
                l = _read(pend[j], 2, table, max_len)
            else:
                l = _read(pend[j], 2, table, max_len)
                if l is None:
                    take(j)
                    l = _read(pend[j], 2, table, max_len)
            if l is None:   # longer than the held bits even after a word: consume them all
                l = len(pend[j])
            del pend[j][:l]
    flags = 0
    if pos != end:
        flags |= OVERRUN if pos > end else UNDERRUN
    if any(any(b) for b in pend):
        flags |= PADDING
    return flags


def chunk_flags(words, offs, lengths, l_min: int, rows: int, cols: int, rows_per_chunk: int, ahead: bool,
                accounting: str) -> list[int]:
    """Flags of every chunk under an accounting of the refill-ahead pairs:
    'chunk' counts pairs from the chunk's start across its rows (the shipped
    loops); 'row' starts the count again at every row."""
    out = []
    ppr = cols // 128
    n_chunks = -(-rows // rows_per_chunk)
    for c in range(n_chunks):
        nr = min(rows_per_chunk, rows - c * rows_per_chunk)
        steps = nr * cols // 64
        early = early_pairs(ahead, steps, l_min)
        if accounting == "chunk":
            rule = lambda k, e=early: k < e
        elif accounting == "row":
            rule = lambda k, e=early: (k % ppr) < min(e, ppr)
        else:
            raise ValueError(accounting)
        out.append(decode_chunk(words, int(offs[c]) // 32, int(offs[c + 1]) // 32, lengths, steps, rule))
    return out
