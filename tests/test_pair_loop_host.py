"""The fused GEMV's pair-loop bookkeeping against the oracle's streams (no
GPU): which pairs of a chunk of whole rows take the refill-ahead rule.

The loops count a chunk's refill-ahead pairs from the chunk's start, across
its rows.  tests/_pair_loop.py runs chunks through a model of the loop that
reads the oracle's words one bit at a time; every chunk must end exactly at
its last word with no bits left over.  The same model with the count started
again at every row fails wherever a chunk's refill-ahead pairs reach past its
first row, which shows that the model sees such a mistake.

A loop variant tried once (each row's loop split by refill-ahead phase)
failed a GPU case with overrun and padding flags on three-row chunks (50 x
256, mixed 4-bit, refilling ahead).  In that case the shortest code is one
bit, so no pair of any chunk takes the refill-ahead rule (32 codes would be
needed, a chunk has 12 per lane): the phase bookkeeping changes no decision
there and cannot have caused those flags.
"""
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from oracle import ccodec, ecw, huffman, quant  # noqa: E402
from tests._pair_loop import chunk_flags, early_pairs  # noqa: E402


def _stream(q, rows, cols, rows_per_chunk, ahead=True):
    q = np.asarray(q, dtype=np.uint8).reshape(rows, cols)
    lengths = huffman.code_lengths(quant.histogram(q, 4), 12)
    words, offs = ccodec.encode(q.ravel(), lengths, cols * rows_per_chunk, 64, threads=1, refill_steps=2,
                                ahead=ahead)
    # the oracle's own decoder reads the stream back
    assert np.array_equal(ecw.decode(words, offs, lengths, q.size, cols * rows_per_chunk, 64, 2, ahead), q.ravel())
    return words, offs, lengths, int(lengths[lengths > 0].min())


def _failing_case():
    rng = np.random.default_rng(32)
    w = (rng.standard_t(4, size=(50, 256)) * 0.02).astype(np.float32)
    return quant.quantize_mixed(w, 4).q


def _uniform_codes(rows, cols, seed):
    return np.random.default_rng(seed).integers(0, 16, size=(rows, cols)).astype(np.uint8)


CASES = [  # (name, codes, rows, cols, rows per chunk)
    ("three-row chunks, mixed 4-bit Student-t", _failing_case, 50, 256, 3),
    ("three-row chunks, uniform codes", lambda: _uniform_codes(31, 256, 1), 31, 256, 3),
    ("two-row chunks, uniform codes", lambda: _uniform_codes(9, 1024, 2), 9, 1024, 2),
    ("seven-row chunks, uniform codes", lambda: _uniform_codes(23, 128, 3), 23, 128, 7),
    ("one-row chunks, uniform codes", lambda: _uniform_codes(5, 2048, 4), 5, 2048, 1),
]


@pytest.mark.parametrize("name,make,rows,cols,rpc", CASES, ids=[c[0] for c in CASES])
def test_chunk_accounting_reads_every_chunk_exactly(name, make, rows, cols, rpc):
    words, offs, lengths, l_min = _stream(make(), rows, cols, rpc)
    assert chunk_flags(words, offs, lengths, l_min, rows, cols, rpc, True, "chunk") == [0] * (len(offs) - 1)


def test_row_restart_fails_where_early_pairs_reach_past_the_first_row():
    rows, cols, rpc = 31, 256, 3
    words, offs, lengths, l_min = _stream(_uniform_codes(rows, cols, 1), rows, cols, rpc)
    assert l_min == 4 and early_pairs(True, rpc * cols // 64, l_min) == 3 > cols // 128
    flags = chunk_flags(words, offs, lengths, l_min, rows, cols, rpc, True, "row")
    assert any(flags[:-1])   # every full chunk's second row starts the refill-ahead pairs again
    # one-row chunks: the two bookkeepings are the same thing
    rows, cols = 5, 2048
    words, offs, lengths, l_min = _stream(_uniform_codes(rows, cols, 4), rows, cols, 1)
    assert chunk_flags(words, offs, lengths, l_min, rows, cols, 1, True, "row") == [0] * rows


def test_the_failing_case_has_no_refill_ahead_pairs():
    rows, cols, rpc = 50, 256, 3
    words, offs, lengths, l_min = _stream(_failing_case(), rows, cols, rpc)
    assert l_min == 1
    for c in range(len(offs) - 1):
        nr = min(rpc, rows - c * rpc)
        assert early_pairs(True, nr * cols // 64, l_min) == 0
    assert chunk_flags(words, offs, lengths, l_min, rows, cols, rpc, True, "row") == [0] * (len(offs) - 1)
