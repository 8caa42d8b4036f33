"""ctypes front end of the oracle's plain C codec (``codec.c``); test infrastructure only.

``build()`` compiles ``codec.c`` with gcc into ``oracle/liboracle_codec.so``.
The functions mirror ``oracle.ecw`` (same layout, same decoder algorithm) and
are cross-checked against it; they exist because the pure-Python version is
too slow for full-size tensors.  ``decode_threaded`` runs independent chunk
ranges on several host threads, the CPU-thread parallel decoding that
EntroLLM describes (gist.science technical summary, Methodology item 3).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "codec.c")
_LIB = os.path.join(_HERE, "liboracle_codec.so")
_lock = threading.Lock()
_lib = None

_ERRORS = {1: "bad parameters", 2: "bad codebook", 3: "stream error", 4: "out of memory"}


class CodecError(ValueError):
    pass


def build() -> str:
    """Compile ``codec.c`` (always) and return the library path."""
    tmp = _LIB + f".tmp{os.getpid()}"
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-o", tmp, _SRC])
    os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
            lib = ctypes.CDLL(_LIB)
            P = ctypes.c_void_p
            U64 = ctypes.c_uint64
            U32 = ctypes.c_uint32
            lib.oc_layout.argtypes = [P, U64, P, U32, U32, U32, P, P]
            lib.oc_encode.argtypes = [P, U64, P, U32, U32, U32, U32, U32, P, P, U64, U64]
            lib.oc_decode.argtypes = [P, U64, P, U64, P, U32, U32, U32, U32, U32, P, U64, U64]
            for f in (lib.oc_layout, lib.oc_encode, lib.oc_decode):
                f.restype = ctypes.c_int
            _lib = lib
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc:
        raise CodecError(f"{what}: {_ERRORS.get(rc, rc)}")


def _split(nc: int, threads: int):
    threads = max(1, min(threads, nc))
    bounds = [nc * i // threads for i in range(threads + 1)]
    return [(bounds[i], bounds[i + 1]) for i in range(threads)]


def layout(q: np.ndarray, lengths: np.ndarray, chunk: int, lanes: int):
    """Chunk offsets and word count of the stream, without writing it ->
    ``(chunk_bit_off uint64, n_words)``; the same offsets as ``encode``."""
    lib = _load()
    q = np.ascontiguousarray(np.asarray(q, dtype=np.uint8).ravel())
    ln = np.ascontiguousarray(np.asarray(lengths, dtype=np.uint8))
    n = q.size
    offs = np.zeros(-(-n // chunk) + 1, dtype=np.uint64)
    nw = np.zeros(1, dtype=np.uint64)
    _check(lib.oc_layout(_ptr(q), n, _ptr(ln), ln.size, chunk, lanes, _ptr(offs), _ptr(nw)), "layout")
    return offs, int(nw[0])


def encode(q: np.ndarray, lengths: np.ndarray, chunk: int, lanes: int, threads: int = 1, refill_steps: int = 1,
           ahead: bool = False):
    """Encode -> ``(words uint32, chunk_bit_off uint64)``; same result as ``oracle.ecw.encode``."""
    lib = _load()
    q = np.ascontiguousarray(np.asarray(q, dtype=np.uint8).ravel())
    ln = np.ascontiguousarray(np.asarray(lengths, dtype=np.uint8))
    n = q.size
    nc = -(-n // chunk)
    offs = np.zeros(nc + 1, dtype=np.uint64)
    nw = np.zeros(1, dtype=np.uint64)
    _check(lib.oc_layout(_ptr(q), n, _ptr(ln), ln.size, chunk, lanes, _ptr(offs), _ptr(nw)), "layout")
    words = np.zeros(int(nw[0]), dtype=np.uint32)
    ranges = _split(nc, threads)

    def run(r):
        return lib.oc_encode(_ptr(q), n, _ptr(ln), ln.size, chunk, lanes, refill_steps, int(ahead), _ptr(offs),
                             _ptr(words), r[0], r[1])

    if len(ranges) == 1:
        _check(run(ranges[0]) if nc else 0, "encode")
    else:
        with ThreadPoolExecutor(len(ranges)) as ex:
            for rc in ex.map(run, ranges):
                _check(rc, "encode")
    return words, offs


def decode(words: np.ndarray, chunk_bit_off: np.ndarray, lengths: np.ndarray,
           n_symbols: int, chunk: int, lanes: int, threads: int = 1,
           chunk_range: tuple[int, int] | None = None, refill_steps: int = 1, ahead: bool = False) -> np.ndarray:
    """Bit-serial decode of all chunks (or ``chunk_range``) -> uint8 codes."""
    lib = _load()
    words = np.ascontiguousarray(words, dtype=np.uint32)
    offs = np.ascontiguousarray(chunk_bit_off, dtype=np.uint64)
    ln = np.ascontiguousarray(np.asarray(lengths, dtype=np.uint8))
    nc = -(-n_symbols // chunk)
    if offs.size != nc + 1 or (nc and int(offs[-1]) != 32 * words.size):
        raise CodecError("chunk offsets do not span the word array")
    out = np.zeros(n_symbols, dtype=np.uint8)
    c0, c1 = chunk_range if chunk_range is not None else (0, nc)
    ranges = [(c0 + a, c0 + b) for a, b in _split(c1 - c0, threads)] if c1 > c0 else []

    def run(r):
        return lib.oc_decode(_ptr(words), words.size, _ptr(offs), n_symbols, _ptr(ln), ln.size,
                             chunk, lanes, refill_steps, int(ahead), _ptr(out), r[0], r[1])

    if len(ranges) == 1:
        _check(run(ranges[0]), "decode")
    elif ranges:
        with ThreadPoolExecutor(len(ranges)) as ex:
            for rc in ex.map(run, ranges):
                _check(rc, "decode")
    return out
