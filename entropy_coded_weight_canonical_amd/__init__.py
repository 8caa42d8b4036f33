"""Python binding of ``libentro.so`` (ctypes; argument marshalling only).

The names mirror the C ABI of ``include/entro.h`` and ``include/entro_encode.h``
without the ``entro_`` prefix.  Every step of the decode path runs in the HIP
kernels of the library; this module only converts arguments.  Device buffers
are torch tensors on the HIP device (``torch.cuda`` is torch's HIP namespace on
ROCm); streams are torch streams.  If the library is missing, every call
raises ``LibraryNotBuilt`` - there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

__all__ = [
    "LibraryNotBuilt", "EntroError", "library_path", "load",
    "Codebook", "Tensor", "GemvItem", "RansTensor", "FLAGS",
    "lut_bytes", "lut_build", "decode", "decode_dequant", "decode_gemv", "GemvCall", "decode_gemm",
    "status_str",
    "quantize", "code_lengths", "encode_layout", "encode",
    "rans_freqs", "rans_table_build", "rans_encode", "rans_decode", "rans_decode_dequant",
    "SCHEME_ASYMMETRIC", "SCHEME_UNSIGNED", "SCHEME_MIXED",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libentro.so")
_lib = None

SCHEME_ASYMMETRIC, SCHEME_UNSIGNED, SCHEME_MIXED = 0, 1, 2
_SCHEME_NAMES = {0: "asymmetric", 1: "unsigned", 2: "mixed"}
_SCHEME_IDS = {v: k for k, v in _SCHEME_NAMES.items()}

FLAGS = {
    "overrun": 0x01, "underrun": 0x02, "badcode": 0x04,
    "padding": 0x08, "offsets": 0x10, "lut": 0x20,
}


class LibraryNotBuilt(RuntimeError):
    pass


class EntroError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_str(status)} ({status})")
        self.status = status


class Codebook(ctypes.Structure):
    _fields_ = [("sym_bits", ctypes.c_uint32), ("max_len", ctypes.c_uint32),
                ("code_len", ctypes.c_void_p), ("scale", ctypes.c_float),
                ("zero_point", ctypes.c_int32)]


class Tensor(ctypes.Structure):
    _fields_ = [("d_lut", ctypes.c_void_p), ("d_words", ctypes.c_void_p),
                ("d_chunk_bit_off", ctypes.c_void_p), ("n_words", ctypes.c_uint64),
                ("n_symbols", ctypes.c_uint64), ("chunk_symbols", ctypes.c_uint32),
                ("lanes", ctypes.c_uint32), ("sym_bits", ctypes.c_uint32),
                ("max_len", ctypes.c_uint32), ("lut_bytes", ctypes.c_uint64),
                ("max_chunk_words", ctypes.c_uint32), ("refill_steps", ctypes.c_uint32),
                ("refill_ahead", ctypes.c_uint32), ("out_cached", ctypes.c_uint32),
                ("d_pair_lut", ctypes.c_void_p)]


class RansTensor(ctypes.Structure):
    _fields_ = [("d_table", ctypes.c_void_p), ("d_units", ctypes.c_void_p),
                ("d_chunk_unit_off", ctypes.c_void_p), ("n_units", ctypes.c_uint64),
                ("n_symbols", ctypes.c_uint64), ("chunk_symbols", ctypes.c_uint32),
                ("lanes", ctypes.c_uint32), ("sym_bits", ctypes.c_uint32),
                ("max_chunk_units", ctypes.c_uint32)]


class GemvItem(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_uint32), ("cols", ctypes.c_uint32),
                ("d_x", ctypes.c_void_p), ("d_y", ctypes.c_void_p)]


def library_path() -> str:
    return _LIB_PATH


def load():
    """Load ``libentro.so`` (raises ``LibraryNotBuilt`` if it is not there)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise LibraryNotBuilt(
            f"{_LIB_PATH} is missing; build it with `python -m entropy_coded_weight_canonical_amd.build`")
    # The device entry points take torch's device pointers and streams, and
    # torch ships its own HIP runtime (same soname).  Load torch first, so that
    # the library binds to that runtime: loaded the other way round, the
    # process holds two HIP runtimes and torch's pointers are foreign to ours.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(_LIB_PATH)
    P, U32, U64, SZ = ctypes.c_void_p, ctypes.c_uint32, ctypes.c_uint64, ctypes.c_size_t
    lib.entro_lut_bytes.argtypes = [P]
    lib.entro_lut_bytes.restype = SZ
    lib.entro_lut_build.argtypes = [P, P, SZ]
    lib.entro_pair_lut_bytes.argtypes = []
    lib.entro_pair_lut_bytes.restype = SZ
    lib.entro_pair_lut_build.argtypes = [P, SZ, P, SZ]
    for name in ("entro_decode", "entro_decode_dequant"):
        getattr(lib, name).argtypes = [P, SZ, P, P, P]
    lib.entro_decode_gemv.argtypes = [P, SZ, P, U32, P, P]
    lib.entro_decode_gemm.argtypes = [P, SZ, P, U32, P, P]
    lib.entro_rans_freqs.argtypes = [P, U32, P]
    lib.entro_rans_table_bytes.argtypes = []
    lib.entro_rans_table_bytes.restype = SZ
    lib.entro_rans_table_build.argtypes = [U32, P, ctypes.c_float, ctypes.c_int32, P, SZ]
    lib.entro_rans_encode.argtypes = [P, U64, P, U32, U32, U32, P, P, U64, P, U32]
    for name in ("entro_rans_decode", "entro_rans_decode_dequant"):
        getattr(lib, name).argtypes = [P, SZ, P, P, P]
    lib.entro_set_max_workgroups.argtypes = [U32]
    lib.entro_set_max_workgroups.restype = U32
    lib.entro_status_str.argtypes = [ctypes.c_int]
    lib.entro_status_str.restype = ctypes.c_char_p
    lib.entro_quantize.argtypes = [P, U64, U32, ctypes.c_int, ctypes.c_float, P, P, P, P]
    lib.entro_code_lengths.argtypes = [P, U64, U32, U32, P]
    lib.entro_encode_layout.argtypes = [P, U64, P, U32, U32, U32, P, P]
    lib.entro_encode.argtypes = [P, U64, P, U32, U32, U32, U32, U32, P, P, U32]
    for name in ("entro_lut_build", "entro_pair_lut_build", "entro_decode", "entro_decode_dequant", "entro_decode_gemv",
                 "entro_decode_gemm", "entro_quantize", "entro_code_lengths", "entro_encode_layout", "entro_encode",
                 "entro_rans_freqs", "entro_rans_table_build", "entro_rans_encode", "entro_rans_decode",
                 "entro_rans_decode_dequant"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def status_str(status: int) -> str:
    return load().entro_status_str(int(status)).decode()


def _check(status: int, what: str):
    if status != 0:
        raise EntroError(status, what)


def _np_ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _codebook(code_len: np.ndarray, sym_bits: int, max_len: int, scale: float, zero_point: int):
    cl = np.ascontiguousarray(code_len, dtype=np.uint8)
    if cl.size != (1 << sym_bits):
        raise ValueError("code_len must have 2**sym_bits entries")
    return Codebook(sym_bits, max_len, cl.ctypes.data, float(scale), int(zero_point)), cl


# --------------------------------------------------------------------------
# decode tables
# --------------------------------------------------------------------------

def lut_bytes(code_len, sym_bits: int, max_len: int, scale: float = 1.0, zero_point: int = 0) -> int:
    cb, _keep = _codebook(code_len, sym_bits, max_len, scale, zero_point)
    return int(load().entro_lut_bytes(ctypes.byref(cb)))


def lut_build(code_len, sym_bits: int, max_len: int, scale: float, zero_point: int) -> np.ndarray:
    """Decode table bytes as a host uint32 array (header + entries)."""
    cb, _keep = _codebook(code_len, sym_bits, max_len, scale, zero_point)
    lib = load()
    nbytes = int(lib.entro_lut_bytes(ctypes.byref(cb)))
    out = np.zeros(max(nbytes, 16) // 4, dtype=np.uint32)
    _check(lib.entro_lut_build(ctypes.byref(cb), _np_ptr(out), out.nbytes), "entro_lut_build")
    return out


# --------------------------------------------------------------------------
# device entry points
# --------------------------------------------------------------------------

def pair_lut_build(lut: np.ndarray) -> np.ndarray:
    """``entro_pair_lut_build``: the two-code table of a 4-bit decode table
    (``lut_build`` output), as uint32 words."""
    lib = load()
    t = np.ascontiguousarray(lut, dtype=np.uint32)
    out = np.zeros(lib.entro_pair_lut_bytes() // 4, dtype=np.uint32)
    _check(lib.entro_pair_lut_build(_np_ptr(t), t.nbytes, _np_ptr(out), out.nbytes), "entro_pair_lut_build")
    return out


def _stream_handle(stream) -> int:
    if stream is None:
        import torch
        stream = torch.cuda.current_stream()
    return int(getattr(stream, "cuda_stream", stream))


def _tensor_array(tensors):
    arr = (Tensor * len(tensors))()
    for i, t in enumerate(tensors):
        arr[i] = t
    return arr


def _ptr_array(ptrs):
    arr = (ctypes.c_void_p * len(ptrs))()
    for i, p in enumerate(ptrs):
        arr[i] = int(p) if p is not None else None
    return arr


def decode(tensors, outs, d_status: int, stream=None) -> None:
    """``entro_decode``: ``tensors`` are ``Tensor`` descriptors, ``outs`` device pointers."""
    ta, oa = _tensor_array(tensors), _ptr_array(outs)
    _check(load().entro_decode(ta, len(tensors), oa, ctypes.c_void_p(d_status),
                               ctypes.c_void_p(_stream_handle(stream))), "entro_decode")


def decode_dequant(tensors, outs, d_status: int, stream=None) -> None:
    """``entro_decode_dequant``: like ``decode`` with bf16 outputs."""
    ta, oa = _tensor_array(tensors), _ptr_array(outs)
    _check(load().entro_decode_dequant(ta, len(tensors), oa, ctypes.c_void_p(d_status),
                                       ctypes.c_void_p(_stream_handle(stream))), "entro_decode_dequant")


def decode_gemv(tensors, items, batch: int, d_status: int, stream=None) -> None:
    """``entro_decode_gemv``: ``items`` are ``GemvItem`` (rows, cols, d_x, d_y)."""
    ta = _tensor_array(tensors)
    ia = (GemvItem * len(items))()
    for i, it in enumerate(items):
        ia[i] = it
    _check(load().entro_decode_gemv(ta, len(tensors), ia, int(batch), ctypes.c_void_p(d_status),
                                    ctypes.c_void_p(_stream_handle(stream))), "entro_decode_gemv")



class GemvCall:
    """``entro_decode_gemv`` over a fixed set of tensors and items, with the
    ctypes argument arrays built once (a caller that repeats the same call,
    such as a per-token loop, then pays no marshalling per call)."""

    def __init__(self, tensors, items, batch: int, d_status: int):
        self._t = _tensor_array(tensors)
        self._i = (GemvItem * len(items))()
        for i, it in enumerate(items):
            self._i[i] = it
        self._n = len(tensors)
        self._batch = int(batch)
        self._st = ctypes.c_void_p(d_status)
        self._fn = load().entro_decode_gemv

    def __call__(self, stream=None) -> None:
        _check(self._fn(self._t, self._n, self._i, self._batch, self._st, ctypes.c_void_p(_stream_handle(stream))),
               "entro_decode_gemv")

def decode_gemm(tensors, items, n_tokens: int, d_status: int, stream=None) -> None:
    """``entro_decode_gemm``: like ``decode_gemv`` for ``n_tokens`` (1..512)
    activation rows at once, products on the matrix cores."""
    ta = _tensor_array(tensors)
    ia = (GemvItem * len(items))()
    for i, it in enumerate(items):
        ia[i] = it
    _check(load().entro_decode_gemm(ta, len(tensors), ia, int(n_tokens), ctypes.c_void_p(d_status),
                                    ctypes.c_void_p(_stream_handle(stream))), "entro_decode_gemm")


def set_max_workgroups(n: int) -> int:
    """``entro_set_max_workgroups``: cap the workgroups of later launches (0:
    no cap); returns the previous cap."""
    return int(load().entro_set_max_workgroups(int(n)))


def _rans_array(tensors):
    arr = (RansTensor * len(tensors))()
    for i, t in enumerate(tensors):
        arr[i] = t
    return arr


def rans_decode(tensors, outs, d_status: int, stream=None) -> None:
    """``entro_rans_decode``: ``tensors`` are ``RansTensor`` descriptors."""
    _check(load().entro_rans_decode(_rans_array(tensors), len(tensors), _ptr_array(outs), ctypes.c_void_p(d_status),
                                    ctypes.c_void_p(_stream_handle(stream))), "entro_rans_decode")


def rans_decode_dequant(tensors, outs, d_status: int, stream=None) -> None:
    """``entro_rans_decode_dequant``: like ``rans_decode`` with bf16 outputs."""
    _check(load().entro_rans_decode_dequant(_rans_array(tensors), len(tensors), _ptr_array(outs),
                                            ctypes.c_void_p(d_status), ctypes.c_void_p(_stream_handle(stream))),
           "entro_rans_decode_dequant")


def rans_freqs(counts: np.ndarray) -> np.ndarray:
    """Histogram -> frequencies summing to 4096 (``entro_rans_freqs``)."""
    c = np.ascontiguousarray(counts, dtype=np.uint64)
    f = np.zeros(c.size, dtype=np.uint32)
    _check(load().entro_rans_freqs(_np_ptr(c), c.size, _np_ptr(f)), "entro_rans_freqs")
    return f


def rans_table_build(freqs: np.ndarray, sym_bits: int, scale: float, zero_point: int) -> np.ndarray:
    f = np.ascontiguousarray(freqs, dtype=np.uint32)
    lib = load()
    nb = int(lib.entro_rans_table_bytes())
    out = np.zeros(nb // 4, dtype=np.uint32)
    _check(lib.entro_rans_table_build(int(sym_bits), _np_ptr(f), ctypes.c_float(scale), int(zero_point),
                                      _np_ptr(out), nb), "entro_rans_table_build")
    return out


def rans_encode(q: np.ndarray, freqs: np.ndarray, sym_bits: int, chunk: int, lanes: int, threads: int = 0):
    """-> ``(units uint16, chunk_unit_off uint64)`` (``entro_rans_encode``)."""
    q = np.ascontiguousarray(q, dtype=np.uint8).ravel()
    f = np.ascontiguousarray(freqs, dtype=np.uint32)
    nc = -(-q.size // chunk) if q.size else 0
    offs = np.zeros(nc + 1, dtype=np.uint64)
    nu = ctypes.c_uint64()
    lib = load()
    _check(lib.entro_rans_encode(_np_ptr(q), q.size, _np_ptr(f), int(sym_bits), int(chunk), int(lanes),
                                 _np_ptr(offs), None, 0, ctypes.byref(nu), int(threads)), "entro_rans_encode")
    units = np.zeros(max(int(nu.value), 1), dtype=np.uint16)
    _check(lib.entro_rans_encode(_np_ptr(q), q.size, _np_ptr(f), int(sym_bits), int(chunk), int(lanes),
                                 _np_ptr(offs), _np_ptr(units), units.size, ctypes.byref(nu), int(threads)),
           "entro_rans_encode")
    return units[: int(nu.value)], offs


@dataclass
class DeviceRansTensor:
    """Device copies of one rANS-coded tensor plus its ``RansTensor`` descriptor."""
    table: object
    units: object
    offs: object
    desc: RansTensor

    @classmethod
    def upload(cls, table: np.ndarray, units: np.ndarray, offs: np.ndarray, n_symbols: int, chunk: int,
               lanes: int, sym_bits: int, device="cuda"):
        import torch

        d_table = torch.from_numpy(np.ascontiguousarray(table).view(np.int32)).to(device)
        u = np.ascontiguousarray(units, dtype=np.uint16)
        d_units = torch.from_numpy(u.view(np.int16) if u.size else np.zeros(8, np.int16)).to(device)
        d_offs = torch.from_numpy(np.ascontiguousarray(offs, dtype=np.uint64).view(np.int64)).to(device)
        o = np.asarray(offs, dtype=np.uint64)
        mcu = int(np.diff(o).max()) if o.size > 1 else 0
        desc = RansTensor(d_table.data_ptr(), d_units.data_ptr(), d_offs.data_ptr(), int(u.size), int(n_symbols),
                          int(chunk), int(lanes), int(sym_bits), mcu)
        return cls(d_table, d_units, d_offs, desc)


# --------------------------------------------------------------------------
# offline encoder (host)
# --------------------------------------------------------------------------

def quantize(w: np.ndarray, bits: int, scheme: str = "mixed", clip: float = 0.0):
    """-> ``(q uint8, scale float32, zero_point int, scheme name)``."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    q = np.empty(w.shape, dtype=np.uint8)
    scale = ctypes.c_float()
    zp = ctypes.c_int32()
    chosen = ctypes.c_int()
    _check(load().entro_quantize(_np_ptr(w), w.size, bits, _SCHEME_IDS[scheme], float(clip), _np_ptr(q),
                                 ctypes.byref(scale), ctypes.byref(zp), ctypes.byref(chosen)), "entro_quantize")
    return q, np.float32(scale.value), int(zp.value), _SCHEME_NAMES[chosen.value]


def code_lengths(q: np.ndarray, bits: int, max_len: int) -> np.ndarray:
    q = np.ascontiguousarray(q, dtype=np.uint8).ravel()
    out = np.zeros(1 << bits, dtype=np.uint8)
    _check(load().entro_code_lengths(_np_ptr(q), q.size, bits, max_len, _np_ptr(out)), "entro_code_lengths")
    return out


def encode_layout(q: np.ndarray, code_len: np.ndarray, bits: int, chunk: int, lanes: int):
    """-> ``(chunk_bit_off uint64[n_chunks + 1], n_words)``."""
    q = np.ascontiguousarray(q, dtype=np.uint8).ravel()
    cl = np.ascontiguousarray(code_len, dtype=np.uint8)
    offs = np.zeros(-(-q.size // chunk) + 1, dtype=np.uint64)
    nw = ctypes.c_uint64()
    _check(load().entro_encode_layout(_np_ptr(q), q.size, _np_ptr(cl), bits, chunk, lanes, _np_ptr(offs),
                                      ctypes.byref(nw)), "entro_encode_layout")
    return offs, int(nw.value)


def encode(q: np.ndarray, code_len: np.ndarray, bits: int, chunk: int, lanes: int, threads: int = 0,
           refill_steps: int = 1, ahead: bool = False):
    """-> ``(words uint32, chunk_bit_off uint64)``."""
    q = np.ascontiguousarray(q, dtype=np.uint8).ravel()
    cl = np.ascontiguousarray(code_len, dtype=np.uint8)
    offs, nw = encode_layout(q, cl, bits, chunk, lanes)
    words = np.zeros(nw, dtype=np.uint32)
    _check(load().entro_encode(_np_ptr(q), q.size, _np_ptr(cl), bits, chunk, lanes, refill_steps, int(ahead),
                               _np_ptr(offs), _np_ptr(words), threads), "entro_encode")
    return words, offs


# --------------------------------------------------------------------------
# convenience: one coded tensor held on the device
# --------------------------------------------------------------------------

@dataclass
class DeviceTensor:
    """Device copies of one coded tensor plus its ``Tensor`` descriptor.

    Holds the torch tensors so that the device memory outlives the calls.
    """
    lut: object
    words: object
    offs: object
    desc: Tensor
    pair_lut: object = None

    @classmethod
    def upload(cls, lut: np.ndarray, words: np.ndarray, offs: np.ndarray, n_symbols: int,
               chunk: int, lanes: int, sym_bits: int, max_len: int, device="cuda", refill_steps: int = 1,
               ahead: bool = False, pair_lut: bool = True):
        """``pair_lut``: for 4-bit tensors, also build the two-code table on
        the host and upload it (``d_pair_lut``); the fused GEMV then loads it
        instead of building it on chip."""
        import torch

        d_lut = torch.from_numpy(np.ascontiguousarray(lut).view(np.int32)).to(device)
        w = np.ascontiguousarray(words, dtype=np.uint32)
        d_words = torch.from_numpy(w.view(np.int32) if w.size else np.zeros(1, np.int32)).to(device)
        d_offs = torch.from_numpy(np.ascontiguousarray(offs, dtype=np.uint64).view(np.int64)).to(device)
        o = np.asarray(offs, dtype=np.uint64)
        max_cw = int(np.diff(o).max() // 32) if o.size > 1 else 0
        desc = Tensor(d_lut.data_ptr(), d_words.data_ptr(), d_offs.data_ptr(), int(w.size), int(n_symbols),
                      int(chunk), int(lanes), int(sym_bits), int(max_len), int(np.asarray(lut).nbytes),
                      max_cw, int(refill_steps), int(ahead))
        d_pair = None
        if pair_lut and int(sym_bits) == 4:
            d_pair = torch.from_numpy(pair_lut_build(lut).view(np.int32)).to(device)
            desc.d_pair_lut = d_pair.data_ptr()
        return cls(d_lut, d_words, d_offs, desc, d_pair)
