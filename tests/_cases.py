"""Coded test cases built only by the oracle (code lengths, stream, expected
values) plus the library's own decode table, and helpers that run the device
entry points through the C ABI."""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

import entropy_coded_weight_canonical_amd as ent
from oracle import ccodec, huffman, quant
from oracle.dequant import dequant_bf16


@dataclass
class Case:
    q: np.ndarray            # flattened uint8 codes (the expected decode)
    bits: int
    max_len: int
    lengths: np.ndarray
    scale: np.float32
    zp: int
    chunk: int
    lanes: int
    words: np.ndarray
    offs: np.ndarray
    lut: np.ndarray
    rows: int = 0
    cols: int = 0
    refill_steps: int = 1
    ahead: bool = False

    @property
    def n(self) -> int:
        return int(self.q.size)

    def expected_bf16(self) -> np.ndarray:
        return dequant_bf16(self.q, self.scale, self.zp)


def make_case(q, bits, chunk, lanes, scale=0.0123, zp=None, max_len=None, lengths=None,
              rows=0, cols=0, refill_steps=1, ahead=False) -> Case:
    q = np.ascontiguousarray(np.asarray(q, dtype=np.uint8).ravel())
    max_len = max_len or (16 if bits == 8 else 12)
    if lengths is None:
        lengths = huffman.code_lengths(quant.histogram(q, bits), max_len) if q.size else None
    if lengths is None:  # empty tensor: any valid codebook
        lengths = np.zeros(1 << bits, dtype=np.int64)
        lengths[0] = 1
    zp = (1 << (bits - 1)) if zp is None else zp
    words, offs = ccodec.encode(q, lengths, chunk, lanes, threads=8, refill_steps=refill_steps, ahead=ahead)
    lut = ent.lut_build(lengths, bits, max_len, np.float32(scale), zp)
    return Case(q, bits, max_len, np.asarray(lengths, dtype=np.uint8), np.float32(scale), int(zp), chunk,
                lanes, words, offs, lut, rows, cols, refill_steps, bool(ahead))


def upload(case: Case, device="cuda", pair_lut=True):
    return ent.DeviceTensor.upload(case.lut, case.words, case.offs, case.n, case.chunk, case.lanes, case.bits,
                                   case.max_len, device=device, refill_steps=case.refill_steps, ahead=case.ahead,
                                   pair_lut=pair_lut)


def _offset_lut(dt, case: Case, offset: int, device):
    """Point ``dt``'s descriptor at a copy of its table ``offset`` words into
    a fresh allocation; returns the allocation (keep it alive)."""
    import torch

    buf = torch.zeros(case.lut.size + offset, dtype=torch.int32, device=device)
    buf[offset:] = torch.from_numpy(np.ascontiguousarray(case.lut).view(np.int32)).to(device)
    dt.desc.d_lut = buf.data_ptr() + 4 * offset
    return buf


def run_decode(cases, mode="u8", device="cuda", cached=None, lut_offset=0):
    """Decode ``cases`` in one call; returns (outputs as numpy, status numpy).
    ``cached``: per case, the descriptor's ``out_cached`` flag (default 0).
    ``lut_offset`` (words) places the decode tables that far past a 256-byte
    aligned allocation."""
    import torch

    dts = [upload(c, device) for c in cases]
    keep = [_offset_lut(d, c, lut_offset, device) for d, c in zip(dts, cases)] if lut_offset else []
    for d, f in zip(dts, cached or []):
        d.desc.out_cached = int(f)
    dtype = torch.uint8 if mode == "u8" else torch.int16
    outs = [torch.empty(max(c.n, 1), dtype=dtype, device=device) for c in cases]
    if mode == "u8":
        for o in outs:
            o.fill_(0xA5)
    else:
        for o in outs:
            o.fill_(0x5A5A)
    status = torch.zeros(len(cases), dtype=torch.int32, device=device)
    fn = ent.decode if mode == "u8" else ent.decode_dequant
    fn([d.desc for d in dts], [o.data_ptr() for o in outs], status.data_ptr())
    torch.cuda.synchronize()
    res = []
    for c, o in zip(cases, outs):
        a = o.cpu().numpy()[: c.n]
        res.append(a if mode == "u8" else a.view(np.uint16))
    return res, status.cpu().numpy().view(np.uint32)


def run_gemv(cases, xs, batch, device="cuda", x_offset=0, lut_offset=0, pair_lut=True, edit=None):
    """Fused GEMV of ``cases`` (each with rows/cols) on bf16 inputs ``xs``.
    ``x_offset`` (elements) and ``lut_offset`` (words) place x and the decode
    table that far past a 256-byte aligned allocation; ``pair_lut``: upload
    the host-built two-code tables of 4-bit tensors; ``edit(i, dt)`` may
    change descriptor i before the call."""
    import torch

    dts = [upload(c, device, pair_lut=pair_lut) for c in cases]
    for i, d in enumerate(dts):
        if edit:
            edit(i, d)
    keep = [_offset_lut(d, c, lut_offset, device) for d, c in zip(dts, cases)] if lut_offset else []
    dx = []
    for x in xs:
        flat = np.ascontiguousarray(x).view(np.int16).ravel()
        buf = torch.zeros(flat.size + x_offset, dtype=torch.int16, device=device)
        buf[x_offset:] = torch.from_numpy(flat).to(device)
        dx.append(buf[x_offset:])
    dy = [torch.full((batch, max(c.rows, 1)), float("nan"), dtype=torch.float32, device=device) for c in cases]
    items = [ent.GemvItem(c.rows, c.cols, x.data_ptr(), y.data_ptr()) for c, x, y in zip(cases, dx, dy)]
    status = torch.zeros(len(cases), dtype=torch.int32, device=device)
    ent.decode_gemv([d.desc for d in dts], items, batch, status.data_ptr())
    torch.cuda.synchronize()
    return [y.cpu().numpy()[:, : c.rows] for c, y in zip(cases, dy)], status.cpu().numpy().view(np.uint32)
