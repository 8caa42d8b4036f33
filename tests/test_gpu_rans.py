"""GPU parity of the interleaved rANS decoder (ECR v1) against the oracle:
codes and bf16 bit-exact over a fuzz grid (both lane counts, both code widths,
every histogram kind, ragged last chunks, several tensors per call), the two
full-size single tensors, and the flags of malformed streams.  Streams and
expected values come from the oracle only; the library contributes its slot
table builder and the kernel under test."""
import sys

import numpy as np
import pytest

import entropy_coded_weight_canonical_amd as ent
from oracle import quant, rans
from oracle.dequant import dequant_bf16
from synth import CODE_KINDS, TensorSpec, fuzz_codes, weights

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ent.load()


class RCase:
    def __init__(self, q, bits, chunk, lanes, scale=0.0123, zp=None):
        self.q = np.ascontiguousarray(np.asarray(q, dtype=np.uint8).ravel())
        self.bits, self.chunk, self.lanes = bits, chunk, lanes
        self.scale = np.float32(scale)
        self.zp = (1 << (bits - 1)) if zp is None else zp
        self.freqs = rans.quantize_freqs(quant.histogram(self.q, bits))
        self.units, self.offs = rans.encode(self.q, self.freqs, chunk, lanes)
        self.table = ent.rans_table_build(self.freqs, bits, self.scale, self.zp)

    @property
    def n(self):
        return int(self.q.size)

    def upload(self):
        return ent.DeviceRansTensor.upload(self.table, self.units, self.offs, self.n, self.chunk, self.lanes,
                                           self.bits)


def run(cases, mode):
    import torch

    dts = [c.upload() for c in cases]
    dtype = torch.uint8 if mode == "u8" else torch.int16
    outs = [torch.full((max(c.n, 1),), 0x5A if mode == "u8" else 0x5A5A, dtype=dtype, device="cuda") for c in cases]
    status = torch.zeros(len(cases), dtype=torch.int32, device="cuda")
    fn = ent.rans_decode if mode == "u8" else ent.rans_decode_dequant
    fn([d.desc for d in dts], [o.data_ptr() for o in outs], status.data_ptr())
    torch.cuda.synchronize()
    res = []
    for c, o in zip(cases, outs):
        a = o.cpu().numpy()[: c.n]
        res.append(a if mode == "u8" else a.view(np.uint16))
    return res, status.cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("lanes", [32, 64])
@pytest.mark.parametrize("bits", [4, 8])
def test_fuzz_grid_bit_exact(lanes, bits):
    cases = []
    for i, kind in enumerate(CODE_KINDS):
        for chunk_mult, extra in ((4, 0), (2, 37), (8, lanes + 5), (1, 0)):
            chunk = lanes * chunk_mult
            n = 5 * chunk + extra
            cases.append(RCase(fuzz_codes(bits * 100 + lanes + i * 7 + chunk_mult, n, bits, kind), bits, chunk, lanes))
    say(f"rANS fuzz grid W={lanes} bits={bits}: {len(cases)} tensors in one call")
    for mode in ("u8", "bf16"):
        outs, st = run(cases, mode)
        assert (st == 0).all(), st
        for c, o in zip(cases, outs):
            exp = c.q if mode == "u8" else dequant_bf16(c.q, c.scale, c.zp)
            assert np.array_equal(o, exp)


@pytest.mark.parametrize("name,bits,scheme,chunk,lanes", [("tensor_4096", 4, "unsigned", 8192, 32),
                                                          ("tensor_2048", 8, "asymmetric", 4096, 32),
                                                          ("tensor_2048", 8, "asymmetric", 4096, 64)])
def test_full_size_tensors(name, bits, scheme, chunk, lanes):
    w = weights(TensorSpec(name, 0, -1, "w", *((4096, 4096) if name == "tensor_4096" else (2048, 2048)), "w"))
    qz = (quant.quantize_unsigned if scheme == "unsigned" else quant.quantize_asymmetric)(w, bits)
    q = qz.q.ravel()
    freqs = rans.quantize_freqs(quant.histogram(q, bits))
    units, offs = ent.rans_encode(q, freqs, bits, chunk, lanes)   # byte-identical to the oracle (host tests)
    c = RCase.__new__(RCase)
    c.q, c.bits, c.chunk, c.lanes, c.scale, c.zp = q, bits, chunk, lanes, qz.scale, qz.zero_point
    c.freqs, c.units, c.offs = freqs, units, offs
    c.table = ent.rans_table_build(freqs, bits, qz.scale, qz.zero_point)
    say(f"rANS {name} W={lanes} x3 tensors")
    outs, st = run([c, c, c], "bf16")
    assert (st == 0).all()
    exp = dequant_bf16(q, qz.scale, qz.zero_point)
    for o in outs:
        assert np.array_equal(o, exp)


def test_malformed_streams_are_flagged_not_fatal():
    good = RCase(fuzz_codes(1, 4000, 8, "skewed"), 8, 512, 32)
    trunc = RCase(fuzz_codes(2, 4000, 8, "skewed"), 8, 512, 32)
    trunc.units = trunc.units[:-3]
    trunc.offs = trunc.offs.copy()
    trunc.offs[-1] -= 3
    flip = RCase(fuzz_codes(3, 4000, 4, "peaked"), 4, 512, 64)
    flip.units = flip.units.copy()
    flip.units[flip.offs[2] + 1] ^= 0x1234        # an initial state of chunk 2
    badoff = RCase(fuzz_codes(4, 4000, 4, "uniform"), 4, 512, 64)
    badoff.offs = badoff.offs.copy()
    badoff.offs[3] = badoff.offs[2] + 3           # a chunk too short for its states
    say("rANS malformed streams")
    outs, st = run([good, trunc, flip, badoff], "u8")
    assert st[0] == 0 and np.array_equal(outs[0], good.q)
    assert st[1] != 0 and st[2] != 0
    assert st[3] & ent.FLAGS["offsets"]


def test_odd_unit_counts_read_the_last_unit():
    """A tensor with an odd number of 16-bit units ends in half a dword; its
    last unit (taken by the last chunk's decoder, often at its first step)
    must still be staged.  Lone last chunks and paired ones, both lane counts."""
    cases = []
    seed = 0
    while len(cases) < 12:
        lanes = 32 if len(cases) % 2 else 64
        chunk = lanes * (2 + len(cases) % 3)
        n = (4 + len(cases) % 2) * chunk + (len(cases) % 4) * 7
        c = RCase(fuzz_codes(900 + seed, n, 4 if seed % 2 else 8, ("uniform", "skewed")[seed % 2]), 4 if seed % 2 else 8,
                  chunk, lanes)
        seed += 1
        if len(c.units) % 2:
            cases.append(c)
    say(f"rANS odd unit counts: {len(cases)} tensors")
    for mode in ("u8", "bf16"):
        outs, st = run(cases, mode)
        assert (st == 0).all(), st
        for c, o in zip(cases, outs):
            assert np.array_equal(o, c.q if mode == "u8" else dequant_bf16(c.q, c.scale, c.zp))


def test_edge_cases_in_one_call():
    """An empty tensor between others, fewer codes than lanes, exactly one
    step, a tensor of one code value (every state stays at L), chunks of one
    step each, both lane counts, both code widths."""
    one = np.full(300, 9, dtype=np.uint8)
    cases = [RCase(fuzz_codes(31, 5, 4, "uniform"), 4, 64, 64),        # 5 codes, 64 lanes
             RCase(fuzz_codes(32, 32, 8, "skewed"), 8, 32, 32),        # one full step
             RCase(one, 4, 128, 32),                                   # a single code value
             RCase(fuzz_codes(33, 64 * 7 + 3, 8, "peaked"), 8, 64, 64),  # one step per chunk, ragged tail
             RCase(fuzz_codes(34, 33, 4, "skewed"), 4, 32, 32)]        # one step and one code
    empty = RCase.__new__(RCase)
    empty.q = np.zeros(0, dtype=np.uint8)
    empty.bits, empty.chunk, empty.lanes, empty.scale, empty.zp = 4, 64, 32, np.float32(0.5), 8
    empty.freqs = cases[0].freqs
    empty.units, empty.offs = np.zeros(0, dtype=np.uint16), np.zeros(1, dtype=np.uint64)
    empty.table = cases[0].table
    cases.insert(2, empty)
    say("rANS edge cases")
    for mode in ("u8", "bf16"):
        outs, st = run(cases, mode)
        assert (st == 0).all(), st
        for c, o in zip(cases, outs):
            assert o.size == c.n
            assert np.array_equal(o, c.q if mode == "u8" else dequant_bf16(c.q, c.scale, c.zp))
