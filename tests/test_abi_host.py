"""Host-side checks of the C ABI (no GPU needed).

* libentro.so loads and exports every function declared in include/*.h;
* entro_lut_build rejects malformed codebooks and its tables decode like the
  oracle's canonical code (prefix match on every index) with the oracle's
  bf16 values;
* the device entry points reject bad descriptors before touching the GPU;
* the library's offline encoder agrees with the oracle: identical codes from
  the quantizer, optimal code lengths of equal cost, byte-identical streams,
  and the oracle decodes what the library writes.
"""
import ctypes
import glob
import os
import re

import numpy as np
import pytest

import entropy_coded_weight_canonical_amd as ent
from oracle import ccodec, ecw, huffman, quant
from oracle.canonical import canonical_codes, codeword_str
from oracle.dequant import dequant_bf16
from synth import TensorSpec, fuzz_codes, weights

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    return ent.load()


def declared_functions():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"\b(entro_[a-z0-9_]+)\s*\(", text):
            names.add(m.group(1))
    return sorted(names)


def test_library_exports_every_declared_function(lib):
    names = declared_functions()
    assert {"entro_decode", "entro_decode_dequant", "entro_decode_gemv", "entro_lut_build",
            "entro_lut_bytes", "entro_status_str"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert ent.status_str(0) == "ok"
    assert "codebook" in ent.status_str(2)


def _expected_entry(lengths, codes, vals, bits_str):
    """The codeword that prefixes ``bits_str`` -> (len, sym, bf16) or None."""
    for s in range(len(lengths)):
        l = int(lengths[s])
        if l and bits_str.startswith(codeword_str(int(codes[s]), l)):
            return l, s, int(vals[s])
    return None


def check_lut(lut, lengths, sym_bits, max_len, scale, zp):
    codes = canonical_codes(lengths)
    vals = dequant_bf16(np.arange(1 << sym_bits), scale, zp)
    assert lut[0] == 0x31574345
    K = int(lut[1]) & 0xFF
    assert (int(lut[1]) >> 8) & 0xFF == sym_bits and (int(lut[1]) >> 16) & 0xFF == max_len
    assert int(lut[1]) >> 24 == min(int(x) for x in lengths if x)
    n_entries, l1 = int(lut[2]), int(lut[3])
    assert l1 == 1 << K and lut.size == 4 + n_entries
    e = lut[4:]
    longest = int(max(lengths))
    for idx in range(l1):
        prefix = format(idx, f"0{K}b")
        ent_ = int(e[idx])
        if ent_ & 0x80:
            sb = (ent_ >> 8) & 31
            base = ent_ >> 16
            assert longest > K
            for i2 in range(1 << sb):
                bits = prefix + format(i2, f"0{sb}b")
                exp = _expected_entry(lengths, codes, vals, bits)
                got = int(e[base + i2])
                assert exp is not None and (got & 31, (got >> 8) & 0xFF, got >> 16) == exp
        else:
            exp = _expected_entry(lengths, codes, vals, prefix)
            if exp is None:
                assert ent_ == 0  # no codeword with this prefix (incomplete code)
            else:
                assert exp[0] <= K
                assert (ent_ & 31, (ent_ >> 8) & 0xFF, ent_ >> 16) == exp


@pytest.mark.parametrize("seed", range(12))
def test_lut_matches_oracle_code(seed):
    rng = np.random.default_rng(seed)
    bits = 8 if seed % 3 else 4
    kind = ["skewed", "peaked", "uniform", "sparse"][seed % 4]
    q = fuzz_codes(seed, 20000, bits, kind)
    max_len = 16 if bits == 8 else 12
    lengths = huffman.code_lengths(quant.histogram(q, bits), max_len)
    scale = np.float32(rng.uniform(1e-4, 1e-1))
    zp = int(rng.integers(0, 1 << bits))
    lut = ent.lut_build(lengths, bits, max_len, scale, zp)
    assert ent.lut_bytes(lengths, bits, max_len, scale, zp) == lut.nbytes
    check_lut(lut, lengths, bits, max_len, scale, zp)


def check_pair_lut(p, lut, lengths, scale, zp):
    """Every entry of a two-code table against the oracle's canonical code:
    the two codewords the 12 index bits begin with (zeros after them), or the
    fallback mark where they do not both lie within the 12 bits."""
    codes = canonical_codes(lengths)
    vals = dequant_bf16(np.arange(16), scale, zp)
    assert p.size == 4 + 2 * 4096 and p[0] == 0x31504345 and p[2] == lut[1] and p[3] == 0
    whole = True
    for i in range(4096):
        bits = format(i, "012b") + "0" * 20
        a = _expected_entry(lengths, codes, vals, bits)
        b = None
        if a is not None and a[0] <= 12:
            b = _expected_entry(lengths, codes, vals, bits[a[0]:] + "0" * a[0])
        if a is None or b is None or a[0] + b[0] > 12:
            exp = (0, 0x80 | 0xFF00)
            whole = False
        else:
            lab = a[0] + b[0]
            exp = (a[2] | (b[2] << 16), (lab << 8) | ((32 - lab) & 31))
        assert (int(p[4 + 2 * i]), int(p[5 + 2 * i])) == exp, i
    assert int(p[1]) == (1 if whole else 0)
    return whole


@pytest.mark.parametrize("seed", range(8))
def test_pair_lut_matches_oracle_code(seed):
    """entro_pair_lut_build over 4-bit codes of every kind: short codes (every
    index a whole pair), long ones (up to the 12-bit cap, two-level decode
    tables) and incomplete codes (indices that begin no codeword)."""
    rng = np.random.default_rng(100 + seed)
    kind = ["skewed", "peaked", "uniform", "sparse"][seed % 4]
    q = fuzz_codes(seed, 20000, 4, kind)
    lengths = huffman.code_lengths(quant.histogram(q, 4), 12)
    if seed >= 4:   # geometric counts: lengths up to the cap
        counts = (2.0 ** np.arange(16, 0, -1)).astype(np.int64)
        lengths = huffman.code_lengths(counts if seed < 6 else counts[::-1].copy(), 12 if seed % 2 else 9)
    scale = np.float32(rng.uniform(1e-4, 1e-1))
    zp = int(rng.integers(0, 16))
    lut = ent.lut_build(lengths, 4, 12, scale, zp)
    check_pair_lut(ent.pair_lut_build(lut), lut, lengths, scale, zp)


def test_pair_lut_cases_and_rejections(lib):
    # uniform 4-bit code: every index holds a whole pair
    lengths = np.full(16, 4, dtype=np.uint8)
    lut = ent.lut_build(lengths, 4, 12, np.float32(0.5), 8)
    assert check_pair_lut(ent.pair_lut_build(lut), lut, lengths, np.float32(0.5), 8)
    # a 12-bit codeword: indices that begin it cannot hold a pair
    counts = (2.0 ** np.arange(16, 0, -1)).astype(np.int64)
    lengths = huffman.code_lengths(counts, 12)
    assert lengths.max() == 12
    lut = ent.lut_build(lengths, 4, 12, np.float32(0.5), 8)
    assert not check_pair_lut(ent.pair_lut_build(lut), lut, lengths, np.float32(0.5), 8)
    out = np.zeros(4 + 8192, dtype=np.uint32)
    P = ctypes.c_void_p
    bad = lut.copy()
    bad[0] ^= 1
    assert lib.entro_pair_lut_build(P(bad.ctypes.data), bad.nbytes, P(out.ctypes.data), out.nbytes) == 1
    assert lib.entro_pair_lut_build(P(lut.ctypes.data), lut.nbytes, P(out.ctypes.data), out.nbytes - 4) == 1
    assert lib.entro_pair_lut_build(P(lut.ctypes.data), 8, P(out.ctypes.data), out.nbytes) == 1
    lut8 = ent.lut_build(np.full(256, 8, dtype=np.uint8), 8, 16, np.float32(0.5), 8)
    assert lib.entro_pair_lut_build(P(lut8.ctypes.data), lut8.nbytes, P(out.ctypes.data), out.nbytes) == 4
    assert lib.entro_pair_lut_bytes() == 16 + 8 * 4096


def test_lut_two_level_with_longest_codes():
    # geometric counts force the 16-bit cap to bind on 8-bit codes
    counts = np.zeros(256, dtype=np.int64)
    counts[:40] = (2.0 ** np.arange(40, 0, -1)).astype(np.int64) // 2 + 1
    lengths = huffman.code_lengths(counts, 16)
    assert lengths.max() == 16
    lut = ent.lut_build(lengths, 8, 16, np.float32(0.01), 3)
    K = int(lut[1]) & 0xFF
    assert K == expected_first_level(lengths) and K < 16
    check_lut(lut, lengths, 8, 16, np.float32(0.01), 3)


def expected_first_level(lengths):
    """First-level width rule of entro_lut_build: smallest k >= 5 whose longer
    codes carry sum 2^-len <= 2^-10, capped at the longest code (<= 12) or 11."""
    ls = [int(l) for l in lengths if l]
    top = max(ls)
    kmax = top if top <= 12 else 11
    for k in range(min(5, kmax), kmax):
        if sum(2.0 ** -l for l in ls if l > k) <= 2.0 ** -10:
            return k
    return kmax


@pytest.mark.parametrize("seed", range(8))
def test_lut_first_level_width_rule(seed):
    bits = 8 if seed % 2 else 4
    q = fuzz_codes(300 + seed, 30000, bits, ["skewed", "peaked", "uniform", "sparse"][seed % 4])
    lengths = huffman.code_lengths(quant.histogram(q, bits), 16 if bits == 8 else 12)
    lut = ent.lut_build(lengths, bits, 16 if bits == 8 else 12, np.float32(0.02), 1)
    assert int(lut[1]) & 0xFF == expected_first_level(lengths)


def test_lut_single_symbol_and_incomplete_code():
    lengths = np.zeros(16, dtype=np.int64)
    lengths[6] = 1
    lut = ent.lut_build(lengths, 4, 12, np.float32(0.5), 8)
    check_lut(lut, lengths, 4, 12, np.float32(0.5), 8)
    lengths = np.zeros(16, dtype=np.int64)
    lengths[[1, 2, 3]] = [2, 2, 3]   # Kraft 5/8
    lut = ent.lut_build(lengths, 4, 12, np.float32(0.5), 8)
    check_lut(lut, lengths, 4, 12, np.float32(0.5), 8)


def test_lut_rejects_bad_codebooks(lib):
    def status(code_len, sym_bits=4, max_len=12):
        cl = np.ascontiguousarray(code_len, dtype=np.uint8)
        cb = ent.Codebook(sym_bits, max_len, cl.ctypes.data, 1.0, 0)
        buf = np.zeros(8192, dtype=np.uint32)
        return lib.entro_lut_build(ctypes.byref(cb), buf.ctypes.data, buf.nbytes)

    ok = np.zeros(16, dtype=np.uint8)
    ok[:2] = 1
    assert status(ok) == 0
    assert status(np.zeros(16)) == 2                      # no symbol
    over = np.zeros(16, dtype=np.uint8)
    over[:3] = 1
    assert status(over) == 2                              # Kraft 3/2
    long_ = ok.copy()
    long_[2] = 13
    assert status(long_) == 2                             # longer than max_len 12
    assert status(ok, sym_bits=5) == 3
    assert status(ok, max_len=17) == 3
    assert status(ok, max_len=0) == 3
    cb = ent.Codebook(4, 12, ok.ctypes.data, 1.0, 0)
    small = np.zeros(2, dtype=np.uint32)
    assert lib.entro_lut_build(ctypes.byref(cb), small.ctypes.data, small.nbytes) == 1
    assert lib.entro_lut_build(None, small.ctypes.data, small.nbytes) == 1
    assert lib.entro_lut_bytes(None) == 0


def test_device_entry_points_validate_before_launch(lib):
    t = ent.Tensor(1, 1, 1, 10, 100, 64, 64, 4, 12, 64)
    arr = (ent.Tensor * 1)(t)
    outs = (ctypes.c_void_p * 1)(1)
    st = ctypes.c_void_p(1)

    def dec(**kw):
        x = ent.Tensor(1, 1, 1, 10, 100, 64, 64, 4, 12, 64)
        for k, v in kw.items():
            setattr(x, k, v)
        return lib.entro_decode((ent.Tensor * 1)(x), 1, outs, st, None)

    assert dec(lanes=3) == 3
    assert dec(lanes=128) == 3
    assert dec(chunk_symbols=96, lanes=64) == 3
    assert dec(chunk_symbols=0) == 3
    assert dec(sym_bits=6) == 3
    assert dec(max_len=17) == 3
    assert dec(refill_steps=3) == 3
    assert dec(refill_ahead=2) == 3
    assert dec(out_cached=2) == 3
    assert dec(d_words=None) == 1
    assert lib.entro_decode(arr, 1, None, st, None) == 1
    assert lib.entro_decode(arr, 1, outs, None, None) == 1
    assert lib.entro_decode(arr, 0, outs, st, None) == 0
    # outputs of neighbouring lanes are stored together: 2-byte aligned codes,
    # 4-byte aligned bf16 (rejected before anything is enqueued)
    assert lib.entro_decode(arr, 1, (ctypes.c_void_p * 1)(0x1001), st, None) == 1
    assert lib.entro_decode_dequant(arr, 1, (ctypes.c_void_p * 1)(0x1002), st, None) == 1
    assert lib.entro_decode_dequant(arr, 1, (ctypes.c_void_p * 1)(0x1001), st, None) == 1
    # GEMV shape checks
    g = (ent.GemvItem * 1)(ent.GemvItem(10, 10, 1, 1))
    assert lib.entro_decode_gemv(arr, 1, g, 1, st, None) == 3      # W=64 does not divide cols=10
    g = (ent.GemvItem * 1)(ent.GemvItem(10, 11, 1, 1))
    assert lib.entro_decode_gemv(arr, 1, g, 1, st, None) == 1      # rows*cols != n
    g = (ent.GemvItem * 1)(ent.GemvItem(1, 100, 1, 1))
    assert lib.entro_decode_gemv(arr, 1, g, 9, st, None) == 1      # batch > 8
    assert lib.entro_decode_gemv(arr, 1, g, 0, st, None) == 1


def test_gemm_entry_point_validates_before_launch(lib):
    st = ctypes.c_void_p(1)

    def gemm(n_tokens=16, rows=2, cols=128, x=0x1000, y=0x2000, **kw):
        t = ent.Tensor(1, 1, 1, 10, rows * cols, cols, 64, 4, 12, 64, 8, 2, 1)
        for k, v in kw.items():
            setattr(t, k, v)
        g = (ent.GemvItem * 1)(ent.GemvItem(rows, cols, x, y))
        return lib.entro_decode_gemm((ent.Tensor * 1)(t), 1, g, n_tokens, st, None)

    assert gemm(n_tokens=0) == 1
    assert gemm(n_tokens=513) == 1
    assert gemm(x=0x1008) == 1                       # activations not 16-byte aligned
    assert gemm(x=0) == 1
    assert gemm(rows=3, n_symbols=256) == 1           # rows * cols != n_symbols
    assert gemm(cols=192, chunk_symbols=192) == 3     # cols not a multiple of 128
    assert gemm(chunk_symbols=256) == 3               # two rows per chunk
    assert gemm(lanes=32) == 4                        # only 64 lanes
    assert gemm(sym_bits=8, max_len=16) == 4          # only 4-bit codes
    assert gemm(refill_steps=1) == 4                  # only pairs of steps
    assert gemm(n_words=1 << 30) == 4                 # a stream of 4 GiB or more
    assert lib.entro_decode_gemm((ent.Tensor * 1)(), 0, None, 16, st, None) == 0


def test_a_call_that_fails_planning_enqueues_nothing(lib):
    """The tensors of a call go out in launches of up to 32; a tensor that a
    later launch cannot take must fail the whole call before the earlier
    launches are enqueued.  On this machine (no GPU) an enqueued launch would
    report ENTRO_E_HIP (5), so ENTRO_E_UNSUPPORTED (4) shows that planning
    rejected the call first."""
    st = ctypes.c_void_p(1)
    good = [ent.Tensor(1, 1, 1, 10, 2 * 128, 128, 64, 4, 12, 64, 8, 2, 1) for _ in range(40)]
    bad = list(good)
    bad[35] = ent.Tensor(1, 1, 1, 1 << 30, 2 * 128, 128, 64, 4, 12, 64, 8, 2, 1)   # a stream of 4 GiB
    g = (ent.GemvItem * 40)(*[ent.GemvItem(2, 128, 0x1000, 0x2000) for _ in range(40)])
    assert lib.entro_decode_gemm((ent.Tensor * 40)(*bad), 40, g, 16, st, None) == 4
    assert lib.entro_decode_gemm((ent.Tensor * 40)(*good), 40, g, 16, st, None) == 5


# --------------------------------------------------------------------------
# the library's offline encoder against the oracle
# --------------------------------------------------------------------------

@pytest.mark.parametrize("bits,scheme,dist", [(8, "asymmetric", "normal"), (8, "unsigned", "t"),
                                              (4, "unsigned", "laplace"), (4, "asymmetric", "t"),
                                              (8, "mixed", "t"), (4, "mixed", "laplace")])
def test_quantizer_matches_oracle(bits, scheme, dist):
    rng = np.random.default_rng(bits * 7 + len(scheme))
    n = 300_000
    w = {"normal": rng.normal(0, 0.02, n), "t": rng.standard_t(4, n) * 0.02,
         "laplace": rng.laplace(0, 0.015, n)}[dist].astype(np.float32)
    q, s, zp, chosen = ent.quantize(w, bits, scheme)
    ref = {"asymmetric": quant.quantize_asymmetric, "unsigned": quant.quantize_unsigned,
           "mixed": quant.quantize_mixed}[scheme](w, bits)
    assert chosen == ref.scheme
    assert s == ref.scale and zp == ref.zero_point
    assert np.array_equal(q, ref.q)


def test_quantizer_clip_and_degenerate_match_oracle():
    w = (np.random.default_rng(1).standard_t(4, 100_000) * 0.02).astype(np.float32)
    c = float(np.float32(1.4 * np.std(w.astype(np.float64))))
    q, s, zp, _ = ent.quantize(w, 4, "unsigned", clip=c)
    ref = quant.quantize_unsigned(w, 4, clip=c)
    assert s == ref.scale and np.array_equal(q, ref.q)
    z = np.full(1000, 0.25, dtype=np.float32)
    for scheme, fn in (("asymmetric", quant.quantize_asymmetric), ("unsigned", quant.quantize_unsigned)):
        q, s, zp, _ = ent.quantize(z, 8, scheme)
        r = fn(z, 8)
        assert s == r.scale and zp == r.zero_point and np.array_equal(q, r.q)


@pytest.mark.parametrize("seed", range(16))
def test_code_lengths_optimal_like_oracle(seed):
    bits = 8 if seed % 2 else 4
    kind = ["skewed", "peaked", "uniform", "sparse", "two", "degenerate"][seed % 6]
    q = fuzz_codes(100 + seed, 50_000, bits, kind)
    max_len = 16 if bits == 8 else 12
    counts = quant.histogram(q, bits)
    mine = ent.code_lengths(q, bits, max_len)
    ref = huffman.code_lengths(counts, max_len)
    assert int(mine.max()) <= max_len
    assert ((mine > 0) == (counts > 0)).all()
    assert huffman.kraft_sum(mine) <= 1.0
    assert int((counts * mine).sum()) == int((counts * ref).sum())


def test_code_lengths_binding_cap_is_optimal():
    counts = np.zeros(16, dtype=np.int64)
    counts[:14] = 2 ** np.arange(14, 0, -1)
    q = np.repeat(np.arange(16, dtype=np.uint8), counts)
    mine = ent.code_lengths(q, 4, 8)
    ref = huffman.package_merge(counts, 8)
    assert mine.max() == 8
    assert int((counts * mine).sum()) == int((counts * ref).sum())


@pytest.mark.parametrize("ahead", [False, True])
@pytest.mark.parametrize("refill_steps", [1, 2])
@pytest.mark.parametrize("lanes,chunk,n", [(1, 64, 1000), (2, 10, 333), (8, 64, 4097), (32, 4096, 70000),
                                           (64, 64, 129), (64, 8192, 100000), (16, 48, 7), (4, 12, 999),
                                           (2, 400, 1000)])
@pytest.mark.parametrize("bits", [4, 8])
def test_encoder_byte_identical_to_oracle(lanes, chunk, n, bits, refill_steps, ahead):
    q = fuzz_codes(lanes + n, n, bits, "skewed")
    lengths = huffman.code_lengths(quant.histogram(q, bits), 16 if bits == 8 else 12)
    words, offs = ent.encode(q, lengths, bits, chunk, lanes, threads=3, refill_steps=refill_steps, ahead=ahead)
    ow, oo = ccodec.encode(q, lengths, chunk, lanes, refill_steps=refill_steps, ahead=ahead)
    assert np.array_equal(offs, oo) and np.array_equal(words, ow)
    assert np.array_equal(ccodec.decode(words, offs, lengths, n, chunk, lanes, refill_steps=refill_steps,
                                        ahead=ahead), q)
    if n <= 1000:
        pw, po = ecw.encode(q, lengths, chunk, lanes, refill_steps, ahead=ahead)
        assert np.array_equal(words, pw)


def test_encoder_rejects_missing_codeword():
    lengths = np.zeros(16, dtype=np.uint8)
    lengths[:2] = 1
    with pytest.raises(ent.EntroError):
        ent.encode(np.array([0, 1, 2], dtype=np.uint8), lengths, 4, 2, 1)
    with pytest.raises(ent.EntroError):
        ent.encode(np.array([0, 1], dtype=np.uint8), lengths, 4, 6, 3)


def test_full_workload_tensor_encodes_like_oracle():
    spec = TensorSpec("tensor_2048", 0, -1, "w", 2048, 2048, "w")
    w = weights(spec)
    q, s, zp, chosen = ent.quantize(w, 8, "asymmetric")
    ref = quant.quantize_asymmetric(w, 8)
    assert np.array_equal(q, ref.q) and s == ref.scale and zp == ref.zero_point
    lengths = huffman.code_lengths(quant.histogram(ref.q, 8), 16)
    words, offs = ent.encode(q, lengths, 8, 4096, 32)
    ow, oo = ccodec.encode(ref.q, lengths, 4096, 32, threads=4)
    assert np.array_equal(words, ow) and np.array_equal(offs, oo)


# --------------------------------------------------------------------------
# rANS variant: host side against the oracle
# --------------------------------------------------------------------------

@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("kind", ["uniform", "skewed", "peaked", "degenerate", "two", "sparse"])
def test_rans_frequencies_and_encoder_match_oracle(bits, kind):
    from oracle import rans
    from synth import fuzz_codes

    q = fuzz_codes(bits * 3 + len(kind), 7000, bits, kind)
    counts = quant.histogram(q, bits)
    f = ent.rans_freqs(counts)
    assert f.tolist() == rans.quantize_freqs(counts).tolist()
    for lanes, chunk in ((32, 256), (64, 640), (1, 64), (8, 1000)):
        units, offs = ent.rans_encode(q, f, bits, chunk, lanes, threads=4)
        ou, oo = rans.encode(q, f, chunk, lanes)
        assert np.array_equal(units, ou) and np.array_equal(offs, oo)


def test_rans_table_layout():
    from oracle import rans
    from oracle.dequant import dequant_bf16

    counts = np.array([0, 5, 1, 90, 0, 3, 1, 0, 0, 0, 0, 0, 0, 0, 0, 900], dtype=np.int64)
    f = ent.rans_freqs(counts)
    t = ent.rans_table_build(f, 4, np.float32(0.0123), 7)
    assert t[0] == 0x31524345 and t[1] == (4 | (12 << 8)) and t[2] == 4096
    cum = rans.cumulative(f)
    vals = dequant_bf16(np.arange(16, dtype=np.uint8), np.float32(0.0123), 7)
    slots = t[4:].reshape(4096, 2)
    for s in range(16):
        for k in range(int(f[s])):
            x, y = int(slots[cum[s] + k, 0]), int(slots[cum[s] + k, 1])
            assert x == (int(vals[s]) << 16) | s
            assert y == int(f[s]) | (k << 16)


def test_rans_host_validation(lib):
    f = np.zeros(16, dtype=np.uint32)
    f[3] = 4096
    q = np.full(10, 3, dtype=np.uint8)
    offs = np.zeros(2, dtype=np.uint64)
    nu = ctypes.c_uint64()
    enc = lambda qq, ff, bits=4, chunk=10, lanes=2: lib.entro_rans_encode(
        qq.ctypes.data, qq.size, ff.ctypes.data, bits, chunk, lanes, offs.ctypes.data, None, 0, ctypes.byref(nu), 1)
    assert enc(q, f) == 0 and nu.value == 4
    assert enc(q, f, lanes=3) == 3
    assert enc(q, f, chunk=9) == 3
    assert enc(q, f, bits=5) == 3
    g = f.copy()
    g[3] = 4095
    assert enc(q, g) == 2                               # frequencies do not sum to 4096
    assert enc(np.full(10, 4, dtype=np.uint8), f) == 2   # a code with frequency 0
    t = np.zeros(4, dtype=np.uint32)
    assert lib.entro_rans_table_build(4, f.ctypes.data, ctypes.c_float(1.0), 0, t.ctypes.data, t.nbytes) == 1
    assert lib.entro_rans_freqs(np.zeros(4, dtype=np.uint64).ctypes.data, 4, f.ctypes.data) == 1
    # device entry points: descriptor checks before launch
    st = ctypes.c_void_p(1)
    outs = (ctypes.c_void_p * 1)(0x1000)

    def dec(**kw):
        x = ent.RansTensor(1, 1, 1, 100, 1000, 256, 32, 4, 100)
        for k, v in kw.items():
            setattr(x, k, v)
        return lib.entro_rans_decode((ent.RansTensor * 1)(x), 1, outs, st, None)

    assert dec(lanes=16) == 3
    assert dec(chunk_symbols=100) == 3
    assert dec(sym_bits=6) == 3
    assert dec(d_units=None) == 1
    assert dec(max_chunk_units=1 << 20) == 4      # larger than the on-chip staging
    assert lib.entro_rans_decode_dequant((ent.RansTensor * 1)(ent.RansTensor(1, 1, 1, 100, 1000, 256, 32, 4, 100)), 1,
                                         (ctypes.c_void_p * 1)(0x1002), st, None) == 1
