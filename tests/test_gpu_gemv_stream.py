"""GPU parity of the streamed fused GEMV kernels: the kernel that multiplies
decoded pairs on the vector ALUs with activations staged whole in LDS
(batch 1, and batches 2..8 while 8 batch slots of x fit, cols <= 4096), and
the matrix-core kernel for 2..8 activation rows whose x is streamed in
512-column slices (one row per chunk, 512 | cols, wider rows).  The library
picks the kernel by itself; the shapes below reach both, often in one call.

Every stream, code length and expected value comes from the oracle; outputs
must lie within 1e-4 (relative, floor-guarded) of the float64 oracle GEMV
over the bf16 weights.  Covered: tile counts that are not multiples of the
workgroup count, rows not multiples of 16, several tensors per call (tiles of
one workgroup in two tensors), codes longer than 6 bits (two-code table
entries that fall back), refilling ahead, wavefronts with more than 64 rows
(with a workgroup cap), results independent of the cap, and a malformed
stream that is flagged while the other tensors of the call stay exact,
and calls of more tensors than one launch holds.
"""
import os
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from oracle import gemv as ogemv  # noqa: E402
from oracle import quant  # noqa: E402
from synth import activations_bf16  # noqa: E402
from tests._cases import make_case, run_gemv  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import entropy_coded_weight_canonical_amd as ent

    ent.load()
    yield
    ent.set_max_workgroups(0)


def say(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def _rows_case(rows, cols, seed, ahead=False, scheme="unsigned"):
    """rows x cols Student-t weights, 4-bit, one row per chunk, 64 lanes,
    refill every two steps."""
    rng = np.random.default_rng(seed)
    w = (rng.standard_t(4, size=(rows, cols)) * 0.02).astype(np.float32)
    qz = quant.quantize_mixed(w, 4) if scheme == "mixed" else quant.quantize_unsigned(w, 4)
    return make_case(qz.q, 4, cols, 64, scale=qz.scale, zp=qz.zero_point, rows=rows, cols=cols,
                     refill_steps=2, ahead=ahead)


def _long_code_case(rows, cols, seed, ahead=False):
    """4-bit codes drawn with probabilities 2^-(s+1): Huffman lengths reach
    the 12-bit cap, so some two-code table entries fall back."""
    rng = np.random.default_rng(seed)
    p = 0.5 ** np.arange(1, 17)
    p /= p.sum()
    q = rng.choice(16, size=rows * cols, p=p).astype(np.uint8)
    return make_case(q, 4, cols, 64, scale=0.01, zp=3, rows=rows, cols=cols, refill_steps=2, ahead=ahead)


def _check(cases, xs, ys, st, tol=1e-4):
    assert (st == 0).all(), st
    for c, x, y in zip(cases, xs, ys):
        ref = ogemv.gemv_f64(c.expected_bf16().reshape(c.rows, c.cols), x)
        err = ogemv.rel_err(y, ref)
        assert err <= tol, (c.rows, c.cols, err)


@pytest.mark.parametrize("pair_lut", [True, False])
@pytest.mark.parametrize("ahead", [False, True])
@pytest.mark.parametrize("batch", [1, 2, 3, 5, 8])
def test_streamed_gemv_shapes_in_one_call(batch, ahead, pair_lut):
    """pair_lut: two-code tables built on the host and loaded, or (False)
    built on chip by every workgroup."""
    shapes = [(1, 1024), (15, 1536), (16, 2048), (17, 4608), (37, 5120), (300, 1024), (64, 3072), (20, 8192),
              (33, 14336), (1, 6144)]
    cases = [_rows_case(r, c, 100 + i, ahead=ahead) for i, (r, c) in enumerate(shapes)]
    xs = [activations_bf16("mistral_stack", 200 + i, c.cols, batch) for i, c in enumerate(cases)]
    say(f"streamed gemv shapes batch={batch} ahead={ahead} pair_lut={pair_lut}")
    ys, st = run_gemv(cases, xs, batch, pair_lut=pair_lut)
    _check(cases, xs, ys, st)


@pytest.mark.parametrize("pair_lut", [True, False])
@pytest.mark.parametrize("batch", [1, 4, 8])
def test_streamed_gemv_codes_longer_than_six_bits(batch, pair_lut):
    cases = [_long_code_case(40, 1024, 7, ahead=True), _long_code_case(23, 2560, 8),
             _long_code_case(19, 5120, 9, ahead=True)]
    assert max(int(c.lengths.max()) for c in cases) > 6
    xs = [activations_bf16("mistral_stack", 300 + i, c.cols, batch) for i, c in enumerate(cases)]
    say(f"streamed gemv long codes batch={batch} pair_lut={pair_lut}")
    ys, st = run_gemv(cases, xs, batch, pair_lut=pair_lut)
    _check(cases, xs, ys, st)


@pytest.mark.parametrize("batch", [1, 8])
def test_streamed_gemv_mismatched_two_code_table_is_flagged(batch):
    """A host-built two-code table of another code is refused (ENTRO_F_LUT,
    tensor not decoded); a misaligned one is ignored (built on chip); the
    other tensors of the call stay exact."""
    cases = [_rows_case(32, 1024, 41), _rows_case(32, 1024, 42), _long_code_case(21, 5120, 43),
             _rows_case(18, 6144, 44)]
    keep = []

    def edit(i, dt):
        import torch

        if i == 1:   # the long-code table of case 2, whose header names another code
            dt.desc.d_pair_lut = None
            p = torch.from_numpy(__import__("entropy_coded_weight_canonical_amd").pair_lut_build(cases[2].lut)
                                 .view(np.int32)).cuda()
            keep.append(p)
            dt.desc.d_pair_lut = p.data_ptr()
        if i == 3:   # an unaligned copy: the kernels build the table themselves
            p = torch.zeros(4 + 8196, dtype=torch.int32, device="cuda")
            p[2:8198] = dt.pair_lut
            keep.append(p)
            dt.desc.d_pair_lut = p.data_ptr() + 8

    xs = [activations_bf16("mistral_stack", 700 + i, c.cols, batch) for i, c in enumerate(cases)]
    say(f"streamed gemv mismatched two-code table batch={batch}")
    ys, st = run_gemv(cases, xs, batch, edit=edit)
    assert st[1] == 0x20, st
    ok = [0, 2, 3]
    _check([cases[i] for i in ok], [xs[i] for i in ok], [ys[i] for i in ok], st[ok])


@pytest.mark.parametrize("cap", [1, 3])
@pytest.mark.parametrize("batch", [1, 8])
def test_streamed_gemv_runs_past_64_rows_per_wavefront(batch, cap):
    """With at most `cap` workgroups each wavefront streams 70 / cap x 16 /
    ... rows: the end offsets are reloaded every 64 rows and y is stored
    every 64 rows."""
    import entropy_coded_weight_canonical_amd as ent

    cases = [_rows_case(16 * 70 * cap + 5, 1024, 11, ahead=True), _rows_case(33, 2048, 12),
             _rows_case(16 * 70 * cap + 3, 4608, 13)]
    xs = [activations_bf16("mistral_stack", 400 + i, c.cols, batch) for i, c in enumerate(cases)]
    say(f"streamed gemv cap={cap} batch={batch} rows={cases[0].rows}")
    prev = ent.set_max_workgroups(cap)
    try:
        ys, st = run_gemv(cases, xs, batch)
    finally:
        ent.set_max_workgroups(prev)
    _check(cases, xs, ys, st)


@pytest.mark.parametrize("batch", [1, 8])
def test_streamed_gemv_calls_of_more_tensors_than_one_launch_holds(batch):
    """20 tensors in one call: the streamed and matrix-core launches hold at
    most 16 each, so the call is split into several launches."""
    shapes = [(17 + 3 * i, (1024, 2048, 4096, 5120)[i % 4]) for i in range(20)]
    cases = [_rows_case(r, c, 900 + i, ahead=i % 2 == 0) for i, (r, c) in enumerate(shapes)]
    xs = [activations_bf16("mistral_stack", 910 + i, c.cols, batch) for i, c in enumerate(cases)]
    say(f"streamed gemv 20 tensors batch={batch}")
    ys, st = run_gemv(cases, xs, batch)
    _check(cases, xs, ys, st)


@pytest.mark.parametrize("batch", [1, 6])
def test_streamed_gemv_results_do_not_depend_on_the_grid(batch):
    import entropy_coded_weight_canonical_amd as ent

    cases = [_rows_case(500, 1024, 21), _rows_case(77, 4096, 22, ahead=True), _rows_case(60, 5120, 23)]
    xs = [activations_bf16("mistral_stack", 500 + i, c.cols, batch) for i, c in enumerate(cases)]
    say(f"streamed gemv grid independence batch={batch}")
    ys0, st0 = run_gemv(cases, xs, batch)
    prev = ent.set_max_workgroups(5)
    try:
        ys1, st1 = run_gemv(cases, xs, batch)
    finally:
        ent.set_max_workgroups(prev)
    _check(cases, xs, ys0, st0)
    assert (st1 == 0).all(), st1
    for a, b in zip(ys0, ys1):
        assert np.array_equal(a, b)


@pytest.mark.parametrize("batch", [1, 8])
def test_streamed_gemv_malformed_stream_is_flagged(batch):
    cases = [_rows_case(48, 1024, 31), _rows_case(48, 1024, 32), _rows_case(20, 2048, 33),
             _rows_case(48, 5120, 34), _rows_case(16, 6144, 35)]
    for i in (1, 3):
        words = cases[i].words.copy()
        words[len(words) // 3:] ^= np.uint32(0x5A5A5A5A)   # the later rows' words no longer decode to their ends
        cases[i].words = words
    xs = [activations_bf16("mistral_stack", 600 + i, c.cols, batch) for i, c in enumerate(cases)]
    say(f"streamed gemv malformed stream batch={batch}")
    ys, st = run_gemv(cases, xs, batch)
    assert st[1] != 0 and st[3] != 0, st
    ok = [0, 2, 4]
    _check([cases[i] for i in ok], [xs[i] for i in ok], [ys[i] for i in ok], st[ok])
