"""GPU parity: the HIP path against the CPU oracle, through the C ABI.

Codes and bf16 values must be bit-exact; fused GEMV outputs within a
floor-guarded relative error of 1e-2 of the float64 oracle (fp32
accumulation gives ~1e-5).  Streams, code lengths and expected values come
from the oracle only; the library contributes its decode table builder and
the kernels under test.
"""
import sys

import numpy as np
import pytest

from oracle import gemv as ogemv
from oracle import quant
from synth import CODE_KINDS, TensorSpec, activations_bf16, fuzz_codes, weights
from tests._cases import make_case, run_decode, run_gemv

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import entropy_coded_weight_canonical_amd as ent

    ent.load()


def say(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


LANE_GRID = [(1, 16), (2, 8), (4, 4), (8, 2), (16, 3), (32, 1), (32, 4), (64, 1), (64, 3)]


@pytest.mark.parametrize("refill_steps", [1, 2])
@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("lanes,mult", LANE_GRID)
def test_fuzz_grid_u8_and_bf16(bits, lanes, mult, refill_steps):
    cases = []
    for i, kind in enumerate(CODE_KINDS):
        chunk = lanes * (mult * 8 + (i % 2))       # even and odd steps per chunk
        n = chunk * (3 + i) + (17 * i + 5) % chunk   # several chunks and a ragged tail
        q = fuzz_codes(1000 * lanes + 10 * mult + i, n, bits, kind)
        cases.append(make_case(q, bits, chunk, lanes, scale=0.0031 * (i + 1), zp=(7 * i) % (1 << bits),
                               refill_steps=refill_steps))
    say(f"fuzz bits={bits} lanes={lanes} mult={mult} refill_steps={refill_steps}")
    outs, st = run_decode(cases, "u8")
    assert (st == 0).all(), st
    for c, o in zip(cases, outs):
        assert np.array_equal(o, c.q)
    outs, st = run_decode(cases, "bf16")
    assert (st == 0).all(), st
    for c, o in zip(cases, outs):
        assert np.array_equal(o, c.expected_bf16())


@pytest.mark.parametrize("refill_steps", [1, 2])
@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("lanes", [1, 2, 8, 32, 64])
def test_refill_ahead_streams(lanes, bits, refill_steps):
    """Streams encoded refilling ahead: long chunks (the early phase covers most
    steps), odd and even step counts, ragged last chunks; the 4-bit
    two-step W = 32 / 64 cases run the LDS loops, the rest the generic path."""
    cases = []
    for i, kind in enumerate(CODE_KINDS):
        steps = [40, 81, 256, 64, 129, 33][i]
        chunk = lanes * steps
        n = chunk * (2 + i % 2) + (29 * i + 7) % chunk
        q = fuzz_codes(7000 + 100 * lanes + 10 * bits + i, n, bits, kind)
        cases.append(make_case(q, bits, chunk, lanes, scale=0.002 * (i + 1), zp=(5 * i) % (1 << bits),
                               refill_steps=refill_steps, ahead=True))
    say(f"refill ahead bits={bits} lanes={lanes} refill_steps={refill_steps}")
    for mode in ("u8", "bf16"):
        outs, st = run_decode(cases, mode)
        assert (st == 0).all(), st
        for c, o in zip(cases, outs):
            assert np.array_equal(o, c.q if mode == "u8" else c.expected_bf16())


@pytest.mark.parametrize("refill_steps", [1, 2])
def test_longest_codes_use_second_level(refill_steps):
    counts = np.zeros(256, dtype=np.int64)
    counts[:40] = (2.0 ** np.arange(40, 0, -1)).astype(np.int64) // 2 + 1
    rng = np.random.default_rng(3)
    q = rng.choice(256, size=200_000, p=counts / counts.sum()).astype(np.uint8)
    # force the rarest symbols in so that 16-bit codes occur in the stream
    q[rng.choice(q.size, 40, replace=False)] = np.arange(40, dtype=np.uint8)
    c = make_case(q, 8, 4096, 32, refill_steps=refill_steps)
    assert c.lengths.max() >= 15
    say(f"two-level table refill_steps={refill_steps}")
    outs, st = run_decode([c], "u8")
    assert st[0] == 0 and np.array_equal(outs[0], c.q)
    outs, st = run_decode([c], "bf16")
    assert st[0] == 0 and np.array_equal(outs[0], c.expected_bf16())


def test_edge_cases_in_one_batch():
    cases = [
        make_case(np.zeros(0, dtype=np.uint8), 4, 64, 64),                 # empty tensor
        make_case(np.full(1000, 9, dtype=np.uint8), 4, 256, 32),           # single symbol
        make_case(fuzz_codes(1, 1, 8, "skewed"), 8, 4096, 64),             # one symbol total
        make_case(fuzz_codes(2, 63, 8, "skewed"), 8, 4096, 64),            # fewer symbols than lanes
        make_case(fuzz_codes(3, 4096 * 3, 4, "uniform"), 4, 4096, 64),     # exact multiple
        make_case(fuzz_codes(4, 100_000, 4, "two"), 4, 64, 64),            # 1-bit codes, short chunks
    ]
    say("edge cases")
    for mode in ("u8", "bf16"):
        outs, st = run_decode(cases, mode)
        assert (st == 0).all(), st
        for c, o in zip(cases, outs):
            exp = c.q if mode == "u8" else c.expected_bf16()
            assert np.array_equal(o, exp)


@pytest.mark.parametrize("lut_offset", [1, 2, 3])
def test_decode_tables_at_any_word_alignment(lut_offset):
    """Decode tables 4, 8 and 12 bytes past 16-byte alignment are fetched
    entry by entry (aligned ones 16 bytes at a time): W = 32 and 64 with the
    two-code table, 8-bit codes, a table whose entry count is not a multiple
    of four, and the same outputs as from aligned tables."""
    cases = [make_case(fuzz_codes(80, 8192 * 5 + 77, 4, "skewed"), 4, 8192, 32, refill_steps=2, ahead=True),
             make_case(fuzz_codes(81, 4096 * 3, 4, "skewed"), 4, 4096, 64, refill_steps=2),
             make_case(fuzz_codes(82, 30_001, 8, "peaked"), 8, 4096, 32),
             make_case(fuzz_codes(83, 5000, 8, "uniform"), 8, 1024, 16)]
    say(f"decode tables at word offset {lut_offset}")
    for mode in ("u8", "bf16"):
        outs, st = run_decode(cases, mode, lut_offset=lut_offset)
        assert (st == 0).all(), st
        for c, o in zip(cases, outs):
            exp = c.q if mode == "u8" else c.expected_bf16()
            assert np.array_equal(o, exp)


def test_more_tensors_than_one_launch_and_mixed_lanes():
    cases = []
    for i in range(45):
        lanes = [64, 32, 64, 8][i % 4]
        bits = 8 if i % 3 else 4
        q = fuzz_codes(50 + i, 5000 + 37 * i, bits, CODE_KINDS[i % len(CODE_KINDS)])
        cases.append(make_case(q, bits, lanes * 32, lanes, scale=0.001 * (i + 1), zp=i % 16,
                               refill_steps=1 + (i % 5 == 2)))
    say("45 tensors")
    outs, st = run_decode(cases, "bf16")
    assert (st == 0).all(), st
    for c, o in zip(cases, outs):
        assert np.array_equal(o, c.expected_bf16())


def test_workgroup_task_ranges_cross_tensor_boundaries():
    """Workgroups take an even share of the launch's tasks, in rounds that
    stay within one tensor, so a share can span several tensors: 32 tensors
    of 40 to 269 tasks (more tasks in all than 16 per CU, so that CUs take
    a second workgroup), lanes 32 (two chunks per task) with a ragged last
    task, then half of the codes with 64 lanes (fewer tasks than that)."""
    cases = []
    for i in range(32):
        n_tasks = 40 + (i * 37) % 230
        n = n_tasks * 2 * 1024 - (i % 3) * 100
        bits = 4 if i % 4 else 8
        q = fuzz_codes(90 + i, n, bits, CODE_KINDS[i % len(CODE_KINDS)])
        cases.append(make_case(q, bits, 1024, 32, refill_steps=2, ahead=bool(i % 2)))
    say("32 tensors, task ranges across tensor boundaries (W 32)")
    outs, st = run_decode(cases, "bf16")
    assert (st == 0).all(), st
    for c, o in zip(cases, outs):
        assert np.array_equal(o, c.expected_bf16())
    cases64 = [make_case(c.q, c.bits, 1024, 64, refill_steps=2) for c in cases[:16]]
    say("16 tensors, task ranges across tensor boundaries (W 64)")
    outs, st = run_decode(cases64, "u8")
    assert (st == 0).all(), st
    for c, o in zip(cases64, outs):
        assert np.array_equal(o, c.q)


def test_cached_output_stores_mixed_with_streamed():
    """out_cached = 1 selects ordinary output stores; tensors of both policies
    in one call are split into separate launches and both decode exactly
    (full tasks and ragged tails, every lane count)."""
    cases, flags = [], []
    for i in range(28):
        lanes = [1, 2, 4, 8, 16, 32, 64][i % 7]
        bits = 4 if i % 2 else 8
        chunk = lanes * (8 + 3 * (i % 3))
        n = chunk * (4 + i % 3) + (11 * i) % chunk
        q = fuzz_codes(700 + i, n, bits, CODE_KINDS[i % len(CODE_KINDS)])
        cases.append(make_case(q, bits, chunk, lanes, scale=0.002 * (i + 1), zp=i % 16,
                               refill_steps=1 + (i % 4 == 1), ahead=(i % 4 == 1)))
        flags.append((i // 7) % 2)
    say("28 tensors, cached and streamed output stores")
    for mode in ("u8", "bf16"):
        outs, st = run_decode(cases, mode, cached=flags)
        assert (st == 0).all(), st
        for c, o in zip(cases, outs):
            assert np.array_equal(o, c.q if mode == "u8" else c.expected_bf16())


def test_faults_are_flagged_not_fatal():
    import entropy_coded_weight_canonical_amd as ent

    base = make_case(fuzz_codes(9, 50_000, 8, "skewed"), 8, 4096, 32)
    cases = []
    # 1. bit flips in the stream
    c = make_case(base.q, 8, 4096, 32)
    rng = np.random.default_rng(0)
    flip = rng.choice(c.words.size, 50, replace=False)
    c.words = c.words.copy()
    c.words[flip] ^= np.uint32(0x00400000)
    cases.append(c)
    # 2. chunk offsets pointing past the stream
    c = make_case(base.q, 8, 4096, 32)
    c.offs = c.offs.copy()
    c.offs[-1] += np.uint64(32 * 1000)
    cases.append(c)
    # 3. offsets not multiples of 32
    c = make_case(base.q, 8, 4096, 32)
    c.offs = c.offs.copy()
    c.offs[3] += np.uint64(5)
    cases.append(c)
    # 4. table built for another code width
    c = make_case(base.q, 8, 4096, 32)
    c.lut = ent.lut_build(np.r_[np.ones(2), np.zeros(14)].astype(np.uint8), 4, 12, 1.0, 0)
    cases.append(c)
    # 5. a word missing from the end (offsets still consistent)
    c = make_case(base.q, 8, 4096, 32)
    c.words = c.words[:-1].copy()
    c.offs = c.offs.copy()
    c.offs[-1] -= np.uint64(32)
    cases.append(c)
    # 6. a clean tensor after the faulty ones
    cases.append(make_case(base.q, 8, 4096, 32))
    say("fault injection")
    outs, st = run_decode(cases, "u8")
    assert st[0] != 0
    assert st[1] & ent.FLAGS["offsets"]
    assert st[2] & ent.FLAGS["offsets"]
    assert st[3] == ent.FLAGS["lut"]
    assert st[4] & (ent.FLAGS["overrun"] | ent.FLAGS["badcode"] | ent.FLAGS["padding"])
    assert st[5] == 0 and np.array_equal(outs[5], base.q)


# --------------------------------------------------------------------------
# full-size workloads, in the launch configuration the benchmark uses
# --------------------------------------------------------------------------

def _spec(workload):
    return {"tensor_2048": TensorSpec("tensor_2048", 0, -1, "w", 2048, 2048, "w"),
            "tensor_4096": TensorSpec("tensor_4096", 0, -1, "w", 4096, 4096, "w")}[workload]


def test_tensor_2048_asymmetric_8bit_full_size():
    qz = quant.quantize_asymmetric(weights(_spec("tensor_2048")), 8)
    cases = [make_case(qz.q, 8, 4096, 32, scale=qz.scale, zp=qz.zero_point),
             make_case(qz.q, 8, 4096, 64, scale=qz.scale, zp=qz.zero_point),
             make_case(qz.q, 8, 4096, 1, scale=qz.scale, zp=qz.zero_point),
             make_case(qz.q, 8, 4096, 32, scale=qz.scale, zp=qz.zero_point, refill_steps=2)]
    say("tensor_2048 W=32/64/1")
    outs, st = run_decode(cases, "u8")
    assert (st == 0).all()
    for c, o in zip(cases, outs):
        assert np.array_equal(o, qz.q.ravel())
    outs, st = run_decode(cases, "bf16")
    assert (st == 0).all()
    for c, o in zip(cases, outs):
        assert np.array_equal(o, c.expected_bf16())


@pytest.mark.parametrize("refill_steps,ahead", [(1, False), (2, False), (2, True)])
def test_tensor_4096_unsigned_4bit_full_size_replicated(refill_steps, ahead):
    qz = quant.quantize_unsigned(weights(_spec("tensor_4096")), 4)
    c = make_case(qz.q, 4, 8192, 32, scale=qz.scale, zp=qz.zero_point, refill_steps=refill_steps, ahead=ahead)
    say(f"tensor_4096 x16 replicas refill_steps={refill_steps} ahead={ahead}")
    outs, st = run_decode([c] * 16, "bf16")
    assert (st == 0).all()
    exp = c.expected_bf16()
    for o in outs:
        assert np.array_equal(o, exp)


# --------------------------------------------------------------------------
# fused GEMV
# --------------------------------------------------------------------------

def _gemv_case(rows, cols, bits, seed, rows_per_chunk=1, lanes=64, scheme="mixed", refill_steps=1, ahead=False):
    rng = np.random.default_rng(seed)
    w = (rng.standard_t(4, size=(rows, cols)) * 0.02).astype(np.float32)
    qz = {"mixed": quant.quantize_mixed, "asymmetric": quant.quantize_asymmetric,
          "unsigned": quant.quantize_unsigned}[scheme](w, bits)
    return make_case(qz.q, bits, cols * rows_per_chunk, lanes, scale=qz.scale, zp=qz.zero_point,
                     rows=rows, cols=cols, refill_steps=refill_steps, ahead=ahead)


@pytest.mark.parametrize("batch", [1, 3, 8])
def test_gemv_small_shapes(batch):
    cases = [_gemv_case(37, 128, 4, 1), _gemv_case(64, 192, 8, 2, rows_per_chunk=3),
             _gemv_case(100, 64, 4, 3, rows_per_chunk=7), _gemv_case(9, 320, 8, 4, lanes=32),
             _gemv_case(33, 48, 4, 5, lanes=16, rows_per_chunk=2), _gemv_case(5, 8, 8, 6, lanes=1),
             _gemv_case(40, 192, 4, 7, refill_steps=2), _gemv_case(21, 96, 8, 8, lanes=32, refill_steps=2)]
    xs = [activations_bf16("phi3_stack", i, c.cols, batch) for i, c in enumerate(cases)]
    say(f"gemv small batch={batch}")
    ys, st = run_gemv(cases, xs, batch)
    assert (st == 0).all(), st
    for c, x, y in zip(cases, xs, ys):
        ref = ogemv.gemv_f64(c.expected_bf16().reshape(c.rows, c.cols), x)
        assert ogemv.rel_err(y, ref) <= 1e-2
        assert ogemv.rel_err(y, ref) <= 1e-4   # fp32 accumulation


@pytest.mark.parametrize("batch", [1, 8])
def test_gemv_refill_ahead(batch):
    cases = [_gemv_case(37, 1024, 4, 31, refill_steps=2, ahead=True),
             _gemv_case(50, 256, 4, 32, rows_per_chunk=3, refill_steps=2, ahead=True),
             _gemv_case(20, 512, 8, 33, refill_steps=2, ahead=True),
             _gemv_case(9, 4096, 4, 34, refill_steps=1, ahead=True, lanes=32)]
    xs = [activations_bf16("phi3_stack", 40 + i, c.cols, batch) for i, c in enumerate(cases)]
    say(f"gemv refill ahead batch={batch}")
    ys, st = run_gemv(cases, xs, batch)
    assert (st == 0).all(), st
    for c, x, y in zip(cases, xs, ys):
        ref = ogemv.gemv_f64(c.expected_bf16().reshape(c.rows, c.cols), x)
        assert ogemv.rel_err(y, ref) <= 1e-4


@pytest.mark.parametrize("ahead", [False, True])
@pytest.mark.parametrize("batch", [2, 8])
def test_gemv_sliced_activations(batch, ahead):
    """Batches of 2..8 whose activations exceed the LDS block (cols * 16 bytes
    > 64 KiB) are walked in column slices by the whole workgroup: one and two
    rows per chunk, a last slice of one pair (4224 = 33 * 128 columns), ragged
    last chunks, and a tensor whose x fits in the same launch."""
    cases = [_gemv_case(70, 5120, 4, 51, refill_steps=2, ahead=ahead),
             _gemv_case(33, 6144, 4, 52, rows_per_chunk=2, refill_steps=2, ahead=ahead, scheme="unsigned"),
             _gemv_case(41, 4224, 4, 53, refill_steps=2, ahead=ahead),
             _gemv_case(50, 1024, 4, 54, rows_per_chunk=3, refill_steps=2, ahead=ahead)]
    xs = [activations_bf16("mistral_stack", 60 + i, c.cols, batch) for i, c in enumerate(cases)]
    say(f"gemv sliced x batch={batch} ahead={ahead}")
    ys, st = run_gemv(cases, xs, batch)
    assert (st == 0).all(), st
    for c, x, y in zip(cases, xs, ys):
        ref = ogemv.gemv_f64(c.expected_bf16().reshape(c.rows, c.cols), x)
        assert ogemv.rel_err(y, ref) <= 1e-4


@pytest.mark.parametrize("batch", [1, 8])
def test_gemv_activations_and_tables_at_any_alignment(batch):
    """x 2 bytes and the decode table 4 bytes past 16-byte alignment take the
    element-wise copies; x at 16 bytes past it takes the 16-byte loads.  The
    LDS path with all of x staged, the column-sliced path (batch 8, 5120
    columns), an 8-bit tensor on the generic path, all within 1e-4 of the
    float64 oracle at every placement."""
    cases = [_gemv_case(37, 1024, 4, 71, refill_steps=2, ahead=True),
             _gemv_case(70, 5120, 4, 72, refill_steps=2, ahead=True),
             _gemv_case(33, 4096, 4, 73, rows_per_chunk=2, refill_steps=2),
             _gemv_case(20, 512, 8, 74, refill_steps=2, ahead=True)]
    xs = [activations_bf16("mistral_stack", 70 + i, c.cols, batch) for i, c in enumerate(cases)]
    refs = [ogemv.gemv_f64(c.expected_bf16().reshape(c.rows, c.cols), x) for c, x in zip(cases, xs)]
    for x_offset, lut_offset in [(1, 1), (1, 0), (0, 3), (8, 4), (0, 0)]:
        say(f"gemv batch={batch} x offset {x_offset} table offset {lut_offset}")
        ys, st = run_gemv(cases, xs, batch, x_offset=x_offset, lut_offset=lut_offset)
        assert (st == 0).all(), st
        for y, ref in zip(ys, refs):
            assert ogemv.rel_err(y, ref) <= 1e-4


@pytest.mark.parametrize("batch", [1, 8])
def test_gemv_task_ranges_cross_tensor_boundaries(batch):
    """Many GEMV tensors in one launch whose row counts do not line up with
    the workgroups' even shares of the tasks: the LDS path (1024 columns)
    and, at batch 8, the column-sliced path (5120 columns), where every
    wavefront of a workgroup takes part in each round, with or without a
    row of its own."""
    cases = []
    for i in range(20):
        cols = 5120 if i % 5 == 0 else 1024
        rows = 90 + (i * 53) % 170
        cases.append(_gemv_case(rows, cols, 4, 200 + i, refill_steps=2, ahead=bool(i % 2)))
    xs = [activations_bf16("mistral_stack", 90 + i, c.cols, batch) for i, c in enumerate(cases)]
    say(f"gemv 20 tensors, task ranges across tensor boundaries, batch={batch}")
    ys, st = run_gemv(cases, xs, batch)
    assert (st == 0).all(), st
    for c, x, y in zip(cases, xs, ys):
        ref = ogemv.gemv_f64(c.expected_bf16().reshape(c.rows, c.cols), x)
        assert ogemv.rel_err(y, ref) <= 1e-4


@pytest.mark.parametrize("batch", [1, 3, 8])
def test_gemv_lds_path_shapes(batch):
    """Tensors the LDS GEMV path takes (W = 64, 4-bit, refill every two steps,
    128 | cols): one or several rows per chunk, a ragged last chunk (generic
    path for that task), and a tensor with 128 not dividing cols in the same
    launch (generic path throughout)."""
    cases = [_gemv_case(37, 128, 4, 11, refill_steps=2),
             _gemv_case(50, 256, 4, 12, rows_per_chunk=3, refill_steps=2),
             _gemv_case(64, 1024, 4, 13, rows_per_chunk=2, refill_steps=2),
             _gemv_case(9, 4096, 4, 14, refill_steps=2, scheme="unsigned"),
             _gemv_case(33, 192, 4, 15, refill_steps=2),
             _gemv_case(129, 384, 4, 16, rows_per_chunk=4, refill_steps=2, scheme="asymmetric")]
    xs = [activations_bf16("mistral_stack", 20 + i, c.cols, batch) for i, c in enumerate(cases)]
    say(f"gemv lds path batch={batch}")
    ys, st = run_gemv(cases, xs, batch)
    assert (st == 0).all(), st
    for c, x, y in zip(cases, xs, ys):
        ref = ogemv.gemv_f64(c.expected_bf16().reshape(c.rows, c.cols), x)
        assert ogemv.rel_err(y, ref) <= 1e-4


@pytest.mark.parametrize("refill_steps", [1, 2])
@pytest.mark.parametrize("batch", [1, 8])
def test_gemv_mistral_shapes_sampled_layer(batch, refill_steps):
    """One layer of the 4-bit Mistral-shaped stack at full size (row-aligned
    chunks, 64 lanes), every output checked against the float64 oracle; with
    refill every two steps the LDS path takes every full chunk (at batch 8 the
    14336-column down projection, whose activations exceed the LDS block, is
    walked in column slices)."""
    specs = [s for s in __import__("synth").tensor_specs("mistral_stack") if s.layer == 0]
    cases, xs = [], []
    for gi, s in enumerate(specs):
        qz = quant.quantize_mixed(weights(s), 4)
        chunk = s.cols * max(1, round(8192 / s.cols))
        cases.append(make_case(qz.q, 4, chunk, 64, scale=qz.scale, zp=qz.zero_point, rows=s.rows, cols=s.cols,
                               refill_steps=refill_steps))
        xs.append(activations_bf16("mistral_stack", gi, s.cols, batch))
    say(f"gemv mistral layer0 batch={batch} refill_steps={refill_steps}")
    ys, st = run_gemv(cases, xs, batch)
    assert (st == 0).all(), st
    for c, x, y in zip(cases, xs, ys):
        ref = ogemv.gemv_f64(c.expected_bf16().reshape(c.rows, c.cols), x)
        assert ogemv.rel_err(y, ref) <= 1e-2


def test_library_loaded_before_torch_shares_torchs_runtime():
    """Loading the library before importing torch must not leave the process
    with a second HIP runtime (torch ships its own): a child process loads
    the library first, then decodes a small tensor from torch memory."""
    import subprocess

    code = r"""
import numpy as np
import entropy_coded_weight_canonical_amd as ent
ent.load()
import torch
from oracle import ccodec, huffman, quant
from synth import fuzz_codes
q = fuzz_codes(9, 5000, 4, "skewed")
L = huffman.code_lengths(quant.histogram(q, 4), 12)
lut = ent.lut_build(L, 4, 12, np.float32(0.01), 8)
w, o = ccodec.encode(q, L, 1024, 32)
t = ent.DeviceTensor.upload(lut, w, o, q.size, 1024, 32, 4, 12)
out = torch.empty(q.size, dtype=torch.uint8, device="cuda")
st = torch.zeros(1, dtype=torch.int32, device="cuda")
ent.decode([t.desc], [out.data_ptr()], st.data_ptr())
torch.cuda.synchronize()
assert int(st.item()) == 0 and np.array_equal(out.cpu().numpy(), q)
print("child ok")
"""
    root = __import__("os").path.dirname(__import__("os").path.dirname(__import__("os").path.abspath(__file__)))
    say("library loaded before torch, in a child process")
    p = subprocess.run([sys.executable, "-c", code], cwd=root, capture_output=True, text=True, timeout=300)
    assert p.returncode == 0 and "child ok" in p.stdout, p.stderr[-2000:]
