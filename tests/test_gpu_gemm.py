"""GPU parity of the fused decode + GEMM (prompt processing on the matrix
cores) against the float64 oracle: token counts around the 16-token groups
and up to the 512 maximum (more than 256 tokens run as several launches),
calls that reach the 16-, 32- and 64-row tiles (the tile height follows the
call's row count against the GPU's CU count), row counts around the tiles,
several matrices per call, streams with and without refilling ahead, long
rows, a malformed stream, and a full-size Mistral-shaped matrix.  Streams
and expected values come from the oracle only."""
import sys

import numpy as np
import pytest

from oracle import gemv as ogemv
from oracle import quant
from synth import TensorSpec, activations_bf16, weights
from tests._cases import make_case, upload

pytestmark = pytest.mark.gpu


def say(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import entropy_coded_weight_canonical_amd as ent

    ent.load()


def _cus():
    import torch

    return torch.cuda.get_device_properties(0).multi_processor_count


def _check(cases, xs, ys, st):
    assert (st == 0).all(), st
    for c, x, y in zip(cases, xs, ys):
        ref = ogemv.gemv_f64(c.expected_bf16().reshape(c.rows, c.cols), x)
        assert not np.isnan(y).any()
        err = ogemv.rel_err(y, ref)
        assert err <= 1e-2
        assert err <= (1e-3 if c.cols > 4096 else 1e-4), (c.rows, c.cols, err)   # fp32 sums; see the long-row test


def _case(rows, cols, seed, scheme="mixed", ahead=True, w=None):
    if w is None:
        rng = np.random.default_rng(seed)
        w = (rng.standard_t(4, size=(rows, cols)) * 0.02).astype(np.float32)
    qz = {"mixed": quant.quantize_mixed, "asymmetric": quant.quantize_asymmetric,
          "unsigned": quant.quantize_unsigned}[scheme](w, 4)
    return make_case(qz.q, 4, cols, 64, scale=qz.scale, zp=qz.zero_point, rows=rows, cols=cols,
                     refill_steps=2, ahead=ahead)


def run_gemm(cases, n_tokens, xs):
    import torch

    import entropy_coded_weight_canonical_amd as ent

    dts = [upload(c) for c in cases]
    dx = [torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda() for x in xs]
    dy = [torch.full((n_tokens, c.rows), float("nan"), dtype=torch.float32, device="cuda") for c in cases]
    items = [ent.GemvItem(c.rows, c.cols, x.data_ptr(), y.data_ptr()) for c, x, y in zip(cases, dx, dy)]
    status = torch.zeros(len(cases), dtype=torch.int32, device="cuda")
    ent.decode_gemm([d.desc for d in dts], items, n_tokens, status.data_ptr())
    torch.cuda.synchronize()
    return [y.cpu().numpy() for y in dy], status.cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("n_tokens", [1, 5, 16, 17, 64, 100, 128, 129, 200, 256, 257, 512])
def test_gemm_matches_oracle(n_tokens):
    cases = [_case(16, 128, 1), _case(37, 256, 2, scheme="asymmetric"), _case(64, 512, 3, ahead=False),
             _case(100, 1024, 4, scheme="unsigned"), _case(5, 384, 5)]
    say(f"decode+GEMM {len(cases)} matrices, {n_tokens} tokens")
    xs = [activations_bf16("mistral_stack", 100 + i, c.cols, n_tokens) for i, c in enumerate(cases)]
    ys, st = run_gemm(cases, n_tokens, xs)
    assert (st == 0).all()
    for c, x, y in zip(cases, xs, ys):
        ref = ogemv.gemv_f64(c.expected_bf16().reshape(c.rows, c.cols), x)
        assert not np.isnan(y).any()
        assert ogemv.rel_err(y, ref) <= 1e-2
        assert ogemv.rel_err(y, ref) <= 1e-4   # fp32 accumulation of exact bf16 products


def test_gemm_flags_a_malformed_stream():
    good, bad = _case(32, 256, 6), _case(48, 256, 7)
    bad.words = np.full_like(bad.words, 0xFFFFFFFF)
    say("decode+GEMM with one malformed stream")
    xs = [activations_bf16("phi3_stack", 200 + i, 256, 16) for i in range(2)]
    ys, st = run_gemm([good, bad], 16, xs)
    assert st[0] == 0 and st[1] != 0
    ref = ogemv.gemv_f64(good.expected_bf16().reshape(good.rows, good.cols), xs[0])
    assert ogemv.rel_err(ys[0], ref) <= 1e-4


@pytest.mark.parametrize("n_tokens", [64, 256, 512])
def test_gemm_mistral_o_full_size(n_tokens):
    """q/o-shaped 4096 x 4096 matrix of the Mistral-shaped stack (layer 0 weights)."""
    spec = TensorSpec("mistral_stack", 3, 0, "L0.o", 4096, 4096, "o")
    c = _case(4096, 4096, 0, w=weights(spec).reshape(4096, 4096))
    say(f"decode+GEMM 4096x4096, {n_tokens} tokens")
    x = activations_bf16("mistral_stack", 300, 4096, n_tokens)
    ys, st = run_gemm([c], n_tokens, [x])
    assert st[0] == 0
    # every row against float64, on a sample of tokens
    toks = np.unique(np.linspace(0, n_tokens - 1, 9).astype(int))
    ref = ogemv.gemv_f64(c.expected_bf16().reshape(4096, 4096), x[toks])
    assert ogemv.rel_err(ys[0][toks], ref) <= 1e-4


@pytest.mark.parametrize("n_tokens", [1, 16, 64, 128, 200])
def test_gemm_long_rows(n_tokens):
    """14336-column rows of uniform 4-bit codes (~1790 words a row, more than
    the down projection at 3.9 bits/weight), streamed through the rings."""
    rng = np.random.default_rng(11)
    q = rng.integers(0, 16, size=(24, 14336), dtype=np.uint8)
    c = make_case(q, 4, 14336, 64, scale=0.01, zp=8, rows=24, cols=14336, refill_steps=2, ahead=True)
    assert c.words.size / 24 > 1700
    say(f"decode+GEMM 24x14336 uniform codes, {n_tokens} tokens")
    x = activations_bf16("mistral_stack", 400, 14336, n_tokens)
    ys, st = run_gemm([c], n_tokens, [x])
    assert st[0] == 0
    ref = ogemv.gemv_f64(c.expected_bf16().reshape(24, 14336), x)
    err = ogemv.rel_err(ys[0], ref)
    assert err <= 1e-2   # the stated bar
    # fp32 accumulation over 448 matrix-core steps of 32 columns: outputs
    # near zero (relative to the 1e-3 floor) show a few e-4
    assert err <= 1e-3, err


@pytest.mark.parametrize("cap", [0, 7])
@pytest.mark.parametrize("n_tokens", [17, 64, 129, 256, 300])
def test_gemm_64_row_tiles(n_tokens, cap):
    """Calls with at least one 64-row tile per CU take the 64-row tiles: rows
    not a multiple of 64, several matrices, streams with and without
    refilling ahead, 14336-column rows; with a workgroup cap of 7 every
    workgroup decodes many tiles one after another."""
    import entropy_coded_weight_canonical_amd as ent

    rng = np.random.default_rng(12)
    q = rng.integers(0, 16, size=(64, 14336), dtype=np.uint8)
    cases = [_case(64 * _cus() - 200, 128, 21), _case(130, 256, 22, scheme="unsigned", ahead=False),
             _case(37, 512, 23), make_case(q, 4, 14336, 64, scale=0.01, zp=8, rows=64, cols=14336, refill_steps=2,
                                           ahead=True)]
    assert sum((c.rows + 63) // 64 for c in cases) >= _cus()
    xs = [activations_bf16("phi3_stack", 500 + i, c.cols, n_tokens) for i, c in enumerate(cases)]
    say(f"decode+GEMM 64-row tiles, {n_tokens} tokens, cap {cap}")
    prev = ent.set_max_workgroups(cap)
    try:
        ys, st = run_gemm(cases, n_tokens, xs)
    finally:
        ent.set_max_workgroups(prev)
    _check(cases, xs, ys, st)


@pytest.mark.parametrize("cap", [0, 5])
@pytest.mark.parametrize("n_tokens", [1, 17, 100, 256, 400])
def test_gemm_32_row_tiles(n_tokens, cap):
    """Calls with 32-row tiles for three quarters of the CUs but fewer 64-row
    tiles than CUs (a Mistral-shaped q/k/v group) take the 32-row tiles."""
    import entropy_coded_weight_canonical_amd as ent

    rng = np.random.default_rng(13)
    q = rng.integers(0, 16, size=(40, 14336), dtype=np.uint8)
    cases = [_case(24 * _cus() + 7, 128, 31), _case(37, 512, 32, ahead=False),
             make_case(q, 4, 14336, 64, scale=0.01, zp=8, rows=40, cols=14336, refill_steps=2, ahead=True)]
    t64, t32 = sum((c.rows + 63) // 64 for c in cases), sum((c.rows + 31) // 32 for c in cases)
    assert t64 < _cus() and 4 * t32 >= 3 * _cus()
    xs = [activations_bf16("phi3_stack", 600 + i, c.cols, n_tokens) for i, c in enumerate(cases)]
    say(f"decode+GEMM 32-row tiles, {n_tokens} tokens, cap {cap}")
    prev = ent.set_max_workgroups(cap)
    try:
        ys, st = run_gemm(cases, n_tokens, xs)
    finally:
        ent.set_max_workgroups(prev)
    _check(cases, xs, ys, st)


@pytest.mark.parametrize("cap", [0, 3])
@pytest.mark.parametrize("n_tokens", [2, 33, 256])
def test_gemm_16_row_tiles_many_per_workgroup(n_tokens, cap):
    """Calls with few rows take the 16-row tiles; with a workgroup cap of 3
    each workgroup decodes tiles of several matrices one after another."""
    import entropy_coded_weight_canonical_amd as ent

    cases = [_case(16 * 20 + 3, 384, 41), _case(16, 128, 42, ahead=False), _case(100, 1024, 43, scheme="unsigned")]
    assert 4 * sum((c.rows + 31) // 32 for c in cases) < 3 * _cus()
    xs = [activations_bf16("mistral_stack", 700 + i, c.cols, n_tokens) for i, c in enumerate(cases)]
    say(f"decode+GEMM 16-row tiles, {n_tokens} tokens, cap {cap}")
    prev = ent.set_max_workgroups(cap)
    try:
        ys, st = run_gemm(cases, n_tokens, xs)
    finally:
        ent.set_max_workgroups(prev)
    _check(cases, xs, ys, st)
