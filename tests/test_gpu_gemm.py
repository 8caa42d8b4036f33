"""GPU parity of the fused decode + GEMM (prompt processing on the matrix
cores) against the float64 oracle: token counts around the 16-token groups
and up to the 512 maximum, row counts around the 16-row tiles, several
matrices per call, streams with and without refilling ahead, a malformed
stream, and a full-size Mistral-shaped matrix.  Streams and expected values
come from the oracle only."""
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


@pytest.mark.parametrize("n_tokens", [1, 5, 16, 17, 64, 100, 256, 257, 512])
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


@pytest.mark.parametrize("n_tokens", [64, 512])
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
