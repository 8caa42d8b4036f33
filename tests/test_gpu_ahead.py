"""GPU parity of decode-ahead streaming (coded matrices consumed by the stock
linear kernel): outputs against the float64 oracle, the staged bf16 weights
bit-exact against the oracle's dequantization, equality with the stock kernel
on the oracle's weights, HIP-graph replays, and decode flags of a malformed
stream.  Streams and expected values come from the oracle only."""
import sys
from types import SimpleNamespace

import numpy as np
import pytest

from oracle import gemv as ogemv
from oracle import quant
from synth import activations_bf16
from tests._cases import make_case, upload


def say(msg):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def _case(rows, cols, bits, seed, chunk=None, lanes=64, refill_steps=2, ahead=True):
    rng = np.random.default_rng(seed)
    w = (rng.standard_t(4, size=(rows, cols)) * 0.02).astype(np.float32)
    qz = quant.quantize_mixed(w, bits)
    return make_case(qz.q, bits, chunk or cols, lanes, scale=qz.scale, zp=qz.zero_point, rows=rows, cols=cols,
                     refill_steps=refill_steps, ahead=ahead)


def _stack():
    return [_case(256, 512, 4, 1), _case(128, 512, 8, 2, chunk=1024), _case(512, 256, 4, 3, lanes=32),
            _case(64, 1024, 4, 4, chunk=2048), _case(96, 320, 8, 5, lanes=32, refill_steps=1, ahead=False)]


def _bf16_tensor(bits_u16, shape):
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits_u16).view(np.int16).reshape(shape)).cuda().view(torch.bfloat16)


def _to_f64(t):
    import torch

    return t.float().cpu().numpy().astype(np.float64)


@pytest.fixture(scope="module")
def torch_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import entropy_coded_weight_canonical_amd as ent

    ent.load()
    return torch


@pytest.mark.gpu
@pytest.mark.parametrize("depth,block_elems", [(2, None), (3, None), (2, 8192), (3, 20000)])
@pytest.mark.parametrize("batch", [1, 8])
def test_decode_ahead_matches_oracle(torch_gpu, depth, block_elems, batch):
    import torch.nn.functional as F

    from entropy_coded_weight_canonical_amd.ahead import DecodeAhead

    cases = _stack()
    say(f"decode-ahead stack of {len(cases)} depth={depth} blocks={block_elems} batch={batch}")
    dts = [upload(c) for c in cases]
    xs_u16 = [activations_bf16("mistral_stack", i, c.cols, batch) for i, c in enumerate(cases)]
    xs = [_bf16_tensor(x, (batch, c.cols)) for x, c in zip(xs_u16, cases)]
    da = DecodeAhead(dts, [(c.rows, c.cols) for c in cases], depth=depth, block_elems=block_elems)
    if block_elems:
        assert len(da.blocks) > 2 * len(cases)
    ys = da.run(xs)
    torch_gpu.cuda.synchronize()
    assert (da.status.cpu().numpy() == 0).all()
    for c, x, xt, y in zip(cases, xs_u16, xs, ys):
        w_bits = c.expected_bf16().reshape(c.rows, c.cols)
        ref = ogemv.gemv_f64(w_bits, x)
        assert y.shape == (batch, c.rows)
        assert ogemv.rel_err(_to_f64(y), ref) <= 1e-2
        # the same stock kernel on the oracle's bf16 weights
        y_stock = F.linear(xt, _bf16_tensor(w_bits, (c.rows, c.cols)))
        assert ogemv.rel_err(_to_f64(y), _to_f64(y_stock)) <= 1e-3


@pytest.mark.gpu
def test_staged_weights_are_the_oracle_dequant(torch_gpu):
    from entropy_coded_weight_canonical_amd.ahead import DecodeAhead

    cases = _stack()[:3]
    say("decode-ahead staging buffers bit-exact")
    dts = [upload(c) for c in cases]
    xs = [_bf16_tensor(activations_bf16("phi3_stack", i, c.cols, 1), (1, c.cols)) for i, c in enumerate(cases)]
    da = DecodeAhead(dts, [(c.rows, c.cols) for c in cases], depth=3)
    da.run(xs)
    torch_gpu.cuda.synchronize()
    for m, c in enumerate(cases):
        staged = da.bufs[m % da.depth][: c.n].view(torch_gpu.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(staged, c.expected_bf16())


@pytest.mark.gpu
def test_chunk_range_views_decode_their_slice(torch_gpu):
    """A descriptor over chunks [c0, c1) of a stream decodes exactly those
    chunks' symbols (offsets are positions in the full stream)."""
    import entropy_coded_weight_canonical_amd as ent
    from entropy_coded_weight_canonical_amd.ahead import chunk_range_view

    torch = torch_gpu
    for c in (_case(96, 256, 4, 11, chunk=512), _case(40, 384, 8, 12, chunk=768, lanes=32),
              _case(33, 64, 4, 13, chunk=128, lanes=16, refill_steps=1, ahead=False)):
        dt = upload(c)
        nc = -(-c.n // c.chunk)
        exp = c.expected_bf16()
        for c0, c1 in ((0, 1), (1, nc), (nc - 1, nc), (nc // 3, 2 * nc // 3 + 1)):
            say(f"chunk range [{c0}, {c1}) of {nc}, W={c.lanes}, {c.bits}-bit")
            v = chunk_range_view(dt.desc, c0, c1)
            out = torch.empty(int(v.n_symbols), dtype=torch.int16, device="cuda")
            st = torch.zeros(1, dtype=torch.int32, device="cuda")
            ent.decode_dequant([v], [out.data_ptr()], st.data_ptr())
            torch.cuda.synchronize()
            assert int(st.item()) == 0
            got = out.cpu().numpy().view(np.uint16)
            assert np.array_equal(got, exp[c0 * c.chunk: min(c1 * c.chunk, c.n)])


@pytest.mark.gpu
def test_decode_ahead_graph_replays(torch_gpu):
    torch = torch_gpu
    from entropy_coded_weight_canonical_amd.ahead import DecodeAhead

    cases = _stack()
    say("decode-ahead captured in a HIP graph, 3 replays")
    dts = [upload(c) for c in cases]
    xs = [_bf16_tensor(activations_bf16("mistral_stack", 20 + i, c.cols, 4), (4, c.cols)) for i, c in enumerate(cases)]
    da = DecodeAhead(dts, [(c.rows, c.cols) for c in cases], depth=2, block_elems=16384)
    eager = [y.clone() for y in da.run(xs)]
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):   # warm-up on a side stream before capture
        da.run(xs)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ys = da.run(xs)
    for r in range(3):
        for y in ys:
            y.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert (da.status.cpu().numpy() == 0).all()
        for y, e in zip(ys, eager):
            assert ogemv.rel_err(_to_f64(y), _to_f64(e)) <= 1e-3
        # eager work between replays: an unrelated run of the same object
        da.run(xs)
        torch.cuda.synchronize()


@pytest.mark.gpu
def test_decode_ahead_flags_a_malformed_matrix(torch_gpu):
    from entropy_coded_weight_canonical_amd.ahead import DecodeAhead

    cases = _stack()[:3]
    bad = cases[1]
    bad = make_case(bad.q.reshape(bad.rows, bad.cols), bad.bits, bad.chunk, bad.lanes, scale=bad.scale, zp=bad.zp,
                    rows=bad.rows, cols=bad.cols, refill_steps=bad.refill_steps, ahead=bad.ahead)
    bad.words = np.full_like(bad.words, 0xFFFFFFFF)
    say("decode-ahead with one malformed stream")
    dts = [upload(c) for c in (cases[0], bad, cases[2])]
    xs = [_bf16_tensor(activations_bf16("phi3_stack", i, c.cols, 1), (1, c.cols))
          for i, c in enumerate((cases[0], bad, cases[2]))]
    da = DecodeAhead(dts, [(c.rows, c.cols) for c in (cases[0], bad, cases[2])], depth=2)
    da.run(xs)
    torch_gpu.cuda.synchronize()
    st = da.status.cpu().numpy()
    assert st[0] == 0 and st[2] == 0 and st[1] != 0


def test_chunk_range_view_fields():
    import entropy_coded_weight_canonical_amd as ent
    from entropy_coded_weight_canonical_amd.ahead import chunk_range_view

    d = ent.Tensor(0x1000, 0x2000, 0x3000, 777, 10 * 64 + 5, 64, 32, 4, 12, 4112, 40, 2, 1)
    v = chunk_range_view(d, 2, 5)
    assert v.d_chunk_bit_off == 0x3000 + 16 and v.n_symbols == 3 * 64
    assert (v.d_words, v.n_words, v.d_lut, v.lanes, v.refill_ahead) == (0x2000, 777, 0x1000, 32, 1)
    last = chunk_range_view(d, 9, 11)
    assert last.n_symbols == 64 + 5 and last.d_chunk_bit_off == 0x3000 + 72
    with pytest.raises(ValueError):
        chunk_range_view(d, 3, 3)
    with pytest.raises(ValueError):
        chunk_range_view(d, 11, 12)


def test_decode_ahead_rejects_mismatched_shapes():
    from entropy_coded_weight_canonical_amd.ahead import DecodeAhead

    t = SimpleNamespace(desc=SimpleNamespace(n_symbols=12))
    with pytest.raises(ValueError):
        DecodeAhead([t], [(3, 5)])
    with pytest.raises(ValueError):
        DecodeAhead([t], [(3, 4)], depth=1)
    with pytest.raises(ValueError):
        DecodeAhead([], [])
