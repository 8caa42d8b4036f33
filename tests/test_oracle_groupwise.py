"""Pins for oracle.groupwise and the entropy study: hand-derived fixture,
per-group round-off bound, reduction to the per-tensor quantizer, the range
stretch that flattens group-wise codes, closed-form side information, and the
pages' claim that tensor-level codes are the more compressible ones."""
import numpy as np
import pytest

from oracle import groupwise, quant
from synth import TensorSpec, weights
from tests._golden import load


def test_golden_tiny():
    g, _ = load("groupwise_tiny.txt")
    w = np.array([[float(x) for x in g["w"][0]]], dtype=np.float32)
    bits, group = int(g["bits"][0][0]), int(g["group"][0][0])
    a = groupwise.quantize_groupwise(w, bits, group, "asymmetric")
    assert a.q[0].tolist() == [int(x) for x in g["asym_q"][0]]
    assert a.zero_points[0].tolist() == [int(x) for x in g["asym_zp"][0]]
    assert a.scales[0].tolist() == [np.float32(2 / 15), np.float32(1 / 15)]
    u = groupwise.quantize_groupwise(w, bits, group, "unsigned")
    assert u.q[0].tolist() == [int(x) for x in g["unsigned_q"][0]]
    assert u.zero_points[0].tolist() == [int(x) for x in g["unsigned_zp"][0]]
    assert u.scales[0].tolist() == [np.float32(1 / 7), np.float32(0.75 / 7)]


def _w(seed, rows=64, cols=512, scale=0.02):
    rng = np.random.default_rng(seed)
    return (rng.standard_t(4, (rows, cols)) * scale).astype(np.float32)


@pytest.mark.parametrize("bits", [4, 8])
@pytest.mark.parametrize("scheme", ["asymmetric", "unsigned"])
@pytest.mark.parametrize("group", [32, 128])
def test_round_off_within_half_a_group_step(bits, scheme, group):
    w = _w(bits * 7 + group)
    gq = groupwise.quantize_groupwise(w, bits, group, scheme)
    Q = (1 << bits) - 1
    err = np.abs(w.astype(np.float64) - groupwise.dequant_groupwise_f64(gq))
    s = np.repeat(gq.scales.astype(np.float64), group, axis=1)
    clamped = (gq.q == 0) | (gq.q == Q)
    assert (err[~clamped] <= 0.5 * s[~clamped] * (1 + 1e-6)).all()
    assert (err <= s * (1 + 1e-6)).all()


@pytest.mark.parametrize("bits", [4, 8])
def test_one_group_per_row_reduces_to_the_tensor_quantizer(bits):
    w = _w(3, rows=1, cols=4096)
    for scheme, f in (("asymmetric", quant.quantize_asymmetric), ("unsigned", quant.quantize_unsigned)):
        gq = groupwise.quantize_groupwise(w, bits, 4096, scheme)
        tq = f(w[0], bits)
        assert gq.q[0].tolist() == tq.q.tolist()
        assert gq.scales[0, 0] == tq.scale and gq.zero_points[0, 0] == tq.zero_point


def test_groups_are_quantized_independently():
    w = _w(4, rows=8, cols=256)
    gq = groupwise.quantize_groupwise(w, 8, 32, "asymmetric")
    for r in (0, 5):
        for k in (0, 3, 7):
            one = quant.quantize_asymmetric(w[r, 32 * k:32 * (k + 1)], 8)
            assert gq.q[r, 32 * k:32 * (k + 1)].tolist() == one.q.tolist()


def test_asymmetric_groups_span_the_code_range():
    """Each group straddling zero is stretched over the whole code range: its
    minimum lands on code 0 and its maximum on Q or Q - 1."""
    w = _w(5)
    for bits in (4, 8):
        Q = (1 << bits) - 1
        gq = groupwise.quantize_groupwise(w, bits, 32, "asymmetric")
        q = gq.q.reshape(w.shape[0], -1, 32)
        g = w.reshape(w.shape[0], -1, 32)
        straddle = (g.min(axis=2) < 0) & (g.max(axis=2) > 0)
        assert straddle.all()
        assert (q.min(axis=2) == 0).all()
        assert (q.max(axis=2) >= Q - 1).all()


def test_side_information_closed_forms():
    w = _w(6, rows=16, cols=256)
    n = w.size
    assert groupwise.tensor_level_stats(w, 4, "unsigned").side_bits == pytest.approx(64 / n)
    assert groupwise.groupwise_stats(w, 4, 32, "asymmetric").side_bits == pytest.approx((16 + 4) / 32)
    assert groupwise.groupwise_stats(w, 8, 128, "asymmetric").side_bits == pytest.approx((16 + 8) / 128)
    assert groupwise.groupwise_stats(w, 8, 128, "unsigned").side_bits == pytest.approx(16 / 128)


def test_entropy_bounds_of_the_capped_code():
    w = _w(7, rows=32, cols=1024)
    for st in (groupwise.tensor_level_stats(w, 8, "mixed"), groupwise.groupwise_stats(w, 8, 32, "asymmetric")):
        # a prefix code is never shorter than the entropy, and the optimal one
        # is within a bit of it (the cap of 16 does not bind at this size)
        assert st.entropy <= st.mean_len < st.entropy + 1


@pytest.mark.parametrize("bits", [4, 8])
def test_tensor_level_codes_are_more_compressible(bits):
    """Tensor-level codes have lower entropy and a shorter Huffman code than
    group-wise codes of the same bit width (gist.science technical summary,
    Methodology item 1), before side information is even counted."""
    w = weights(TensorSpec("tensor_2048", 0, -1, "w", 2048, 2048, "w"))[:256].reshape(256, 2048)
    t = groupwise.tensor_level_stats(w, bits, "mixed")
    for group in (32, 128):
        for scheme in ("asymmetric", "unsigned"):
            g = groupwise.groupwise_stats(w, bits, group, scheme)
            assert t.entropy < g.entropy and t.mean_len < g.mean_len
