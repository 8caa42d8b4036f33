"""Pins for oracle.dequant and oracle.gemv: hand-derived fixtures, torch's bf16
cast, exact float64 products, and exactly rounded sums (math.fsum)."""
import math

import numpy as np
import pytest
import torch

from oracle import dequant, gemv
from tests._golden import load


def test_golden_bf16_rne():
    _, rows = load("bf16_rne.txt")
    f = np.array([int(r[0], 16) for r in rows], dtype=np.uint32).view(np.float32)
    expect = [int(r[1], 16) for r in rows]
    assert dequant.f32_to_bf16_rne(f).tolist() == expect


def test_golden_dequant():
    _, rows = load("dequant_tiny.txt")
    for sb, zp, q, out in rows:
        scale = np.array([int(sb, 16)], dtype=np.uint32).view(np.float32)[0]
        got = dequant.dequant_bf16(np.array([int(q)], dtype=np.uint8), scale, int(zp))
        assert int(got[0]) == int(out, 16)


@pytest.mark.parametrize("bits", [4, 8])
def test_all_codes_match_torch_bf16_cast(bits):
    rng = np.random.default_rng(bits)
    q = np.arange(1 << bits, dtype=np.uint8)
    for _ in range(200):
        scale = np.float32(rng.uniform(1e-5, 1e-1) * (10.0 ** rng.integers(-3, 3)))
        zp = int(rng.integers(0, 1 << bits))
        p = dequant.dequant_f32(q, scale, zp)
        # exact product in float64 (24 + 9 bits fit), one rounding to float32
        exact = (np.float64(scale) * (q.astype(np.float64) - zp)).astype(np.float32)
        assert np.array_equal(p.view(np.uint32), exact.view(np.uint32))
        tb = torch.from_numpy(p).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
        assert np.array_equal(dequant.dequant_bf16(q, scale, zp), tb)


def test_bf16_to_f64_round_trip():
    rng = np.random.default_rng(0)
    b = rng.integers(0, 1 << 16, size=4096).astype(np.uint16)
    b = b[(b & 0x7F80) != 0x7F80]  # finite only
    f = dequant.bf16_to_f64(b)
    assert np.array_equal(dequant.f32_to_bf16_rne(f.astype(np.float32)), b)


def _bf16(x):
    return dequant.f32_to_bf16_rne(np.asarray(x, dtype=np.float32))


def test_gemv_against_exact_sums():
    rng = np.random.default_rng(1)
    rows, cols, batch = 37, 300, 3
    w = _bf16(rng.normal(0, 0.02, (rows, cols)))
    x = _bf16(rng.normal(0, 1, (batch, cols)))
    y = gemv.gemv_f64(w, x)
    wf = dequant.bf16_to_f64(w)
    xf = dequant.bf16_to_f64(x)
    for b in range(batch):
        for o in range(rows):
            exact = math.fsum(float(wf[o, i]) * float(xf[b, i]) for i in range(cols))
            assert abs(y[b, o] - exact) <= 1e-12 * max(1.0, abs(exact))
    # one-hot inputs pick out columns exactly
    onehot = np.zeros((1, cols), dtype=np.uint16)
    onehot[0, 17] = 0x3F80
    assert np.array_equal(gemv.gemv_f64(w, onehot)[0], wf[:, 17])


def test_rel_err_metric():
    y = np.array([[1.0, -2.0, 4.0]])
    assert gemv.rel_err(y * (1 + 1e-3), y) == pytest.approx(1e-3)
    # entries far below the row's largest magnitude are measured against 1e-3 of it
    r = np.array([[1000.0, 0.0]])
    assert gemv.rel_err(np.array([[1000.0, 0.5]]), r) == pytest.approx(0.5)
    assert gemv.rel_err(r, r) == 0.0
