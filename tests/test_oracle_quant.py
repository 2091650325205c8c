"""Pins of the per-token fp8 quantiser oracle (CPU only)."""
import numpy as np
import pytest
import torch

import oracle
from oracle.formats import e4m3fn_table

MAG = e4m3fn_table()[:0x7F]


def torch_e4m3(y):
    return torch.from_numpy(np.asarray(y, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_encode_matches_torch_on_every_midpoint():
    # every representable magnitude, every midpoint between neighbours (the
    # ties), and values just either side of each midpoint, both signs
    mids = (MAG[1:] + MAG[:-1]) / 2
    eps = np.abs(mids) * 2.0 ** -20
    vals = np.concatenate([MAG, mids, mids - eps, mids + eps]).astype(np.float32)
    vals = np.concatenate([vals, -vals])
    assert np.array_equal(oracle.e4m3fn_encode(vals), torch_e4m3(vals))


def test_encode_matches_torch_random():
    rng = np.random.default_rng(3)
    vals = np.concatenate([rng.uniform(-448, 448, 50000), rng.standard_normal(50000),
                           rng.uniform(-2.0 ** -6, 2.0 ** -6, 50000)]).astype(np.float32)
    assert np.array_equal(oracle.e4m3fn_encode(vals), torch_e4m3(vals))


def test_encode_extremes():
    enc = oracle.e4m3fn_encode
    assert enc(np.float32(448.0)) == 0x7E and enc(np.float32(-448.0)) == 0xFE
    assert enc(np.float32(1e9)) == 0x7E                     # clamped, never the NaN code
    assert enc(np.float32(2.0 ** -9)) == 0x01               # smallest subnormal
    assert enc(np.float32(2.0 ** -10)) == 0x00              # tie with 0 -> even code 0
    assert enc(np.float32(3 * 2.0 ** -10)) == 0x02          # tie 1.5 steps -> even code 2
    assert enc(np.float32(-0.0)) == 0x80


def test_quantize_rows_properties():
    rng = np.random.default_rng(4)
    x = (rng.standard_normal((40, 256)) * 10.0 ** rng.uniform(-3, 3, (40, 1))).astype(np.float32)
    x[3] = 0.0
    bits = torch.from_numpy(x).to(torch.bfloat16).view(torch.uint16).numpy()
    codes, scale = oracle.quantize_rows_fp8(bits)
    xb = oracle.bf16_to_f64(bits)
    assert codes.dtype == np.uint8 and scale.dtype == np.float32
    assert scale[3] == 1.0 and np.all(codes[3] == 0)
    deq = oracle.e4m3fn_to_f64(codes) * scale[:, None].astype(np.float64)
    for r in range(40):
        if r == 3:
            continue
        j = int(np.argmax(np.abs(xb[r])))
        assert codes[r, j] & 0x7F == 0x7E                   # the row maximum maps to 448
        # each element is within half an e4m3 step of its scaled value
        y = np.abs(xb[r]) / scale[r]
        step = np.where(y < 2.0 ** -6, 2.0 ** -9, 2.0 ** (np.floor(np.log2(np.maximum(y, 2.0 ** -6))) - 3))
        assert np.all(np.abs(deq[r] - xb[r]) <= 0.5 * step * scale[r] * (1 + 1e-6) + 1e-30)


def test_truncating_mutant_is_caught():
    vals = ((MAG[1:] + MAG[:-1]) / 2 + 2.0 ** -12).astype(np.float32)
    trunc = np.searchsorted(MAG, np.abs(vals), side="right") - 1
    assert not np.array_equal(trunc.astype(np.uint8), torch_e4m3(vals))
