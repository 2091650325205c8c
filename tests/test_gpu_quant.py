"""GPU parity of the per-token fp8 quantiser (dsa_quantize_fp8_rows) against
the oracle: codes and scales bit for bit."""
import numpy as np
import pytest
import torch

import oracle
from dsa_inputs import host_bits
from _gpu_helpers import say

pytestmark = pytest.mark.gpu


def check(dsa, x, rows_to_check=None):
    codes, scale = dsa.quantize_fp8_rows(x)
    torch.cuda.synchronize()
    cols = x.shape[-1]
    x2, c2, s2 = x.reshape(-1, cols), codes.view(torch.uint8).reshape(-1, cols), scale.reshape(-1)
    rows = torch.arange(x2.shape[0]) if rows_to_check is None else torch.as_tensor(rows_to_check)
    rows = rows.to(x.device)
    ref_c, ref_s = oracle.quantize_rows_fp8(host_bits(x2[rows]))   # only the checked rows leave the GPU
    got_c = c2[rows].cpu().numpy()
    got_s = s2[rows].cpu().numpy()
    assert np.array_equal(got_s.view(np.uint32), ref_s.view(np.uint32)), "scales differ"
    bad = np.argwhere(got_c != ref_c)
    assert bad.size == 0, f"{len(bad)} codes differ, first at {bad[:3].tolist()}"
    assert not np.any((got_c & 0x7F) == 0x7F), "NaN code"


def test_quant_random_rows(dsa):
    say("quant random")
    g = torch.Generator(device="cuda").manual_seed(1_000_000 * 11 + 1)
    x = torch.randn(300, 1024, generator=g, device="cuda")
    x *= torch.logspace(-8, 8, 300, device="cuda")[:, None]        # rows over 16 decades
    x[7] = 0.0                                                      # zero row -> scale 1
    x[9] = -0.0
    x[11, ::3] = 0.0
    check(dsa, x.to(torch.bfloat16))


def test_quant_small_cols_and_ties(dsa):
    say("quant ties")
    # rows whose scaled values land on e4m3 midpoints: x = 448 and half-steps
    mags = oracle.formats.e4m3fn_table()[:0x7F]
    mids = (mags[1:] + mags[:-1]) / 2
    vals = np.concatenate([[448.0], mids[-63:]]).astype(np.float32)   # 64 values, max 448 -> scale 1
    x = torch.from_numpy(np.stack([vals, -vals, vals / 64, vals * 2.0 ** 20])).to(torch.bfloat16).cuda()
    check(dsa, x)


def test_quant_q_idx_shape_200k(dsa):
    """The 200K layer's q_idx as the quantiser sees it: [L, H_I * d_I] = [200000, 8192]."""
    say("quant 200K q_idx")
    g = torch.Generator(device="cuda").manual_seed(1_000_000 * 12 + 1)
    x = torch.randn(200000, 64 * 128, generator=g, device="cuda", dtype=torch.bfloat16)
    rows = [0, 1, 4095, 100000, 199999] + np.random.default_rng(0).choice(200000, 27, replace=False).tolist()
    check(dsa, x, rows)
    del x
    torch.cuda.empty_cache()


def test_quant_k_idx_rows(dsa):
    say("quant k_idx")
    g = torch.Generator(device="cuda").manual_seed(1_000_000 * 12 + 2)
    x = torch.randn(5003, 128, generator=g, device="cuda", dtype=torch.bfloat16)
    check(dsa, x)


def test_quant_empty(dsa):
    x = torch.empty(0, 128, device="cuda", dtype=torch.bfloat16)
    codes, scale = dsa.quantize_fp8_rows(x)
    assert codes.shape == (0, 128) and scale.shape == (0,)


def test_quant_long_rows(dsa):
    """Rows longer than the register path (two passes over memory)."""
    say("quant long rows")
    g = torch.Generator(device="cuda").manual_seed(1_000_000 * 12 + 3)
    x = torch.randn(37, 16400, generator=g, device="cuda") * torch.logspace(-3, 3, 37, device="cuda")[:, None]
    check(dsa, x.to(torch.bfloat16))


def test_quant_every_bf16_value(dsa):
    """Every finite bf16 pattern in rows whose maxima sweep 60 binades (2^-30 ..
    2^29, mantissas varied), and rows with the smallest scales (where the
    kernel divides exactly): codes and scales bit for bit."""
    say("quant every bf16 value")
    pats = np.arange(65536, dtype=np.uint32)
    x_all = (pats << 16).view(np.float32)
    x_all = x_all[np.isfinite(x_all)]
    rng = np.random.default_rng(1_000_000 * 11 + 7)
    amaxes = [np.float32(2.0 ** e * (1 + rng.integers(0, 128) / 128)) for e in range(-30, 30)]
    amaxes += [np.float32(2.0 ** -120), np.float32(1.5 * 2.0 ** -126), np.float32(2.0 ** -130)]
    rows = []
    for a in amaxes:
        a = np.float32(torch.tensor(float(a)).to(torch.bfloat16).float().item())  # a bf16 value
        v = x_all[np.abs(x_all) <= a]
        row = np.zeros(65536, dtype=np.float32)
        row[:v.size] = v
        row[-1] = a          # the row's maximum is a
        rows.append(row)
    x = torch.from_numpy(np.stack(rows)).to(torch.bfloat16).cuda()
    check(dsa, x)
