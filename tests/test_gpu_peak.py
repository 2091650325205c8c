"""The rate probes the benchmark measures peaks with compute what they claim:
the copy and the read touch every byte, the gather reads every listed row,
the MFMA loop runs to completion with the same result in every workgroup."""
import ctypes
import os

import numpy as np
import pytest
import torch

from _gpu_helpers import say

pytestmark = pytest.mark.gpu
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def plib():
    lib = ctypes.CDLL(os.path.join(ROOT, "dsa_indexer_top_amd", "libdsa_peak.so"))
    lib.dsa_peak_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                  ctypes.POINTER(ctypes.c_double), ctypes.c_void_p]
    lib.dsa_peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    lib.dsa_peak_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.dsa_peak_gather.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                    ctypes.c_void_p, ctypes.c_void_p]
    return lib


def test_copy_and_read(plib):
    say("peak probes: copy, read")
    s = torch.cuda.current_stream().cuda_stream
    n = (1 << 20) * 16 + 48          # a ragged tail after the 4-word rounds
    src = torch.randint(-2**31, 2**31 - 1, (n // 4,), dtype=torch.int32, device="cuda")
    dst = torch.zeros_like(src)
    assert plib.dsa_peak_copy(src.data_ptr(), dst.data_ptr(), n, 64, s) == 0
    blocks = 64
    red = torch.zeros(blocks, dtype=torch.int32, device="cuda")
    assert plib.dsa_peak_read(src.data_ptr(), n, blocks, red.data_ptr(), s) == 0
    torch.cuda.synchronize()
    assert torch.equal(dst, src)
    want = int(np.bitwise_xor.reduce(src.cpu().numpy().view(np.uint32)))
    got = int(np.bitwise_xor.reduce(red.cpu().numpy().view(np.uint32)))
    assert got == want


@pytest.mark.parametrize("dtype", [0, 1])
def test_mfma_loop(plib, dtype):
    say(f"peak probes: mfma dtype {dtype}")
    s = torch.cuda.current_stream().cuda_stream
    blocks, iters = 8, 64
    out = torch.full((blocks * 256,), float("nan"), device="cuda")
    flop = ctypes.c_double()
    assert plib.dsa_peak_mfma(dtype, blocks, iters, out.data_ptr(), ctypes.byref(flop), s) == 0
    torch.cuda.synchronize()
    per = 2 * 32 * 32 * (64 if dtype else 16)
    assert flop.value == per * 4 * iters * 4 * blocks
    o = out.view(blocks, 256)
    assert torch.isfinite(o).all() and (o != 0).any()
    assert torch.equal(o, o[0:1].expand_as(o))


def test_gather(plib):
    say("peak probes: gather")
    s = torch.cuda.current_stream().cuda_stream
    rows, n, blocks = 1000, 100003, 32     # n: a ragged tail after the 8-row rounds
    g = torch.Generator().manual_seed(7)
    table = torch.randint(-2**31, 2**31 - 1, (rows, 64), dtype=torch.int32, generator=g)
    idx = torch.randint(0, rows, (n,), dtype=torch.int32, generator=g)
    idx[5], idx[n - 1] = -1, rows + 7       # out of range: read the last row
    red = torch.zeros(blocks, dtype=torch.int32, device="cuda")
    td, idd = table.cuda(), idx.cuda()
    assert plib.dsa_peak_gather(td.data_ptr(), rows, idd.data_ptr(), n, blocks, red.data_ptr(), s) == 0
    assert plib.dsa_peak_gather(td.data_ptr(), 0, idd.data_ptr(), n, blocks, red.data_ptr(), s) == 1
    torch.cuda.synchronize()
    folded = np.bitwise_xor.reduce(table.numpy().view(np.uint32), axis=1)
    i = idx.numpy()
    want = int(np.bitwise_xor.reduce(folded[np.where((i < 0) | (i >= rows), rows - 1, i)]))
    got = int(np.bitwise_xor.reduce(red.cpu().numpy().view(np.uint32)))
    assert got == want
