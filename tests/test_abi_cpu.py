"""C-ABI checks that need no GPU: the library loads, exports every symbol that
include/dsa.h declares, resolves patterns like the oracle, and rejects invalid
arguments on the host before any HIP call (outputs untouched)."""
import ctypes
import os
import random
import re
import subprocess

import pytest

import oracle
from oracle import PatternError
import dsa_indexer_top_amd as dsa
from dsa_indexer_top_amd import _lib as L
from dsa_indexer_top_amd.api import attn_args, indexer_args

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def lib():
    return dsa.load()


def _declared_functions(header="dsa.h"):
    src = open(os.path.join(ROOT, "include", header)).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dsa_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol(lib):
    declared = _declared_functions()
    assert set(declared) == set(L.EXPORTS)
    for name in declared:
        assert hasattr(lib, name), name
    assert lib.dsa_abi_version() == 1


def test_peak_probe_library_exports():
    """The rate-probe library the benchmark measures peaks with loads and
    exports what include/dsa_peak.h declares; invalid arguments are refused
    before any launch."""
    path = os.path.join(ROOT, "dsa_indexer_top_amd", "libdsa_peak.so")
    plib = ctypes.CDLL(path)
    declared = _declared_functions("dsa_peak.h")
    assert declared == ["dsa_peak_copy", "dsa_peak_gather", "dsa_peak_mfma", "dsa_peak_read"]
    for name in declared:
        assert hasattr(plib, name), name
    plib.dsa_peak_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                   ctypes.POINTER(ctypes.c_double), ctypes.c_void_p]
    plib.dsa_peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    plib.dsa_peak_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    assert plib.dsa_peak_mfma(2, 1, 1, 16, None, None) == 1          # unknown dtype
    assert plib.dsa_peak_mfma(0, 0, 1, 16, None, None) == 1          # no blocks
    assert plib.dsa_peak_copy(16, 32, 17, 1, None) == 1              # not a multiple of 16
    assert plib.dsa_peak_copy(None, 32, 16, 1, None) == 1
    assert plib.dsa_peak_read(16, 16, 1, None, None) == 1            # no output


def _c_layout(tmp_path, struct, fields):
    """sizeof/offsetof of a dsa.h struct as the C compiler lays it out."""
    src = tmp_path / "layout.c"
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "dsa.h"', "int main(void){",
             f'printf("%zu\\n", sizeof({struct}));']
    lines += [f'printf("%zu\\n", offsetof({struct}, {f}));' for f in fields]
    lines.append("return 0;}")
    src.write_text("\n".join(lines))
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-std=c99", "-I", os.path.join(ROOT, "include"), str(src), "-o", str(exe)],
                   check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split()
    return [int(x) for x in out]


@pytest.mark.parametrize("cls,struct", [(L.IndexerArgs, "dsa_indexer_args"),
                                        (L.AttnArgs, "dsa_attn_args"),
                                        (L.StackArgs, "dsa_stack_args"),
                                        (L.PagedKVArgs, "dsa_paged_kv")])
def test_ctypes_layout_matches_header(tmp_path, cls, struct):
    fields = [f for f, _ in cls._fields_]
    got = [ctypes.sizeof(cls)] + [getattr(cls, f).offset for f in fields]
    assert got == _c_layout(tmp_path, struct, fields)


def test_status_strings(lib):
    assert lib.dsa_status_string(0) == b"DSA_OK"
    assert lib.dsa_status_string(3) == b"DSA_ERR_BAD_PATTERN"


def test_pattern_resolution_matches_oracle():
    rng = random.Random(4)
    cases = [(47, None, 0), (47, None, 2), (47, None, 4), (47, None, 1), (5, None, 7),
             (78, "FFSFSSSFSSFFFSSSFFFSFSSSSSSFFSFFSFFSSFFFFFFSFFFFFSFFSSSSSSFSFFFSFSSSFSFFSFFSSS", 0)]
    for _ in range(30):
        n = rng.randint(1, 60)
        cases.append((n, "F" + "".join(rng.choice("FS") for _ in range(n - 1)), 0))
    for n, pat, freq in cases:
        assert dsa.resolve_pattern(n, pat, freq) == oracle.resolve_pattern(n, pat, freq)


@pytest.mark.parametrize("n,pat,freq,status", [
    (4, "FSF", 0, L.DSA_ERR_BAD_PATTERN),
    (4, "FSFSF", 0, L.DSA_ERR_BAD_PATTERN),
    (4, "FSXF", 0, L.DSA_ERR_BAD_PATTERN),
    (4, "fsfs", 0, L.DSA_ERR_BAD_PATTERN),
    (4, "SFFF", 0, L.DSA_ERR_BAD_PATTERN),
    (4, "FSFS", 2, L.DSA_ERR_INVALID_ARGUMENT),
    (4, None, -1, L.DSA_ERR_INVALID_ARGUMENT),
    (0, None, 0, L.DSA_ERR_INVALID_ARGUMENT),
])
def test_pattern_errors(n, pat, freq, status):
    with pytest.raises(dsa.DsaError) as ei:
        dsa.resolve_pattern(n, pat, freq)
    assert ei.value.status == status
    with pytest.raises(PatternError):
        oracle.resolve_pattern(n, pat, freq)


FAKE = 0x10000  # aligned non-NULL address; never dereferenced (validation fails first)


def _idx_args(**kw):
    d = dict(B=1, n_q=64, n_k=64, pos_offset=0, H=64, D=128, topk=16, code=L.DSA_BF16)
    d.update(kw)
    a = indexer_args(d["B"], d["n_q"], d["n_k"], d["pos_offset"], d["H"], d["D"], d["topk"], d["code"])
    a.q = a.k = a.w = a.out_idx = FAKE
    return a


def _call_idx(lib, a):
    return lib.dsa_indexer_scores_topk(ctypes.byref(a), None)


@pytest.mark.parametrize("mut,status", [
    (lambda a: setattr(a, "struct_size", 8), L.DSA_ERR_INVALID_ARGUMENT),
    (lambda a: setattr(a, "q", None), L.DSA_ERR_INVALID_ARGUMENT),
    (lambda a: setattr(a, "out_idx", None), L.DSA_ERR_INVALID_ARGUMENT),
    (lambda a: setattr(a, "k", FAKE + 8), L.DSA_ERR_INVALID_ARGUMENT),        # misaligned
    (lambda a: setattr(a, "n_q", 0), L.DSA_ERR_INVALID_ARGUMENT),
    (lambda a: setattr(a, "q_pos_offset", 1), L.DSA_ERR_INVALID_ARGUMENT),    # offset + n_q > n_k
    (lambda a: setattr(a, "q_pos_offset", -1), L.DSA_ERR_INVALID_ARGUMENT),
    (lambda a: setattr(a, "head_dim", 96), L.DSA_ERR_UNSUPPORTED),
    (lambda a: setattr(a, "n_heads", 65), L.DSA_ERR_UNSUPPORTED),
    (lambda a: setattr(a, "topk", 0), L.DSA_ERR_UNSUPPORTED),
    (lambda a: setattr(a, "topk", 2049), L.DSA_ERR_UNSUPPORTED),
    (lambda a: setattr(a, "dtype", 7), L.DSA_ERR_UNSUPPORTED),
    (lambda a: setattr(a, "q_scale", FAKE), L.DSA_ERR_INVALID_ARGUMENT),      # scales with bf16
    (lambda a: (setattr(a, "dtype", L.DSA_FP8_E4M3FN), setattr(a, "head_dim", 32)), L.DSA_ERR_UNSUPPORTED),
    (lambda a: setattr(a, "dtype", L.DSA_FP8_E4M3FN), L.DSA_ERR_INVALID_ARGUMENT),  # fp8 without scales
    (lambda a: None, L.DSA_ERR_WORKSPACE),                                       # no workspace
    (lambda a: (setattr(a, "workspace", FAKE), setattr(a, "workspace_bytes", 100)), L.DSA_ERR_WORKSPACE),
    (lambda a: (setattr(a, "B", 70000)), L.DSA_ERR_INVALID_ARGUMENT),
])
def test_indexer_validation(lib, mut, status):
    a = _idx_args()
    mut(a)
    assert _call_idx(lib, a) == status
    assert lib.dsa_last_error() != b""


def test_size_overflow_rejected(lib):
    a = _idx_args(B=65535, n_q=2 ** 31 - 1, n_k=2 ** 31 - 1, H=64, D=128)
    n = ctypes.c_size_t(0)
    assert lib.dsa_indexer_workspace_size(ctypes.byref(a), ctypes.byref(n)) == L.DSA_ERR_INVALID_ARGUMENT


def test_workspace_size_is_reported():
    n = dsa.indexer_workspace_size(1, 1024, 1024, 64, 128, 2048)
    assert n >= 2 * 1024 * 4096 * 4
    assert dsa.indexer_workspace_size(2, 1, 5000, 64, 128, 2048) > 2 * 5000 * 4
    # attention splits each row over about 2048 / rows waves (at most 64, at
    # least one 32-entry chunk each); partials: one per split below 8 splits,
    # none at 8 (one 8-wave workgroup), one per 4-wave workgroup from 16 on
    part = 4 * (128 + 4) * 16
    assert dsa.attn_workspace_size(1, 16384, 16384, 16, 128, 2048) == 0     # one wave per row
    assert dsa.attn_workspace_size(1, 2048, 16384, 16, 128, 2048) == 0      # 2048 rows: one split
    assert dsa.attn_workspace_size(1, 1024, 1024, 16, 128, 2048) == 1024 * 2 * part  # 2 splits
    assert dsa.attn_workspace_size(1, 512, 1024, 16, 128, 2048) == 512 * 4 * part    # 4 splits
    assert dsa.attn_workspace_size(256, 1, 5000, 16, 128, 2048) == 0        # 8 splits: one workgroup
    assert dsa.attn_workspace_size(128, 1, 5000, 16, 128, 2048) == 128 * 4 * part  # 16 splits: 4 workgroups
    assert dsa.attn_workspace_size(64, 1, 5000, 16, 128, 2048) == 64 * 8 * part    # 32 splits: 8 workgroups
    assert dsa.attn_workspace_size(2, 1, 5000, 16, 128, 2048) == 2 * 16 * part     # 64 splits: 16 workgroups
    assert dsa.attn_workspace_size(1, 1, 5000, 16, 128, 64) == 2 * part     # two chunks: 2 splits
    assert dsa.attn_workspace_size(4, 1, 5000, 16, 128, 16) == 0            # one chunk


@pytest.mark.parametrize("mut,status", [
    (lambda a: setattr(a, "n_heads", 17), L.DSA_ERR_UNSUPPORTED),
    (lambda a: setattr(a, "head_dim", 32), L.DSA_ERR_UNSUPPORTED),
    (lambda a: setattr(a, "topk", 4097), L.DSA_ERR_UNSUPPORTED),
    (lambda a: setattr(a, "scale", -1.0), L.DSA_ERR_INVALID_ARGUMENT),
    (lambda a: setattr(a, "scale", float("nan")), L.DSA_ERR_INVALID_ARGUMENT),
    (lambda a: setattr(a, "idx", None), L.DSA_ERR_INVALID_ARGUMENT),
    (lambda a: setattr(a, "v", FAKE + 4), L.DSA_ERR_INVALID_ARGUMENT),
])
def test_attn_validation(lib, mut, status):
    a = attn_args(1, 64, 64, 0, 16, 128, 64, 0.0)
    a.q = a.k = a.v = a.idx = a.out = FAKE
    mut(a)
    assert lib.dsa_sparse_attn(ctypes.byref(a), None) == status


def test_stack_validation(lib):
    a = L.StackArgs()
    a.struct_size = ctypes.sizeof(L.StackArgs)
    a.n_layers = 4
    a.indexer = indexer_args(1, 64, 64, 0, 4, 32, 16, L.DSA_BF16)
    a.attn = attn_args(1, 64, 64, 0, 4, 64, 16, 0.0)
    # bad pattern is reported before anything else is looked at
    assert lib.dsa_layer_stack_run(ctypes.byref(a), b"SFFF", 0, None) == L.DSA_ERR_BAD_PATTERN
    assert lib.dsa_layer_stack_run(ctypes.byref(a), b"FSFS", 2, None) == L.DSA_ERR_INVALID_ARGUMENT
    # missing per-layer arrays
    assert lib.dsa_layer_stack_run(ctypes.byref(a), b"FSFS", 0, None) == L.DSA_ERR_INVALID_ARGUMENT
    # shapes that disagree between indexer and attention
    a.attn = attn_args(1, 64, 64, 0, 4, 64, 32, 0.0)
    assert lib.dsa_layer_stack_run(ctypes.byref(a), None, 0, None) == L.DSA_ERR_INVALID_ARGUMENT
    # the workspace does not depend on the pattern: its size call takes none
    a.attn = attn_args(1, 64, 64, 0, 4, 64, 16, 0.0)
    n = ctypes.c_size_t(0)
    assert lib.dsa_stack_workspace_size(ctypes.byref(a), ctypes.byref(n)) == 0
    assert n.value == max(dsa.indexer_workspace_size(1, 64, 64, 4, 32, 16),
                          dsa.attn_workspace_size(1, 64, 64, 4, 64, 16))


def test_quantize_validation(lib):
    FAKE = 1 << 20  # aligned, never dereferenced: validation fails first
    q = lib.dsa_quantize_fp8_rows
    assert q(FAKE, -1, 128, FAKE, FAKE, None) == L.DSA_ERR_INVALID_ARGUMENT
    assert q(FAKE, 4, 100, FAKE, FAKE, None) == L.DSA_ERR_UNSUPPORTED          # not a multiple of 8
    assert q(FAKE, 4, 0, FAKE, FAKE, None) == L.DSA_ERR_UNSUPPORTED
    assert q(FAKE, 4, (1 << 24) + 8, FAKE, FAKE, None) == L.DSA_ERR_UNSUPPORTED
    assert q(None, 4, 128, FAKE, FAKE, None) == L.DSA_ERR_INVALID_ARGUMENT
    assert q(FAKE + 8, 4, 128, FAKE, FAKE, None) == L.DSA_ERR_INVALID_ARGUMENT  # x not 16-byte aligned
    assert q(FAKE, 4, 128, FAKE + 4, FAKE, None) == L.DSA_ERR_INVALID_ARGUMENT  # out not 8-byte aligned
    assert q(FAKE, 0, 128, None, None, None) == L.DSA_OK                        # nothing to do, no launch


def _kv(**kw):
    kv = L.PagedKVArgs()
    kv.struct_size = ctypes.sizeof(L.PagedKVArgs)
    kv.max_seq_len, kv.page_size, kv.max_pages, kv.num_pages = 256, 64, 4, 16
    kv.seq_lens = kv.block_table = FAKE
    for k, v in kw.items():
        setattr(kv, k, v)
    return kv


@pytest.mark.parametrize("kvmut,amut,status", [
    (dict(struct_size=4), None, L.DSA_ERR_INVALID_ARGUMENT),
    (dict(page_size=48), None, L.DSA_ERR_UNSUPPORTED),                 # not a multiple of 32
    (dict(page_size=0), None, L.DSA_ERR_UNSUPPORTED),
    (dict(max_pages=3), None, L.DSA_ERR_INVALID_ARGUMENT),             # 3 * 64 < max_seq_len
    (dict(num_pages=0), None, L.DSA_ERR_INVALID_ARGUMENT),
    (dict(num_pages=2 ** 30), None, L.DSA_ERR_INVALID_ARGUMENT),       # pool rows overflow int32
    (dict(max_seq_len=300), None, L.DSA_ERR_INVALID_ARGUMENT),         # n_k != max_seq_len
    (dict(seq_lens=None), None, L.DSA_ERR_INVALID_ARGUMENT),
    (dict(block_table=FAKE + 2), None, L.DSA_ERR_INVALID_ARGUMENT),    # misaligned
    (dict(), lambda a: (setattr(a, "n_q", 2), setattr(a, "q_pos_offset", 254)), L.DSA_ERR_UNSUPPORTED),
    (dict(), None, L.DSA_ERR_WORKSPACE),                                # valid layout, no workspace
])
def test_paged_validation(lib, kvmut, amut, status):
    kv = _kv(**kvmut)
    a = _idx_args(B=2, n_q=1, n_k=256, pos_offset=255, topk=64)
    if amut:
        amut(a)
    assert lib.dsa_paged_indexer_topk(ctypes.byref(a), ctypes.byref(kv), None) == status
    assert lib.dsa_last_error() != b""
    at = attn_args(2, 1, 256, 255, 16, 128, 64, 0.0)
    at.q = at.k = at.v = at.idx = at.out = FAKE
    if amut:
        amut(at)
    assert lib.dsa_paged_sparse_attn(ctypes.byref(at), ctypes.byref(kv), None) == (
        L.DSA_ERR_WORKSPACE if status == L.DSA_ERR_WORKSPACE else status)
    assert lib.dsa_paged_indexer_topk(ctypes.byref(a), None, None) == L.DSA_ERR_INVALID_ARGUMENT


def test_paged_append_validation(lib):
    ap = lib.dsa_paged_append_rows
    kv = _kv()
    assert ap(FAKE, 0, 256, FAKE, ctypes.byref(kv), None) == L.DSA_ERR_INVALID_ARGUMENT
    assert ap(FAKE, 2, 6, FAKE, ctypes.byref(kv), None) == L.DSA_ERR_UNSUPPORTED     # not a multiple of 4
    assert ap(None, 2, 256, FAKE, ctypes.byref(kv), None) == L.DSA_ERR_INVALID_ARGUMENT
    assert ap(FAKE, 2, 256, FAKE + 2, ctypes.byref(kv), None) == L.DSA_ERR_INVALID_ARGUMENT
    assert ap(FAKE, 2, 256, FAKE, None, None) == L.DSA_ERR_INVALID_ARGUMENT
    bad = _kv(page_size=16)
    assert ap(FAKE, 2, 256, FAKE, ctypes.byref(bad), None) == L.DSA_ERR_UNSUPPORTED


def test_paged_stack_validation(lib):
    a = L.StackArgs()
    a.struct_size = ctypes.sizeof(L.StackArgs)
    a.n_layers = 2
    a.indexer = indexer_args(2, 1, 256, 255, 4, 32, 16, L.DSA_BF16)
    a.attn = attn_args(2, 1, 256, 255, 4, 64, 16, 0.0)
    kv = _kv()
    assert lib.dsa_paged_layer_stack_run(ctypes.byref(a), ctypes.byref(kv), b"SF", 0, None) == L.DSA_ERR_BAD_PATTERN
    assert lib.dsa_paged_layer_stack_run(ctypes.byref(a), None, b"FS", 0, None) == L.DSA_ERR_INVALID_ARGUMENT
    # layout fine, per-layer arrays missing
    assert lib.dsa_paged_layer_stack_run(ctypes.byref(a), ctypes.byref(kv), b"FS", 0, None) == \
        L.DSA_ERR_INVALID_ARGUMENT


def _stack_args(B=1, n_q=64, n_k=64, off=0, layers=4):
    a = L.StackArgs()
    a.struct_size = ctypes.sizeof(L.StackArgs)
    a.n_layers = layers
    a.indexer = indexer_args(B, n_q, n_k, off, 4, 32, 16, L.DSA_BF16)
    a.attn = attn_args(B, n_q, n_k, off, 4, 64, 16, 0.0)
    return a


def test_chunked_stack_validation(lib):
    run = lib.dsa_layer_stack_run_chunked
    a = _stack_args(B=2)
    assert run(ctypes.byref(a), 16, None, 0, None) == L.DSA_ERR_UNSUPPORTED          # one sequence only
    a = _stack_args()
    assert run(ctypes.byref(a), 0, None, 0, None) == L.DSA_ERR_INVALID_ARGUMENT      # chunk_rows < 1
    assert run(ctypes.byref(a), 16, b"SFFF", 0, None) == L.DSA_ERR_BAD_PATTERN
    assert run(ctypes.byref(a), 16, b"FSFS", 0, None) == L.DSA_ERR_INVALID_ARGUMENT  # no per-layer arrays
    a.layer_events = FAKE
    assert run(ctypes.byref(a), 16, None, 0, None) == L.DSA_ERR_INVALID_ARGUMENT     # events do not span chunks
    a.layer_events = None
    n = ctypes.c_size_t(0)
    assert lib.dsa_chunked_stack_workspace_size(ctypes.byref(a), 0, ctypes.byref(n)) == L.DSA_ERR_INVALID_ARGUMENT


def test_chunked_stack_workspace_is_one_chunk(lib):
    """The chunked workspace covers the largest chunk shape (a full chunk or
    the ragged last one), not the whole prompt."""
    def ws(a, rows):
        n = ctypes.c_size_t(0)
        assert lib.dsa_chunked_stack_workspace_size(ctypes.byref(a), rows, ctypes.byref(n)) == 0
        return n.value
    L_, k = 9000, 16
    a = _stack_args(n_q=L_, n_k=L_)
    full = ws(a, L_)
    n = ctypes.c_size_t(0)
    assert lib.dsa_stack_workspace_size(ctypes.byref(a), ctypes.byref(n)) == 0
    assert full == n.value
    chunk = ws(a, 3000)
    assert chunk < full
    one = dict(idx=dsa.indexer_workspace_size(1, 3000, L_, 4, 32, k),
               attn=dsa.attn_workspace_size(1, 3000, L_, 4, 64, k))
    assert chunk == max(one.values())
    # a one-row last chunk takes the decode path: its workspace counts too
    dec = dsa.indexer_workspace_size(1, 1, L_, 4, 32, k)
    assert ws(a, 2999) >= dec   # 9000 = 3 * 2999 + 3 rows
    assert ws(a, 8999) >= dec   # last chunk of one row


# ---- the Python binding checks every caller tensor before anything is launched
import torch  # noqa: E402


def _cpu_inputs(B=1, n_q=8, n_k=8, H=4, D=32):
    return dict(q=torch.zeros(B, n_q, H, D, dtype=torch.bfloat16), k=torch.zeros(B, n_k, D, dtype=torch.bfloat16),
                w=torch.zeros(B, n_q, H))


@pytest.mark.parametrize("bad,msg", [
    (dict(k=torch.zeros(1, 8, 16, dtype=torch.bfloat16)), "k must have shape"),
    (dict(w=torch.zeros(1, 8, 5)), "w must have shape"),
    (dict(w=torch.zeros(1, 8, 4, dtype=torch.float64)), "w must be"),
    (dict(out_idx=torch.zeros(1, 8, 15, dtype=torch.int32)), "out_idx must have shape"),
    (dict(out_scores=torch.zeros(1, 8, 17)), "out_scores must have shape"),
    (dict(debug_full_scores=torch.zeros(1, 8, 9)), "debug_full_scores must have shape"),
    (dict(debug_full_scores=torch.zeros(1, 8, 8, dtype=torch.float16)), "debug_full_scores must be"),
    (dict(q_scale=torch.ones(1, 8)), "for fp8 inputs only"),
    (dict(), "q must be a GPU tensor"),                     # every shape right: the device check fires
])
def test_binding_indexer_argument_checks(bad, msg):
    d = _cpu_inputs()
    kw = {k: v for k, v in bad.items() if k not in d}
    d.update({k: v for k, v in bad.items() if k in d})
    with pytest.raises((ValueError, TypeError), match=msg):
        dsa.indexer_scores_topk(d["q"], d["k"], d["w"], 16, **kw)


@pytest.mark.parametrize("bad,msg", [
    (dict(v=torch.zeros(1, 9, 64, dtype=torch.bfloat16)), "v must have shape"),
    (dict(idx=torch.zeros(1, 7, 16, dtype=torch.int32)), "idx must have shape"),
    (dict(out=torch.zeros(1, 8, 4, 32, dtype=torch.bfloat16)), "out must have shape"),
    (dict(lse=torch.zeros(1, 8, 5)), "lse must have shape"),
    (dict(), "q must be a GPU tensor"),
])
def test_binding_attention_argument_checks(bad, msg):
    d = dict(q=torch.zeros(1, 8, 4, 64, dtype=torch.bfloat16), k=torch.zeros(1, 8, 64, dtype=torch.bfloat16),
             v=torch.zeros(1, 8, 64, dtype=torch.bfloat16), idx=torch.zeros(1, 8, 16, dtype=torch.int32))
    kw = {k: v for k, v in bad.items() if k not in d}
    d.update({k: v for k, v in bad.items() if k in d})
    with pytest.raises((ValueError, TypeError), match=msg):
        dsa.sparse_attn(d["q"], d["k"], d["v"], d["idx"], **kw)


def _layers(n=2, n_q=8, n_k=8, fp8=False):
    dt = torch.float8_e4m3fn if fp8 else torch.bfloat16
    out = []
    for _ in range(n):
        out.append(dict(q_idx=torch.zeros(1, n_q, 4, 32, dtype=dt), k_idx=torch.zeros(1, n_k, 32, dtype=dt),
                        w=torch.zeros(1, n_q, 4),
                        q_scale=torch.ones(1, n_q) if fp8 else None, k_scale=torch.ones(1, n_k) if fp8 else None,
                        q=torch.zeros(1, n_q, 4, 64, dtype=torch.bfloat16),
                        k=torch.zeros(1, n_k, 64, dtype=torch.bfloat16),
                        v=torch.zeros(1, n_k, 64, dtype=torch.bfloat16)))
    return out


@pytest.mark.parametrize("layer,name,val,msg", [
    (1, "k_idx", torch.zeros(1, 9, 32, dtype=torch.bfloat16), r"layers\[1\].k_idx must have shape"),
    (1, "w", torch.zeros(1, 8, 3), r"layers\[1\].w must have shape"),
    (1, "v", torch.zeros(1, 8, 32, dtype=torch.bfloat16), r"layers\[1\].v must have shape"),
    (1, "k", torch.zeros(1, 8, 64, dtype=torch.float32), r"layers\[1\].k must be"),
    (0, "q_scale", torch.ones(1, 8), "fp8 inputs only"),
    (1, "q", torch.zeros(1, 8, 4, 64, dtype=torch.bfloat16), "layers.0..q_idx must be a GPU tensor"),
])
def test_binding_stack_argument_checks(layer, name, val, msg):
    ls = _layers()
    ls[layer][name] = val
    with pytest.raises((ValueError, TypeError), match=msg):
        dsa.LayerStack(ls, 16)


def test_binding_stack_fp8_scales_checked():
    ls = _layers(fp8=True)
    ls[1]["k_scale"] = torch.ones(1, 7)
    with pytest.raises(ValueError, match=r"layers\[1\].k_scale must have shape"):
        dsa.LayerStack(ls, 16)
    ls = _layers(fp8=True)
    ls[0]["q_scale"] = None
    with pytest.raises(TypeError, match=r"layers\[0\].q_scale must be a torch.Tensor"):
        dsa.LayerStack(ls, 16)


def test_binding_chunked_stack_arguments():
    with pytest.raises(ValueError, match="chunk_rows"):
        dsa.LayerStack(_layers(), 16, chunk_rows=0)
    with pytest.raises(ValueError, match="chunk_rows"):
        dsa.LayerStack(_layers(), 16, chunk_rows=4, events=True)


def test_binding_other_argument_checks():
    with pytest.raises(ValueError, match="out must have shape"):
        dsa.topk_overlap(torch.zeros(3, 2, 4, dtype=torch.int32), 10, out=torch.zeros(3, 2, dtype=torch.int64))
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        dsa.topk_overlap(torch.zeros(3, 2, 4, dtype=torch.int32), 10)
    x = torch.zeros(4, 64, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="out must have shape"):
        dsa.quantize_fp8_rows(x, out=torch.zeros(4, 32, dtype=torch.float8_e4m3fn))
    with pytest.raises(ValueError, match="one entry per row"):
        dsa.quantize_fp8_rows(x, scale=torch.zeros(5))
    with pytest.raises(ValueError, match="must be a GPU tensor"):
        dsa.quantize_fp8_rows(x)


def test_static_scratch_entry_validation(lib):
    """The no-allocation entry point validates like dsa_indexer_scores_topk,
    refuses a workspace, and rejects shapes beyond its static scratch before
    any HIP call."""
    f = lib.dsa_indexer_scores_topk_static
    a = _idx_args()
    a.q = None
    assert f(ctypes.byref(a), None) == L.DSA_ERR_INVALID_ARGUMENT
    a = _idx_args()
    a.workspace, a.workspace_bytes = FAKE, 1 << 20
    assert f(ctypes.byref(a), None) == L.DSA_ERR_INVALID_ARGUMENT
    a = _idx_args(n_q=4096, n_k=4096, topk=2048)
    assert dsa.indexer_workspace_size(1, 4096, 4096, 64, 128, 2048) > L.DSA_STATIC_SCRATCH_BYTES
    assert f(ctypes.byref(a), None) == L.DSA_ERR_WORKSPACE
    assert b"static scratch" in lib.dsa_last_error()
    # decode of 32 requests over 200K tokens fits
    assert dsa.indexer_workspace_size(32, 1, 200000, 64, 128, 2048) <= L.DSA_STATIC_SCRATCH_BYTES
