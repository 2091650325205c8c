#!/usr/bin/env python3
"""Benchmark of the DSA indexer + top-k hot path on one MI355X.

Headline (the JSON line's `value`): single-layer prefill lightning indexer fused
with exact top-k at L = 200000 tokens, H_I = 64 indexer heads, d_I = 128,
top-k = 2048, fp8 e4m3 q_idx/k_idx with per-token fp32 scales (causal). A step
is one dsa_indexer_scores_topk call over the whole layer (score kernel +
selection kernel) with inputs resident in HBM; value = L / step time.

`roofline` is for the dominant kernel (the fused score + streaming-filter
kernel): its algorithmic work is L(L+1)/2 * H_I * d_I * 2 flop per launch (the
causal triangle only), timed live with HIP events recorded by the library on
the stream it launches on; `peak` is the published one and `peak_measured` the
rate of a dense MFMA loop of the same dtype on this GPU. `cpu_baseline` times
the fp64 CPU oracle on a bounded sample of the same layer's query rows and
extrapolates by the number of causal keys. `extra` adds the measured peaks
(MFMA loops, HBM copy and read), the single-layer L = 10240 bf16 layer with
the CPU oracle timed over all of it, the bf16 200K layer, the 47-layer F/S
prefill stack at L = 61440 (all-F, index_topk_freq 2 and 4) and at 200K (all-F,
the seeded 12-F pattern, and that pattern prefilled in chunks of 25000 rows),
decode at 200K context (per-kernel times warm and over rotating layer sets)
and paged decode of 32 requests with ragged context lengths up to 200K, and
the cross-layer top-k overlap of 47 layers.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--quick]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "indexer+top-k queries/sec & fraction of MFMA peak at 200K; stack prefill time F/S"
PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0}   # MI355X dense MFMA
PEAK_HBM_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "indexer_prefill_fp8_L200000_traffic.json")
PEAK_LIB = os.path.join(ROOT, "dsa_indexer_top_amd", "libdsa_peak.so")
KERNEL_SOURCES = ["dsa_indexer_top_amd/csrc/indexer_prefill.hip", "dsa_indexer_top_amd/csrc/dsa_device.h"]


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def kernel_source_hash():
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def causal_flops(L, H, D):
    return L * (L + 1) // 2 * H * D * 2


def time_indexer(dsa, torch, inp, topk, steps, warmup):
    """Returns (ms per step wall-clock, mean score-kernel ms, mean select ms, idx)."""
    g = inp
    B, n_q, H, D = g.q.shape
    n_k = g.k.shape[1]
    code = 1 if g.dtype == "fp8" else 0
    ws = torch.empty(dsa.indexer_workspace_size(B, n_q, n_k, H, D, topk, code), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((B, n_q, topk), dtype=torch.int32, device="cuda")
    call = lambda ev=None: dsa.indexer_scores_topk(g.q, g.k, g.w, topk, q_scale=g.q_scale,
                                                   k_scale=g.k_scale, pos_offset=g.pos_offset,
                                                   out_idx=out, workspace=ws, phase_events=ev)
    for _ in range(warmup):
        call()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        call(evs[i])
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    k_ms = sum(e[0].elapsed_time(e[1]) for e in evs) / steps
    s_ms = sum(e[1].elapsed_time(e[2]) for e in evs) / steps
    del ws
    return wall, k_ms, s_ms, out


def traffic_for_current_kernel():
    """HBM bytes per launch of the score kernel from the committed rocprofv3
    counter summary, or None if the kernel source changed since it was taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha256") != kernel_source_hash():
        return None
    return t.get("traffic_bytes_per_launch")


def cpu_info():
    """CPU model, the threads this process may use and the BLAS numpy calls."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = []
    try:
        from threadpoolctl import threadpool_info
        blas = [{k: p.get(k) for k in ("internal_api", "version", "num_threads", "threading_layer", "architecture")}
                for p in threadpool_info() if p.get("user_api") == "blas"]
    except Exception:
        pass
    return {"cpu_model": model, "logical_cpus": os.cpu_count(),
            "cpus_available": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None,
            "blas": blas}


def blas_threads():
    try:
        from threadpoolctl import threadpool_info
        return max([p.get("num_threads", 1) for p in threadpool_info() if p.get("user_api") == "blas"] or [1])
    except Exception:
        return 1


def measured_peaks(torch):
    """Rates of the probes in libdsa_peak.so on this GPU (best of 3 timed
    launches after one untimed): dense MFMA loops in bf16 and fp8 (two
    workgroups of four waves per CU, four independent accumulators per wave),
    an HBM copy and read of 2 GiB with 16-byte nontemporal accesses (the
    best of four grid sizes), and a gather of 256-byte rows (bf16 rows of 128)
    with the prefill attention's access pattern over tables of the K and V rows
    of 61440 and of 200000 tokens (the best of three grid sizes)."""
    import ctypes
    lib = ctypes.CDLL(PEAK_LIB)
    lib.dsa_peak_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                  ctypes.POINTER(ctypes.c_double), ctypes.c_void_p]
    lib.dsa_peak_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    lib.dsa_peak_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.dsa_peak_gather.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                    ctypes.c_void_p, ctypes.c_void_p]
    stream = torch.cuda.current_stream().cuda_stream
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def best_ms(launch, reps=3):
        launch()
        ms = []
        for _ in range(reps):
            e0.record()
            launch()
            e1.record()
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        return min(ms)

    cus = torch.cuda.get_device_properties(0).multi_processor_count
    res = {"cus": cus}
    out = torch.empty(2 * cus * 256, dtype=torch.float32, device="cuda")
    for code, name, iters in ((0, "bf16", 40000), (1, "fp8", 20000)):
        flop = ctypes.c_double()

        def run():
            if lib.dsa_peak_mfma(code, 2 * cus, iters, out.data_ptr(), ctypes.byref(flop), stream) != 0:
                raise RuntimeError("dsa_peak_mfma failed")
        ms = best_ms(run)
        res[f"mfma_{name}_TFLOPs"] = flop.value / (ms * 1e-3) / 1e12
    n = 2 << 30
    src = torch.ones(n // 4, dtype=torch.int32, device="cuda")
    dst = torch.empty_like(src)
    red = torch.empty(16384, dtype=torch.int32, device="cuda")
    copy_best = read_best = 0.0
    for blocks in (1024, 2048, 4096, 8192):
        def cp():
            if lib.dsa_peak_copy(src.data_ptr(), dst.data_ptr(), n, blocks, stream) != 0:
                raise RuntimeError("dsa_peak_copy failed")

        def rd():
            if lib.dsa_peak_read(src.data_ptr(), n, blocks, red.data_ptr(), stream) != 0:
                raise RuntimeError("dsa_peak_read failed")
        copy_best = max(copy_best, 2 * n / best_ms(cp) / 1e6)
        read_best = max(read_best, n / best_ms(rd) / 1e6)
    res["hbm_copy_GBps"] = copy_best
    res["hbm_read_GBps"] = read_best
    del dst
    gen = torch.Generator(device="cuda")
    gen.manual_seed(12345)
    res["gather_GBps"] = {}
    for tokens in (61440, 200000):
        # the attention's access pattern without its arithmetic: 4096 query
        # rows t drawn uniformly and taken in increasing order (as the
        # attention's workgroups go), each listing 2048 keys drawn uniformly
        # from [0, t], each key's K row (table rows [0, tokens)) and V row
        # (rows [tokens, 2 tokens)) in turn
        rows = 2 * tokens
        t = torch.randint(0, tokens, (4096,), device="cuda", generator=gen).sort().values.unsqueeze(1)
        key = (torch.rand((4096, 2048), device="cuda", generator=gen) * (t + 1)).long().clamp_(max=tokens - 1)
        idx = torch.stack((key, key + tokens), dim=-1).flatten().to(torch.int32)
        ng = idx.numel()
        del t, key
        g_best = 0.0
        for blocks in (2048, 4096, 8192):
            def ga():
                if lib.dsa_peak_gather(src.data_ptr(), rows, idx.data_ptr(), ng, blocks, red.data_ptr(), stream) != 0:
                    raise RuntimeError("dsa_peak_gather failed")
            g_best = max(g_best, 256 * ng / best_ms(ga) / 1e6)
        res["gather_GBps"][f"kv_{tokens}_tokens"] = g_best
        del idx
    res["published"] = {"mfma_bf16_TFLOPs": PEAK_TFLOPS["bf16"], "mfma_fp8_TFLOPs": PEAK_TFLOPS["fp8"],
                        "hbm_GBps": PEAK_HBM_GBS}
    log(f"measured peaks: MFMA bf16 {res['mfma_bf16_TFLOPs']:.0f} TFLOP/s, fp8 {res['mfma_fp8_TFLOPs']:.0f} "
        f"TFLOP/s; HBM copy {copy_best:.0f} GB/s, read {read_best:.0f} GB/s; row gather "
        + ", ".join(f"{k} {v:.0f} GB/s" for k, v in res["gather_GBps"].items()))
    del src, red, out
    torch.cuda.empty_cache()
    return res


def cpu_c2_full(L=10240, topk=2048):
    """The fp64 oracle over every query row of the L = 10240 bf16 layer
    (scores and top-k), timed in full on this host."""
    import oracle
    from dsa_inputs import host_bits, make_indexer_inputs
    inp = make_indexer_inputs(1, L, L, 64, 128, config=2, dtype="bf16", w_std=0.125)
    q, k, w = host_bits(inp.q), host_bits(inp.k), host_bits(inp.w)
    t0 = time.perf_counter()
    oracle.indexer_topk(q, k, w, topk)
    t = time.perf_counter() - t0
    log(f"CPU oracle, L={L} bf16 layer in full: {t:.1f} s")
    return {"value": L / t, "unit": "queries/s", "seconds": t, "cores": blas_threads(), "kind": "oracle",
            "sample": f"all {L} query rows of the layer (scores and top-k), not extrapolated", **cpu_info()}


def cpu_baseline(inp_host, L, topk, budget_s):
    """Times the fp64 oracle on seeded random query rows of the layer until the
    time budget is spent, and extrapolates to the whole layer by causal keys."""
    import numpy as np
    import oracle
    threads = blas_threads()
    rng = np.random.default_rng(2024)
    order = rng.permutation(L)
    done_rows, done_keys, spent = 0, 0, 0.0
    q, k, w, qs, ks, dt = inp_host
    i = 0
    while spent < budget_s and i < L:
        rows = sorted(int(r) for r in order[i:i + 4])
        i += 4
        t0 = time.perf_counter()
        sc = oracle.indexer_scores_rows(q, k, w, rows, dtype=dt, q_scale=qs, k_scale=ks)
        oracle.topk_from_scores(sc, topk, rows=rows)
        spent += time.perf_counter() - t0
        done_rows += len(rows)
        done_keys += sum(r + 1 for r in rows)
    total_keys = L * (L + 1) // 2
    est_s = spent / done_keys * total_keys
    return {"value": L / est_s, "unit": "queries/s", "cores": threads, "kind": "oracle",
            "sample": (f"{done_rows} seeded-random query rows of the same layer ({done_keys} causal "
                       f"keys, {spent:.1f} s of fp64 oracle: scores + top-k), extrapolated to all "
                       f"{L} rows by causal-key count (layer estimate {est_s:.0f} s)"), **cpu_info()}


def stack_bench(dsa, torch, L, n_layers, topk, steps, warmup, config=3, dtype="bf16", patterns=None,
                chunked=None):
    """47-layer prefill stack, per-layer tensors seeded independently, one shared
    index buffer. patterns: list of (name, run kwargs); default all-F vs
    index_topk_freq 2 and 4. Reports each pattern's best wall time and mean
    per-layer event times of its F and S layers. chunked: list of (name, run
    kwargs, chunk_rows): the same layers prefilled chunk by chunk (each chunk's
    rows over the keys up to its last row, a per-chunk index buffer)."""
    from dsa_inputs import make_attn_inputs, make_indexer_inputs
    if patterns is None:
        patterns = [("all_F", {}), ("freq2", {"freq": 2}), ("freq4", {"freq": 4})]
    layers = []
    for l in range(n_layers):
        ii = make_indexer_inputs(1, L, L, 64, 128, config=config, layer=l, dtype=dtype, w_std=0.125,
                                 device="cuda")
        aa = make_attn_inputs(1, L, L, 16, 128, config=config, layer=l, device="cuda")
        layers.append(dict(q_idx=ii.q, k_idx=ii.k, w=ii.w, q_scale=ii.q_scale, k_scale=ii.k_scale,
                           q=aa.q, k=aa.k, v=aa.v))
    st = dsa.LayerStack(layers, topk, shared_out=True, events=True)
    res = {}
    for name, kw in patterns:
        for _ in range(warmup):
            st.run(**kw)
        torch.cuda.synchronize()
        times, per_layer = [], None
        for _ in range(steps):
            t0 = time.perf_counter()
            st.run(**kw)
            torch.cuda.synchronize()
            times.append(time.perf_counter() - t0)
            per_layer = st.layer_times_ms()
        pat = dsa.resolve_pattern(n_layers, kw.get("pattern"), kw.get("freq", 0))
        f_ms = [t for t, c in zip(per_layer, pat) if c == "F"]
        s_ms = [t for t, c in zip(per_layer, pat) if c == "S"]
        res[name] = {"pattern": pat, "pattern_F": pat.count("F"), "time_s": min(times),
                     "mean_F_layer_ms": sum(f_ms) / len(f_ms),
                     "mean_S_layer_ms": (sum(s_ms) / len(s_ms)) if s_ms else None}
        log(f"stack L={L} {name}: {min(times):.3f} s")
    for name, _ in patterns[1:]:
        res[name]["speedup_vs_all_F"] = res["all_F"]["time_s"] / res[name]["time_s"]
    del st
    torch.cuda.empty_cache()
    for name, kw, rows in chunked or []:
        stc = dsa.LayerStack(layers, topk, shared_out=True, chunk_rows=rows)
        for _ in range(warmup):
            stc.run(**kw)
        torch.cuda.synchronize()
        times = []
        for _ in range(steps):
            t0 = time.perf_counter()
            stc.run(**kw)
            torch.cuda.synchronize()
            times.append(time.perf_counter() - t0)
        pat = dsa.resolve_pattern(n_layers, kw.get("pattern"), kw.get("freq", 0))
        res[name] = {"pattern": pat, "pattern_F": pat.count("F"), "chunk_rows": rows,
                     "chunks": (L + rows - 1) // rows, "time_s": min(times)}
        log(f"stack L={L} {name} (chunks of {rows}): {min(times):.3f} s")
        del stc
        torch.cuda.empty_cache()
    del layers
    torch.cuda.empty_cache()
    return res


def decode_bench(dsa, torch, B, T, n_layers, topk, steps, warmup, config=4):
    """One decode token over n_layers with a seeded 12-F pattern; independent
    caches per request. B = 1 uses distinct tensors for every layer; larger B
    rotates two distinct layer sets (each far larger than the 256 MB MALL)."""
    from dsa_inputs import make_attn_inputs, make_indexer_inputs, seeded_pattern
    n_sets = n_layers if B == 1 else 2
    sets = []
    for l in range(n_sets):
        ii = make_indexer_inputs(B, 1, T, 64, 128, config=config, layer=l, w_std=0.125, device="cuda")
        aa = make_attn_inputs(B, 1, T, 16, 128, config=config, layer=l, device="cuda")
        sets.append(dict(q_idx=ii.q, k_idx=ii.k, w=ii.w, q_scale=None, k_scale=None,
                         q=aa.q, k=aa.k, v=aa.v))
    layers = [sets[l % n_sets] for l in range(n_layers)]
    pat = seeded_pattern(n_layers, 12, seed=1_000_000 * config + 9)
    # per-kernel HBM rates on one layer
    l0 = sets[0]
    evi = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    eva = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    k_ms = a_ms = 0.0
    idx = None
    for i in range(warmup + steps):
        r = dsa.indexer_scores_topk(l0["q_idx"], l0["k_idx"], l0["w"], topk, phase_events=evi)
        idx = r.idx
        dsa.sparse_attn(l0["q"], l0["k"], l0["v"], idx, phase_events=eva)
        torch.cuda.synchronize()
        if i >= warmup:
            k_ms += evi[0].elapsed_time(evi[1]) / steps
            a_ms += eva[0].elapsed_time(eva[1]) / steps
    idx_bytes = B * T * 128 * 2 + B * T * 4                 # k_idx read + score keys written
    att_bytes = B * topk * 2 * 128 * 2                      # gathered K and V rows
    # cold: each call on the next distinct layer set (B = 1: 47 sets of 154 MB;
    # B = 32: two sets of 4.9 GB), so no call finds its inputs in the 256 MB
    # memory-side cache
    kc_ms = ac_ms = 0.0
    n_cold = max(2 * n_sets, 8) if B > 1 else n_sets
    for i in range(n_cold + 1):
        s_ = sets[i % n_sets]
        r = dsa.indexer_scores_topk(s_["q_idx"], s_["k_idx"], s_["w"], topk, phase_events=evi)
        dsa.sparse_attn(s_["q"], s_["k"], s_["v"], r.idx, phase_events=eva)
        torch.cuda.synchronize()
        if i >= 1:
            kc_ms += evi[0].elapsed_time(evi[1]) / n_cold
            ac_ms += eva[0].elapsed_time(eva[1]) / n_cold
    st = dsa.LayerStack(layers, topk, shared_out=True)
    for _ in range(warmup):
        st.run(pat)
    torch.cuda.synchronize()
    times = []
    for _ in range(steps):
        t0 = time.perf_counter()
        st.run(pat)
        torch.cuda.synchronize()
        times.append(time.perf_counter() - t0)
    step = min(times)
    res = {"B": B, "context": T, "pattern": pat,
           "indexer_kernel_ms": k_ms, "indexer_hbm_GBps": idx_bytes / k_ms / 1e6,
           "indexer_hbm_frac": idx_bytes / k_ms / 1e6 / PEAK_HBM_GBS,
           "attn_ms": a_ms, "attn_gather_GBps": att_bytes / a_ms / 1e6,
           "attn_gather_hbm_frac": att_bytes / a_ms / 1e6 / PEAK_HBM_GBS,
           "cold": {"sets": n_sets, "calls": n_cold,
                    "indexer_kernel_ms": kc_ms, "indexer_hbm_GBps": idx_bytes / kc_ms / 1e6,
                    "indexer_hbm_frac": idx_bytes / kc_ms / 1e6 / PEAK_HBM_GBS,
                    "attn_ms": ac_ms, "attn_gather_GBps": att_bytes / ac_ms / 1e6,
                    "attn_gather_hbm_frac": att_bytes / ac_ms / 1e6 / PEAK_HBM_GBS},
           "step_ms_47_layers": step * 1e3, "tok_per_s_per_request": 1.0 / step,
           "tok_per_s_total": B / step}
    log(f"decode B={B}: indexer {k_ms:.3f} ms warm / {kc_ms:.3f} ms cold ({idx_bytes / kc_ms / 1e6:.0f} GB/s), "
        f"attn {a_ms:.3f} ms warm / {ac_ms:.3f} ms cold, 47-layer step {step*1e3:.2f} ms")
    del st, layers, sets
    torch.cuda.empty_cache()
    return res


def decode_gather_bench(dsa, torch, B, T, topk, steps, warmup, config=4):
    """Decode attention alone at a batch large enough to load the HBM: B
    requests over T-token caches (K and V: B * T * 512 bytes), k uniform random
    indices per request (on the synthetic scores the indexer's picks are
    spread the same way)."""
    from dsa_inputs import make_attn_inputs
    a = make_attn_inputs(B, 1, T, 16, 128, config=config, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(1_000_000 * config + 13)
    # four index sets: the warm figure repeats the first, the cold one rotates
    # them (each call gathers rows the previous three calls did not touch)
    idxs = [torch.randint(0, T, (B, 1, topk), generator=g, device="cuda", dtype=torch.int32) for _ in range(4)]
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ms, cold = [], []
    for i in range(warmup + steps):
        dsa.sparse_attn(a.q, a.k, a.v, idxs[0], phase_events=ev)
        torch.cuda.synchronize()
        if i >= warmup:
            ms.append(ev[0].elapsed_time(ev[1]))
    for i in range(1, 1 + 2 * len(idxs)):
        dsa.sparse_attn(a.q, a.k, a.v, idxs[i % len(idxs)], phase_events=ev)
        torch.cuda.synchronize()
        cold.append(ev[0].elapsed_time(ev[1]))
    a_ms = sum(ms) / len(ms)
    c_ms = sum(cold) / len(cold)
    att_bytes = B * topk * 2 * 128 * 2  # gathered K and V rows
    res = {"B": B, "context": T, "topk": topk, "attn_ms": a_ms, "attn_gather_GBps": att_bytes / a_ms / 1e6,
           "attn_gather_hbm_frac": att_bytes / a_ms / 1e6 / PEAK_HBM_GBS,
           "cold": {"index_sets": len(idxs), "attn_ms": c_ms, "attn_gather_GBps": att_bytes / c_ms / 1e6,
                    "attn_gather_hbm_frac": att_bytes / c_ms / 1e6 / PEAK_HBM_GBS}}
    log(f"decode attention B={B}: {a_ms * 1e3:.1f} us warm, {c_ms * 1e3:.1f} us cold "
        f"({att_bytes / c_ms / 1e6:.0f} GB/s of gathered rows)")
    del a, idxs
    torch.cuda.empty_cache()
    return res


def paged_decode_bench(dsa, torch, B, T, n_layers, topk, steps, warmup, page_size=64, config=6):
    """One decode token of B requests with seeded ragged context lengths
    (uniform in [2048, T]) over paged pools (page_size tokens, pages handed out
    in a seeded random order), 47 layers with the seeded 12-F pattern; two
    distinct layer sets rotate. Pools hold N(0,1) draws: the rows are the
    requests' caches. Algorithmic indexer bytes = sum of lengths * (256 k_idx
    bytes + 4 score-key bytes)."""
    import numpy as np
    from dsa_inputs import make_paged_layout, seeded_pattern, seed_for, randn
    rng = np.random.default_rng(1_000_000 * config + 11)
    lens = rng.integers(2048, T + 1, size=B)
    lay = make_paged_layout(lens.tolist(), page_size, T, seed=1_000_000 * config + 12).to("cuda")
    kv = dsa.PagedKV(lay.seq_lens, lay.block_table, page_size, lay.num_pages, T)
    sets = []
    for l in range(2):
        def pool(name, D=128):
            return randn((lay.num_pages, page_size, D), seed_for(config, l, name), "cuda").to(torch.bfloat16)
        q_idx = randn((B, 1, 64, 128), seed_for(config, l, "q_idx"), "cuda").to(torch.bfloat16)
        w = randn((B, 1, 64), seed_for(config, l, "w"), "cuda") * 0.125
        q = randn((B, 1, 16, 128), seed_for(config, l, "q"), "cuda").to(torch.bfloat16)
        sets.append(dict(q_idx=q_idx, k_idx=pool("k_idx"), w=w, q_scale=None, k_scale=None,
                         q=q, k=pool("k"), v=pool("v")))
    layers = [sets[l % 2] for l in range(n_layers)]
    pat = seeded_pattern(n_layers, 12, seed=1_000_000 * config + 9)
    l0 = sets[0]
    evi = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
    eva = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    k_ms = a_ms = 0.0
    for i in range(warmup + steps):
        r = dsa.paged_indexer_topk(l0["q_idx"], l0["k_idx"], l0["w"], topk, kv, phase_events=evi)
        dsa.paged_sparse_attn(l0["q"], l0["k"], l0["v"], r.idx, kv, phase_events=eva)
        torch.cuda.synchronize()
        if i >= warmup:
            k_ms += evi[0].elapsed_time(evi[1]) / steps
            a_ms += eva[0].elapsed_time(eva[1]) / steps
    total = int(lens.sum())
    idx_bytes = total * (128 * 2 + 4)
    att_bytes = B * topk * 2 * 128 * 2
    st = dsa.LayerStack(layers, topk, shared_out=True, kv=kv)
    for _ in range(warmup):
        st.run(pat)
    torch.cuda.synchronize()
    times = []
    for _ in range(steps):
        t0 = time.perf_counter()
        st.run(pat)
        torch.cuda.synchronize()
        times.append(time.perf_counter() - t0)
    step = min(times)
    res = {"B": B, "max_context": T, "page_size": page_size, "context_sum": total,
           "context_mean": total / B, "pattern": pat,
           "indexer_kernel_ms": k_ms, "indexer_hbm_GBps": idx_bytes / k_ms / 1e6,
           "indexer_hbm_frac": idx_bytes / k_ms / 1e6 / PEAK_HBM_GBS,
           "attn_ms": a_ms, "attn_gather_GBps": att_bytes / a_ms / 1e6,
           "step_ms_47_layers": step * 1e3, "tok_per_s_total": B / step}
    log(f"paged decode B={B} (mean context {total / B:.0f}): indexer {k_ms:.3f} ms "
        f"({res['indexer_hbm_GBps']:.0f} GB/s), attn {a_ms:.3f} ms, 47-layer step {step*1e3:.2f} ms")
    del st, layers, sets
    torch.cuda.empty_cache()
    return res


def overlap_bench(dsa, torch, steps, n=47, R=256, k=2048, n_k=200000):
    """Cross-layer top-k overlap of 47 layers' indices for 256 sampled query
    rows (k = 2048 of a 200K context; synthetic correlated random-walk index
    sets), then the 12-F similarity pattern from it. Bytes: every workgroup
    (row, layer a) reads the rows of layers b >= a, (n + 1) n / 2 rows of k
    int32 per query row, from L2; n R k int32 are the compulsory HBM reads."""
    from dsa_inputs import make_correlated_topk
    idx = torch.from_numpy(make_correlated_topk(n, R, k, n_k, swap=0.1, seed=47, reset_every=6)).cuda()
    out = dsa.topk_overlap(idx, n_k)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        dsa.topk_overlap(idx, n_k, out=out)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    t0 = time.perf_counter()
    pat = dsa.similarity_pattern(out, 12)
    pat_ms = (time.perf_counter() - t0) * 1e3
    l2_bytes = R * (n + 1) * n // 2 * k * 4
    res = {"layers": n, "rows": R, "topk": k, "n_k": n_k, "ms": ms, "l2_read_GBps": l2_bytes / ms / 1e6,
           "compulsory_hbm_GBps": n * R * k * 4 / ms / 1e6, "pattern_12F": pat, "pattern_host_ms": pat_ms}
    log(f"topk overlap {n} layers x {R} rows: {ms:.3f} ms ({res['l2_read_GBps']:.0f} GB/s of index rows), "
        f"pattern {pat_ms:.2f} ms on the host")
    del idx, out
    torch.cuda.empty_cache()
    return res


def quant_bench(dsa, torch, L, steps):
    """Per-token fp8 quantisation of the 200K layer's q_idx ([L, 64 * 128] bf16):
    algorithmic HBM bytes = 2 read + 1 written per element + 4 per row."""
    g = torch.Generator(device="cuda").manual_seed(1_000_000 * 5 + 1)
    x = torch.randn(L, 64 * 128, generator=g, device="cuda", dtype=torch.bfloat16)
    codes = torch.empty(x.shape, dtype=torch.float8_e4m3fn, device="cuda")
    scale = torch.empty(L, dtype=torch.float32, device="cuda")
    dsa.quantize_fp8_rows(x, out=codes, scale=scale)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(steps):
        dsa.quantize_fp8_rows(x, out=codes, scale=scale)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    nbytes = x.numel() * 3 + L * 4
    del x, codes, scale
    torch.cuda.empty_cache()
    return {"rows": L, "cols": 64 * 128, "ms": ms, "hbm_GBps": nbytes / ms / 1e6,
            "hbm_frac": nbytes / ms / 1e6 / PEAK_HBM_GBS}


def c2_bench(dsa, torch, steps, warmup, peaks=None, L=10240, topk=2048):
    """The single-layer L = 10240 bf16 layer (H_I = 64, d_I = 128, k = 2048):
    queries/s of the fused indexer + top-k step and the score kernel's MFMA
    fraction (causal flop / kernel time) against the published and the
    measured bf16 peak."""
    from dsa_inputs import make_indexer_inputs
    inp = make_indexer_inputs(1, L, L, 64, 128, config=2, dtype="bf16", w_std=0.125, device="cuda")
    wall, k_ms, s_ms, _ = time_indexer(dsa, torch, inp, topk, steps, warmup)
    flops = causal_flops(L, 64, 128)
    a = flops / (k_ms * 1e-3) / 1e12
    step_tf = flops / (wall * 1e-3) / 1e12
    res = {"L": L, "dtype": "bf16", "topk": topk, "ms_per_step": wall, "queries_per_s": L / (wall * 1e-3),
           "score_kernel_ms": k_ms, "select_kernel_ms": s_ms, "score_kernel_TFLOPs": a,
           "mfma_frac": a / PEAK_TFLOPS["bf16"], "step_mfma_frac": step_tf / PEAK_TFLOPS["bf16"]}
    if peaks:
        res["mfma_frac_of_measured"] = a / peaks["mfma_bf16_TFLOPs"]
        res["step_mfma_frac_of_measured"] = step_tf / peaks["mfma_bf16_TFLOPs"]
    log(f"L={L} bf16: {wall:.3f} ms/step ({L / (wall * 1e-3):.0f} queries/s), score kernel {k_ms:.3f} ms "
        f"({a:.0f} TFLOP/s, {a / PEAK_TFLOPS['bf16']:.3f} of peak)")
    del inp
    torch.cuda.empty_cache()
    return res


def stack200k(dsa, torch, L, topk, args):
    """The 47-layer stack at L = 200000 with the fp8 indexer: all-F vs a seeded
    pattern with 12 F layers (layer 0 and 11 of layers 1..46)."""
    from dsa_inputs import seeded_pattern
    pat = seeded_pattern(47, 12, seed=1_000_000 * 5 + 9)
    res = {"L": L, "layers": 47, "dtype": "fp8 indexer, bf16 attention", "attn": "16 heads, d=128, 1 KV head",
           **stack_bench(dsa, torch, L, 47, topk, 1, 1, config=5, dtype="fp8",
                         patterns=[("all_F", {}), ("seeded_quarter_F", {"pattern": pat})],
                         chunked=[("seeded_quarter_F_chunked", {"pattern": pat}, 25000)])}
    res["seeded_quarter_F_chunked"]["time_vs_one_shot"] = (res["seeded_quarter_F_chunked"]["time_s"]
                                                           / res["seeded_quarter_F"]["time_s"])
    return res


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--L", type=int, default=200000)
    ap.add_argument("--dtype", default="fp8", choices=["fp8", "bf16"])
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="headline only")
    ap.add_argument("--quick", action="store_true", help="headline + CPU baseline only")
    ap.add_argument("--stack-L", type=int, default=61440)
    ap.add_argument("--stack-layers", type=int, default=47)
    ap.add_argument("--only", choices=["stack", "stack200k", "decode", "paged", "quant", "overlap", "peaks", "c2"],
                    default=None,
                    help="run only the stack or only the decode measurement and print its JSON "
                         "(for profiling one part; not the benchmark line)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only copy a MIB-MiB device buffer 3 times (reference dispatch for "
                         "rocprofv3 FETCH_SIZE / WRITE_SIZE scaling) and exit")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: this build measures one GPU only; --gpus N > 1 (or WORLD_SIZE > 1) is not "
              "supported (the path has no multi-GPU mode)", file=sys.stderr)
        sys.exit(2)

    import torch
    import dsa_indexer_top_amd as dsa
    from dsa_inputs import host_bits, make_indexer_inputs
    dsa.load()
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.randint(0, 255, (n,), dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        assert torch.equal(dst, src)
        print(json.dumps({"copy_bytes": n, "copies": 3}), flush=True)
        return
    L, H, D, topk = args.L, 64, 128, 2048
    if args.only == "stack":
        print(json.dumps(stack_bench(dsa, torch, args.stack_L, args.stack_layers, topk,
                                     max(1, args.steps // 2), 1)), flush=True)
        return
    if args.only == "quant":
        print(json.dumps(quant_bench(dsa, torch, L, max(2, args.steps))), flush=True)
        return
    if args.only == "stack200k":
        print(json.dumps(stack200k(dsa, torch, L, topk, args)), flush=True)
        return
    if args.only == "decode":
        res = {f"decode_B{B}": decode_bench(dsa, torch, B, 200000, 47, topk, args.steps, 2) for B in (1, 32)}
        res["decode_attn_B256"] = decode_gather_bench(dsa, torch, 256, 200000, topk, max(3, args.steps), 2)
        print(json.dumps(res), flush=True)
        return
    if args.only == "peaks":
        print(json.dumps(measured_peaks(torch)), flush=True)
        return
    if args.only == "c2":
        print(json.dumps(c2_bench(dsa, torch, max(5, args.steps), args.warmup)), flush=True)
        return
    if args.only == "overlap":
        print(json.dumps(overlap_bench(dsa, torch, max(2, args.steps))), flush=True)
        return
    if args.only == "paged":
        print(json.dumps(paged_decode_bench(dsa, torch, 32, 200000, 47, topk, args.steps, 2)), flush=True)
        return

    peaks = None
    if not (args.no_extra or args.quick):
        peaks = measured_peaks(torch)
    log(f"generating the L={L} {args.dtype} layer")
    inp = make_indexer_inputs(1, L, L, H, D, config=5, dtype=args.dtype, w_std=0.125, device="cuda")
    torch.cuda.synchronize()
    log("timing the headline")
    wall_ms, k_ms, s_ms, _ = time_indexer(dsa, torch, inp, topk, args.steps, args.warmup)
    flops = causal_flops(L, H, D)
    achieved = flops / (k_ms * 1e-3) / 1e12
    log(f"headline: {wall_ms:.2f} ms/step, score kernel {k_ms:.2f} ms ({achieved:.1f} TFLOP/s), "
        f"select {s_ms:.2f} ms")
    result = {
        "metric": METRIC,
        "value": L / (wall_ms * 1e-3),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": args.dtype,
        "data": "synthetic: seeded N(0,1) q_idx/k_idx"
                + (" clipped to +-8 and cast to e4m3 with per-token fp32 scales U[0.5,2)"
                   if args.dtype == "fp8" else " in bf16") + ", w ~ N(0,1)/8",
        "config": {"workload": f"single-layer prefill indexer + exact top-k, L={L}, H_I={H}, d_I={D}, "
                               f"k={topk}, causal, {args.dtype}",
                   "L": L, "H_I": H, "d_I": D, "topk": topk},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_TFLOPS[args.dtype],
                     "unit": "TFLOP/s", "frac": achieved / PEAK_TFLOPS[args.dtype],
                     "traffic": traffic_for_current_kernel() if (args.dtype == "fp8" and L == 200000)
                     else None,
                     "kernel": "indexer_prefill_kernel", "kernel_ms": k_ms,
                     "flop_per_launch": flops,
                     "peak_measured": peaks[f"mfma_{args.dtype}_TFLOPs"] if peaks else None,
                     "frac_of_measured": achieved / peaks[f"mfma_{args.dtype}_TFLOPs"] if peaks else None},
        "select_kernel_ms": s_ms,
    }
    if not args.no_cpu:
        log("CPU oracle baseline")
        hb = (host_bits(inp.q[:, :]), host_bits(inp.k), host_bits(inp.w), host_bits(inp.q_scale),
              host_bits(inp.k_scale), inp.dtype)
        result["cpu_baseline"] = cpu_baseline(hb, L, topk, args.cpu_seconds)
    del inp
    torch.cuda.empty_cache()

    if not (args.no_extra or args.quick):
        extra = {"measured_peaks": peaks}
        log("L=10240 bf16 layer")
        extra["C2_L10240_bf16"] = c2_bench(dsa, torch, max(10, 2 * args.steps), args.warmup, peaks)
        if not args.no_cpu:
            extra["cpu_oracle_L10240_bf16_full"] = cpu_c2_full()
        other = "bf16" if args.dtype == "fp8" else "fp8"
        log(f"generating the L={L} {other} layer")
        inp2 = make_indexer_inputs(1, L, L, H, D, config=5, dtype=other, w_std=0.125, device="cuda")
        w2, k2, s2, _ = time_indexer(dsa, torch, inp2, topk, max(2, args.steps // 2), 1)
        a2 = flops / (k2 * 1e-3) / 1e12
        st2 = flops / (w2 * 1e-3) / 1e12
        extra[f"{other}_L{L}"] = {"ms_per_step": w2, "queries_per_s": L / (w2 * 1e-3),
                                  "score_kernel_ms": k2, "select_kernel_ms": s2,
                                  "TFLOPs": a2, "mfma_frac": a2 / PEAK_TFLOPS[other],
                                  "step_mfma_frac": st2 / PEAK_TFLOPS[other],
                                  "mfma_frac_of_measured": a2 / peaks[f"mfma_{other}_TFLOPs"],
                                  "step_mfma_frac_of_measured": st2 / peaks[f"mfma_{other}_TFLOPs"],
                                  "frac_of_bf16_peak": a2 / PEAK_TFLOPS["bf16"]}
        log(f"{other}: {w2:.2f} ms/step, kernel {k2:.2f} ms ({a2:.1f} TFLOP/s)")
        del inp2
        torch.cuda.empty_cache()
        log(f"stack prefill L={args.stack_L}, {args.stack_layers} layers")
        extra["stack_prefill"] = {"L": args.stack_L, "layers": args.stack_layers, "dtype": "bf16",
                                  "attn": "16 heads, d=128, 1 KV head",
                                  **stack_bench(dsa, torch, args.stack_L, args.stack_layers, topk,
                                                max(1, args.steps // 2), 1)}
        extra["quantize_fp8_q_idx"] = quant_bench(dsa, torch, L, max(2, args.steps))
        log(f"quantize q_idx: {extra['quantize_fp8_q_idx']['ms']:.3f} ms "
            f"({extra['quantize_fp8_q_idx']['hbm_GBps']:.0f} GB/s)")
        log(f"stack prefill L={L}, 47 layers, fp8 indexer")
        extra["stack_prefill_200k"] = stack200k(dsa, torch, L, topk, args)
        for B in (1, 32):
            log(f"decode B={B}")
            extra[f"decode_B{B}"] = decode_bench(dsa, torch, B, 200000, 47, topk, args.steps, 2)
        extra["decode_attn_B256"] = decode_gather_bench(dsa, torch, 256, 200000, topk, max(3, args.steps), 2)
        log("paged ragged decode B=32")
        extra["decode_paged_ragged_B32"] = paged_decode_bench(dsa, torch, 32, 200000, 47, topk, args.steps, 2)
        extra["topk_overlap_47_layers"] = overlap_bench(dsa, torch, max(2, args.steps))
        # HBM-bound figures against the rates measured on this GPU as well
        rd, cp = peaks["hbm_read_GBps"], peaks["hbm_copy_GBps"]
        for key in ("decode_B1", "decode_B32"):
            for part in (extra[key], extra[key]["cold"]):
                part["indexer_frac_of_measured_read"] = part["indexer_hbm_GBps"] / rd
                part["attn_gather_frac_of_measured_read"] = part["attn_gather_GBps"] / rd
        for part in (extra["decode_attn_B256"], extra["decode_attn_B256"]["cold"]):
            part["attn_gather_frac_of_measured_read"] = part["attn_gather_GBps"] / rd
        extra["quantize_fp8_q_idx"]["frac_of_measured_copy"] = extra["quantize_fp8_q_idx"]["hbm_GBps"] / cp
        # an S layer is the sparse attention alone: its gathered K and V rows
        # (min(t + 1, k) of 256 bytes each per query row) against the row-gather
        # probe over a table of the same size
        for key, pat, tokens in (("stack_prefill", "freq4", args.stack_L),
                                 ("stack_prefill_200k", "seeded_quarter_F", L)):
            s_ms = extra[key][pat]["mean_S_layer_ms"]
            entries = topk * (tokens - topk) + topk * (topk + 1) // 2 if tokens >= topk else tokens * (tokens + 1) // 2
            rate = entries * 2 * 256 / s_ms / 1e6
            probe = peaks["gather_GBps"].get(f"kv_{tokens}_tokens")
            extra[key]["S_layer_gather_GBps"] = rate
            extra[key]["S_layer_gather_frac_of_measured_gather"] = rate / probe if probe else None
        result["extra"] = extra
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
