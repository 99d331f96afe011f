"""Benchmark of the DSA hot path on one MI355X.

One step = one pass of the hot path over the 4K-token prefill workload
(one causal sequence T=4096, bf16): lightning-indexer scores -> per-row top-k
(index_topk 2048) -> sparse MLA (128 heads, d_qk 576, d_v 512).  The indexer
operands are prepared once (key LayerNorm + RoPE + bf16) by the library's prep
kernel before timing; all inputs are seeded synthetic data resident in HBM.

Printed: ONE JSON line.  ``value`` is the step throughput in indexer q.k pairs
per second (valid causal (t, s) pairs / step time); ``components`` holds the
three per-stage rates of the metric, each timed with HIP events around its own
launches on the launch stream; ``roofline`` is for the dominant kernel;
``cpu_baseline`` is the float64 CPU oracle timed on a row sample of the same
workload on this host.

``roofline.onbox`` holds what plain library work reaches on the same box (a bf16
GEMM through torch.matmul and a device copy), so that the kernel's fraction can
be read against the box as well as against the published peak.

    python bench.py [--gpus 1] [--steps 300] [--warmup 20] [--no-cpu]
"""
from __future__ import annotations

import argparse
import dataclasses
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
FP8_PEAK_TFLOPS = 5000.0
FP4_PEAK_TFLOPS = 10100.0
MLA_FLOP_PER_PAIR = 2 * 128 * (576 + 512)   # 278,528


KERNEL_SOURCES = {                      # kernel -> the sources its code is built from
    "mla_bf16_kernel": ["mla.hip", "dsa_device.h"],
    "indexer_rows_kernel": ["indexer.hip", "indexer_core.h", "dsa_device.h"],
    "topk_rows_kernel": ["topk.hip", "topk_select.h", "dsa_device.h"],
}


def kernel_source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "sparse_attention_08_amd", "csrc")
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile(kernel: str):
    """HBM bytes per launch from the committed counter summary, or None when the
    kernel's sources changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "counters_prefill4k.json")
    try:
        with open(path) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    k = d.get("kernels", {}).get(kernel)
    if k is None or k.get("source_hash") != kernel_source_hash(kernel):
        return None
    return k.get("hbm_bytes_per_launch")


def onbox_peaks(torch, np) -> dict:
    """What the box reaches with plain library work, timed like the stages (HIP
    events, median): a bf16 GEMM through torch.matmul (hipBLASLt; M=32768,
    N=K=8192, both operands K-contiguous, the fastest of the shapes and layouts
    tried on MI355X, about 1.65 PFLOP/s) and a 1 GiB device-to-device copy (read
    + write bytes).  Neither is this library's code; they calibrate the published
    peaks against this box."""
    def timed(f, reps):
        for _ in range(3):
            f()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            f()
            e1.record()
            ts.append((e0, e1))
        torch.cuda.synchronize()
        return float(np.median([x.elapsed_time(y) for x, y in ts]))
    m, n, k = 32768, 8192, 8192
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    a = torch.randn((m, k), device="cuda", generator=g).to(torch.bfloat16).contiguous()
    bt = torch.randn((n, k), device="cuda", generator=g).to(torch.bfloat16).contiguous()
    c = torch.empty((m, n), device="cuda", dtype=torch.bfloat16)
    gemm_ms = timed(lambda: torch.matmul(a, bt.t(), out=c), 10)
    del a, bt, c
    src = torch.empty(1 << 28, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    copy_ms = timed(lambda: dst.copy_(src), 10)
    nbytes = 2 * src.numel() * 4
    del src, dst
    return {"bf16_gemm_tflops": 2 * m * n * k / (gemm_ms * 1e-3) / 1e12,
            "copy_gbs": nbytes / (copy_ms * 1e-3) / 1e9,
            "how": "torch.matmul bf16 32768x8192x8192, both operands K-contiguous (median of 10), "
                   "and a 1 GiB device copy (median of 10, read + write bytes), after the timed "
                   "steps"}


def with_onbox(roof: dict, ob: dict) -> dict:
    """roofline + the fraction of what the box reaches with plain library work
    (the GEMM for an MFMA-bound kernel, the copy for an HBM-bound one)."""
    if roof["bound"] == "hbm":
        peak = ob["copy_gbs"]
    elif roof["unit"] == "TFLOP/s" and roof["peak"] == BF16_PEAK_TFLOPS:
        peak = ob["bf16_gemm_tflops"]
    else:
        peak = None   # no fp8 / fp4 library reference
    roof["onbox"] = {"peak": peak, "frac": roof["achieved"] / peak if peak else None,
                     "bf16_gemm_tflops": ob["bf16_gemm_tflops"], "copy_gbs": ob["copy_gbs"],
                     "how": ob["how"]}
    return roof


def blas_threads() -> int:
    """Threads of the BLAS numpy calls into (the oracle's matrix products)."""
    try:
        from threadpoolctl import threadpool_info
        return max([i.get("num_threads", 1) for i in threadpool_info() if i.get("user_api") == "blas"]
                   or [1])
    except Exception:
        return len(os.sched_getaffinity(0))


def cpu_baseline(host_inputs, seconds: float = 12.0, threads: int | None = None):
    """Oracle (float64 numpy) over a row sample of the same workload (the same
    seeded inputs the GPU run uses): indexer scores of each sampled row, its
    top-k, and sparse attention over the selection.  Rate in the unit of
    ``value``: indexer pairs per second of oracle time.  threads: BLAS thread
    limit (None = the library default, all cores)."""
    import contextlib
    try:
        from threadpoolctl import threadpool_limits
        ctx = threadpool_limits(limits=threads, user_api="blas") if threads else contextlib.nullcontext()
    except Exception:
        ctx = contextlib.nullcontext()
    with ctx:
        return _cpu_baseline(host_inputs, seconds)


def _cpu_baseline(host_inputs, seconds):
    import numpy as np
    import synth
    from oracle import indexer as o_idx, mla as o_mla, prep as o_prep, topk as o_topk, windows as o_win
    cores = blas_threads()
    w = synth.WORKLOADS["prefill4k"]
    lay = synth.layout(w)
    rows = host_inputs["rows"]
    rs, re = o_win.row_windows(lay.cu_q, lay.cu_k)
    kv = o_prep.round_bf16(host_inputs["mla_kv"])
    pk = o_prep.prepare_indexer_inputs(np.zeros((1, w.n_heads, w.head_dim)), host_inputs["k_raw"],
                                       np.zeros((1, w.n_heads)), np.zeros(1), lay.key_positions(),
                                       "bf16", w.rope_dim, w.rope_main_dim, w.rope_theta)
    t0 = time.perf_counter()
    pairs = 0
    done = 0
    for i, t in enumerate(rows):
        t = int(t)
        pq = o_prep.prepare_indexer_inputs(host_inputs["q_raw"][i:i + 1], pk["k"][:1],
                                           host_inputs["w"][i:i + 1], np.array([t]), np.zeros(1),
                                           "bf16", w.rope_dim, w.rope_main_dim, w.rope_theta)
        a, b = int(rs[t]), int(re[t])
        s = o_idx.score_row(pq["q"][0], pk["k"][a:b], pq["w"][0])
        full = np.full(lay.n_k, -np.inf, np.float32)
        full[a:b] = s
        idx = o_topk.topk_row(full, a, b, w.index_topk)
        o_mla.attend_row(o_prep.round_bf16(host_inputs["mla_q"][i]), kv, idx, w.sm_scale, w.d_v)
        pairs += b - a
        done += 1
        if time.perf_counter() - t0 > seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": pairs / dt, "unit": "indexer pairs/s", "cores": int(cores), "kind": "oracle",
            "blas_threads": int(cores),
            "sample": f"{done} of {lay.n_q} query rows in a seeded random order (stopped after "
                      f"{seconds:.0f} s or all rows), each through indexer scores, top-k and sparse "
                      f"MLA in float64: {pairs} indexer pairs in {dt:.1f} s"}


def stage_cpu_baseline(w, lay, inp, fp8_kv: bool, seconds: float = 10.0, wall_s: float = 60.0):
    """Oracle (float64) on a seeded random sample of the workload's query rows:
    per row, query prep, indexer scores over its window, top-k and sparse MLA
    over the selection.  Key prep (and the fp8 latent quantisation) is done once
    per key in the pipeline, so it runs outside the timed part (each key once,
    cached in chunks), as do the device-to-host copies of the row's operands.
    Stops after ``seconds`` of oracle time or ``wall_s`` in all.  Rate: indexer
    pairs per second of oracle time; ``full_workload_s`` extrapolates it by
    pair count."""
    import numpy as np
    import torch
    from oracle import indexer as o_idx, mla as o_mla, prep as o_prep, topk as o_topk, windows as o_win
    rs, re = o_win.row_windows(lay.cu_q, lay.cu_k)
    pos_q, pos_k = lay.positions(), lay.key_positions()
    H, D, C = w.n_heads, w.head_dim, 4096
    chunks = {}

    def keys(a, b):
        """prepared keys [a, b) (codes / values and scales), prepared once per chunk"""
        for c in range(a // C, (b - 1) // C + 1):
            if c not in chunks:
                lo, hi = c * C, min(c * C + C, lay.n_k)
                pk = o_prep.prepare_indexer_inputs(
                    np.zeros((1, H, D)), inp["k_raw"][lo:hi].double().cpu().numpy(),
                    np.zeros((1, H)), np.zeros(1), pos_k[lo:hi], w.dtype, w.rope_dim,
                    w.rope_main_dim, w.rope_theta)
                chunks[c] = (pk["k"], pk["k_scale"])
        ks = [chunks[c] for c in range(a // C, (b - 1) // C + 1)]
        k = np.concatenate([x[0] for x in ks])[a - (a // C) * C:][:b - a]
        sc = None if ks[0][1] is None else np.concatenate([x[1] for x in ks])[a - (a // C) * C:][:b - a]
        return k, sc

    order = np.random.default_rng(7).permutation(lay.n_q)
    t_or, pairs, done = 0.0, 0, 0
    wall0 = time.perf_counter()
    for t in order:
        t = int(t)
        a, b = int(rs[t]), int(re[t])
        if b <= a:
            continue
        q_raw = inp["q_raw"][t:t + 1].double().cpu().numpy()
        wt = inp["w"][t:t + 1].double().cpu().numpy()
        k, k_scale = keys(a, b)
        t0 = time.perf_counter()
        pq = o_prep.prepare_indexer_inputs(q_raw, k[:1], wt, np.array([pos_q[t]]), np.zeros(1),
                                           w.dtype, w.rope_dim, w.rope_main_dim, w.rope_theta)
        sc = o_idx.score_row(pq["q"][0], k, pq["w"][0], k_scale)
        full = np.full(lay.n_k, -np.inf, np.float32)
        full[a:b] = sc
        idx = o_topk.topk_row(full, a, b, w.index_topk)
        t_or += time.perf_counter() - t0
        sel = idx[idx >= 0]
        kv = o_prep.round_bf16(inp["mla_kv"][torch.from_numpy(sel).to(inp["mla_kv"].device)]
                               .double().cpu().numpy())
        if fp8_kv:
            kv = o_prep.dequant_mla_kv(*o_prep.mla_kv_quant(kv))
        mq = o_prep.round_bf16(inp["mla_q"][t].double().cpu().numpy())
        t0 = time.perf_counter()
        o_mla.attend_row(mq, kv, np.arange(sel.size), w.sm_scale, w.d_v)
        t_or += time.perf_counter() - t0
        pairs += b - a
        done += 1
        if t_or > seconds or time.perf_counter() - wall0 > wall_s:
            break
    total = int(np.maximum(np.asarray(re, np.int64) - np.asarray(rs, np.int64), 0).sum())
    rate = pairs / t_or
    return {"value": rate, "unit": "indexer pairs/s", "cores": blas_threads(), "kind": "oracle",
            "blas_threads": blas_threads(), "full_workload_s": total / rate,
            "sample": f"{done} of {lay.n_q} query rows in a seeded random order, each through query "
                      f"prep, indexer scores, top-k and sparse MLA in float64 ({pairs} of {total} "
                      f"indexer pairs, {t_or:.1f} s of oracle time)"}


def stage_bench(args, dsa, synth, np, torch):
    """Each stage of the path timed on its own on one of the other workloads (THD
    varlen prefill, decode, fp8 64K prefill).  HBM-bound stages (all of decode,
    and every standalone top-k) get a 1 GiB read between repetitions so that
    their inputs are not served from the 256 MB last-level cache.  Each stage is
    repeated at least --steps times and until --min-time seconds have passed;
    the median is reported, with p10 / p90 in components["stage_ms_stats"]."""
    dev = "cuda"
    fp8_cache = args.workload == "decode_fp8"
    mx = args.workload == "mxfp4_64k"
    base = "decode" if fp8_cache else ("fp8_64k" if mx else args.workload.replace("_stages", ""))
    w = synth.WORKLOADS[base]
    if mx:  # the 64K prefill with MXFP4 indexer operands (no index rope)
        w = dataclasses.replace(w, dtype="mxfp4")
    lay = synth.layout(w)
    i32 = lambda x: torch.from_numpy(np.asarray(x, np.int32)).to(dev)
    inp = synth.device_inputs(w, dev, lay)
    tdt = {"bf16": torch.bfloat16, "fp8": torch.float8_e4m3fn, "mxfp4": "mxfp4"}[w.dtype]
    rs, re = dsa.dsa_row_windows(i32(lay.cu_q), i32(lay.cu_k), lay.n_q)
    insert_ms = None
    if fp8_cache:
        # the index-key cache in e4m3 + power-of-two scales, written by the fused
        # norm -> quant -> insert from the bf16 key projections (timed once)
        w = dataclasses.replace(w, dtype="fp8")
        k_in = inp["k_raw"].to(torch.bfloat16)
        slots = torch.arange(lay.n_k, dtype=torch.int64, device=dev)
        k = torch.empty((lay.n_k, w.head_dim), dtype=torch.float8_e4m3fn, device=dev)
        ks = torch.empty(lay.n_k, dtype=torch.float32, device=dev)
        dsa.dsa_indexer_k_insert(k_in, slots, k, ks)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dsa.dsa_indexer_k_insert(k_in, slots, k, ks)
        e1.record()
        torch.cuda.synchronize()
        insert_ms = e0.elapsed_time(e1)
        del k_in
        q, _, wt, _ = dsa.dsa_indexer_prep(inp["q_raw"], None, inp["w"], out_dtype=torch.float8_e4m3fn)
    else:
        q, k, wt, ks = dsa.dsa_indexer_prep(inp["q_raw"], inp["k_raw"], inp["w"],
                                            i32(lay.positions()), i32(lay.key_positions()), tdt,
                                            w.rope_dim, w.rope_main_dim, w.rope_theta)
    mq = inp["mla_q"].to(torch.bfloat16)
    mkv = inp["mla_kv"].to(torch.bfloat16)
    inp_w_nonneg = (inp["w"] >= 0).all(dim=1).cpu().numpy()
    cpu_inp = None if args.no_cpu else {n: inp[n] for n in ("q_raw", "k_raw", "w", "mla_q", "mla_kv")}
    del inp
    mla_insert_ms, mcache = None, None
    if fp8_cache:
        # the latent cache in fp8 (656-byte rows), written from the bf16 rows (timed once)
        slots = torch.arange(lay.n_k, dtype=torch.int64, device=dev)
        mcache = torch.empty((lay.n_k, dsa.MLA_FP8_ROW_BYTES), dtype=torch.uint8, device=dev)
        dsa.dsa_mla_kv_insert(mkv, slots, mcache)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        dsa.dsa_mla_kv_insert(mkv, slots, mcache)
        e1.record()
        torch.cuda.synchronize()
        mla_insert_ms = e0.elapsed_time(e1)
        del slots
    K = w.index_topk
    scores = torch.full((lay.n_q, lay.n_k), float("-inf"), dtype=torch.float32, device=dev)
    idx = torch.empty((lay.n_q, K), dtype=torch.int32, device=dev)
    out = torch.empty((lay.n_q, w.mla_heads, w.d_v), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((lay.n_q, w.mla_heads), dtype=torch.float32, device=dev)
    ws = torch.empty(max(dsa.sparse_mla_workspace(lay.n_q, w.mla_heads, w.d_qk, w.d_v, K, 1), 1),
                     dtype=torch.uint8, device=dev)
    # Cache flush for the HBM-bound stages: a 1 GiB read.  A write would leave up to
    # the size of the last-level cache in dirty lines, whose write-back would then
    # run inside the timed region and halve the bandwidth the stage sees.
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    flush.sum()
    torch.cuda.synchronize()
    hbm_bound = {"indexer": w.decode, "topk": True, "mla": w.decode}
    fns = {
        "indexer": lambda: dsa.dsa_indexer_scores(q, k, wt, rs, re, k_scale=ks, scores=scores),
        "topk": lambda: dsa.dsa_topk(scores, rs, re, K, out=idx),
        "mla": lambda: dsa.dsa_sparse_mla_fwd(mq, mkv if mcache is None else mcache, idx,
                                              w.sm_scale, w.d_v, out=out, lse=lse, workspace=ws),
    }
    if mcache is not None:   # the same attention over the bf16 rows, for comparison
        out_b = torch.empty_like(out)
        fns["mla_bf16_kv"] = lambda: dsa.dsa_sparse_mla_fwd(mq, mkv, idx, w.sm_scale, w.d_v,
                                                            out=out_b, lse=lse, workspace=ws)
        hbm_bound["mla_bf16_kv"] = True
    fused = True                     # the fused indexer + top-k: decode and prefill kernels
    if fused:
        idx2 = torch.empty_like(idx)
        code = {"bf16": 1, "fp8": 2, "mxfp4": 3}[w.dtype]
        fws = torch.empty(max(dsa.indexer_topk_workspace(lay.n_q, lay.n_k, w.n_heads, w.head_dim,
                                                         code, K), 1), dtype=torch.uint8, device=dev)
        fns["indexer_topk"] = lambda: dsa.dsa_indexer_topk(q, k, wt, rs, re, K, k_scale=ks, out=idx2,
                                                           workspace=fws)
        hbm_bound["indexer_topk"] = w.decode
    ms, ms_stats = {}, {}
    for name in fns:
        f = fns[name]
        for _ in range(args.warmup):
            f()
        torch.cuda.synchronize()
        times = []
        t_start = time.perf_counter()
        while True:
            for _ in range(args.steps):
                if hbm_bound[name]:
                    flush.sum()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                f()
                e1.record()
                times.append((e0, e1))
            torch.cuda.synchronize()
            if time.perf_counter() - t_start >= args.min_time or len(times) >= 4000:
                break
        v = [a.elapsed_time(b) for a, b in times]
        ms[name] = float(np.median(v))
        ms_stats[name] = {"median": round(ms[name], 5), "p10": round(float(np.percentile(v, 10)), 5),
                          "p90": round(float(np.percentile(v, 90)), 5), "reps": len(v)}
    rs_h, re_h = rs.cpu().numpy().astype(np.int64), re.cpu().numpy().astype(np.int64)
    pairs = int((re_h - rs_h).sum())
    sel = int((idx >= 0).sum().item())
    hd = w.n_heads * w.head_dim
    elt = {"bf16": 2.0, "fp8": 1.0, "mxfp4": 0.5 + 1 / 32}[w.dtype]   # bytes per element (+ scales)
    idx_flop = pairs * 2 * hd
    key_bytes = int(lay.n_k * (w.head_dim * elt + (4 if w.dtype == "fp8" else 0)))  # codes + scale
    idx_bytes = int(lay.n_q * hd * elt) + key_bytes + lay.n_q * w.n_heads * 4 + pairs * 4
    topk_bytes = pairs * 4 + lay.n_q * K * 4
    mla_flop = sel * MLA_FLOP_PER_PAIR
    row_bytes = dsa.MLA_FP8_ROW_BYTES if mcache is not None else w.d_qk * 2
    gather = sel * row_bytes
    mla_compulsory = mq.numel() * 2 + out.numel() * 2 + lse.numel() * 4 + idx.numel() * 4
    mfma_peak = {"bf16": BF16_PEAK_TFLOPS, "fp8": FP8_PEAK_TFLOPS, "mxfp4": FP4_PEAK_TFLOPS}[w.dtype]
    t = {n: v * 1e-3 for n, v in ms.items()}
    if fused:
        assert torch.equal(idx, idx2), "fused and unfused indexer + top-k disagree"
    comp = {
        "indexer": {"ms": ms["indexer"], "pairs_per_s": pairs / t["indexer"],
                    "tflops": idx_flop / t["indexer"] / 1e12,
                    "frac_mfma_peak": idx_flop / t["indexer"] / 1e12 / mfma_peak,
                    "gbs": idx_bytes / t["indexer"] / 1e9,
                    "frac_hbm": idx_bytes / t["indexer"] / 1e9 / HBM_PEAK_GBS},
        "topk": {"ms": ms["topk"], "rows_per_s": lay.n_q / t["topk"],
                 "gbs": topk_bytes / t["topk"] / 1e9,
                 "frac_hbm": topk_bytes / t["topk"] / 1e9 / HBM_PEAK_GBS},
        "mla": {"ms": ms["mla"], "tflops": mla_flop / t["mla"] / 1e12,
                "frac_bf16_peak": mla_flop / t["mla"] / 1e12 / BF16_PEAK_TFLOPS,
                "gather_gbs": (gather + mla_compulsory) / t["mla"] / 1e9,
                "frac_hbm": (gather + mla_compulsory) / t["mla"] / 1e9 / HBM_PEAK_GBS},
    }
    comp["stage_ms_stats"] = ms_stats   # per stage: median, p10, p90 (ms) and repetitions
    if mcache is not None:
        gb = sel * w.d_qk * 2
        comp["mla"]["kv_row_bytes"] = row_bytes
        comp["mla_bf16_kv"] = {"ms": ms["mla_bf16_kv"], "kv_row_bytes": w.d_qk * 2,
                               "gather_gbs": (gb + mla_compulsory) / t["mla_bf16_kv"] / 1e9,
                               "fp8_speedup": ms["mla_bf16_kv"] / ms["mla"]}
        mb = lay.n_k * (w.d_qk * 2 + 8 + row_bytes)          # bf16 rows + slot in, fp8 rows out
        comp["mla_kv_insert"] = {"ms": mla_insert_ms, "rows_per_s": lay.n_k / (mla_insert_ms * 1e-3),
                                 "gbs": mb / (mla_insert_ms * 1e-3) / 1e9,
                                 "frac_hbm": mb / (mla_insert_ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    if insert_ms is not None:
        ib = lay.n_k * (w.head_dim * 2 + 8 + w.head_dim + 4)  # bf16 keys + slot in, codes + scale out
        comp["k_insert"] = {"ms": insert_ms, "keys_per_s": lay.n_k / (insert_ms * 1e-3),
                            "gbs": ib / (insert_ms * 1e-3) / 1e9,
                            "frac_hbm": ib / (insert_ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
    if fused:
        fb = idx_bytes - pairs * 4 + lay.n_q * K * 4       # q + k + w read, indices written
        # rows the fused kernels write without scoring: windows of at most k keys
        # with no negative head weight (the prefill kernel skips a block of four
        # rows only when all four are such rows)
        wn = np.asarray(inp_w_nonneg)
        whole = ((re_h - rs_h) <= K) & wn
        if lay.n_q > 256:
            nb = (lay.n_q + 3) // 4
            pad = np.ones(nb * 4, bool)
            pad[:lay.n_q] = whole
            whole = np.repeat(pad.reshape(nb, 4).all(axis=1), 4)[:lay.n_q]
        scored = pairs - int((re_h - rs_h)[whole].sum())
        comp["indexer_topk_fused"] = {"ms": ms["indexer_topk"],
                                      "pairs_per_s": pairs / t["indexer_topk"],
                                      "pairs_scored": scored,
                                      "tflops": scored * 2 * hd / t["indexer_topk"] / 1e12,
                                      "frac_mfma_peak": scored * 2 * hd / t["indexer_topk"] / 1e12 / mfma_peak,
                                      "gbs": fb / t["indexer_topk"] / 1e9,
                                      "frac_hbm": fb / t["indexer_topk"] / 1e9 / HBM_PEAK_GBS,
                                      "vs_unfused": (ms["indexer"] + ms["topk"]) / ms["indexer_topk"]}
        ms_path = {"indexer_topk": ms["indexer_topk"], "mla": ms["mla"]}
    else:
        ms_path = {"indexer": ms["indexer"], "topk": ms["topk"], "mla": ms["mla"]}
    dom = max(ms_path, key=ms_path.get)
    if dom == "indexer_topk" and w.decode:
        ach = comp["indexer_topk_fused"]["gbs"]
        roof = {"kernel": "indexer_topk_chunk_kernel", "bound": "hbm", "achieved": ach,
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS, "traffic": None}
    elif dom == "indexer_topk":
        ach = comp["indexer_topk_fused"]["tflops"]
        roof = {"kernel": "indexer_topk_rows_kernel", "bound": "mfma", "achieved": ach,
                "peak": mfma_peak, "unit": "TFLOP/s", "frac": ach / mfma_peak, "traffic": None}
    elif dom == "indexer" and not w.decode:
        ach = comp["indexer"]["tflops"]
        roof = {"kernel": "indexer_rows_kernel", "bound": "mfma", "achieved": ach, "peak": mfma_peak,
                "unit": "TFLOP/s", "frac": ach / mfma_peak, "traffic": None}
    elif dom == "indexer":
        ach = comp["indexer"]["gbs"]
        roof = {"kernel": "indexer_rowsplit_kernel", "bound": "hbm", "achieved": ach,
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS, "traffic": None}
    elif dom == "mla" and not w.decode:
        ach = comp["mla"]["tflops"]
        roof = {"kernel": "mla_bf16_kernel", "bound": "mfma", "achieved": ach,
                "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": ach / BF16_PEAK_TFLOPS,
                "traffic": None}
    elif dom == "mla":
        ach = comp["mla"]["gather_gbs"]
        roof = {"kernel": "mla_bf16_kernel" if mcache is None else "mla_fp8_kernel",
                "bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": ach / HBM_PEAK_GBS, "traffic": None}
    else:
        ach = comp["topk"]["gbs"]
        roof = {"kernel": "topk_rows_kernel", "bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": ach / HBM_PEAK_GBS, "traffic": None}
    roof = with_onbox(roof, onbox_peaks(torch, np))
    total = sum(ms_path.values())
    extra = {}
    if cpu_inp is not None:
        extra["cpu_baseline"] = stage_cpu_baseline(w, lay, cpu_inp, mcache is not None)
    res = {
        "metric": "indexer q·k pairs/s + top-k rows/s + sparse-MLA TFLOP/s (per stage)",
        "value": pairs / (total * 1e-3), "unit": "indexer pairs/s (sum of the stage medians)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": total,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": f"{args.workload}: n_q={lay.n_q} n_k={lay.n_k} index {w.n_heads}x{w.head_dim} "
                               f"{w.dtype}, index_topk {K}, sparse MLA {w.mla_heads} heads "
                               f"{w.d_qk}/{w.d_v} bf16" +
                               (" over the fp8 latent cache (656-B rows)" if mcache is not None else ""),
                   "valid_pairs": pairs, "selected_pairs": sel,
                   "parallelism": "none (1 GPU)"},
        "components": comp, "roofline": roof,
    }
    res.update(extra)
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300,
                    help="timed steps (prefill4k: about 0.5 s); per stage the minimum repetitions")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--min-time", type=float, default=0.5,
                    help="stage workloads: repeat each stage until this many seconds have passed")
    ap.add_argument("--workload", default="prefill4k",
                    choices=["prefill4k", "prefill4k_stages", "thd", "decode", "decode_fp8",
                             "fp8_64k", "mxfp4_64k"],
                    help="prefill4k: the benchmark step; the others time each stage on its own")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first run a plain 1 GiB device copy (reference for HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import sparse_attention_08_amd as dsa
    import synth

    dsa.load()
    dev = "cuda"
    if args.copy_calibration:
        src = torch.empty(1 << 28, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(2):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.workload != "prefill4k":
        print(json.dumps(stage_bench(args, dsa, synth, np, torch)), flush=True)
        return
    w = synth.WORKLOADS["prefill4k"]
    lay = synth.layout(w)
    i32 = lambda x: torch.from_numpy(np.asarray(x, np.int32)).to(dev)
    inp = synth.device_inputs(w, dev, lay)
    rs, re = dsa.dsa_row_windows(i32(lay.cu_q), i32(lay.cu_k), lay.n_q)
    q, k, wt, _ = dsa.dsa_indexer_prep(inp["q_raw"], inp["k_raw"], inp["w"], i32(lay.positions()),
                                       i32(lay.key_positions()), torch.bfloat16, w.rope_dim,
                                       w.rope_main_dim, w.rope_theta)
    mq = inp["mla_q"].to(torch.bfloat16)
    mkv = inp["mla_kv"].to(torch.bfloat16)
    host_inputs = None
    if not args.no_cpu:
        rows = np.random.default_rng(5).permutation(lay.n_q)   # seeded order, time-bounded
        rt = torch.from_numpy(rows).to(dev)
        host_inputs = {"rows": rows, "k_raw": inp["k_raw"].cpu().numpy(),
                       "mla_kv": inp["mla_kv"].cpu().numpy(),
                       "q_raw": inp["q_raw"][rt].cpu().numpy(), "w": inp["w"][rt].cpu().numpy(),
                       "mla_q": inp["mla_q"][rt].cpu().numpy()}
    del inp
    K = w.index_topk
    scores = torch.full((lay.n_q, lay.n_k), float("-inf"), dtype=torch.float32, device=dev)
    idx = torch.empty((lay.n_q, K), dtype=torch.int32, device=dev)
    out = torch.empty((lay.n_q, w.mla_heads, w.d_v), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((lay.n_q, w.mla_heads), dtype=torch.float32, device=dev)
    ws_bytes = dsa.sparse_mla_workspace(lay.n_q, w.mla_heads, w.d_qk, w.d_v, K, 1)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device=dev)

    ev = lambda: torch.cuda.Event(enable_timing=True)
    stage_ms = {"indexer": [], "topk": [], "mla": [], "step": []}

    def step(record: bool):
        e = [ev() for _ in range(4)]
        e[0].record()
        dsa.dsa_indexer_scores(q, k, wt, rs, re, scores=scores)
        e[1].record()
        dsa.dsa_topk(scores, rs, re, K, out=idx)
        e[2].record()
        dsa.dsa_sparse_mla_fwd(mq, mkv, idx, w.sm_scale, w.d_v, out=out, lse=lse, workspace=ws)
        e[3].record()
        return e if record else None

    for _ in range(args.warmup):
        step(False)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    evs = [step(True) for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    for e in evs:
        stage_ms["indexer"].append(e[0].elapsed_time(e[1]))
        stage_ms["topk"].append(e[1].elapsed_time(e[2]))
        stage_ms["mla"].append(e[2].elapsed_time(e[3]))
        stage_ms["step"].append(e[0].elapsed_time(e[3]))
    ms_step = wall * 1e3 / args.steps
    step_ev = stage_ms.pop("step")

    # the fused indexer + top-k (no score matrix), timed after the steps on the
    # same inputs and checked against the composed selection of the last step
    idx_f = torch.empty_like(idx)
    for _ in range(args.warmup):
        dsa.dsa_indexer_topk(q, k, wt, rs, re, K, out=idx_f)
    fused_ev = []
    for _ in range(args.steps):
        e0, e1 = ev(), ev()
        e0.record()
        dsa.dsa_indexer_topk(q, k, wt, rs, re, K, out=idx_f)
        e1.record()
        fused_ev.append((e0, e1))
    e0, e1 = ev(), ev()                      # and back to back, one event pair
    e0.record()
    for _ in range(args.steps):
        dsa.dsa_indexer_topk(q, k, wt, rs, re, K, out=idx_f)
    e1.record()
    torch.cuda.synchronize()
    assert torch.equal(idx_f, idx), "fused and composed indexer + top-k disagree"
    fused_ms = [a.elapsed_time(b) for a, b in fused_ev]
    fused_b2b = e0.elapsed_time(e1) / args.steps

    pairs = lay.n_q * (lay.n_q + 1) // 2                               # valid (t, s), s <= t
    mla_pairs = sum(min(t + 1, K) for t in range(lay.n_q))            # selected (t, j)
    avg = {s: float(np.mean(v)) for s, v in stage_ms.items()}
    pct = lambda v, q: round(float(np.percentile(v, q)), 4)
    stats = {s: {"mean": round(float(np.mean(v)), 4), "p10": pct(v, 10), "median": pct(v, 50),
                 "p90": pct(v, 90)} for s, v in list(stage_ms.items()) + [("step", step_ev)]}
    idx_flop = pairs * 2 * w.n_heads * w.head_dim
    mla_flop = mla_pairs * MLA_FLOP_PER_PAIR
    topk_bytes = pairs * 4 + lay.n_q * K * 4                          # valid scores read + idx written
    components = {
        "indexer_pairs_per_s": pairs / (avg["indexer"] * 1e-3),
        "indexer_tflops": idx_flop / (avg["indexer"] * 1e-3) / 1e12,
        "topk_rows_per_s": lay.n_q / (avg["topk"] * 1e-3),
        "topk_gbs": topk_bytes / (avg["topk"] * 1e-3) / 1e9,
        "sparse_mla_tflops": mla_flop / (avg["mla"] * 1e-3) / 1e12,
        "stage_ms": {s: round(v, 4) for s, v in avg.items()},
        # per-launch HIP-event times over the timed steps (ms): mean, p10, median, p90
        "stage_ms_stats": stats,
        # dsa_indexer_topk on the same inputs: the scores stay in LDS (no score
        # matrix); a row whose window holds at most k keys and whose head weights
        # are >= 0 is its whole window and is written without scoring
        "indexer_topk_fused": {
            "ms": {"mean": round(float(np.mean(fused_ms)), 4), "p10": pct(fused_ms, 10),
                   "median": pct(fused_ms, 50), "p90": pct(fused_ms, 90)},
            # a launch this short can wait on the host (its events then span the
            # wait): the medians, and the mean of launches back to back
            "back_to_back_mean": round(fused_b2b, 4),
            "composed_over_fused": (stats["indexer"]["median"] + stats["topk"]["median"]) /
                                   float(np.median(fused_ms)),
            "pairs_scored": pairs - sum(t + 1 for t in range(min(lay.n_q, K))),
            "step_ms_with_fused": float(np.median(fused_ms)) + stats["mla"]["median"],
        },
    }
    # dominant kernel of the step
    dom = max(avg, key=avg.get)
    if dom == "mla":
        ach = mla_flop / (avg["mla"] * 1e-3) / 1e12
        roof = {"kernel": "mla_bf16_kernel", "bound": "mfma", "achieved": ach,
                "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": ach / BF16_PEAK_TFLOPS,
                "traffic": traffic_from_profile("mla_bf16_kernel")}
    elif dom == "indexer":
        ach = idx_flop / (avg["indexer"] * 1e-3) / 1e12
        roof = {"kernel": "indexer_rows_kernel", "bound": "mfma", "achieved": ach,
                "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": ach / BF16_PEAK_TFLOPS,
                "traffic": traffic_from_profile("indexer_rows_kernel")}
    else:
        ach = topk_bytes / (avg["topk"] * 1e-3) / 1e9
        roof = {"kernel": "topk_rows_kernel", "bound": "hbm", "achieved": ach,
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": ach / HBM_PEAK_GBS,
                "traffic": traffic_from_profile("topk_rows_kernel")}

    line = {
        "metric": "indexer q·k pairs/s + top-k rows/s + sparse-MLA TFLOP/s (4K prefill)",
        "value": pairs / (ms_step * 1e-3),
        "unit": "indexer pairs/s (whole step: indexer + top-k + sparse MLA)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": ms_step,
        "ms_per_step_p10_median_p90": [stats["step"]["p10"], stats["step"]["median"],
                                        stats["step"]["p90"]],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "prefill4k: one causal sequence T=4096, bf16; indexer 64 heads x 128 "
                               "(RoPE on 64 dims), fp32 head weights; index_topk 2048; sparse MLA "
                               "128 heads, d_qk 576, d_v 512",
                   "global_batch": 1, "seq_len": lay.n_q, "parallelism": "none (1 GPU)"},
        "components": components,
        "roofline": with_onbox(roof, onbox_peaks(torch, np)),
    }
    if not args.no_cpu:
        # all cores (the BLAS default), then one BLAS thread on the same sample order
        line["cpu_baseline"] = cpu_baseline(host_inputs)
        line["cpu_baseline"]["one_core"] = cpu_baseline(host_inputs, threads=1)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
