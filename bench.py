#!/usr/bin/env python3
"""TurboQuant hot-path benchmark on one MI355X.

A step is one pass of the whole path over one batch of synthetic keys: quantize a whole
key cache (rotation, Lloyd-Max, residual, QJL signs, packing) and score every query head
of one decode step against all keys (query prep + quantized-key logits).

Default workload (long_context, the largest single-GPU configuration): 16 sequences x 8 KV
heads x 131072 tokens x d = 128, bf16 keys drawn N(0, 1) with 4 outlier channels per head
scaled x20, b = 3 bits (2-bit Lloyd-Max + 1-bit QJL), 32 query heads per sequence in GQA
groups of 4.  --workload decode_layer: one sequence x 8 KV heads x 32768 tokens, b = 4;
--workload decode_batch16: 16 sequences x 8 KV heads x 8192 tokens, b = 2 (--bits 3 for b = 3).

--workload embedding_search: a step quantizes 10^6 unit vectors in R^1536 (float32, low
rank + noise) and returns the top-10 of 1000 queries by the estimated inner product (flat
scan over the codes); b = 4 unless --bits says otherwise.

--workload decode_attention: one tq_attention decode step at the decode-layer shapes.
--workload fractional_kv: decode_layer's keys and queries at a fractional rate (--rate 2.5
or 3.5 bits per channel): channels 0..63 at the higher b and 64..127 at the lower one, each
group its own TurboQuant instance; a step is tq_quantize_split + the split scoring
(tq_score_split_prepare on a second stream beside the quantize, then
tq_score_ip_split_prepared), as the KV workloads split tq_score_ip.
--workload toy: 4096 float32 unit vectors in R^128 at b = 4 and all 64 x 4096 logits of 64
unit queries (latency-bound; its replicas fit the MALL, so it is reported, not held to a roofline).
--workload ubench: achievable HBM and MFMA rates of the GPU.

Prints one JSON line.  Kernel durations come from HIP events recorded on the stream the
kernels run on; every per-launch timing of the other workloads cycles through more than
512 MB of distinct inputs, so that the 256 MB MALL does not serve them from cache.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
BF16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA, TFLOP/s
FP16_MFMA_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 MFMA, TFLOP/s


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long_context",
                    choices=["long_context", "decode_layer", "decode_batch16", "embedding_search",
                             "decode_attention", "fractional_kv", "toy", "ubench"])
    ap.add_argument("--rate", type=float, default=3.5, help="fractional_kv: bits per channel (2.5 or 3.5)")
    ap.add_argument("--bits", type=int, default=0,
                    help="b of workloads defined at several (embedding_search: 4, decode_batch16: 2)")
    ap.add_argument("--replicas", type=int, default=8, help="resident input copies cycled per step")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="oracle CPU baseline budget")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy-mb", type=int, default=0,
                    help="also run one device copy of this many MiB (HBM counter calibration)")
    return ap.parse_args()


def cpu_model() -> str:
    """The host CPU's model name (from /proc/cpuinfo), for the oracle baseline's record."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def measured_copy_gbs(torch, mib: int = 1024, reps: int = 10) -> float:
    """Achievable HBM rate on this GPU: a device copy of `mib` MiB, read + write bytes."""
    a = torch.ones(mib * 1024 * 1024 // 4, dtype=torch.float32, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(2):
        b.copy_(a)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b
    return 2.0 * mib * 1024 * 1024 / (ms * 1e-3) / 1e9


def measured_gemm_tflops(torch, dtype, m: int = 8192, reps: int = 5) -> float:
    """Achievable dense MFMA rate on this GPU for dtype: a library GEMM of m x m x m."""
    x = torch.randn(m, m, device="cuda:0").to(dtype)
    y = torch.randn(m, m, device="cuda:0").to(dtype)
    for _ in range(2):
        torch.mm(x, y)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        torch.mm(x, y)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del x, y
    return 2.0 * m ** 3 / (ms * 1e-3) / 1e12


def with_measured_peak(roof: dict, measured: float, what: str) -> dict:
    """Adds the achievable rate measured in this run next to the published peak."""
    roof["measured_peak"] = measured
    roof["frac_of_measured_peak"] = roof["achieved"] / measured
    roof["measured_peak_source"] = what
    return roof


def bench_ubench(args):
    """Achievable peaks of this MI355X next to the published ones: HBM from a 2 GiB device
    copy (read + write bytes), dense bf16 / fp16 MFMA from a library GEMM (8192^3)."""
    import torch
    dev = torch.device("cuda:0")

    def median_ms(fn, reps=20):
        ts = []
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        for _ in range(reps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

    n = (2 << 30) // 4
    a = torch.ones(n, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    copy_ms = median_ms(lambda: b.copy_(a))
    copy_gbs = 2 * n * 4 / (copy_ms * 1e-3) / 1e9
    del a, b
    out = {}
    for name, dt in (("bf16", torch.bfloat16), ("fp16", torch.float16)):
        m = 8192
        x = torch.randn(m, m, device=dev).to(dt)
        y = torch.randn(m, m, device=dev).to(dt)
        ms = median_ms(lambda: torch.mm(x, y), reps=10)
        out[name] = 2.0 * m ** 3 / (ms * 1e-3) / 1e12
        del x, y
    result = {
        "metric": "achievable MI355X peaks (device copy, library GEMM), 1 MI355X",
        "value": copy_gbs, "unit": "GB/s", "n_gpus": 1, "higher_is_better": True,
        "hbm_copy_gbs": copy_gbs, "hbm_copy_frac_of_published": copy_gbs / HBM_PEAK_GBS,
        "bf16_gemm_tflops": out["bf16"], "bf16_frac_of_published": out["bf16"] / BF16_MFMA_PEAK_TFLOPS,
        "fp16_gemm_tflops": out["fp16"], "fp16_frac_of_published": out["fp16"] / FP16_MFMA_PEAK_TFLOPS,
        "note": "published: HBM 8000 GB/s, dense bf16/fp16 MFMA 2500 TFLOP/s; the rooflines of the other "
                "workloads are quoted against the published figures",
    }
    print(json.dumps(result), flush=True)


def time_per_launch(torch, fn, R: int, K: int, min_calls: int = 8) -> float:
    """Average duration (ms) of one call fn(r): M = max(R, min_calls) calls fn(i % R) are
    captured into one HIP graph (so the graph launch overhead is paid once per M calls, not
    per call) and the graph is replayed until about K calls ran, between two events on the
    current stream."""
    M = max(R, min_calls)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(M):
            fn(i % R)
    g.replay()
    torch.cuda.synchronize()
    reps = max(1, K // M)
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (reps * M)


def time_steps(torch, fn, R: int, K: int) -> float:
    """Wall-clock ms per step over exactly K steps fn(0), fn(1), ... (step i works on replica
    i % R).  The steps are replayed from HIP graphs (one node per kernel launch) so that
    Python launch overhead does not pace the GPU: one graph holds the R steps of a cycle
    through the replicas, so a graph launch is paid once per R steps; the K steps are K // R
    replays of it and one replay of a graph of the first K % R steps."""
    def capture(rs):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for r in rs:
                fn(r)
        return g

    full = capture(range(R))
    part = capture(range(K % R)) if K % R else None
    full.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(K // R):
        full.replay()
    if part is not None:
        part.replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / K


def calibration_copy(torch, dev, mib: int) -> None:
    """A device copy of known size (mib MiB each way) in the run, for scaling HBM byte counters."""
    a = torch.empty(mib * 1024 * 1024 // 4, dtype=torch.float32, device=dev)
    bb = torch.empty_like(a)
    a.fill_(1.0)
    torch.cuda.synchronize()
    bb.copy_(a)
    torch.cuda.synchronize()
    del a, bb


def source_hash(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "kv_cache_embedding_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel_files, workload: str):
    """HBM bytes per launch measured by rocprofv3 counters (profiles/traffic.json, keyed
    "<source file[+source file...]>:<workload>"), if they were taken on the current sources;
    else None."""
    files = (kernel_files,) if isinstance(kernel_files, str) else tuple(kernel_files)
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        rec = json.load(open(path)).get(f"{'+'.join(files)}:{workload}")
    except Exception:
        return None
    if not rec or rec.get("source_hash") != source_hash(*files):
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(workload, b: int, seconds: float):
    """The oracle (float64 NumPy) on a bounded sample: whole KV heads, one at a time."""
    import oracle
    from workloads import gen
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    w = workload
    d = w.d
    Pi = gen.haar_orthogonal(d, w.cfg)
    S = gen.gaussian_matrix(d, d, w.cfg)
    c, t = oracle.codebook(b - 1, d)
    chans = gen.outlier_channels(w.cfg, w.n_kv, d)
    q = gen.bf16_bits_to_f32(gen.kv_queries(w.cfg, w.n_seq, w.n_q_heads, d)).astype(np.float64)
    q = q.reshape(w.groups, w.G, d)
    groups = 0
    logits = 0
    vectors = 0
    elapsed = 0.0
    # whole (sequence, KV head) groups in cache order until the time budget is spent
    while groups < w.groups and elapsed < seconds:
        s_, h = divmod(groups, w.n_kv)
        keys = gen.bf16_bits_to_f32(gen.kv_keys_chunk(w.cfg, s_, h, w.T, d, chans[h]))
        t0 = time.perf_counter()
        r = oracle.quantize(keys.astype(np.float64), Pi, S, c, t)
        est = oracle.estimate_ip(q[groups], Pi, S, r["idx"], r["z"], r["nu"], r["gamma"], c)
        elapsed += time.perf_counter() - t0
        groups += 1
        vectors += w.T
        logits += est.size
    return {
        "value": logits / elapsed, "unit": "logits/s", "cores": int(cores), "cpu_model": cpu_model(), "kind": "oracle",
        "sample": f"{groups} of {w.groups} (sequence, KV head) groups ({vectors} keys quantized, {logits} "
                  f"logits), float64 NumPy oracle, {elapsed:.1f} s",
        "vectors_per_s": vectors / elapsed,
    }


def cpu_baseline_search(w, b, seconds: float):
    """The oracle on a bounded sample of the search workload: quantize 16384-vector blocks
    and score all queries against them, until the time budget is spent."""
    import oracle
    from workloads import gen
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    d = w.d
    rank, snr = w.lowrank
    Pi = gen.haar_orthogonal(d, w.cfg)
    S = gen.gaussian_matrix(d, d, w.cfg)
    c, t = oracle.codebook(b - 1, d)
    basis = gen.lowrank_basis(d, rank, w.cfg)
    q = gen.lowrank_queries(w.nq, d, rank, snr, cfg=w.cfg).astype(np.float64)
    blocks, vectors, pairs, elapsed = 0, 0, 0, 0.0
    # one sample per seeded block (its first 2048 vectors), while blocks remain
    while elapsed < seconds and blocks * gen.LOWRANK_BLOCK < w.n:
        x = gen.lowrank_block(blocks, d, rank, snr, w.cfg, 0, basis, n_total=w.n).astype(np.float64)
        x = x[:2048]
        t0 = time.perf_counter()
        r = oracle.quantize(x, Pi, S, c, t)
        est = oracle.estimate_ip(q, Pi, S, r["idx"], r["z"], r["nu"], r["gamma"], c)
        oracle.topk(est, w.k)
        elapsed += time.perf_counter() - t0
        blocks += 1
        vectors += x.shape[0]
        pairs += est.size
    return {
        "value": pairs / elapsed, "unit": "scores/s", "cores": int(cores), "cpu_model": cpu_model(), "kind": "oracle",
        "sample": f"{vectors} of {w.n} vectors (first 2048 of {blocks} seeded blocks) quantized and "
                  f"scored against all {w.nq} queries with top-{w.k}, float64 NumPy oracle, {elapsed:.1f} s",
        "vectors_per_s": vectors / elapsed,
    }


def search_recall(torch, x, q, idx, k: int, chunk: int = 65536) -> float:
    """Mean |returned top-k & exact top-k| / k over the queries; exact = float32 inner
    products of the unquantized vectors (library GEMM in key chunks, running top-k)."""
    nq = q.shape[0]
    best_s = torch.full((nq, k), -float("inf"), device=q.device)
    best_i = torch.zeros((nq, k), dtype=torch.int64, device=q.device)
    for c0 in range(0, x.shape[0], chunk):
        cs, ci = torch.topk(q @ x[c0:c0 + chunk].T, k, dim=1)
        alls = torch.cat([best_s, cs], 1)
        alli = torch.cat([best_i, ci + c0], 1)
        o = torch.topk(alls, k, dim=1)
        best_s, best_i = o.values, torch.gather(alli, 1, o.indices)
    ex = best_i.cpu().numpy()
    got = idx.to(torch.int64).cpu().numpy()
    return float(np.mean([len(set(ex[i]) & set(got[i])) / k for i in range(nq)]))


def bench_search(args):
    import torch

    import kv_cache_embedding_amd as tq
    from workloads import gen

    w = gen.EMBED_SEARCH
    b = args.bits or 4
    if b not in w.bits:
        raise SystemExit(f"embedding_search is defined for b in {w.bits}")
    d, n, nq, k = w.d, w.n, w.nq, w.k
    rank, snr = w.lowrank
    dev = torch.device("cuda:0")
    Pi = gen.haar_orthogonal(d, w.cfg)
    S = gen.gaussian_matrix(d, d, w.cfg)
    c, t = tq.tq_codebook_build(b - 1, d)
    params = torch.empty(tq.tq_params_bytes(d, b), dtype=torch.uint8, device=dev)
    tq.tq_prepare(d, b, Pi, S, c, t, params)
    basis = gen.lowrank_basis(d, rank, w.cfg)
    x = torch.empty((n, d), dtype=torch.float32, device=dev)
    nblk = (n + gen.LOWRANK_BLOCK - 1) // gen.LOWRANK_BLOCK
    for blk in range(nblk):
        lo = blk * gen.LOWRANK_BLOCK
        xb = gen.lowrank_block(blk, d, rank, snr, w.cfg, 0, basis, n_total=n)
        x[lo:lo + xb.shape[0]] = torch.from_numpy(xb).to(dev)
        if blk % 16 == 15:
            print(f"# generated {lo + xb.shape[0]} / {n} vectors", file=sys.stderr, flush=True)
    q = torch.from_numpy(gen.lowrank_queries(nq, d, rank, snr, cfg=w.cfg)).to(dev)
    codes = torch.empty(n * (d // 32) * b, dtype=torch.int32, device=dev)
    nu = torch.empty(n, dtype=torch.float32, device=dev)
    gamma = torch.empty(n, dtype=torch.float32, device=dev)
    idx = torch.empty(nq * k, dtype=torch.int32, device=dev)
    score = torch.empty(nq * k, dtype=torch.float32, device=dev)
    ws = torch.empty(tq.tq_topk_ws_bytes(d, b, nq, n, k), dtype=torch.uint8, device=dev)

    def quantize():
        tq.tq_quantize(params, d, b, x, codes, nu, gamma)

    def topk():
        tq.tq_topk(params, d, b, q, codes, nu, gamma, n, k, tq.TQ_EST_PROD, idx, score, ws)

    if args.calibrate_copy_mb:   # a device copy of known size, for scaling HBM byte counters
        calibration_copy(torch, dev, args.calibrate_copy_mb)

    for _ in range(max(args.warmup, 1)):
        quantize()
        topk()
    torch.cuda.synchronize()
    print("# warmup done", file=sys.stderr, flush=True)

    K = args.steps
    t0 = time.perf_counter()
    for _ in range(K):
        quantize()
        topk()
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / K

    def timed(fn):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(K):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / K

    q_ms = timed(quantize)
    t_ms = timed(topk)
    recall = search_recall(torch, x, q, idx.view(nq, k), k)
    pairs = nq * n
    q_flops = n * 4.0 * d * d                      # Pi x and S' r': 2 d^2 each
    t_flops = pairs * 3.0 * d                      # 2d (MSE dot) + d (signed QJL sum) per pair
    q_bytes = n * (d * 4 + d // 8 * b + 8)
    t_bytes = n * (d // 8 * b + 8)
    t_tflops = t_flops / (t_ms * 1e-3) / 1e12
    q_tflops = q_flops / (q_ms * 1e-3) / 1e12
    result = {
        "metric": "quantized-key scores/s of a flat top-k scan + vectors quantized/s, 1 MI355X",
        "value": pairs / (ms_step * 1e-3),
        "unit": "scores/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic (seeded low-rank + noise unit vectors, float32; random rotation and QJL matrix)",
        "config": {
            "workload": f"{w.name}: {n} x d={d} float32 unit vectors (rank {rank}, SNR {snr}), b={b}, "
                        f"{nq} queries, top-{k}",
            "n": n, "d": d, "bits": b, "queries": nq, "k": k,
        },
        "roofline": {
            "kernel": "tq_topk (query prep + fused score/select scan + merge)",
            "bound": "mfma", "achieved": t_tflops, "peak": FP16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": t_tflops / FP16_MFMA_PEAK_TFLOPS,
            "traffic": traffic_from_profiles("topk.hip", w.name),
            "note": "algorithmic 3 d flop per (query, key) pair; timed over the whole call; traffic = "
                    "counter-measured bytes per call (the codes are read once per 256-query tile)",
        },
        "roofline_quantize": {
            "kernel": "quantize_gemm (tq_quantize, d=1536)",
            "bound": "mfma", "achieved": q_tflops, "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": q_tflops / BF16_MFMA_PEAK_TFLOPS,
            "traffic": traffic_from_profiles("quantize_gemm.hip", w.name),
            "note": "algorithmic 4 d^2 flop/vector; float32 inputs execute 3 + 3 bf16 MFMA passes; "
                    "traffic = counter-measured bytes per call, including the per-chunk scratch round "
                    "trips of the bf16 split rows and the residual",
        },
        "quantize": {"ms": q_ms, "vectors_per_s": n / (q_ms * 1e-3),
                     "hbm_gbs": q_bytes / (q_ms * 1e-3) / 1e9},
        "topk": {"ms": t_ms, "scores_per_s": pairs / (t_ms * 1e-3), "hbm_gbs": t_bytes / (t_ms * 1e-3) / 1e9},
        "recall_at_k": {"value": recall, "k": k, "queries": nq,
                        "note": "mean overlap of the returned top-k with the exact top-k of the float32 "
                                "inner products (chunked library GEMM), after the timed region"},
    }
    with_measured_peak(result["roofline"], measured_gemm_tflops(torch, torch.float16),
                       "8192^3 fp16 library GEMM in this run")
    with_measured_peak(result["roofline_quantize"], measured_gemm_tflops(torch, torch.bfloat16),
                       "8192^3 bf16 library GEMM in this run")
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_search(w, b, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def cpu_baseline_attention(w, b_k, b_v, seconds: float):
    """The oracle on a bounded sample of the decode-attention workload: whole KV heads (keys
    and values quantized, logits, softmax, values aggregated), until the budget is spent."""
    import oracle
    from workloads import gen
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    d = w.d
    Pk, Sk = gen.haar_orthogonal(d, w.cfg), gen.gaussian_matrix(d, d, w.cfg)
    Pv, Sv = gen.haar_orthogonal(d, w.cfg, rep=1), gen.gaussian_matrix(d, d, w.cfg, rep=1)
    ck, tk = oracle.codebook(b_k - 1, d)
    cv, tv = oracle.codebook(b_v - 1, d)
    del Sv
    chans = gen.outlier_channels(w.cfg, w.n_kv, d)
    q = gen.bf16_bits_to_f32(gen.kv_queries(w.cfg, 1, w.n_q_heads, d)[0]).astype(np.float64)
    heads, pairs, elapsed = 0, 0, 0.0
    while heads < w.n_kv and elapsed < seconds:
        keys = gen.bf16_bits_to_f32(gen.kv_keys_chunk(w.cfg, 0, heads, w.T, d, chans[heads]))
        vals = gen.bf16_bits_to_f32(gen.kv_keys_chunk(w.cfg, w.n_seq, heads, w.T, d, chans[heads], scale=1.0))
        t0 = time.perf_counter()
        rk = oracle.quantize(keys.astype(np.float64), Pk, Sk, ck, tk)
        rv = oracle.quantize_mse(vals.astype(np.float64), Pv, cv, tv)
        qh = q[heads * w.G:(heads + 1) * w.G]
        lg = oracle.estimate_ip(qh, Pk, Sk, rk["idx"], rk["z"], rk["nu"], rk["gamma"], ck)
        vh = oracle.dequantize_mse(Pv, rv["idx"], rv["nu"], cv)
        oracle.attention_decode(lg[None], vh[None], 1.0 / np.sqrt(d))
        elapsed += time.perf_counter() - t0
        heads += 1
        pairs += lg.size
    return {
        "value": pairs / elapsed, "unit": "pairs/s", "cores": int(cores), "cpu_model": cpu_model(), "kind": "oracle",
        "sample": f"{heads} of {w.n_kv} KV heads ({heads * w.T} keys and values quantized, {pairs} "
                  f"(query head, key) pairs attended), float64 NumPy oracle, {elapsed:.1f} s",
    }


def bench_attention(args):
    """One decode step of attention over a quantized KV cache at the decode-layer shapes:
    keys b = 4 (TurboQuant-prod), values 3 index bits (TurboQuant-mse, a block prepared for
    b = 4); a step is one tq_attention call (logits, softmax, value aggregation)."""
    import torch

    import kv_cache_embedding_amd as tq
    from workloads import gen

    w = gen.DECODE_LAYER
    dev = torch.device("cuda:0")
    d, b_k, b_v = w.d, 4, 4
    groups, G, T = w.groups, w.G, w.T
    n = w.n_keys
    scale = 1.0 / float(np.sqrt(d))

    def prep(bits, rep):
        Pi = gen.haar_orthogonal(d, w.cfg, rep=rep)
        S = gen.gaussian_matrix(d, d, w.cfg, rep=rep)
        c, t = tq.tq_codebook_build(bits - 1, d)
        prm = torch.empty(tq.tq_params_bytes(d, bits), dtype=torch.uint8, device=dev)
        tq.tq_prepare(d, bits, Pi, S, c, t, prm)
        return prm

    pk, pv = prep(b_k, 0), prep(b_v, 1)
    chans = gen.outlier_channels(w.cfg, w.n_kv, d)
    keys = torch.empty((n, d), dtype=torch.bfloat16, device=dev)
    vals = torch.empty((n, d), dtype=torch.bfloat16, device=dev)
    for s in range(w.n_seq):
        for h in range(w.n_kv):
            gi = s * w.n_kv + h
            kc = gen.kv_keys_chunk(w.cfg, s, h, T, d, chans[h])
            vc = gen.kv_keys_chunk(w.cfg, w.n_seq + s, h, T, d, chans[h], scale=1.0)
            keys[gi * T:(gi + 1) * T] = torch.from_numpy(kc.view(np.int16)).to(dev).view(torch.bfloat16)
            vals[gi * T:(gi + 1) * T] = torch.from_numpy(vc.view(np.int16)).to(dev).view(torch.bfloat16)
    q = torch.from_numpy(gen.kv_queries(w.cfg, w.n_seq, w.n_q_heads, d).reshape(-1, d).view(np.int16))
    q = q.to(dev).view(torch.bfloat16)

    per_key = d // 8 * b_k + 8 + d // 8 * (b_v - 1) + 4     # key codes, nu, gamma, value codes, nu
    R = max(1, min(max(args.replicas, 12), int(2 * 1024**3 // (n * per_key))))
    ck = [torch.empty(n * (d // 32) * b_k, dtype=torch.int32, device=dev) for _ in range(R)]
    nk = [torch.empty(n, dtype=torch.float32, device=dev) for _ in range(R)]
    gk = [torch.empty(n, dtype=torch.float32, device=dev) for _ in range(R)]
    cv = [torch.empty(n * (d // 32) * (b_v - 1), dtype=torch.int32, device=dev) for _ in range(R)]
    nv = [torch.empty(n, dtype=torch.float32, device=dev) for _ in range(R)]
    for r in range(R):
        tq.tq_quantize(pk, d, b_k, keys, ck[r], nk[r], gk[r])
        tq.tq_quantize_mse(pv, d, b_v, vals, cv[r], nv[r])
    out = torch.empty(groups * G * d, dtype=torch.float32, device=dev)
    ws = torch.empty(tq.tq_attention_ws_bytes(d, b_k, groups, G, T), dtype=torch.uint8, device=dev)

    def attend(r):
        tq.tq_attention(pk, pv, d, b_k, b_v, q, ck[r], nk[r], gk[r], cv[r], nv[r], groups, G, T, scale,
                        tq.TQ_EST_PROD, out, ws)

    def vquant(r):
        tq.tq_quantize_mse(pv, d, b_v, vals, cv[r], nv[r])

    # one decode step's cache write: the newest token of every group, key and value
    k_tok = keys.view(groups, T, d)[:, T - 1, :].contiguous()
    v_tok = vals.view(groups, T, d)[:, T - 1, :].contiguous()
    ws_app = torch.empty(max(tq.tq_append_ws_bytes(d, b_k, groups), tq.tq_append_ws_bytes(d, b_v, groups)),
                         dtype=torch.uint8, device=dev)

    def append(r):
        tq.tq_append(pk, d, b_k, tq.TQ_EST_PROD, k_tok, T, T - 1, ck[r], nk[r], gk[r], ws_app)
        tq.tq_append(pv, d, b_v, tq.TQ_EST_MSE, v_tok, T, T - 1, cv[r], nv[r], None, ws_app)

    for i in range(max(args.warmup, 1)):
        attend(i % R)
    torch.cuda.synchronize()
    if args.calibrate_copy_mb:
        calibration_copy(torch, dev, args.calibrate_copy_mb)

    K = args.steps
    ms_step = time_steps(torch, attend, R, K)
    a_ms = time_per_launch(torch, attend, R, K)
    vq_ms = time_per_launch(torch, vquant, R, K)
    app_ms = time_steps(torch, append, R, K)
    pairs = groups * G * T
    a_bytes = n * per_key + groups * G * d * 4
    a_gbs = a_bytes / (a_ms * 1e-3) / 1e9
    vq_bytes = n * (d * 2 + d // 8 * (b_v - 1) + 4)
    result = {
        "metric": "decode attention over a TurboQuant KV cache: (query head, key) pairs/s "
                  "(GB/s vs HBM peak), 1 MI355X",
        "value": pairs / (ms_step * 1e-3),
        "unit": "pairs/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded N(0,1) keys with outlier channels and N(0,1) values, bf16; "
                "random rotations and QJL matrix)",
        "config": {
            "workload": f"decode_attention: {w.n_kv} KV heads x {T} tokens x d={d}, keys b={b_k} "
                        f"(prod), values {b_v - 1} index bits (mse), {w.n_q_heads} query heads "
                        f"(GQA {G}), softmax scale 1/sqrt(d)",
            "keys": n, "d": d, "key_bits": b_k, "value_index_bits": b_v - 1, "replicas": R,
        },
        "roofline": {
            "kernel": "tq_attention (query prep + fused score/softmax/value blocks + combine)",
            "bound": "hbm", "achieved": a_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": a_gbs / HBM_PEAK_GBS,
            "traffic": traffic_from_profiles(("score.hip", "score_tile.h", "attention.hip"), "decode_attention"),
            "note": f"algorithmic bytes per key: {d // 8 * b_k} B key codes + 8 B nu, gamma + "
                    f"{d // 8 * (b_v - 1)} B value codes + 4 B nu; the block partials in the "
                    "workspace are implementation traffic; timed over the whole call; traffic = "
                    "counter-measured bytes per call (query prep + block kernel + combine)",
        },
        "value_quantize": {"ms": vq_ms, "vectors_per_s": n / (vq_ms * 1e-3),
                           "hbm_gbs": vq_bytes / (vq_ms * 1e-3) / 1e9},
        "append": {"us": app_ms * 1e3,
                   "note": f"tq_append of one token per group ({groups} groups): key (prod) + value "
                           "(mse), as one decode step writes them"},
    }
    with_measured_peak(result["roofline"], measured_copy_gbs(torch), "1 GiB device copy in this run (read + write bytes)")
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_attention(w, b_k, b_v, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def cpu_baseline_fractional(w, b0, b1, seconds: float):
    """The oracle's split quantize + split estimate on whole KV heads, one at a time."""
    import oracle
    from workloads import gen
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        cores = os.cpu_count() or 1
    d, d0 = w.d, w.d // 2
    gdefs = []
    for k, (off, wd, b) in enumerate(((0, d0, b0), (d0, d - d0, b1))):
        c, t = oracle.codebook(b - 1, wd)
        gdefs.append({"off": off, "width": wd, "Pi": gen.haar_orthogonal(wd, w.cfg + k),
                      "S": gen.gaussian_matrix(wd, wd, w.cfg + k), "centroids": c, "thresholds": t})
    chans = gen.outlier_channels(w.cfg, w.n_kv, d)
    q = gen.bf16_bits_to_f32(gen.kv_queries(w.cfg, 1, w.n_q_heads, d)[0]).astype(np.float64)
    heads = logits = vectors = 0
    elapsed = 0.0
    while heads < w.n_kv and elapsed < seconds:
        keys = gen.bf16_bits_to_f32(gen.kv_keys_chunk(w.cfg, 0, heads, w.T, d, chans[heads]))
        t0 = time.perf_counter()
        codes = oracle.quantize_split(keys.astype(np.float64), gdefs)
        est = oracle.estimate_ip_split(q[heads * w.G:(heads + 1) * w.G], gdefs, codes)
        elapsed += time.perf_counter() - t0
        heads += 1
        vectors += w.T
        logits += est.size
    return {
        "value": logits / elapsed, "unit": "logits/s", "cores": int(cores), "cpu_model": cpu_model(), "kind": "oracle",
        "sample": f"{heads} of {w.n_kv} KV heads ({vectors} keys quantized, {logits} logits), "
                  f"float64 NumPy oracle, {elapsed:.1f} s",
    }


def bench_fractional(args):
    import torch

    import kv_cache_embedding_amd as tq
    from workloads import gen

    if args.rate not in (2.5, 3.5):
        print("--rate must be 2.5 or 3.5", file=sys.stderr)
        sys.exit(2)
    w = gen.DECODE_LAYER
    dev = torch.device("cuda:0")
    d, d0 = w.d, w.d // 2
    b0, b1 = int(args.rate + 0.5), int(args.rate - 0.5)
    groups, G, T = w.groups, w.G, w.T
    n = w.n_keys
    params = []
    for k, (wd, b) in enumerate(((d0, b0), (d - d0, b1))):
        c, t = tq.tq_codebook_build(b - 1, wd)
        p = torch.empty(tq.tq_params_bytes(wd, b), dtype=torch.uint8, device=dev)
        tq.tq_prepare(wd, b, gen.haar_orthogonal(wd, w.cfg + k), gen.gaussian_matrix(wd, wd, w.cfg + k),
                      c, t, p)
        params.append(p)
    chans = gen.outlier_channels(w.cfg, w.n_kv, d)
    x = torch.empty((n, d), dtype=torch.bfloat16, device=dev)
    for s in range(w.n_seq):
        for h in range(w.n_kv):
            gi = s * w.n_kv + h
            chunk = gen.kv_keys_chunk(w.cfg, s, h, T, d, chans[h])
            x[gi * T:(gi + 1) * T] = torch.from_numpy(chunk.view(np.int16)).to(dev).view(torch.bfloat16)
    q = torch.from_numpy(gen.kv_queries(w.cfg, w.n_seq, w.n_q_heads, d).reshape(-1, d).view(np.int16))
    q = q.to(dev).view(torch.bfloat16)

    R = max(1, min(args.replicas, int(2 * 1024**3 // (n * d * 2))))
    xs = [x] + [x.clone() for _ in range(R - 1)]

    def group_bufs(wd, b):
        return ([torch.empty(n * (wd // 32) * b, dtype=torch.int32, device=dev) for _ in range(R)],
                [torch.empty(n, dtype=torch.float32, device=dev) for _ in range(R)],
                [torch.empty(n, dtype=torch.float32, device=dev) for _ in range(R)])
    g0 = group_bufs(d0, b0)
    g1 = group_bufs(d - d0, b1)
    logits = [torch.empty(groups * G * T, dtype=torch.float32, device=dev) for _ in range(R)]
    ws = torch.empty(tq.tq_score_split_ws_bytes(d, d0, b0, b1, groups, G, T), dtype=torch.uint8, device=dev)

    def quantize(r):
        tq.tq_quantize_split(params[0], params[1], d, d0, b0, b1, xs[r], g0[0][r], g0[1][r], g0[2][r],
                             g1[0][r], g1[1][r], g1[2][r])

    def score(r):       # the whole scoring call: both groups' query prep + one scan
        tq.tq_score_ip_split(params[0], params[1], d, d0, b0, b1, q, g0[0][r], g0[1][r], g0[2][r],
                             g1[0][r], g1[1][r], g1[2][r], groups, G, T, tq.TQ_EST_PROD, logits[r], ws)

    def prepare():      # the query prep alone (depends on q only)
        tq.tq_score_split_prepare(params[0], params[1], d, d0, b0, b1, q, groups, G, ws)

    def scan(r):        # the scan against the prepared query operands
        tq.tq_score_ip_split_prepared(params[0], params[1], d, d0, b0, b1, g0[0][r], g0[1][r], g0[2][r],
                                      g1[0][r], g1[1][r], g1[2][r], groups, G, T, tq.TQ_EST_PROD, logits[r], ws)

    for i in range(max(args.warmup, 1)):
        quantize(i % R)
        score(i % R)
    torch.cuda.synchronize()

    # steps as in the KV workloads: serial (the query prep on a second stream beside the quantize
    # of batch r, then the scan of batch r) and pipelined (batch r quantized while the second
    # stream prepares the queries and scans batch r - 1)
    side = torch.cuda.Stream()

    def serial(r):
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            prepare()
        quantize(r)
        torch.cuda.current_stream().wait_stream(side)
        scan(r)

    def pipe(r):
        side.wait_stream(torch.cuda.current_stream())
        quantize(r)
        with torch.cuda.stream(side):
            prepare()
            scan((r - 1) % R)
        torch.cuda.current_stream().wait_stream(side)

    if args.calibrate_copy_mb:
        calibration_copy(torch, dev, args.calibrate_copy_mb)
    K = args.steps
    plain_ms = time_steps(torch, lambda r: (quantize(r), score(r)), R, K)
    serial_ms = time_steps(torch, serial, R, K)
    pipe_ms = time_steps(torch, pipe, R, K)
    ms_step = min(serial_ms, pipe_ms)

    q_ms = time_per_launch(torch, quantize, R, K)
    s_ms = time_per_launch(torch, score, R, K)
    n_logits = groups * G * T
    code_bytes = (d0 * b0 + (d - d0) * b1) // 8 + 16          # both groups' codes, nu, gamma
    q_bytes = n * (d * 2 + code_bytes)
    # 64 + 64 with whole quads of heads: one scan sums both groups' estimates before its single
    # store; otherwise the general path, whose second group reads the logits back to add to them
    int_path = d == 128 and d0 == 64 and G % 4 == 0
    s_bytes = n * code_bytes + n_logits * 4 * (1 if int_path else 2)
    q_flops = n * 4.0 * (d0 * d0 + (d - d0) ** 2)
    q_gbs = q_bytes / (q_ms * 1e-3) / 1e9
    s_gbs = s_bytes / (s_ms * 1e-3) / 1e9
    rq = {"kernel": "tq_quantize_split (fused d = 128 encoder, split mode: both groups in one pass)",
          "bound": "hbm",
          "achieved": q_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": q_gbs / HBM_PEAK_GBS,
          "traffic": traffic_from_profiles("quantize.hip", f"fractional_kv_{args.rate}"),
          "note": f"algorithmic bytes per vector: {d * 2} B bf16 key in, {code_bytes} B codes, nu and gamma "
                  f"of both groups out; {q_flops / n:.0f} flop per vector"}
    rs = {"kernel": "tq_score_ip_split (" + ("integer MFMA scan, both channel groups per key tile" if int_path
                                             else "general scoring path, two channel groups") + ")",
          "bound": "hbm",
          "achieved": s_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": s_gbs / HBM_PEAK_GBS,
          "traffic": traffic_from_profiles(("score_split.hip", "score_tile.h"), f"fractional_kv_{args.rate}")
          if int_path else None,
          "note": f"algorithmic bytes per key: {code_bytes} B codes, nu and gamma of both groups in; "
                  + ("fp32 logits written once" if int_path
                     else "fp32 logits written and, by the second group, read back")}
    dominant, other = (rq, rs) if q_ms >= s_ms else (rs, rq)

    # the value side of the same cache: values as two channel groups through the MSE quantizer,
    # each group at the key group's bit count in index bits, capped at 3 (a block prepared for
    # b carries b - 1 of them), and one decode step of attention over the split keys and values
    bv = [min(b0 + 1, 4), min(b1 + 1, 4)]
    pvs = []
    for k, (wd, b) in enumerate(((d0, bv[0]), (d - d0, bv[1]))):
        c, t = tq.tq_codebook_build(b - 1, wd)
        p = torch.empty(tq.tq_params_bytes(wd, b), dtype=torch.uint8, device=dev)
        tq.tq_prepare(wd, b, gen.haar_orthogonal(wd, w.cfg + 2 + k), gen.gaussian_matrix(wd, wd, w.cfg + 2 + k),
                      c, t, p)
        pvs.append(p)
    vals = torch.empty((n, d), dtype=torch.bfloat16, device=dev)
    for s_ in range(w.n_seq):
        for h in range(w.n_kv):
            gi = s_ * w.n_kv + h
            vc = gen.kv_keys_chunk(w.cfg, w.n_seq + s_, h, T, d, chans[h], scale=1.0)
            vals[gi * T:(gi + 1) * T] = torch.from_numpy(vc.view(np.int16)).to(dev).view(torch.bfloat16)
    cv = [[torch.empty(n * (wd // 32) * (b - 1), dtype=torch.int32, device=dev) for _ in range(R)]
          for wd, b in ((d0, bv[0]), (d - d0, bv[1]))]
    nv = [[torch.empty(n, dtype=torch.float32, device=dev) for _ in range(R)] for _ in range(2)]
    scale = 1.0 / float(np.sqrt(d))
    out = torch.empty(groups * G * d, dtype=torch.float32, device=dev)
    wsa = torch.empty(tq.tq_attention_split_ws_bytes(d, d0, b0, b1, groups, G, T), dtype=torch.uint8, device=dev)

    def vquant(r):
        tq.tq_quantize_mse_split(pvs[0], pvs[1], d, d0, bv[0], bv[1], vals, cv[0][r], nv[0][r], cv[1][r], nv[1][r])

    def attend(r):
        tq.tq_attention_split(params[0], params[1], pvs[0], pvs[1], d, d0, b0, b1, bv[0], bv[1], q, g0[0][r],
                              g0[1][r], g0[2][r], g1[0][r], g1[1][r], g1[2][r], cv[0][r], nv[0][r], cv[1][r],
                              nv[1][r], groups, G, T, scale, tq.TQ_EST_PROD, out, wsa)

    for r in range(R):
        vquant(r)
        attend(r)
    torch.cuda.synchronize()
    vq_ms = time_per_launch(torch, vquant, R, K)
    a_ms = time_per_launch(torch, attend, R, K)

    result = {
        "metric": "quantized-key logits/s at a fractional rate (two channel groups), 1 MI355X",
        "value": n_logits / (ms_step * 1e-3),
        "unit": "logits/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) keys with outlier channels, bf16; random rotations and QJL matrices)",
        "config": {
            "workload": f"fractional_kv: {w.name} keys ({w.n_seq} seq x {w.n_kv} KV heads x {T} tokens x d={d} "
                        f"bf16, 4 outlier channels x20) at {args.rate} bits per channel: channels 0..{d0 - 1} "
                        f"at b={b0}, {d0}..{d - 1} at b={b1}; {w.n_q_heads} query heads (GQA {G})",
            "keys": n, "d": d, "rate": args.rate, "groups": [[d0, b0], [d - d0, b1]], "replicas": R,
        },
        "roofline": dominant,
        "roofline_other": other,
        "quantize": {"ms": q_ms, "vectors_per_s": n / (q_ms * 1e-3), "hbm_gbs": q_gbs},
        "score": {"ms": s_ms, "logits_per_s": n_logits / (s_ms * 1e-3), "hbm_gbs": s_gbs},
        "steps_timing": {"serial_ms": serial_ms, "pipelined_ms": pipe_ms, "one_stream_ms": plain_ms,
                         "note": "ms_per_step is the faster of: serial (both groups' query prep on a second "
                                 "stream beside the quantize of batch i, then the scan of batch i) and "
                                 "pipelined (batch i's quantize beside the query prep and scan of batch i-1 "
                                 "on a second stream); one_stream: quantize then tq_score_ip_split"},
        "value_quantize": {"ms": vq_ms, "vectors_per_s": n / (vq_ms * 1e-3),
                           "index_bits": [[d0, bv[0] - 1], [d - d0, bv[1] - 1]]},
        "attention": {"ms": a_ms, "pairs_per_s": n_logits / (a_ms * 1e-3),
                      "note": "tq_attention_split: split-key logits, softmax, per-group value sums"},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline_fractional(w, b0, b1, args.cpu_seconds)
    copy_gbs = measured_copy_gbs(torch)
    for key in ("roofline", "roofline_other"):
        with_measured_peak(result[key], copy_gbs, "1 GiB device copy in this run (read + write bytes)")
    print(json.dumps(result), flush=True)


def kv_keys_on_device(torch, w, chans, dev):
    """The whole bf16 key cache of a KV workload on the GPU, generated chunk by chunk on host
    threads from the seeded generator."""
    import concurrent.futures

    from workloads import gen
    x = torch.empty((w.n_keys, w.d), dtype=torch.bfloat16, device=dev)

    def one(gi):
        s_, h = divmod(gi, w.n_kv)
        return gi, gen.kv_keys_chunk(w.cfg, s_, h, w.T, w.d, chans[h])

    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        for gi, chunk in ex.map(one, range(w.groups)):
            x[gi * w.T:(gi + 1) * w.T] = torch.from_numpy(chunk.view(np.int16)).to(dev).view(torch.bfloat16)
    return x


#: working set cycled by every per-launch timing: above the 256 MB MALL by a wide margin
MIN_WORKING_SET = 640 * 1024 * 1024


def bench_kv(args):
    """A decode-step workload: quantize the whole key cache, then score every query head."""
    import torch

    import kv_cache_embedding_amd as tq
    from workloads import gen

    w = {"decode_layer": gen.DECODE_LAYER, "decode_batch16": gen.DECODE_BATCH16,
         "long_context": gen.LONG_CONTEXT}[args.workload]
    dev = torch.device("cuda:0")
    d = w.d
    b = args.bits or w.bits[0]
    if b not in w.bits:
        raise SystemExit(f"{w.name} is defined for b in {w.bits}")
    # counter records of a workload defined at several b are kept per b
    traffic_key = w.name if len(w.bits) == 1 else f"{w.name}_b{b}"
    groups, G, T = w.groups, w.G, w.T
    n = w.n_keys

    # ---- parameters and resident inputs
    Pi = gen.haar_orthogonal(d, w.cfg)
    S = gen.gaussian_matrix(d, d, w.cfg)
    c, t = tq.tq_codebook_build(b - 1, d)
    params = torch.empty(tq.tq_params_bytes(d, b), dtype=torch.uint8, device=dev)
    tq.tq_prepare(d, b, Pi, S, c, t, params)
    chans = gen.outlier_channels(w.cfg, w.n_kv, d)
    t_gen = time.perf_counter()
    x = kv_keys_on_device(torch, w, chans, dev)
    print(f"# generated {n} keys in {time.perf_counter() - t_gen:.1f} s", file=sys.stderr, flush=True)
    q = torch.from_numpy(gen.kv_queries(w.cfg, w.n_seq, w.n_q_heads, d).reshape(-1, d).view(np.int16))
    q = q.to(dev).view(torch.bfloat16)

    # Replicas: the inputs of the quantize launches and the code sets of the scoring launches
    # each cycle through more than MIN_WORKING_SET distinct bytes, so no per-launch timing is
    # served from the MALL.  Step r quantizes input copy r % Rx into code set r.
    n_logits = groups * G * T
    in_bytes = n * d * 2
    score_in_bytes = n * (d // 8 * b + 8) + n_logits * 4
    Rx = max(1, min(16, -(-MIN_WORKING_SET // in_bytes)))
    R = max(Rx, min(64, -(-MIN_WORKING_SET // score_in_bytes)))
    xs = [x] + [x.clone() for _ in range(Rx - 1)]
    wc = d // 32 * b
    codes = [torch.empty(n * wc, dtype=torch.int32, device=dev) for _ in range(R)]
    nus = [torch.empty(n, dtype=torch.float32, device=dev) for _ in range(R)]
    gms = [torch.empty(n, dtype=torch.float32, device=dev) for _ in range(R)]
    logits = [torch.empty(n_logits, dtype=torch.float32, device=dev) for _ in range(R)]
    ws = torch.empty(tq.tq_score_ws_bytes(d, b, groups, G, T), dtype=torch.uint8, device=dev)

    def quantize(r):
        tq.tq_quantize(params, d, b, xs[r % Rx], codes[r], nus[r], gms[r])

    def score(r):       # the whole scoring call: query prep + scan
        tq.tq_score_ip(params, d, b, q, codes[r], nus[r], gms[r], groups, G, T, tq.TQ_EST_PROD,
                       logits[r], ws)

    def prepare():      # the query prep alone (depends on q only)
        tq.tq_score_prepare(params, d, b, q, groups, G, ws)

    def scan(r):        # the scan against the prepared query operands
        tq.tq_score_ip_prepared(params, d, b, codes[r], nus[r], gms[r], groups, G, T, tq.TQ_EST_PROD,
                                logits[r], ws)

    if args.calibrate_copy_mb:
        calibration_copy(torch, dev, args.calibrate_copy_mb)

    for r in range(R):
        quantize(r)
        score(r)
    for i in range(args.warmup):
        quantize(i % R)
        score(i % R)
    torch.cuda.synchronize()

    # Serial steps: the query prep (which depends on the queries only) on a second stream
    # (default priority, forked and joined inside the graph) beside the quantize of batch r,
    # then the scan of batch r.
    side = torch.cuda.Stream()

    def serial(r):
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            prepare()
        quantize(r)
        torch.cuda.current_stream().wait_stream(side)
        scan(r)

    # Pipelined steps: step r quantizes batch r while the second stream prepares the queries
    # and scans batch r - 1, which the previous step quantized; each step is one quantize +
    # one query prep + one scan
    def pipe(r):
        side.wait_stream(torch.cuda.current_stream())
        quantize(r)
        with torch.cuda.stream(side):
            prepare()
            scan((r - 1) % R)
        torch.cuda.current_stream().wait_stream(side)

    K = args.steps
    serial_ms = time_steps(torch, serial, R, K)
    pipe_ms = time_steps(torch, pipe, R, K)

    q_ms = time_per_launch(torch, quantize, R, K)
    s_ms = time_per_launch(torch, score, R, K)
    scan_ms = time_per_launch(torch, scan, R, K)
    ms_step = min(serial_ms, pipe_ms)

    # The pages' comparison (attention logits with 4-bit keys against 32-bit keys): the same
    # logits from a float32 copy of the cache by a library batched GEMM, K q^T per group (the
    # cache is the contiguous left operand), beside the tq_score_ip call on the b-bit codes.
    # long_context only: its 8.6 GB of float32 keys cannot be served from the 256 MB MALL.
    keys32 = None
    if args.workload == "long_context":
        kf = xs[0].view(groups, T, d).float()
        qt = q.view(groups, G, d).float().transpose(1, 2).contiguous()
        o32 = torch.empty((groups, T, G), dtype=torch.float32, device=dev)
        for _ in range(2):
            torch.bmm(kf, qt, out=o32)
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            torch.bmm(kf, qt, out=o32)
        e1.record()
        torch.cuda.synchronize()
        ms32 = e0.elapsed_time(e1) / 5
        keys32 = {"fp32_keys_ms": ms32, "fp32_keys_gbs": n * d * 4 / (ms32 * 1e-3) / 1e9,
                  "tq_score_ms": s_ms, "speedup": ms32 / s_ms,
                  "note": "logits of all query heads: float32 keys through torch.bmm vs b-bit TurboQuant "
                          "codes through tq_score_ip (query prep included); the pages report up to 8x "
                          "for 4-bit vs 32-bit keys on another GPU"}
        del kf, o32
        torch.cuda.empty_cache()

    # algorithmic work per launch
    q_flops = n * 4.0 * d * d                       # Pi x and S' r': 2 d^2 each
    q_bytes = n * (d * 2 + d // 8 * b + 8)          # bf16 keys in, codes + nu + gamma out
    s_bytes = score_in_bytes                        # codes + nu + gamma in, fp32 logits out
    q_tflops = q_flops / (q_ms * 1e-3) / 1e12
    q_gbs = q_bytes / (q_ms * 1e-3) / 1e9
    s_gbs = s_bytes / (s_ms * 1e-3) / 1e9

    result = {
        "metric": "quantized-key logits/s (GB/s vs HBM peak) + vectors quantized/s, 1 MI355X",
        "value": n_logits / (ms_step * 1e-3),
        "unit": "logits/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) keys with outlier channels, bf16; random rotation and QJL matrix)",
        "config": {
            "workload": f"{w.name}: {w.n_seq} seq x {w.n_kv} KV heads x {T} tokens x d={d} bf16 keys "
                        f"(4 outlier channels x20), b={b}, {w.n_q_heads} query heads per sequence (GQA {G})",
            "keys": n, "d": d, "bits": b, "query_heads": w.n_seq * w.n_q_heads,
            "input_copies": Rx, "code_sets": R,
        },
        "roofline": {
            "kernel": "quantize_d128 (tq_quantize)",
            "bound": "hbm", "achieved": q_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": q_gbs / HBM_PEAK_GBS,
            "traffic": traffic_from_profiles("quantize.hip", traffic_key),
            "note": f"algorithmic bytes per vector: {d * 2} B bf16 key in, {d // 8 * b} B codes and 8 B "
                    f"nu, gamma out; at 4 d^2 flop per vector the arithmetic intensity "
                    f"({4 * d * d / (d * 2 + d // 8 * b + 8):.0f} flop/B) is below the MFMA ridge "
                    f"({BF16_MFMA_PEAK_TFLOPS / HBM_PEAK_GBS * 1e3:.0f} flop/B), so HBM binds; "
                    "roofline_mfma gives the same launch against the bf16 MFMA peak",
        },
        "roofline_mfma": {
            "kernel": "quantize_d128 (tq_quantize)",
            "bound": "mfma", "achieved": q_tflops, "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": q_tflops / BF16_MFMA_PEAK_TFLOPS,
            "executed": q_tflops * 2.5,
            "note": "algorithmic 4 d^2 flop/vector; the kernel executes 10 d^2 on bf16 MFMA "
                    "(hi/lo operand splits for float32-accurate rotation and projection): 'executed' "
                    "is that rate, 'executed_frac_of_measured_peak' its fraction of a library bf16 GEMM's",
        },
        "roofline_score": {
            "kernel": "score_qprep + score (tq_score_ip)",
            "bound": "hbm", "achieved": s_gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": s_gbs / HBM_PEAK_GBS, "traffic": traffic_from_profiles("score.hip", traffic_key),
            "note": f"the whole call (query prep + scan) over {R} code sets of "
                    f"{score_in_bytes / 2**20:.0f} MiB cycled per launch",
        },
        "steps_timing": {"serial_ms": serial_ms, "pipelined_ms": pipe_ms,
                         "note": "ms_per_step is the faster of: serial (the query prep on a second stream beside "
                                 "the quantize of batch i, then the scan of batch i) and pipelined (batch i's "
                                 "quantize beside the query prep and scan of batch i-1 on a second stream)"},
        "quantize": {"ms": q_ms, "vectors_per_s": n / (q_ms * 1e-3), "hbm_gbs": q_gbs,
                     "hbm_frac": q_gbs / HBM_PEAK_GBS},
        "score": {"ms": s_ms, "logits_per_s": n_logits / (s_ms * 1e-3), "keys_per_s": n / (s_ms * 1e-3),
                  "hbm_gbs": s_gbs},
        "scan": {"ms": scan_ms, "hbm_gbs": s_bytes / (scan_ms * 1e-3) / 1e9,
                 "hbm_frac": s_bytes / (scan_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
                 "note": "tq_score_ip_prepared alone (the query operands prepared once)"},
        "context": "pages: up to 8x faster attention logits with 4-bit keys vs 32-bit keys on H100 "
                   "(no absolute numbers); not a target",
    }
    if keys32 is not None:
        result["vs_fp32_keys"] = keys32
    copy_gbs = measured_copy_gbs(torch)
    with_measured_peak(result["roofline"], copy_gbs, "1 GiB device copy in this run (read + write bytes)")
    with_measured_peak(result["roofline_score"], copy_gbs, "1 GiB device copy in this run (read + write bytes)")
    rm = with_measured_peak(result["roofline_mfma"], measured_gemm_tflops(torch, torch.bfloat16),
                            "8192^3 library bf16 GEMM in this run")
    rm["executed_frac_of_measured_peak"] = rm["executed"] / rm["measured_peak"]
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, b, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def bench_toy(args):
    """The toy configuration: 4096 float32 unit vectors in R^128 at b = 4 and 64 unit queries; a
    step quantizes the vectors and computes all 64 x 4096 logits (one group of 64 query heads).
    At 3.7 MB per step it is launch- and latency-bound: reported, not held to a roofline."""
    import torch

    import kv_cache_embedding_amd as tq
    import oracle
    from workloads import gen

    w = gen.TOY
    dev = torch.device("cuda:0")
    d, b, n, nq = w.d, w.bits[0], w.n, w.nq
    Pi = gen.haar_orthogonal(d, w.cfg)
    S = gen.gaussian_matrix(d, d, w.cfg)
    c, t = tq.tq_codebook_build(b - 1, d)
    params = torch.empty(tq.tq_params_bytes(d, b), dtype=torch.uint8, device=dev)
    tq.tq_prepare(d, b, Pi, S, c, t, params)
    xh = gen.unit_sphere(n, d, cfg=w.cfg, role=gen.ROLE_DATA)
    qh = gen.unit_sphere(nq, d, cfg=w.cfg, role=gen.ROLE_QUERY)
    R = 64
    xs = [torch.from_numpy(xh).to(dev) for _ in range(R)]
    q = torch.from_numpy(qh).to(dev)
    codes = [torch.empty(n * d // 32 * b, dtype=torch.int32, device=dev) for _ in range(R)]
    nus = [torch.empty(n, dtype=torch.float32, device=dev) for _ in range(R)]
    gms = [torch.empty(n, dtype=torch.float32, device=dev) for _ in range(R)]
    logits = [torch.empty(nq * n, dtype=torch.float32, device=dev) for _ in range(R)]
    ws = torch.empty(tq.tq_score_ws_bytes(d, b, 1, nq, n), dtype=torch.uint8, device=dev)

    def quantize(r):
        tq.tq_quantize(params, d, b, xs[r], codes[r], nus[r], gms[r])

    def score(r):
        tq.tq_score_ip(params, d, b, q, codes[r], nus[r], gms[r], 1, nq, n, tq.TQ_EST_PROD, logits[r], ws)

    def step(r):
        quantize(r)
        score(r)

    for i in range(max(args.warmup, 1)):
        step(i % R)
    torch.cuda.synchronize()
    K = args.steps
    ms_step = time_steps(torch, step, R, K)
    q_ms = time_per_launch(torch, quantize, R, K)
    s_ms = time_per_launch(torch, score, R, K)
    step_bytes = n * (d * 4 + d // 8 * b + 8) + n * (d // 8 * b + 8) + nq * n * 4
    gbs = step_bytes / (ms_step * 1e-3) / 1e9
    result = {
        "metric": "quantized-key logits/s (GB/s vs HBM peak) + vectors quantized/s, 1 MI355X",
        "value": nq * n / (ms_step * 1e-3),
        "unit": "logits/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded N(0, I) vectors and queries scaled to unit length, float32; random "
                "rotation and QJL matrix)",
        "config": {"workload": f"toy: {n} x d={d} float32 unit vectors, b={b}, {nq} unit queries, all "
                               f"{nq} x {n} logits", "n": n, "d": d, "bits": b, "queries": nq, "replicas": R},
        "roofline": {
            "kernel": "tq_quantize + tq_score_ip (whole step)",
            "bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
            "traffic": None,
            "note": f"algorithmic bytes of a step: float32 vectors in, codes + nu + gamma out and back in, "
                    f"fp32 logits out ({step_bytes / 1e6:.2f} MB); at this size two kernel launches and one "
                    "memory round trip each set the time, so the fraction is not a bandwidth figure "
                    f"(the {R} replicas fit the MALL)",
        },
        "quantize": {"ms": q_ms, "vectors_per_s": n / (q_ms * 1e-3)},
        "score": {"ms": s_ms, "logits_per_s": nq * n / (s_ms * 1e-3)},
    }
    if not args.no_cpu_baseline:
        t0 = time.perf_counter()
        c64, t64 = oracle.codebook(b - 1, d)
        r = oracle.quantize(xh.astype(np.float64), Pi, S, c64, t64)
        oracle.estimate_ip(qh.astype(np.float64), Pi, S, r["idx"], r["z"], r["nu"], r["gamma"], c64)
        el = time.perf_counter() - t0
        try:
            from threadpoolctl import threadpool_info
            cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        except Exception:
            cores = os.cpu_count() or 1
        result["cpu_baseline"] = {"value": nq * n / el, "unit": "logits/s", "cores": int(cores),
                                  "cpu_model": cpu_model(), "kind": "oracle",
                                  "sample": f"the whole workload ({n} vectors quantized, {nq * n} logits), "
                                            f"float64 NumPy oracle, {el:.1f} s"}
    print(json.dumps(result), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              f"(asked for --gpus {args.gpus}); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    run = {"embedding_search": bench_search, "decode_attention": bench_attention,
           "fractional_kv": bench_fractional, "ubench": bench_ubench,
           "toy": bench_toy}.get(args.workload, bench_kv)
    run(args)


if __name__ == "__main__":
    main()
