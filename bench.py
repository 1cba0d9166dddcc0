#!/usr/bin/env python3
"""Benchmark of the QSA hot path on one MI355X.

A step is one pass of the whole layer (compress of the block the new token completes,
indexer scoring, top-512 block selection, sparse GQA attention) over one batch of the
decode workload: 16 sequences at 262,144 tokens of context, one query token each.
Inputs are seeded and synthetic and sit in HBM before timing starts. Consecutive steps
rotate over R distinct query sets and R copies of the compressed-key cache, so that a
step never finds the previous step's 168 MB working set in the 256 MB Infinity Cache.

Prints one JSON line: throughput (query-tokens/s), the median and minimum step times, a
roofline entry for the dominant kernel (algorithmic bytes / its mean HIP-event duration)
and the whole step's HBM fraction, the CPU oracle timed on a bounded sample, and the
other measurements: decode at 1M tokens, with 4 query tokens per sequence and from the
FP8 cache; compression of the full 16 x 262,144-token key cache; the ragged
65,535/40,001/8,190/3 prefill (with its FP8 and backward variants and its own oracle
baseline); and the 1x1024, 1x16384 and 1x262144 prefills and the 1x32768 decode.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "QSA query-tokens/s: decode @256K ctx + prefill @64K; % of HBM/MFMA peak"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2516.6  # dense bf16, 256 CU x 2.4 GHz x 4096 flop/clk

HQ, HKV, D, HI, DI, BS, TOPK = 24, 2, 128, 4, 64, 4, 512
HOST_THREADS = 16   # host threads for the oracle baseline: one GPU's share of the host

# HBM bytes per dispatch (FETCH_SIZE + WRITE_SIZE, each scaled by the factor the counter
# reads on a plain 512 MiB copy) from rocprofv3 --pmc runs of this benchmark, with the
# fingerprint of the kernel sources they were taken on; reported only while it matches.
TRAFFIC = {
    "score": {"bytes": 134_762_000, "sources_sha256": "de17aaecc9d0f5de9b401caaa2257983ffe1a8b2ef34d6ed03e08cf069885dc6"},
}


# The sources the dominant (scoring) kernel and its launch are built from: its translation
# unit, the headers it includes and the host code that sizes its grid. The dense-regime and
# backward kernels live in translation units of their own and do not enter it.
SCORE_SOURCES = ("qsa_api.hip", "qsa_device.h", "qsa_kernels.hip", "qsa_launch.h")


def sources_sha256():
    """SHA-256 of the scoring kernel's sources' code: comments removed and white space
    collapsed, so that only a change of code invalidates a stored measurement."""
    import hashlib
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "long_context_block_qsa_amd", "csrc")
    for name in SCORE_SOURCES:
        with open(os.path.join(csrc, name), encoding="utf-8") as f:
            code = f.read()
        code = re.sub(r"/\*.*?\*/", " ", code, flags=re.S)
        code = re.sub(r"//[^\n]*", " ", code)
        code = " ".join(code.split())
        h.update(name.encode() + b"\0" + code.encode())
    return h.hexdigest()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=48)
    ap.add_argument("--warmup", type=int, default=8)
    ap.add_argument("--rotate", type=int, default=4, help="distinct query sets / cache copies")
    ap.add_argument("--prefill-steps", type=int, default=3)
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the lines of the other workloads (1x1024, 1x32768 decode, "
                         "1x16384, 1x262144)")
    ap.add_argument("--no-1m", action="store_true", help="skip the 1M-context decode line")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8 KV cache lines")
    ap.add_argument("--no-mtp", action="store_true",
                    help="skip the multi-query decode line (4 query tokens per sequence)")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the prefill's attention backward line")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--trace-steps", type=int, default=8)
    ap.add_argument("--no-graph", action="store_true",
                    help="launch every step from Python instead of replaying HIP graphs")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run 4 plain device copies of MIB MiB (reference for HBM "
                         "byte counters) and exit")
    return ap.parse_args()


def copy_calibration(torch, mib):
    """Plain copy kernels of a known size: each dispatch reads and writes mib MiB, so
    HBM byte counters read on it give the counter's scale."""
    n = mib * 2**20 // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(4):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_mib": mib, "dispatches": 4,
                      "bytes_read_per_dispatch": n * 4, "bytes_written_per_dispatch": n * 4}),
          flush=True)


# ---------------------------------------------------------------- decode workload

def decode_algorithmic_bytes(batch, ctx):
    """Bytes the decode step must move (no intermediate spills):
    score: every visible compressed key (128 B per block) + q_idx and w;
    attend: 512 blocks x 4 tokens x (K + V, 2 heads x 128 x bf16) + Q (bf16) + O (fp32)."""
    nblk = ctx // BS
    score = batch * (nblk * DI * 2 + HI * DI * 2 + HI * 4)
    attend = batch * (TOPK * BS * HKV * D * 2 * 2 + HQ * D * 2 + HQ * D * 4)
    return {"score": score, "attend": attend, "total": score + attend}


def run_decode(args, torch, qsa, gen):
    cfg = gen.WORKLOADS["decode_16x262144"]
    lens, batch = cfg["lens"], len(cfg["lens"])
    ctx = lens[0]
    t0 = time.time()
    p = gen.workload_problem("decode_16x262144")
    log(f"generated decode inputs in {time.time() - t0:.1f}s")
    dev16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    seqs = qsa.Seqs(p.cu_q, p.cu_k)
    k, v, k_idx = dev16(p.k), dev16(p.v), dev16(p.k_idx)
    R = max(1, args.rotate)
    sets = []
    k_blk0 = torch.empty((seqs.n_blocks, DI), dtype=torch.int16, device="cuda")
    qsa.compress(seqs, k_idx, k_blk0)
    for r in range(R):
        if r == 0:
            q, q_idx, w = p.q, p.q_idx, p.w
        else:
            s2 = 50_000 + r
            q = gen.normal_bf16(s2, gen.TID_Q, batch * HQ * D).reshape(batch, HQ, D)
            q_idx = gen.uniform_int_bf16(s2, gen.TID_QIDX, batch * HI * DI, -3, 3).reshape(
                batch, HI, DI)
            w = gen.weights(s2, gen.TID_W, batch * HI).reshape(batch, HI)
        kb = k_blk0 if r == 0 else k_blk0.clone()
        sets.append(dict(q=dev16(q), q_idx=dev16(q_idx), w=torch.from_numpy(w).cuda(), k_blk=kb,
                         sel=torch.empty((batch, TOPK), dtype=torch.int32, device="cuda"),
                         out=torch.empty((batch, HQ, D), dtype=torch.float32, device="cuda"),
                         lse=torch.empty((batch, HQ), dtype=torch.float32, device="cuda")))
    ws = qsa.alloc_workspace(seqs, TOPK)
    torch.cuda.synchronize()
    log(f"decode inputs resident: K/V {2 * k.numel() * 2 / 2**30:.2f} GiB, "
        f"{R} cache copies of {k_blk0.numel() * 2 / 2**20:.0f} MiB")

    def step(i):
        s = sets[i % R]
        qsa.forward(seqs, s["q"], k, v, s["q_idx"], s["w"], k_idx, s["k_blk"], s["sel"],
                    s["out"], s["lse"], ws, TOPK)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # one HIP graph holding R consecutive steps (one per rotation set): a replay runs the
    # library's kernels for R steps as recorded, with one launch
    graph = None
    if not args.no_graph:
        if args.steps % R:
            sys.exit(f"--steps must be a multiple of --rotate ({R}) with graph replay")
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for r in range(R):
                step(r)
        torch.cuda.synchronize()
        for _ in range(max(1, args.warmup // R)):
            graph.replay()
        torch.cuda.synchronize()
    # correctness guard on the timed configuration: needles of set 0 selected
    sel0 = sets[0]["sel"].cpu().numpy()
    for b, needles in p.needles.items():
        if not set(needles) <= set(sel0[b].tolist()):
            raise RuntimeError(f"needle blocks of sequence {b} not selected")

    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    ev0.record()
    if graph is None:
        for i in range(args.steps):
            step(i)
    else:
        for _ in range(args.steps // R):
            graph.replay()
    ev1.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    gpu_ms = ev0.elapsed_time(ev1)
    log(f"decode: {args.steps} steps ({'eager' if graph is None else 'graph replay'}), "
        f"wall {wall * 1e3:.2f} ms, events {gpu_ms:.2f} ms")
    # per-step distribution (outside the timed region): HIP events around each replay of
    # R steps, or around each eager step
    if graph is None:
        ctr = [0]

        def one():
            step(ctr[0])
            ctr[0] += 1

        per_step = event_times(torch, one, args.steps)
    else:
        per_step = [t / R for t in event_times(torch, graph.replay, max(1, args.steps // R))]

    # instrumented pass: per-kernel durations with HIP events on the library's stream
    with qsa.trace(4096) as tr:
        for i in range(args.trace_steps):
            step(i)
    torch.cuda.synchronize()
    long_ctx = None if args.no_1m else run_decode_1m(args, torch, qsa, gen, k, v, k_idx, sets)
    mtp = None if args.no_mtp else run_decode_mtp(args, torch, qsa, gen, k, v, k_idx, sets)
    fp8 = None if args.no_fp8 else run_decode_fp8(args, torch, qsa, seqs, k, v, k_idx, sets)
    return dict(p=p, batch=batch, ctx=ctx, wall_s=wall, gpu_ms=gpu_ms,
                kernels=tr.mean_ms(), kernel_total=tr.total_ms(), seqs=seqs, sets=sets,
                long_ctx=long_ctx, fp8=fp8, mtp=mtp, per_step=per_step, k_idx=k_idx)


def time_steps(args, torch, step, R, n):
    """Runs n steps (a multiple of R) and returns (ms per step, launch mode): replays of one
    HIP graph holding R consecutive steps, as for the main decode line, or with --no-graph
    launches from Python."""
    if args.no_graph:
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(n):
            step(i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / n, "eager"
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for r in range(R):
            step(r)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n // R):
        graph.replay()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / n
    del graph
    return ms, "hip graph replay"


def run_decode_fp8(args, torch, qsa, seqs, k, v, k_idx, sets):
    """The decode workload with K and V read from the FP8 cache (built once, outside the
    timed region, like the compressed indexer keys)."""
    nk = seqs.n_k
    k8 = torch.empty((nk, HKV, D), dtype=torch.uint8, device="cuda")
    v8 = torch.empty_like(k8)
    ks = torch.empty((nk, HKV), dtype=torch.float32, device="cuda")
    vs = torch.empty_like(ks)
    qsa.quantize_kv(seqs, k, v, k8, v8, ks, vs)
    ws = qsa.alloc_workspace(seqs, TOPK)
    R = len(sets)

    def step(i):
        s = sets[i % R]
        qsa.forward_fp8(seqs, s["q"], k8, v8, ks, vs, s["q_idx"], s["w"], k_idx, s["k_blk"],
                        s["sel"], s["out"], s["lse"], ws, TOPK)

    for i in range(max(args.warmup, R)):
        step(i)
    torch.cuda.synchronize()
    n = max(R, args.steps // R * R)
    ms, mode = time_steps(args, torch, step, R, n)
    with qsa.trace(64) as tr:
        for i in range(R):
            step(i)
    torch.cuda.synchronize()
    batch = seqs.n_q
    nblk = seqs.n_blocks // batch
    nbytes = batch * (nblk * DI * 2 + HI * DI * 2 + HI * 4) + \
        batch * (TOPK * BS * HKV * (2 * D + 2 * 4) + HQ * D * 2 + HQ * D * 4)
    gbs = nbytes / (ms / 1e3) / 1e9
    log(f"decode fp8: {n} steps, {ms * 1e3:.1f} us/step")
    del k8, v8, ks, vs
    return {"workload": "decode as above, K/V from the FP8 (E4M3 + per-row scale) cache",
            "steps": n, "launch": mode, "ms_per_step": round(ms, 5),
            "query_tokens_per_s": round(batch / (ms / 1e3), 1), "algorithmic_bytes": nbytes,
            "achieved_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "kernel_mean_ms": {k2: round(v2, 5) for k2, v2 in tr.mean_ms().items()}}


def run_decode_1m(args, torch, qsa, gen, k, v, k_idx, sets):
    """Decode at 1,048,576 tokens of context (the extended window): the resident
    4,194,304-token K/V, indexer keys and compressed caches, read as 4 sequences of
    1,048,576 tokens with fresh query tokens; same rotation and timing protocol."""
    L, batch = 1 << 20, 4
    if k.shape[0] != L * batch:
        return None
    dev16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    cu_k = np.arange(batch + 1, dtype=np.int32) * L
    cu_q = np.arange(batch + 1, dtype=np.int32)
    seqs = qsa.Seqs(cu_q, cu_k)
    R = len(sets)
    qs = []
    for r in range(R):
        s2 = 60_000 + r
        qs.append(dict(
            q=dev16(gen.normal_bf16(s2, gen.TID_Q, batch * HQ * D).reshape(batch, HQ, D)),
            q_idx=dev16(gen.uniform_int_bf16(s2, gen.TID_QIDX, batch * HI * DI, -3, 3).reshape(
                batch, HI, DI)),
            w=torch.from_numpy(gen.weights(s2, gen.TID_W, batch * HI).reshape(batch, HI)).cuda(),
            sel=torch.empty((batch, TOPK), dtype=torch.int32, device="cuda"),
            out=torch.empty((batch, HQ, D), dtype=torch.float32, device="cuda"),
            lse=torch.empty((batch, HQ), dtype=torch.float32, device="cuda")))
    ws = qsa.alloc_workspace(seqs, TOPK)

    def step(i):
        s, kb = qs[i % R], sets[i % R]["k_blk"]
        qsa.forward(seqs, s["q"], k, v, s["q_idx"], s["w"], k_idx, kb, s["sel"], s["out"],
                    s["lse"], ws, TOPK)

    for i in range(max(args.warmup, R)):
        step(i)
    torch.cuda.synchronize()
    n = max(R, args.steps // 2 // R * R)
    ms, mode = time_steps(args, torch, step, R, n)
    ab = decode_algorithmic_bytes(batch, L)
    gbs = ab["total"] / (ms / 1e3) / 1e9
    log(f"decode 1M: {n} steps, {ms * 1e3:.1f} us/step")
    return {"workload": "decode: 4 sequences x 1,048,576 tokens of context, 1 query token "
                        "each, budget 512 blocks", "steps": n, "launch": mode,
            "ms_per_step": round(ms, 5), "query_tokens_per_s": round(batch / (ms / 1e3), 1),
            "algorithmic_bytes": ab["total"], "achieved_gbs": round(gbs, 1),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}


def run_decode_mtp(args, torch, qsa, gen, k, v, k_idx, sets, nq=4):
    """Multi-query decode (several draft tokens verified per step): the resident
    16 x 262,144-token K/V, indexer keys and compressed caches, with the last nq tokens of
    every sequence as queries (fresh query tensors); the sequence's rows share the scan of
    its compressed keys. Same rotation and timing protocol as the 1M line."""
    batch, L = 16, 262144
    if k.shape[0] != L * batch:
        return None
    dev16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    cu_k = np.arange(batch + 1, dtype=np.int32) * L
    cu_q = np.arange(batch + 1, dtype=np.int32) * nq
    seqs = qsa.Seqs(cu_q, cu_k)
    rows = batch * nq
    R = len(sets)
    qs = []
    for r in range(R):
        s2 = 70_000 + r
        qs.append(dict(
            q=dev16(gen.normal_bf16(s2, gen.TID_Q, rows * HQ * D).reshape(rows, HQ, D)),
            q_idx=dev16(gen.uniform_int_bf16(s2, gen.TID_QIDX, rows * HI * DI, -3, 3).reshape(
                rows, HI, DI)),
            w=torch.from_numpy(gen.weights(s2, gen.TID_W, rows * HI).reshape(rows, HI)).cuda(),
            sel=torch.empty((rows, TOPK), dtype=torch.int32, device="cuda"),
            out=torch.empty((rows, HQ, D), dtype=torch.float32, device="cuda"),
            lse=torch.empty((rows, HQ), dtype=torch.float32, device="cuda")))
    ws = qsa.alloc_workspace(seqs, TOPK)

    def step(i):
        s, kb = qs[i % R], sets[i % R]["k_blk"]
        qsa.forward(seqs, s["q"], k, v, s["q_idx"], s["w"], k_idx, kb, s["sel"], s["out"],
                    s["lse"], ws, TOPK)

    for i in range(max(args.warmup, R)):
        step(i)
    torch.cuda.synchronize()
    n = max(R, args.steps // 2 // R * R)
    ms, mode = time_steps(args, torch, step, R, n)
    with qsa.trace(64) as tr:
        for i in range(R):
            step(i)
    torch.cuda.synchronize()
    one = decode_algorithmic_bytes(batch, L)
    nbytes = one["score"] + batch * (nq - 1) * (HI * DI * 2 + HI * 4) + nq * one["attend"]
    gbs = nbytes / (ms / 1e3) / 1e9
    log(f"decode {nq} queries/sequence: {n} steps, {ms * 1e3:.1f} us/step")
    return {"workload": f"decode: 16 sequences x 262,144 tokens of context, {nq} query tokens "
                        "each (the last ones), budget 512 blocks", "steps": n, "launch": mode,
            "ms_per_step": round(ms, 5), "query_tokens_per_s": round(rows / (ms / 1e3), 1),
            "algorithmic_bytes": nbytes, "achieved_gbs": round(gbs, 1),
            "hbm_frac": round(gbs / HBM_PEAK_GBS, 4),
            "kernel_mean_ms": {k2: round(v2, 5) for k2, v2 in tr.mean_ms().items()}}


# ---------------------------------------------------------------- prefill workloads

# Random 256-byte row gathers from a 67 MB table, measured on this part with a probe
# kernel of the attention's access shape (16 lanes per row): the beyond-L2 ceiling the
# sparse rows' gathers are compared against.
GATHER_CEILING_GBS = 7900.0


def step_stats(ms_list):
    a = np.asarray(ms_list, dtype=np.float64)
    return {"n": int(a.size), "median_ms": round(float(np.median(a)), 5),
            "min_ms": round(float(a.min()), 5), "mean_ms": round(float(a.mean()), 5)}


def event_times(torch, fn, n):
    """HIP-event time of each of n calls of fn on torch's current stream (ms)."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    for e0, e1 in evs:
        e0.record()
        fn()
        e1.record()
    torch.cuda.synchronize()
    return [e0.elapsed_time(e1) for e0, e1 in evs]


def prefill_work(cu_k):
    """Attended (query, key) pairs of a prefill (every token a query), split into rows
    that keep every visible block (dense) and the others, and scored (query, block)
    pairs."""
    dense = sparse = scored = 0
    for L in np.diff(np.asarray(cu_k, dtype=np.int64)):
        t = np.arange(int(L), dtype=np.int64)
        nv = (t + 1) // BS
        keys = np.minimum(nv, TOPK) * BS + (t + 1 - BS * nv)
        dm = nv <= TOPK
        dense += int(keys[dm].sum())
        sparse += int(keys[~dm].sum())
        scored += int(nv[~dm].sum())
    return dense, sparse, scored


# Prefill forwards whose attention of each selection pass runs on a second stream (the FP8
# cache, long-row passes) overlap kernels: their kernel times add up to more than the step.
OVERLAP_NOTE = ("the attention of each selection pass ran on a second stream, concurrently "
                "with the later passes' score + select: kernel times overlap, and the attention "
                "figures divide by its kernel spans under that sharing")


def overlapped(km, st):
    """Kernel times that add up to clearly more than a step of at least a millisecond (in
    short steps each kernel's traced time includes its launch gap)."""
    return st["median_ms"] >= 1.0 and sum(km.values()) > 1.1 * st["median_ms"]


def measure_prefill(args, torch, qsa, gen, name, steps, extras=False):
    """One prefill workload through qsa_forward (compress, score + select in passes,
    attention): step times by HIP events, per-kernel totals of one traced step, the
    attention's MFMA fraction (attended pairs x 12,288 flop) and its gather rate."""
    t0 = time.time()
    p = gen.workload_problem(name)
    log(f"{name}: inputs generated in {time.time() - t0:.1f}s")
    dev16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    seqs = qsa.Seqs(p.cu_q, p.cu_k)
    q, k, v, q_idx, k_idx = (dev16(x) for x in (p.q, p.k, p.v, p.q_idx, p.k_idx))
    w = torch.from_numpy(p.w).cuda()
    k_blk = torch.empty((seqs.n_blocks, DI), dtype=torch.int16, device="cuda")
    sel = torch.empty((seqs.n_q, TOPK), dtype=torch.int32, device="cuda")
    out = torch.empty((seqs.n_q, HQ, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((seqs.n_q, HQ), dtype=torch.float32, device="cuda")
    ws = qsa.alloc_workspace(seqs, TOPK)

    def step():
        qsa.forward(seqs, q, k, v, q_idx, w, k_idx, k_blk, sel, out, lse, ws, TOPK)

    step()
    torch.cuda.synchronize()
    times = event_times(torch, step, max(1, steps))
    with qsa.trace(8192) as tr:
        step()
    torch.cuda.synchronize()
    km = tr.total_ms()
    dense, sparse, scored = prefill_work(p.cu_k)
    pairs = dense + sparse
    att_flop = pairs * HQ * D * 4
    att_ms = km.get("attend", 0.0) + km.get("attend_dense", 0.0) + km.get("combine", 0.0)
    sparse_ms = km.get("attend", 0.0) + km.get("combine", 0.0)
    st = step_stats(times)
    res = {
        "workload": name, "ms_per_step": st["median_ms"], "step_ms": st,
        "query_tokens_per_s": round(seqs.n_q / (st["median_ms"] / 1e3), 1),
        "kernel_ms": {k2: round(v2, 4) for k2, v2 in km.items()},
        "attention_pairs": {"dense_rows": dense, "sparse_rows": sparse},
        "attention_tflops": round(att_flop / (att_ms / 1e3) / 1e12, 2),
        "attention_mfma_frac": round(att_flop / (att_ms / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "score_select_ms": round(km.get("score_select", 0.0), 4),
        "score_tflops_incl_select": (round(scored * HI * DI * 2 / (km["score_select"] / 1e3) / 1e12,
                                           2) if km.get("score_select") else None),
        "workspace_bytes": int(ws.numel()),
    }
    if dense and km.get("attend_dense"):
        f = dense * HQ * D * 4 / (km["attend_dense"] / 1e3) / 1e12
        res["dense_rows_tflops"] = round(f, 2)
        res["dense_rows_mfma_frac"] = round(f / MFMA_BF16_PEAK_TFLOPS, 4)
    if sparse and sparse_ms > 0:
        g = sparse * HKV * D * 2 * 2 / (sparse_ms / 1e3) / 1e9   # K and V rows of both heads
        res["sparse_rows_gather_gbs"] = round(g, 1)
        res["sparse_rows_gather_frac"] = round(g / GATHER_CEILING_GBS, 4)
    if overlapped(km, st):
        res["kernel_ms_note"] = OVERLAP_NOTE
    log(f"{name}: {st['median_ms']:.3f} ms per step (median of {st['n']})")
    if extras:
        res["fp8_kv"] = None if args.no_fp8 else run_prefill_fp8(
            args, torch, qsa, seqs, q, k, v, q_idx, w, k_idx, k_blk, sel, out, lse, ws, steps,
            att_flop, sparse)
        res["backward"] = None if args.no_backward else run_prefill_backward(
            args, torch, qsa, gen, p, seqs, q, k, v, sel, out, lse, steps, pairs)
    return res


def run_prefill_fp8(args, torch, qsa, seqs, q, k, v, q_idx, w, k_idx, k_blk, sel, out, lse, ws,
                    steps, att_flop, sparse):
    """The same prefill with K and V read from the FP8 (E4M3 + per-row scale) cache."""
    k8 = torch.empty((seqs.n_k, HKV, D), dtype=torch.uint8, device="cuda")
    v8 = torch.empty_like(k8)
    ks = torch.empty((seqs.n_k, HKV), dtype=torch.float32, device="cuda")
    vs = torch.empty_like(ks)
    qsa.quantize_kv(seqs, k, v, k8, v8, ks, vs)

    def step8():
        qsa.forward_fp8(seqs, q, k8, v8, ks, vs, q_idx, w, k_idx, k_blk, sel, out, lse, ws, TOPK)

    step8()
    torch.cuda.synchronize()
    st = step_stats(event_times(torch, step8, max(1, steps)))
    with qsa.trace(8192) as tr8:
        step8()
    torch.cuda.synchronize()
    km8 = tr8.total_ms()
    att8 = km8.get("attend", float("nan")) + km8.get("combine", 0.0)
    note = {"kernel_ms_note": OVERLAP_NOTE} if overlapped(km8, st) else {}
    return {**note, "ms_per_step": st["median_ms"], "step_ms": st,
            "query_tokens_per_s": round(seqs.n_q / (st["median_ms"] / 1e3), 1),
            "kernel_ms": {k2: round(v2, 4) for k2, v2 in km8.items()},
            "attention_tflops": round(att_flop / (att8 / 1e3) / 1e12, 2),
            "attention_gather_gbs": round(sparse * HKV * (2 * D + 8) / (att8 / 1e3) / 1e9, 1)}


def run_decode_32k(args, torch, qsa, gen):
    """Decode of one sequence at 32,768 tokens of context (16 needle blocks); its 3.2 MB
    working set stays in the caches between steps. ms_per_step: replays of one HIP graph of
    4 consecutive forwards, as for the main decode line; single_replay_ms: replays of a graph
    of one forward, each paying its own graph launch (a one-step latency)."""
    p = gen.workload_problem("decode_1x32768")
    dev16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    seqs = qsa.Seqs(p.cu_q, p.cu_k)
    q, k, v, q_idx, k_idx = (dev16(x) for x in (p.q, p.k, p.v, p.q_idx, p.k_idx))
    w = torch.from_numpy(p.w).cuda()
    k_blk = torch.empty((seqs.n_blocks, DI), dtype=torch.int16, device="cuda")
    qsa.compress(seqs, k_idx, k_blk)
    sel = torch.empty((1, TOPK), dtype=torch.int32, device="cuda")
    out = torch.empty((1, HQ, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((1, HQ), dtype=torch.float32, device="cuda")
    ws = qsa.alloc_workspace(seqs, TOPK)

    def step():
        qsa.forward(seqs, q, k, v, q_idx, w, k_idx, k_blk, sel, out, lse, ws, TOPK)

    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    g.replay()
    torch.cuda.synchronize()
    single = step_stats(event_times(torch, g.replay, max(8, args.steps)))
    g4 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g4):
        for _ in range(4):
            step()
    g4.replay()
    torch.cuda.synchronize()
    st = step_stats([t / 4 for t in event_times(torch, g4.replay, max(8, args.steps // 4))])
    if not set(p.needles[0]) <= set(sel.cpu().numpy()[0].tolist()):
        raise RuntimeError("decode_1x32768: needle blocks not selected")
    nbytes = decode_algorithmic_bytes(1, 32768)["total"]
    with qsa.trace(64) as tr:
        step()
    torch.cuda.synchronize()
    return {"workload": "decode_1x32768", "launch": "hip graph replay (4 steps per graph)",
            "ms_per_step": st["median_ms"], "step_ms": st,
            "single_replay_ms": single["median_ms"],
            "query_tokens_per_s": round(1 / (st["median_ms"] / 1e3), 1),
            "algorithmic_bytes": nbytes,
            "achieved_gbs": round(nbytes / (st["median_ms"] / 1e3) / 1e9, 1),
            "hbm_frac": round(nbytes / (st["median_ms"] / 1e3) / 1e9 / HBM_PEAK_GBS, 4),
            "kernel_ms": {k2: round(v2, 5) for k2, v2 in tr.total_ms().items()}}


def run_compress_full(torch, qsa, d):
    """Compression of the whole 16 x 262,144-token indexer-key cache (4,194,304 tokens ->
    1,048,576 blocks): 512 B read and 128 B written per block."""
    seqs, k_idx = d["seqs"], d["k_idx"]
    k_blk = torch.empty((seqs.n_blocks, DI), dtype=torch.int16, device="cuda")

    def run():
        qsa.compress(seqs, k_idx, k_blk)

    run()
    torch.cuda.synchronize()
    st = step_stats(event_times(torch, run, 10))
    nbytes = seqs.n_blocks * (BS * DI * 2 + DI * 2)
    gbs = nbytes / (st["median_ms"] / 1e3) / 1e9
    return {"workload": "compress of the decode_16x262144 indexer keys (full context)",
            "algorithmic_bytes": nbytes, "ms": st["median_ms"], "step_ms": st,
            "achieved_gbs": round(gbs, 1), "hbm_frac": round(gbs / HBM_PEAK_GBS, 4)}


def run_prefill_backward(args, torch, qsa, gen, p, seqs, q, k, v, sel, out, lse, n, pairs):
    """Attention backward over the prefill's own selection, out and lse, with a seeded
    bf16 dout: dq, dk, dv of all 113,729 rows."""
    dev16 = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda()
    dout = dev16(gen.make_dout(p, 900))
    dq = torch.empty((seqs.n_q, HQ, D), dtype=torch.float32, device="cuda")
    dk = torch.empty((seqs.n_k, HKV, D), dtype=torch.float32, device="cuda")
    dv = torch.empty_like(dk)
    bws = qsa.alloc_backward_workspace(seqs, TOPK)

    def stepb():
        qsa.attend_backward(seqs, q, k, v, sel, out, lse, dout, dq, dk, dv, bws, TOPK)

    stepb()
    torch.cuda.synchronize()
    st = step_stats(event_times(torch, stepb, max(1, n)))
    ms = st["median_ms"]
    with qsa.trace(64) as tr:
        stepb()
    torch.cuda.synchronize()
    km = tr.total_ms()   # the dK/dV kernel runs once per row window
    # five contractions per attended (query head, key): S and dP recomputed, dQ, dK, dV
    flop = pairs * HQ * D * 2 * 5
    note = {"kernel_ms_note": "dQ ran on a second stream, concurrently with the dK/dV launches: "
                              "kernel times overlap"} if overlapped(km, st) else {}
    # dkv_row_gbs: rows x kept blocks per KV head (the dK/dV kernel's row visits)
    return {**note, "ms_per_step": round(ms, 3), "step_ms": st,
            "query_tokens_per_s": round(seqs.n_q / (ms / 1e3), 1),
            "kernel_ms": {k2: round(v2, 4) for k2, v2 in km.items()},
            "tflops": round(flop / (ms / 1e3) / 1e12, 2),
            "mfma_frac": round(flop / (ms / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "dq_gather_gbs": round(pairs * HKV * D * 2 * 2 / (km.get("bwd_dq", float("nan")) / 1e3)
                                   / 1e9, 1),
            "dkv_row_gbs": round(pairs / BS * HQ * D * 2 * 2 /
                                 (km.get("bwd_dkv", float("nan")) / 1e3) / 1e9, 1)}


# ---------------------------------------------------------------- CPU baseline

def run_cpu_baseline(args, d, oracle):
    """The oracle timed on host cores: the decode step's select + attend for the 16
    rows against the prebuilt compressed cache, repeated for a bounded time."""
    p = d["p"]
    dims = oracle.Dims()
    k_blk = oracle.compress(dims, p.cu_k, p.k_idx)
    threads = min(os.cpu_count() or 1, p.n_q, HOST_THREADS)
    reps, t0 = 0, time.perf_counter()
    while True:
        sel = oracle.select(dims, p.cu_q, p.cu_k, p.q_idx, p.w, k_blk, threads=threads)
        oracle.attend(dims, p.cu_q, p.cu_k, p.q, p.k, p.v, sel, threads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= args.cpu_seconds:
            break
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
    except OSError:
        pass
    return {"value": round(reps * p.n_q / el, 3), "unit": "query-tokens/s", "cores": threads,
            "cpu_model": model, "host_cpus": os.cpu_count(), "kind": "oracle",
            "sample": f"{reps} decode step(s) of 16 rows at 262,144 context (score + select + "
                      f"attend over the prebuilt compressed cache), {el:.1f} s wall"}


def run_cpu_baseline_prefill(args, oracle, gen, stride=8):
    """The oracle on a bounded sample of the ragged 64K prefill: every stride-th query row
    (compress of all blocks, then score + select + attend of the sampled rows)."""
    p = gen.workload_problem("prefill_ragged_65535_40001_8190_3")
    rows = np.arange(0, p.n_q, stride, dtype=np.int64)
    threads = min(os.cpu_count() or 1, HOST_THREADS)
    t0 = time.perf_counter()
    oracle.forward(oracle.Dims(), p.cu_q, p.cu_k, p.q, p.k, p.v, p.q_idx, p.w, p.k_idx,
                   rows=rows, threads=threads)
    el = time.perf_counter() - t0
    return {"value": round(rows.size / el, 3), "unit": "query-tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"every {stride}th row of the ragged 65,535/40,001/8,190/3 prefill "
                      f"({rows.size} rows: compress of every block, then score, select and "
                      f"attend of those rows), {el:.1f} s wall"}


def traffic_of(kernel):
    rec = TRAFFIC.get(kernel)
    if rec is None or rec["sources_sha256"] != sources_sha256():
        return None
    return rec["bytes"]


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU: the library "
                                   "has no multi-GPU path (its sharding is a design only)",
                          "n_gpus": args.gpus}),
              flush=True)
        sys.exit(2)
    import torch
    import long_context_block_qsa_amd as qsa
    import qsa_inputs as gen
    if not torch.cuda.is_available():
        sys.exit("bench.py needs a GPU")
    if args.copy_calibration > 0:
        copy_calibration(torch, args.copy_calibration)
        return
    qsa.lib()

    d = run_decode(args, torch, qsa, gen)
    step_ms = d["wall_s"] * 1e3 / args.steps
    value = d["batch"] / (step_ms / 1e3)
    ab = decode_algorithmic_bytes(d["batch"], d["ctx"])

    # dominant kernel (largest total traced time) and its algorithmic bytes per launch
    kern = d["kernels"]
    dom = max(d["kernel_total"], key=d["kernel_total"].get)
    per_launch = {"score": ab["score"],
                  "attend": ab["attend"] - d["batch"] * HQ * D * 4,
                  "select": d["batch"] * ((d["ctx"] // BS) * 4 + TOPK * 4),
                  "combine": d["batch"] * HQ * (D + 1) * 4,
                  "compress": d["batch"] * (BS * DI * 2 + DI * 2),
                  "prep": d["batch"] * 40}
    achieved = per_launch[dom] / (kern[dom] / 1e3) / 1e9
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": traffic_of(dom), "algorithmic_bytes_per_launch": per_launch[dom],
                "mean_ms": round(kern[dom], 5)}
    step_gbs = ab["total"] / (step_ms / 1e3) / 1e9

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "query-tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "decode: 16 sequences x 262,144 tokens of context, 1 query "
                               "token each, budget 512 blocks of 4 tokens",
                   "batch": d["batch"], "context": d["ctx"], "budget_blocks": TOPK,
                   "rotation_sets": args.rotate,
                   "launch": "eager" if args.no_graph else "hip graph replay"},
        "roofline": roofline,
        "step_hbm": {"algorithmic_bytes": ab["total"], "achieved_gbs": round(step_gbs, 1),
                     "frac": round(step_gbs / HBM_PEAK_GBS, 4)},
        "step_ms": step_stats(d["per_step"]),
        "kernel_mean_ms": {k2: round(v2, 5) for k2, v2 in kern.items()},
    }
    if d["long_ctx"] is not None:
        line["decode_1m"] = d["long_ctx"]
    if d["mtp"] is not None:
        line["decode_multi_query"] = d["mtp"]
    if d["fp8"] is not None:
        line["decode_fp8"] = d["fp8"]
    line["compress_full_context"] = run_compress_full(torch, qsa, d)
    if not args.no_prefill:
        log("prefill workloads")
        line["prefill"] = measure_prefill(args, torch, qsa, gen,
                                          "prefill_ragged_65535_40001_8190_3",
                                          args.prefill_steps, extras=True)
    if not args.no_workloads:
        w = {"decode_1x32768": run_decode_32k(args, torch, qsa, gen)}
        for name, n in (("prefill_1x1024", 20), ("prefill_1x16384", 5),
                        ("prefill_1x262144", 2)):
            if name == "prefill_1x262144" and args.no_prefill:
                continue
            w[name] = measure_prefill(args, torch, qsa, gen, name, n)
            torch.cuda.empty_cache()
        line["workloads"] = w
    if not args.no_cpu_baseline:
        import oracle
        log("CPU oracle baseline")
        line["cpu_baseline"] = run_cpu_baseline(args, d, oracle)
        if not args.no_prefill:
            line["cpu_baseline_prefill"] = run_cpu_baseline_prefill(args, oracle, gen)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
