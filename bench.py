#!/usr/bin/env python3
"""Benchmark of the QSA hot path on one MI355X.

A step is one pass of the whole layer (compress of the block the new token completes,
indexer scoring, top-512 block selection, sparse GQA attention) over one batch of the
decode workload: 16 sequences at 262,144 tokens of context, one query token each.
Inputs are seeded and synthetic and sit in HBM before timing starts. Consecutive steps
rotate over R distinct query sets and R copies of the compressed-key cache, so that a
step never finds the previous step's 168 MB working set in the 256 MB Infinity Cache.

Prints one JSON line: throughput (query-tokens/s), a roofline entry for the dominant
kernel (algorithmic bytes / its mean HIP-event duration), the CPU oracle timed on a
bounded sample, and a secondary prefill measurement (ragged 65,535/40,001/8,190/3).

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

# HBM bytes per dispatch (FETCH_SIZE + WRITE_SIZE, each scaled by the factor the counter
# reads on a plain 512 MiB copy) from rocprofv3 --pmc runs of this benchmark, with the
# fingerprint of the kernel sources they were taken on; reported only while it matches.
TRAFFIC = {
    "score": {"bytes": 135_080_000, "sources_sha256": "ed8549b398cc8cdd4f8153c3ef6564e38bb32af532bc19b81f08f2a57e00e32c"},
}


def sources_sha256():
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "long_context_block_qsa_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
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
                long_ctx=long_ctx, fp8=fp8, mtp=mtp)


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


# ---------------------------------------------------------------- prefill workload

def run_prefill(args, torch, qsa, gen):
    p = gen.workload_problem("prefill_ragged_65535_40001_8190_3")
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
    n = max(1, args.prefill_steps)
    t0 = time.perf_counter()
    for _ in range(n):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / n
    with qsa.trace(4096) as tr:
        step()
    torch.cuda.synchronize()
    # algorithmic work: attended (query, key) pairs and scored (query, block) pairs
    pairs, scored = 0, 0
    for b in range(len(p.cu_k) - 1):
        L = int(p.cu_k[b + 1] - p.cu_k[b])
        for t in range(L):
            nv = (t + 1) // BS
            pairs += min(nv, TOPK) * BS + (t + 1 - BS * nv)
            scored += nv if nv > TOPK else 0
    att_flop = pairs * HQ * D * 4
    score_flop = scored * HI * DI * 2
    km = tr.total_ms()   # score and select run once per pass of score tiles
    att_ms = km.get("attend", float("nan")) + km.get("combine", 0.0)
    fp8 = None
    if not args.no_fp8:
        k8 = torch.empty((seqs.n_k, HKV, D), dtype=torch.uint8, device="cuda")
        v8 = torch.empty_like(k8)
        ks = torch.empty((seqs.n_k, HKV), dtype=torch.float32, device="cuda")
        vs = torch.empty_like(ks)
        qsa.quantize_kv(seqs, k, v, k8, v8, ks, vs)

        def step8():
            qsa.forward_fp8(seqs, q, k8, v8, ks, vs, q_idx, w, k_idx, k_blk, sel, out, lse, ws,
                            TOPK)

        step8()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(n):
            step8()
        torch.cuda.synchronize()
        ms8 = (time.perf_counter() - t0) * 1e3 / n
        with qsa.trace(4096) as tr8:
            step8()
        torch.cuda.synchronize()
        km8 = tr8.total_ms()
        att8 = km8.get("attend", float("nan")) + km8.get("combine", 0.0)
        fp8 = {"ms_per_step": round(ms8, 3),
               "query_tokens_per_s": round(seqs.n_q / (ms8 / 1e3), 1),
               "kernel_ms": {k2: round(v2, 4) for k2, v2 in km8.items()},
               "attention_tflops": round(att_flop / (att8 / 1e3) / 1e12, 2),
               "attention_gather_gbs": round(pairs * HKV * (2 * D + 8) / (att8 / 1e3) / 1e9, 1)}
    bwd = None if args.no_backward else run_prefill_backward(args, torch, qsa, gen, p, seqs, q, k,
                                                             v, sel, out, lse, n, pairs)
    return {
        "fp8_kv": fp8,
        "backward": bwd,
        "workload": "ragged prefill 65,535/40,001/8,190/3 tokens, budget 512 blocks",
        "ms_per_step": round(ms, 3),
        "query_tokens_per_s": round(seqs.n_q / (ms / 1e3), 1),
        "kernel_ms": {k2: round(v2, 4) for k2, v2 in km.items()},
        "attention_pairs": pairs,
        "attention_tflops": round(att_flop / (att_ms / 1e3) / 1e12, 2),
        "attention_mfma_frac": round(att_flop / (att_ms / 1e3) / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
        "attention_gather_gbs": round(pairs * HKV * D * 2 * 2 / (att_ms / 1e3) / 1e9, 1),
        # score and select of the passes run in the same launches
        "score_select_ms": round(km.get("score_select", float("nan")), 4),
        "score_tflops_incl_select": round(score_flop / (km.get("score_select", float("nan")) / 1e3)
                                          / 1e12, 2),
    }


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
    t0 = time.perf_counter()
    for _ in range(n):
        stepb()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / n
    with qsa.trace(64) as tr:
        stepb()
    torch.cuda.synchronize()
    km = tr.total_ms()   # the dK/dV kernel runs once per row window
    # five contractions per attended (query head, key): S and dP recomputed, dQ, dK, dV
    flop = pairs * HQ * D * 2 * 5
    # rows x kept blocks per KV head (the dK/dV kernel's row visits)
    return {"ms_per_step": round(ms, 3),
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
    threads = min(os.cpu_count() or 1, p.n_q)
    reps, t0 = 0, time.perf_counter()
    while True:
        sel = oracle.select(dims, p.cu_q, p.cu_k, p.q_idx, p.w, k_blk, threads=threads)
        oracle.attend(dims, p.cu_q, p.cu_k, p.q, p.k, p.v, sel, threads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= args.cpu_seconds or reps >= 50:
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
        "kernel_mean_ms": {k2: round(v2, 5) for k2, v2 in kern.items()},
    }
    if d["long_ctx"] is not None:
        line["decode_1m"] = d["long_ctx"]
    if d["mtp"] is not None:
        line["decode_multi_query"] = d["mtp"]
    if d["fp8"] is not None:
        line["decode_fp8"] = d["fp8"]
    if not args.no_prefill:
        log("prefill workload")
        line["prefill"] = run_prefill(args, torch, qsa, gen)
    if not args.no_cpu_baseline:
        import oracle
        log("CPU oracle baseline")
        line["cpu_baseline"] = run_cpu_baseline(args, d, oracle)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
