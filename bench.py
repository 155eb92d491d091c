#!/usr/bin/env python3
"""Benchmark of the paged-attention hot path on one MI355X.

Default workload (the headline): LLaMA-7B-shaped paged decode, 64 sequences,
32 heads MHA, head_dim 128, fp16, context lengths U[128, 2048], 16-token
blocks scattered through a pool of 1.2x demand.  A step is one pa_decode call
over the whole batch; inputs are resident in HBM before timing starts.

Timing protocol: W untimed warm-up steps, then K timed steps.  Before every
step (outside its timed region) a 512 MiB buffer is read, which evicts the
256 MB Infinity Cache, so each step reads its K/V from HBM as a decode step
in a real model would (the layers in between stream their weights through
the cache).  Each step is bracketed by HIP events on the stream the kernels
run on; ms_per_step is their mean.  --warm-cache drops the eviction.

Prints ONE JSON line: KV GB/s (algorithmic bytes: sum_s L_s * 2 * Hkv * D *
2 per step, divided by the measured step time), us/step, the roofline of the
dominant kernel, and the fp64 CPU oracle timed on a bounded sample of the
same workload on this host's cores.

Other workloads (--workload): llama8b_gqa, llama13b_shared (prefix sharing
built through the block pool), mixed (slot-mapped write + 2 prefill chunks +
4096 decode sequences, each call timed), tiny, prefill (the mixed step's
two 2048-row chunks alone, without its decode batch: the MFMA-bound part,
reported against the matrix-core roofline), and prefix_cache (a RAG-shaped
batch of 32 requests sharing one 1024-token document, written and prefilled
with and without automatic prefix caching), and swap (scattered blocks to
pinned host memory and back, against the host link's rate), and beam (beam
search at width 4: fork, copy-on-write, write and decode per step, and the
memory that sharing saves).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, 8 TB/s
MFMA_16BIT_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16 matrix peak
METRIC = "paged-decode KV GB/s (% of HBM peak) + \u00b5s/step, batch 64 LLaMA-7B shape"
# Every other workload names its own shape in its metric; only the 7B batch
# carries the headline metric.
WORKLOAD_METRIC = {
    "llama7b": METRIC,
    "llama8b_gqa": "paged-decode KV GB/s (% of HBM peak) + \u00b5s/step, batch 256 Llama-3.1-8B GQA shape",
    "llama13b_shared": "paged-decode KV GB/s (% of HBM peak on unique bytes) + \u00b5s/step, batch 128 "
                       "LLaMA-13B shape with shared prompt prefixes",
    "mixed": "mixed-step decode KV GB/s (% of HBM peak) + \u00b5s/step, 8192-token chunked-prefill + decode "
             "step, Llama-3.1-8B GQA shape",
    "tiny": "paged-decode KV GB/s + \u00b5s/step, 4 sequences, 4 heads, head_dim 64 (latency-bound)",
    "llama8b_long": "paged-decode KV GB/s (% of HBM peak) + \u00b5s/step, 32 sequences of 8192-32768 tokens, "
                    "Llama-3.1-8B GQA shape",
    "prefill": "chunked-prefill TFLOP/s (% of MFMA peak) + \u00b5s/step, 2 chunks of 2048 rows over 1024 cached "
               "tokens, Llama-3.1-8B GQA shape",
}
FLUSH_BYTES = 512 << 20
DECODE_SOURCES = ("paged_kv_cache_422_amd/csrc/decode.hip", "paged_kv_cache_422_amd/csrc/common.hpp",
                  "paged_kv_cache_422_amd/csrc/launch.hpp", "paged_kv_cache_422_amd/csrc/capi.cpp")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama7b",
                    choices=["llama7b", "llama8b_gqa", "llama13b_shared", "mixed", "tiny", "prefill",
                             "prefix_cache", "swap", "beam", "llama8b_long"])
    ap.add_argument("--partition", type=int, default=-1,
                    help="partition size in tokens (-1: the workload's own, 0: library default)")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle work for the cpu_baseline sample (0: skip)")
    ap.add_argument("--warm-cache", action="store_true",
                    help="do not evict the Infinity Cache between steps")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured into a HIP graph and replayed")
    ap.add_argument("--overlap", action="store_true",
                    help="mixed step: also time it with the prefill chunks on a second stream, "
                         "concurrent with the decode")
    ap.add_argument("--settle", type=float, default=5.0,
                    help="seconds to wait before building the workload, so that memory an earlier process "
                         "freed on the GPU has been reclaimed (0: no wait)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run 5 device copies of 1 GiB (torch's copy kernel), the known-size "
                         "reference that scales rocprofv3 FETCH_SIZE / WRITE_SIZE to bytes")
    return ap.parse_args()


def copy_calibration(torch):
    """Five copies of 1 GiB: each reads and writes exactly 2^30 bytes."""
    src = torch.ones(1 << 28, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": 1 << 30, "copy_calibration_bytes_written": 1 << 30,
                      "launches": 5}), flush=True)
    return 0


def source_digest(paths) -> str:
    h = hashlib.sha256()
    for p in paths:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def profiled_traffic(name: str, paths):
    """HBM bytes per launch from a committed rocprofv3 PMC summary, or None
    when there is none or the kernel source changed since it was taken."""
    path = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_b = re.search(r"^traffic_bytes_per_launch:\s*(\d+)", text, re.M)
    m_h = re.search(r"^source_sha256:\s*([0-9a-f]{64})", text, re.M)
    if not (m_b and m_h) or m_h.group(1) != source_digest(paths):
        return None
    return int(m_b.group(1))


class StepTimer:
    """Per-step HIP events on the current stream, with an optional cache
    eviction (a full read of a 512 MiB buffer) before each step."""

    def __init__(self, torch, evict: bool):
        self.torch = torch
        self.junk = torch.ones(FLUSH_BYTES // 4, dtype=torch.float32, device="cuda") if evict else None

    def evict(self):
        if self.junk is not None:
            self.junk.sum()

    def run(self, steps, fns):
        """fns: list of callables forming one step; returns per-call ms lists."""
        t = self.torch
        ev = [[t.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)] for _ in range(steps)]
        t.cuda.synchronize()
        t0 = time.perf_counter()
        for e in ev:
            self.evict()
            e[0].record()
            for i, fn in enumerate(fns):
                fn()
                e[i + 1].record()
        t.cuda.synchronize()
        wall = (time.perf_counter() - t0) / steps * 1e3
        per = [[e[i].elapsed_time(e[i + 1]) for e in ev] for i in range(len(fns))]
        total = [e[0].elapsed_time(e[-1]) for e in ev]
        return per, total, wall


def achievable_copy_gbs(torch, nbytes=2 << 30, reps=10):
    """Device-to-device copy of 2 GiB (read + write bytes per second): the
    achievable HBM rate on this machine, beside the 8 TB/s peak."""
    a = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    gbs = 2 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, b
    return gbs


def achievable_gemm_tflops(torch, n=8192, reps=10):
    """bf16 n x n x n matrix product through torch (hipBLASLt): the achievable
    matrix-core rate on this machine, beside the 2.5 PFLOP/s peak."""
    a = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    b = torch.randn(n, n, device="cuda").to(torch.bfloat16)
    c = a @ b
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        c = a @ b
    e1.record()
    torch.cuda.synchronize()
    del a, b, c
    return 2 * n ** 3 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e12


def mean(xs):
    return sum(xs) / max(len(xs), 1)


def median(xs):
    s = sorted(xs)
    return s[len(s) // 2] if s else 0.0


def percentile(xs, q):
    """Nearest-rank percentile (q in 0..100) of a list of step times."""
    s = sorted(xs)
    if not s:
        return 0.0
    k = max(0, min(len(s) - 1, math.ceil(q / 100 * len(s)) - 1))
    return s[k]


def step_stats(total_ms):
    """Mean, median, p10 and p90 of per-step times, in us."""
    return {"us_per_step": round(mean(total_ms) * 1e3, 2), "us_per_step_median": round(median(total_ms) * 1e3, 2),
            "us_per_step_p10": round(percentile(total_ms, 10) * 1e3, 2),
            "us_per_step_p90": round(percentile(total_ms, 90) * 1e3, 2)}


def host_info():
    """The host the oracle runs on: cores this process may use, CPU model,
    and numpy's BLAS library and its thread count."""
    info = {"host_cores": len(os.sched_getaffinity(0)), "cpu_model": None, "blas": None}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    info["cpu_model"] = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        blas = [b for b in threadpool_info() if b.get("user_api") == "blas"]
        if blas:
            info["blas"] = {"library": blas[0].get("internal_api"), "version": blas[0].get("version"),
                            "threads": blas[0].get("num_threads")}
    except Exception:  # pragma: no cover - threadpoolctl missing
        pass
    return info


def cpu_baseline_line(value, unit, threads, sample, **extra):
    line = {"value": value, "unit": unit, "cores": threads, "threads_used": threads, "kind": "oracle",
            "sample": sample}
    line.update(host_info())
    line.update(extra)
    return line


def bits(t):
    import numpy as np
    import torch
    t = t.detach().cpu().contiguous()
    return t.numpy() if t.dtype == torch.float16 else t.view(torch.int16).numpy().view(np.uint16)


def cpu_oracle_decode(q, kc, vc, block_tables, context_lens, scale, dtype, budget_s, seqs=None):
    """fp64 oracle over sequences in order (wrapping around) until the time
    budget is spent.  Device -> host copies are not timed.  Returns (KV GB/s
    processed, sequences done, wall seconds, threads used)."""
    import numpy as np
    import torch
    from oracle import attention as A

    order = list(range(len(context_lens))) if seqs is None else list(seqs)
    per_seq = {}
    qh = bits(q)
    Hkv, D = vc.shape[1], vc.shape[3]
    t0 = time.perf_counter()
    c0 = time.process_time()
    done = bytes_done = 0
    spent = 0.0
    while spent < budget_s:
        s = order[done % len(order)]
        if s not in per_seq:
            L = int(context_lens[s])
            nb = -(-L // 16)
            idx = torch.from_numpy(block_tables[s, :nb].astype(np.int64)).to(kc.device)
            pause = time.perf_counter()
            per_seq[s] = (L, bits(kc[idx]), bits(vc[idx]), np.arange(nb, dtype=np.int32)[None])
            t0 += time.perf_counter() - pause          # copy-back is not oracle work
        L, kh, vh, bt = per_seq[s]
        A.decode(qh[s:s + 1], kh, vh, bt, [L], scale, dtype)
        bytes_done += L * 2 * Hkv * D * 2
        done += 1
        spent = time.perf_counter() - t0
    cpu = time.process_time() - c0
    threads = max(1, round(cpu / spent)) if spent > 0 else 1
    return bytes_done / spent / 1e9, done, spent, threads


def cpu_oracle_mixed(w, kc, vc, q_dec, q_pre, n_decode=256, seed=5):
    """fp64 oracle over the mixed step's work after its write: both prefill
    chunks in full (every row and head) plus a seeded sample of n_decode
    decode sequences.  Only the blocks they read are copied back (not
    timed).  Returns (prefill s, decode s, decode KV bytes, sequences,
    threads used)."""
    import numpy as np
    import torch
    from oracle import attention as A

    rng = np.random.default_rng(seed)
    seqs = sorted(rng.choice(w.num_decode, n_decode, replace=False).tolist())
    need = set()
    for s_ in seqs:
        need.update(w.decode_bt[s_, :-(-int(w.decode_lens[s_]) // 16)].tolist())
    for c in range(w.num_chunks):
        need.update(w.prefill_bt[c, :-(-int(w.prefill_seq_lens[c]) // 16)].tolist())
    need = np.array(sorted(need), dtype=np.int64)
    remap = np.zeros(w.num_blocks, dtype=np.int64)
    remap[need] = np.arange(len(need))
    idx = torch.from_numpy(need).to(kc.device)
    kh, vh = bits(kc[idx]), bits(vc[idx])
    qd, qp = bits(q_dec), bits(q_pre)
    pbt = remap[w.prefill_bt].astype(np.int32)
    dbt = remap[w.decode_bt].astype(np.int32)
    c0, t0 = time.process_time(), time.perf_counter()
    A.prefill(qp, kh, vh, pbt, w.q_start_loc, w.prefill_seq_lens, w.scale, w.dtype)
    t1 = time.perf_counter()
    A.decode(qd, kh, vh, dbt, w.decode_lens, w.scale, w.dtype, seqs=seqs)
    t2 = time.perf_counter()
    cpu = time.process_time() - c0
    threads = max(1, round(cpu / (t2 - t0))) if t2 > t0 else 1
    dec_bytes = int(sum(int(w.decode_lens[s_]) for s_ in seqs)) * 2 * w.num_kv_heads * w.head_dim * 2
    return t1 - t0, t2 - t1, dec_bytes, len(seqs), threads


def build_shared_cache(torch, pa, w, k_tok, v_tok):
    """Lay the prefix-sharing workload out through the block pool: each
    group's prompt is appended once, forked to the other members, then every
    member appends its own tokens (copy-on-write for the shared partial
    block)."""
    pool = pa.BlockPool(w.num_blocks, 16, 7)
    H, D = w.num_kv_heads, w.head_dim
    kc = torch.zeros(pa.k_cache_shape(w.num_blocks, H, D), dtype=k_tok.dtype, device="cuda")
    vc = torch.zeros(pa.v_cache_shape(w.num_blocks, H, D), dtype=k_tok.dtype, device="cuda")
    seqs = [None] * w.num_seqs

    def write(i, sid, lo, hi):
        slots, cow = pool.append(sid, hi - lo)
        if cow:
            pa.copy_blocks(kc, vc, torch.tensor(cow, dtype=torch.int32, device="cuda"))
        rows = torch.from_numpy(w.token_rows[i][lo:hi]).cuda()
        pa.write_kv(k_tok[rows], v_tok[rows], kc, vc, torch.tensor(slots, dtype=torch.int64, device="cuda"))

    G = w.group_size
    for k in range(w.num_seqs // G):
        P = int(w.prefix_lens[k])
        members = list(range(k * G, (k + 1) * G))
        root = pool.create()
        write(members[0], root, 0, P)
        seqs[members[0]] = root
        for s in members[1:]:
            seqs[s] = pool.fork(root)
        for s in members:
            write(s, seqs[s], P, int(w.context_lens[s]))
    bt, ctx = pool.block_tables(seqs, w.bt_stride, pad=0)
    torch.cuda.synchronize()
    used = pool.num_blocks - pool.num_free
    return kc, vc, bt, ctx, used


def bench_prefix_cache(args, np, torch, pa):
    """RAG-shaped batch: R requests = one shared 1024-token document + a
    unique 256-token query each, 8B-GQA shape, bf16.  A request served
    earlier left the document's blocks in the cache (untimed set-up), so with
    prefix caching each request writes and prefills only its 256 new tokens
    over 1024 cached keys; without it, all 1280.  A step = pa_write_kv of the
    batch's new tokens + pa_prefill_chunk of its chunks; host admission
    (pool calls) is timed separately."""
    R, DOC, QRY, Hq, Hkv, D, B = 32, 1024, 256, 32, 8, 128, 16
    L = DOC + QRY
    rng = np.random.Generator(np.random.PCG64(4230))
    doc = rng.integers(0, 32000, DOC).tolist()
    queries = [rng.integers(0, 32000, QRY).tolist() for _ in range(R + 1)]
    num_blocks = int(1.2 * (R + 1) * (L // B))
    g = torch.Generator(device="cuda").manual_seed(4230)
    dt = torch.bfloat16
    kc = torch.randn(pa.k_cache_shape(num_blocks, Hkv, D, B), generator=g, device="cuda").to(dt)
    vc = torch.randn(pa.v_cache_shape(num_blocks, Hkv, D, B), generator=g, device="cuda").to(dt)

    def admit(caching):
        pool = pa.BlockPool(num_blocks, B, 4230, prefix_caching=caching)
        warm = pool.create()
        pool.append_tokens(warm, doc + queries[R], L - 1)
        pool.free(warm)
        t0 = time.perf_counter()
        seqs, slots, hits = [], [], []
        for r in range(R):
            sid = pool.create()
            sl, cow, hit = pool.append_tokens(sid, doc + queries[r], L - 1)
            seqs.append(sid)
            slots += sl[hit:]
            hits.append(hit)
        tabs, ctx = pool.block_tables(seqs, stride=L // B)
        host_us = (time.perf_counter() - t0) * 1e6 / R
        return tabs, ctx, np.array(slots, np.int64), hits, host_us

    def prefill_flop(n_cached, n):
        return Hq * 4 * D * (n * n_cached + n * (n + 1) // 2)

    results = {}
    for caching in (True, False):
        tabs, ctx, slots, hits, host_us = admit(caching)
        host = [admit(caching)[4] for _ in range(5)]
        n_new = [L - h for h in hits]
        T = sum(n_new)
        k_new = torch.randn(T, Hkv, D, generator=g, device="cuda").to(dt)
        v_new = torch.randn(T, Hkv, D, generator=g, device="cuda").to(dt)
        q = torch.randn(T, Hq, D, generator=g, device="cuda").to(dt)
        out = torch.empty_like(q)
        sm = torch.from_numpy(slots).cuda()
        bt = torch.from_numpy(tabs).cuda()
        qsl = torch.from_numpy(np.concatenate([[0], np.cumsum(n_new)]).astype(np.int32)).cuda()
        sl_t = torch.from_numpy(ctx).cuda()
        scale = 1.0 / math.sqrt(D)
        fns = [lambda: pa.write_kv(k_new, v_new, kc, vc, sm),
               lambda: pa.prefill_chunk(out, q, kc, vc, bt, qsl, sl_t, max(n_new), L, scale)]
        timer = StepTimer(torch, evict=not args.warm_cache)
        timer.run(args.warmup, fns)
        per, total, wall = timer.run(args.steps, fns)
        flop = sum(prefill_flop(h, n) for h, n in zip(hits, n_new))
        results[caching] = {
            **step_stats(total), "write_kv_us": round(mean(per[0]) * 1e3, 2),
            "prefill_us": round(mean(per[1]) * 1e3, 2), "new_tokens": T, "cached_tokens": sum(hits),
            "prefill_flop": int(flop), "prefill_tflops": round(flop / (mean(per[1]) * 1e-3) / 1e12, 1),
            "host_admit_us_per_request": round(float(np.median(host)), 2), "wall_ms_per_step": round(wall, 5)}
    on, off = results[True], results[False]
    tflops = on["prefill_tflops"]
    line = {
        "metric": "prefill step time of a RAG-shaped batch with automatic prefix caching",
        "value": on["us_per_step"], "unit": "us", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(on["us_per_step"] / 1e3, 5), "higher_is_better": False, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"prefix_cache: {R} requests of one shared {DOC}-token document + a unique "
                               f"{QRY}-token query, {Hq} query heads over {Hkv} KV heads, head_dim {D}, bf16; "
                               "step = slot-mapped write of the new tokens + chunked prefill",
                   "cache": "warm" if args.warm_cache else "Infinity Cache evicted before each step",
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "mfma", "achieved": tflops, "peak": MFMA_16BIT_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / MFMA_16BIT_PEAK_TFLOPS, 4), "traffic": None,
                     "kernel": "pa_prefill_chunk (prefill_kernel), cached prefix"},
        "with_prefix_cache": on, "without_prefix_cache": off,
        "speedup": round(off["us_per_step"] / on["us_per_step"], 2),
        "cpu_baseline": None,
    }
    line["settle_s"] = args.settle
    print(json.dumps(line), flush=True)
    return 0


PCIE_PEAK_GBS = 64.0   # PCIe 5.0 x16, one direction


def bench_swap(args, np, torch, pa):
    """Swap traffic at the 8B-GQA cache shape (8 KV heads, head_dim 128,
    bf16, 64 KiB of K + V per block): 4096 scattered device blocks go to
    scattered blocks of a pinned host swap space and back, each direction one
    pa_swap_blocks launch.  A contiguous DMA copy of the same byte count
    (torch's pinned <-> device copy) is timed beside it as the achievable
    host-link rate."""
    N, NH, NSW, H, D, B = 6144, 4608, 4096, 8, 128, 16
    rng = np.random.Generator(np.random.PCG64(4231))
    dev_ids = rng.permutation(N)[:NSW].astype(np.int32)
    host_ids = rng.permutation(NH)[:NSW].astype(np.int32)
    g = torch.Generator(device="cuda").manual_seed(4231)
    dt = torch.bfloat16
    kc = torch.randn(pa.k_cache_shape(N, H, D, B), generator=g, device="cuda").to(dt)
    vc = torch.randn(pa.v_cache_shape(N, H, D, B), generator=g, device="cuda").to(dt)
    hk = torch.empty(pa.k_cache_shape(NH, H, D, B), dtype=dt).pin_memory()
    hv = torch.empty(pa.v_cache_shape(NH, H, D, B), dtype=dt).pin_memory()
    out_pairs = torch.from_numpy(np.stack([dev_ids, host_ids], 1)).cuda()
    in_pairs = torch.from_numpy(np.stack([host_ids, dev_ids], 1)).cuda()
    nbytes = NSW * 2 * H * B * D * 2
    flat_h = torch.empty(nbytes // 2, dtype=dt).pin_memory()
    flat_d = torch.empty(nbytes // 2, dtype=dt, device="cuda")
    timer = StepTimer(torch, evict=not args.warm_cache)
    fns = {
        "swap_out": lambda: pa.swap_blocks(kc, vc, hk, hv, out_pairs, pa.PA_SWAP_OUT),
        "swap_in": lambda: pa.swap_blocks(kc, vc, hk, hv, in_pairs, pa.PA_SWAP_IN),
        "dma_d2h": lambda: flat_h.copy_(flat_d, non_blocking=True),
        "dma_h2d": lambda: flat_d.copy_(flat_h, non_blocking=True),
    }
    res = {}
    for k, fn in fns.items():
        timer.run(args.warmup, [fn])
        per, total, wall = timer.run(args.steps, [fn])
        ms = mean(total)
        res[k] = {"us": round(ms * 1e3, 1), "GB/s": round(nbytes / (ms * 1e-3) / 1e9, 2), **step_stats(total)}
    rt_ms = (res["swap_out"]["us"] + res["swap_in"]["us"]) / 1e3
    gbs = round(2 * nbytes / (rt_ms * 1e-3) / 1e9, 2)
    line = {
        "metric": "KV swap GB/s over the host link (swap-out + swap-in of scattered blocks)",
        "value": gbs, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(rt_ms, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"swap: {NSW} scattered blocks of {N} (8 KV heads, head_dim 128, bf16, 64 KiB "
                               f"each) to scattered blocks of a {NH}-block pinned host swap space and back; "
                               "step = one swap-out + one swap-in launch",
                   "bytes_each_way": nbytes, "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "pcie", "achieved": gbs, "peak": PCIE_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / PCIE_PEAK_GBS, 4), "traffic": None,
                     "kernel": "pa_swap_blocks (copy_blocks_kernel over mapped host memory)"},
        "directions": res,
        "cpu_baseline": None,
    }
    line["settle_s"] = args.settle
    print(json.dumps(line), flush=True)
    return 0


def bench_beam(args, np, torch, pa):
    """Beam search at width 4 over 64 requests with 1024-token prompts
    (8B-GQA shape, bf16): every step each new beam picks a parent (seeded,
    beam 0 likeliest), a parent taken twice is forked, unchosen beams are
    freed, and every beam appends one token (copy-on-write of a shared last
    block).  Device work per step: the block copies, the slot-mapped write of
    256 tokens and a decode over the 256 beams.  Reports the step time and
    the blocks the shared layout holds against private copies per beam."""
    R, WID, PROMPT, Hq, Hkv, D, B = 64, 4, 1024, 32, 8, 128, 16
    steps_total = args.warmup + args.steps
    max_len = PROMPT + steps_total + 1
    N = int(1.2 * R * WID * (-(-max_len // B)))
    rng = np.random.Generator(np.random.PCG64(4232))
    parent_p = np.array([0.4, 0.3, 0.2, 0.1])
    g = torch.Generator(device="cuda").manual_seed(4232)
    dt = torch.bfloat16
    kc = torch.randn(pa.k_cache_shape(N, Hkv, D, B), generator=g, device="cuda").to(dt)
    vc = torch.randn(pa.v_cache_shape(N, Hkv, D, B), generator=g, device="cuda").to(dt)
    pool = pa.BlockPool(N, B, 4232)
    beams = []
    for _ in range(R):
        sid = pool.create()
        pool.append(sid, PROMPT)          # prompt K/V: the cache's random contents stand in for it
        beams.append([sid] + [pool.fork(sid) for _ in range(WID - 1)])
    k_new = torch.randn(R * WID, Hkv, D, generator=g, device="cuda").to(dt)
    v_new = torch.randn(R * WID, Hkv, D, generator=g, device="cuda").to(dt)
    q = torch.randn(R * WID, Hq, D, generator=g, device="cuda").to(dt)
    out = torch.empty_like(q)
    scale = 1.0 / math.sqrt(D)
    stride = -(-max_len // B)
    ws = torch.empty(max(pa.decode_workspace_size(R * WID, Hq, D, max_len, 0, Hkv), 1),
                     dtype=torch.uint8, device="cuda")

    # Parent choices drawn up front, so the timed host work is the pool's.
    choices = np.sort(rng.choice(WID, (steps_total, R, WID), p=parent_p), axis=-1).tolist()

    def host_step(i):
        """Beam bookkeeping for step i (the selection itself is the
        harness's part); returns the step's pool outputs and the time spent
        in pool calls."""
        to_fork, to_free, fork_at = [], [], set()
        for r in range(R):
            taken = set()
            for j, p in enumerate(choices[i][r]):
                if p in taken:
                    to_fork.append(beams[r][p])
                    fork_at.add((r, j))
                else:
                    taken.add(p)
            to_free += [beams[r][p] for p in range(WID) if p not in taken]
        t0 = time.perf_counter()
        children = pool.fork_many(to_fork)
        pool.free_many(to_free)
        t_pool = time.perf_counter() - t0
        children = iter(children)
        for r in range(R):
            old = beams[r]
            beams[r] = [next(children) if (r, j) in fork_at else old[p] for j, p in enumerate(choices[i][r])]
        seqs = [s for req in beams for s in req]
        t0 = time.perf_counter()
        slots, cows = pool.append_many(seqs, [1] * len(seqs))
        tabs, ctx = pool.block_tables(seqs, stride=stride)
        t_pool += time.perf_counter() - t0
        return slots, cows, tabs, ctx, t_pool

    # Per-step host outputs go up through two alternating pinned staging sets
    # (asynchronous copies on the stream); a set is refilled only after the
    # copies that read it have run.
    nb = R * WID
    stage = [{"slots": torch.empty(nb, dtype=torch.int64).pin_memory(),
              "cows": torch.empty(nb, 2, dtype=torch.int32).pin_memory(),
              "tabs": torch.empty(nb, stride, dtype=torch.int32).pin_memory(),
              "ctx": torch.empty(nb, dtype=torch.int32).pin_memory()} for _ in range(2)]
    dev = [{k: torch.empty_like(v, device="cuda") for k, v in st.items()} for st in stage]
    done = [None, None]
    host_us, cow_counts, dev_ms, wall_ms = [], [], [], []
    t_wall = None
    for i in range(steps_total):
        if i == args.warmup:
            torch.cuda.synchronize()
            t_wall = time.perf_counter()
        slots, cows, tabs, ctx, host = host_step(i)
        sb, db = stage[i % 2], dev[i % 2]
        if done[i % 2] is not None:
            done[i % 2].synchronize()
        sb["slots"].numpy()[:] = slots
        sb["tabs"].numpy()[:] = tabs
        sb["ctx"].numpy()[:] = ctx
        if cows:
            sb["cows"].numpy()[:len(cows)] = cows
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for k in sb:
            db[k].copy_(sb[k], non_blocking=True)
        done[i % 2] = torch.cuda.Event()
        done[i % 2].record()
        if cows:
            pa.copy_blocks(kc, vc, db["cows"][:len(cows)])
        pa.write_kv(k_new, v_new, kc, vc, db["slots"])
        pa.decode(out, q, kc, vc, db["tabs"], db["ctx"], max_len, scale, 0, ws)
        e1.record()
        if i >= args.warmup:
            host_us.append(host * 1e6)
            cow_counts.append(len(cows))
            dev_ms.append((e0, e1))
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t_wall) / args.steps * 1e3
    dev = [a.elapsed_time(b) for a, b in dev_ms]
    seqs = [s for req in beams for s in req]
    used = N - pool.num_free
    private = sum(-(-pool.block_table(s)[1] // B) for s in seqs)
    kv_bytes = int(sum(pool.block_table(s)[1] for s in seqs)) * 2 * Hkv * D * 2
    # Each physical block counted once, with the slots its holders use: a
    # prompt block shared by four beams is read from HBM once, then from cache.
    filled = {}
    for sq in seqs:
        tab, n_tok = pool.block_table(sq)
        for j, phys in enumerate(tab):
            filled[phys] = max(filled.get(phys, 0), min(B, n_tok - B * j))
    unique_bytes = int(sum(filled.values())) * 2 * Hkv * D * 2
    uniq_gbs = unique_bytes / (mean(dev) * 1e-3) / 1e9
    line = {
        "metric": "beam-search step (width 4): fork / copy-on-write / write / decode, and memory saved by sharing",
        "value": round(mean(dev) * 1e3, 2), "unit": "us", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        **step_stats(dev),
        "ms_per_step": round(mean(dev), 5), "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": f"beam: {R} requests x {WID} beams, {PROMPT}-token prompts, 32 query heads over 8 KV "
                               "heads, head_dim 128, bf16; step = parent choice, fork/free, one token per beam "
                               "(copy-on-write), block copies + slot-mapped write + decode of all beams",
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": round(uniq_gbs, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(uniq_gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "bytes": "unique physical KV bytes the last step's decode reads (each shared block once), "
                              "over the whole device step",
                     "kernel": "whole device step (block copies + write + decode)"},
        "logical_kv_bytes": kv_bytes, "unique_kv_bytes": unique_bytes,
        "logical_GBps": round(kv_bytes / (mean(dev) * 1e-3) / 1e9, 2),
        "host_pool_us_per_step": round(float(np.median(host_us)), 1),
        "copy_on_write_pairs_per_step": round(mean(cow_counts), 2),
        "wall_ms_per_step": round(wall, 5),
        "blocks_in_use": int(used), "blocks_if_private": int(private),
        "memory_saved_by_sharing": round(1 - used / private, 4),
        "cpu_baseline": None,
    }
    line["settle_s"] = args.settle
    print(json.dumps(line), flush=True)
    return 0


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only (asked for --gpus {args.gpus}); "
              "the path shards by sequence or KV head with no exchange inside attention, "
              "but runs on more than one GPU are not part of it.", file=sys.stderr)
        return 2
    import numpy as np
    import torch
    import paged_kv_cache_422_amd as pa
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    if args.copy_calibration:
        return copy_calibration(torch)
    if args.settle > 0:
        # The driver reclaims device memory that an earlier process freed in
        # the background, for a few seconds after that process ends, and the
        # reclaim takes HBM bandwidth: right after a process that touched
        # 64-160 GiB exited, the 7B batch read 196-197 us per step, six
        # seconds later 193 us (same box).  The test suite is such a process.
        time.sleep(args.settle)
    name = args.workload
    if name == "prefix_cache":
        return bench_prefix_cache(args, np, torch, pa)
    if name == "swap":
        return bench_swap(args, np, torch, pa)
    if name == "beam":
        return bench_beam(args, np, torch, pa)
    w = W.mixed(num_decode=0) if name == "prefill" else W.make_workload(name)
    timer = StepTimer(torch, evict=not args.warm_cache)
    extra = {}

    if name == "prefill":
        kc, vc, k_new, v_new, q_dec, q_pre = w.make_tensors("cuda")
        sm = torch.from_numpy(w.slot_mapping).cuda()
        pbt = torch.from_numpy(w.prefill_bt).cuda()
        qsl = torch.from_numpy(w.q_start_loc).cuda()
        psl = torch.from_numpy(w.prefill_seq_lens).cuda()
        out_pre = torch.empty_like(q_pre)
        pa.write_kv(k_new, v_new, kc, vc, sm)
        fns = [lambda: pa.prefill_chunk(out_pre, q_pre, kc, vc, pbt, qsl, psl, w.prefill_chunk,
                                        w.prefill_cached + w.prefill_chunk, w.scale)]
        timer.run(args.warmup, fns)
        per, total, wall = timer.run(args.steps, fns)
        ms = mean(total)
        tflops = w.prefill_flops / (ms * 1e-3) / 1e12
        line = {
            "metric": WORKLOAD_METRIC["prefill"], "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
            **step_stats(total),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": w.dtype,
            "data": "synthetic",
            "config": {"workload": f"prefill: {w.num_chunks} chunks of {w.prefill_chunk} query rows over "
                                   f"{w.prefill_cached} cached tokens, {w.num_q_heads} query heads over "
                                   f"{w.num_kv_heads} KV heads, head_dim {w.head_dim}, {w.dtype}",
                       "flop_per_step": int(w.prefill_flops),
                       "cache": "warm" if args.warm_cache else "Infinity Cache evicted before each step",
                       "parallelism": "none (1 GPU)"},
            "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": MFMA_16BIT_PEAK_TFLOPS,
                         "unit": "TFLOP/s", "frac": round(tflops / MFMA_16BIT_PEAK_TFLOPS, 4),
                         "traffic": None, "kernel": "pa_prefill_chunk (prefill_kernel)"},
            "cpu_baseline": None,
            "wall_ms_per_step": round(wall, 5),
        }
        gemm = achievable_gemm_tflops(torch)
        line["achievable"] = {"bf16_gemm_tflops": round(gemm, 1), "frac_of_gemm": round(tflops / gemm, 4),
                              "reference": "torch bf16 8192^3 matrix product (hipBLASLt), same run"}
        line["settle_s"] = args.settle
        print(json.dumps(line), flush=True)
        return 0

    if name == "mixed":
        kc, vc, k_new, v_new, q_dec, q_pre = w.make_tensors("cuda")
        sm = torch.from_numpy(w.slot_mapping).cuda()
        pbt = torch.from_numpy(w.prefill_bt).cuda()
        qsl = torch.from_numpy(w.q_start_loc).cuda()
        psl = torch.from_numpy(w.prefill_seq_lens).cuda()
        dbt = torch.from_numpy(w.decode_bt).cuda()
        dctx = torch.from_numpy(w.decode_lens).cuda()
        P = w.partition_size if args.partition < 0 else args.partition
        ws = torch.empty(max(pa.decode_workspace_size(w.num_decode, w.num_q_heads, w.head_dim,
                                                      w.max_model_len, P, w.num_kv_heads), 1),
                         dtype=torch.uint8, device="cuda")
        out_pre, out_dec = torch.empty_like(q_pre), torch.empty_like(q_dec)
        fns = [lambda: pa.write_kv(k_new, v_new, kc, vc, sm),
               lambda: pa.prefill_chunk(out_pre, q_pre, kc, vc, pbt, qsl, psl, w.prefill_chunk,
                                        w.prefill_cached + w.prefill_chunk, w.scale),
               lambda: pa.decode(out_dec, q_dec, kc, vc, dbt, dctx, w.max_model_len, w.scale, P, ws)]
        kv_bytes = w.decode_kv_bytes
        q_dec_t, kc_t, vc_t, bt_np, ctx_np = q_dec, kc, vc, w.decode_bt, w.decode_lens
        num_seqs, Hq, Hkv, D = w.num_decode, w.num_q_heads, w.num_kv_heads, w.head_dim
    else:
        if name == "llama13b_shared":
            q, k_tok, v_tok = w.make_tensors("cuda")
            kc, vc, bt_np, ctx_np, used = build_shared_cache(torch, pa, w, k_tok, v_tok)
            del k_tok, v_tok
            P = 0 if args.partition < 0 else args.partition
            extra["unique_kv_bytes_per_step"] = w.unique_kv_bytes
            extra["pool_blocks_used"] = int(used)
        else:
            q, kc, vc = w.make_tensors("cuda")
            bt_np, ctx_np = w.block_tables, w.context_lens
            P = w.partition_size if args.partition < 0 else args.partition
        bt = torch.from_numpy(bt_np).cuda()
        ctx = torch.from_numpy(ctx_np).cuda()
        ws = torch.empty(max(pa.decode_workspace_size(w.num_seqs, w.num_q_heads, w.head_dim,
                                                      w.max_model_len, P, w.num_kv_heads), 1),
                         dtype=torch.uint8, device="cuda")
        out = torch.empty_like(q)
        fns = [lambda: pa.decode(out, q, kc, vc, bt, ctx, w.max_model_len, w.scale, P, ws)]
        kv_bytes = w.kv_bytes
        q_dec_t, kc_t, vc_t = q, kc, vc
        num_seqs, Hq, Hkv, D = w.num_seqs, w.num_q_heads, w.num_kv_heads, w.head_dim

    timer.run(args.warmup, fns)
    per, total, wall = timer.run(args.steps, fns)
    ms = mean(total)
    dec_ms = mean(per[-1])                       # pa_decode is the last call of every step
    gbs = kv_bytes / (dec_ms * 1e-3) / 1e9

    if name in ("llama7b", "llama8b_gqa"):
        # The same decode over the same context lengths with every sequence's
        # blocks consecutive and in order: what the scattered layout costs.
        nb_s = (ctx_np.astype(np.int64) + 15) // 16
        starts = np.concatenate([[0], np.cumsum(nb_s)[:-1]])
        bt_c = np.zeros_like(bt_np)
        for s_i in range(len(ctx_np)):
            bt_c[s_i, :nb_s[s_i]] = starts[s_i] + np.arange(nb_s[s_i])
        assert int(nb_s.sum()) <= kc_t.shape[0]
        bt_ct = torch.from_numpy(bt_c).cuda()
        fn_c = [lambda: pa.decode(out, q, kc, vc, bt_ct, ctx, w.max_model_len, w.scale, P, ws)]
        timer.run(args.warmup, fn_c)
        _, tot_c, _ = timer.run(args.steps, fn_c)
        gbs_c = kv_bytes / (mean(tot_c) * 1e-3) / 1e9
        copy = achievable_copy_gbs(torch)
        extra["achievable"] = {
            "copy_GBps": round(copy, 1), "frac_of_copy": round(gbs / copy, 4),
            "contiguous_blocks_GBps": round(gbs_c, 1), "frac_of_contiguous": round(gbs / gbs_c, 4),
            "reference": "2 GiB device-to-device copy (read + write bytes); the same decode with each "
                         "sequence's blocks consecutive in memory, same run"}

    if args.overlap and name == "mixed":
        # The prefill chunks and the decode only read the cache once the
        # write is done, so a caller can run them concurrently: the prefill on
        # a second stream (default priority) that waits for the write, the
        # decode on this one, and this stream waits for the second at the end.
        side = torch.cuda.Stream()
        written = torch.cuda.Event()

        def step_two_streams():
            fns[0]()
            written.record()
            side.wait_event(written)
            with torch.cuda.stream(side):
                fns[1]()
            fns[2]()
            torch.cuda.current_stream().wait_stream(side)

        timer.run(args.warmup, [step_two_streams])
        _, tot_o, wall_o = timer.run(args.steps, [step_two_streams])
        extra["two_streams"] = {"us_per_step": round(mean(tot_o) * 1e3, 2), "wall_ms_per_step": round(wall_o, 5),
                                "one_stream_us_per_step": round(ms * 1e3, 2)}

    if args.graph:
        # The same calls captured once into a HIP graph; each step replays it.
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for fn in fns:
                fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for fn in fns:
                fn()
        timer.run(args.warmup, [graph.replay])
        _, tot_g, wall_g = timer.run(args.steps, [graph.replay])
        extra["hip_graph"] = {"us_per_step": round(mean(tot_g) * 1e3, 2), "wall_ms_per_step": round(wall_g, 5),
                              "eager_us_per_step": round(ms * 1e3, 2), "eager_wall_ms_per_step": round(wall, 5)}

    if name == "llama8b_gqa" and P != 0:
        # The workload fixes 512-token split-KV partitions; also time the same
        # batch with the library's default partitioning for comparison.
        P_def = pa.default_partition_size(num_seqs, Hq, Hkv, D, w.max_model_len)
        ws_def = torch.empty(max(pa.decode_workspace_size(w.num_seqs, Hq, D, w.max_model_len, 0, Hkv), 1),
                             dtype=torch.uint8, device="cuda")
        fn_def = [lambda: pa.decode(out, q, kc, vc, bt, ctx, w.max_model_len, w.scale, 0, ws_def)]
        timer.run(args.warmup, fn_def)
        _, tot_def, _ = timer.run(args.steps, fn_def)
        gbs_def = kv_bytes / (mean(tot_def) * 1e-3) / 1e9
        extra["library_default_partition"] = {"partition_size": P_def, "us_per_step": round(mean(tot_def) * 1e3, 2),
                                              "GB/s": round(gbs_def, 2), "frac_hbm": round(gbs_def / HBM_PEAK_GBS, 4)}

    if name == "mixed":
        w_ms, p_ms = mean(per[0]), mean(per[1])
        extra["calls_us"] = {"write_kv": round(w_ms * 1e3, 2), "prefill_chunk": round(p_ms * 1e3, 2),
                             "decode": round(dec_ms * 1e3, 2)}
        extra["write_kv"] = {"bytes": w.write_bytes, "GB/s": round(w.write_bytes / (w_ms * 1e-3) / 1e9, 1),
                             "frac_hbm": round(w.write_bytes / (w_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
        tflops = w.prefill_flops / (p_ms * 1e-3) / 1e12
        extra["prefill_chunk"] = {"flop": w.prefill_flops, "TFLOP/s": round(tflops, 1),
                                  "frac_mfma": round(tflops / MFMA_16BIT_PEAK_TFLOPS, 4)}

    cpu = None
    if args.cpu_budget > 0 and name == "mixed":
        print("bench.py: fp64 oracle on both prefill chunks and 256 decode sequences", file=sys.stderr,
              flush=True)
        t_pre, t_dec, dec_bytes, n_seq, threads = cpu_oracle_mixed(w, kc, vc, q_dec, q_pre)
        cpu = cpu_baseline_line(
            round(dec_bytes / t_dec / 1e9, 6), "GB/s", threads,
            f"both prefill chunks in full ({w.num_chunks} x {w.prefill_chunk} rows, all {Hq} query heads) in "
            f"{t_pre:.1f} s, then {n_seq} seeded decode sequences of the {num_seqs} (all {Hq} query heads "
            f"each) in {t_dec:.1f} s; value = decode KV GB/s of that sample",
            prefill_s=round(t_pre, 3), decode_sample_s=round(t_dec, 3),
            step_s_extrapolated=round(t_pre + t_dec * num_seqs / n_seq, 2),
            extrapolation="prefill time + sample decode time x (decode sequences / sample); the write is a "
                          "bit copy and not timed")
    elif args.cpu_budget > 0:
        gbs_cpu, n_seq, wall_cpu, threads = cpu_oracle_decode(
            q_dec_t, kc_t, vc_t, bt_np, ctx_np, w.scale, w.dtype, args.cpu_budget)
        cpu = cpu_baseline_line(
            round(gbs_cpu, 6), "GB/s", threads,
            f"{n_seq} single-sequence fp64 decodes (all {Hq} query heads each) over the {num_seqs} "
            f"sequences of this workload in order, in {wall_cpu:.1f} s; KV GB/s of the sample")

    traffic = profiled_traffic(f"decode_{name}_pmc.md", DECODE_SOURCES)
    # A shared prompt's blocks are read once per sequence that shares them,
    # partly from cache, so the HBM roofline of the shared-prefix workload
    # counts each physical block once; `value` keeps the logical bytes.
    roof_gbs, roof_bytes = gbs, "logical KV bytes (sum over sequences of L x 2 x Hkv x D x 2)"
    if "unique_kv_bytes_per_step" in extra:
        roof_gbs = extra["unique_kv_bytes_per_step"] / (dec_ms * 1e-3) / 1e9
        roof_bytes = "unique physical KV bytes (each shared block once)"
    line = {
        "metric": WORKLOAD_METRIC[name],
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        **step_stats(total),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{name}: paged decode of {num_seqs} sequences, {Hq} query heads over {Hkv} "
                        f"KV heads, head_dim {D}, 16-token blocks, {w.dtype}"
                        + (" (plus slot-mapped write of 8192 tokens and 2 prefill chunks of 2048)"
                           if name == "mixed" else ""),
            "num_seqs": num_seqs,
            "kv_bytes_per_step": int(kv_bytes),
            "partition_size": P or pa.default_partition_size(num_seqs, Hq, Hkv, D, w.max_model_len),
            "cache": "warm" if args.warm_cache else "Infinity Cache evicted before each step",
            "parallelism": "none (1 GPU)",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(roof_gbs, 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(roof_gbs / HBM_PEAK_GBS, 4),
            "bytes": roof_bytes,
            "traffic": traffic,
            "kernel": "pa_decode, every kernel of one call (partition kernel, or the single-pass kernel "
                      "when partition states are merged on chip, plus the merge pass when there is one)",
        },
        "cpu_baseline": cpu,
        "wall_ms_per_step": round(wall, 5),
        **extra,
    }
    line["settle_s"] = args.settle
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
