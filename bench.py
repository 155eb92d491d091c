#!/usr/bin/env python3
"""Benchmark of the paged-attention hot path on one MI355X.

Default workload: LLaMA-7B-shaped paged decode, 64 sequences, 32 heads MHA,
head_dim 128, fp16, context lengths U[128, 2048], 16-token blocks scattered
through a pool of 1.2x demand.  A step is one pa_decode call (partition
kernel + log-sum-exp merge kernel) over the whole batch; inputs are resident
in HBM before timing starts.

Prints ONE JSON line: KV GB/s (algorithmic bytes: sum_s L_s * 2 * Hkv * D * 2
per step, divided by the measured step time), us/step, the roofline of the
dominant kernel, and the fp64 CPU oracle timed on a bounded sample of the
same workload on this host's cores.

Other workloads (--workload): llama8b_gqa, llama13b_shared (not for the
headline), mixed (write + 2 prefill chunks + 4096 decode), tiny.
"""
from __future__ import annotations

import argparse
import json
import os
import resource
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16/fp16 matrix peak


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama7b",
                    choices=["llama7b", "llama8b_gqa", "llama13b_shared", "mixed", "tiny"])
    ap.add_argument("--partition", type=int, default=-1,
                    help="partition size in tokens (-1: the workload's own, 0: library default)")
    ap.add_argument("--cpu-budget", type=float, default=15.0,
                    help="seconds of oracle work for the cpu_baseline sample (0: skip)")
    return ap.parse_args()


class Timer:
    """HIP events on the stream the kernels run on (torch's current stream)."""

    def __init__(self, torch):
        self.torch = torch
        self.pairs = []

    def __call__(self, fn):
        t = self.torch
        a, b = t.cuda.Event(enable_timing=True), t.cuda.Event(enable_timing=True)
        a.record()
        fn()
        b.record()
        self.pairs.append((a, b))

    def mean_ms(self):
        return sum(a.elapsed_time(b) for a, b in self.pairs) / max(len(self.pairs), 1)


def cpu_oracle_sample(w, q, kc, vc, budget_s):
    """fp64 oracle over the workload's sequences in order (wrapping around for
    further passes) until the time budget is spent.  Returns (GB/s of KV
    processed, sequences done, wall seconds, cores used)."""
    import numpy as np
    import torch
    from oracle import attention as A

    def bits(t):
        t = t.detach().cpu().contiguous()
        return t.numpy() if t.dtype == torch.float16 else t.view(torch.int16).numpy().view(np.uint16)

    # Copy back each sequence's blocks once (device -> host is not timed).
    per_seq = []
    qh = bits(q)
    for s in range(w.num_seqs):
        L = int(w.context_lens[s])
        nb = -(-L // 16)
        it = torch.from_numpy(w.block_tables[s, :nb].astype(np.int64)).to(kc.device)
        per_seq.append((L, bits(kc[it]), bits(vc[it]), np.arange(nb, dtype=np.int32)[None]))
    t0, c0 = time.perf_counter(), time.process_time()
    done = bytes_done = 0
    while True:
        s = done % w.num_seqs
        L, kh, vh, bt = per_seq[s]
        A.decode(qh[s:s + 1], kh, vh, bt, [L], w.scale, w.dtype)
        bytes_done += L * 2 * w.num_kv_heads * w.head_dim * 2
        done += 1
        if time.perf_counter() - t0 > budget_s:
            break
    wall = time.perf_counter() - t0
    cpu = time.process_time() - c0
    cores = max(1, round(cpu / wall)) if wall > 0 else 1
    return bytes_done / wall / 1e9, done, wall, cores


def bench_decode(args, torch, pa, w):
    dev = "cuda"
    q, kc, vc = w.make_tensors(dev)
    bt = torch.from_numpy(w.block_tables).to(dev)
    ctx = torch.from_numpy(w.context_lens).to(dev)
    P = w.partition_size if args.partition < 0 else args.partition
    need = pa.decode_workspace_size(w.num_seqs, w.num_q_heads, w.head_dim, w.max_model_len, P,
                                    w.num_kv_heads)
    ws = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    out = torch.empty_like(q)

    def step():
        pa.decode(out, q, kc, vc, bt, ctx, w.max_model_len, w.scale, P, ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    timer = Timer(torch)
    t0 = time.perf_counter()
    for _ in range(args.steps):
        timer(step)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    ms = timer.mean_ms()
    kv = w.kv_bytes
    gbs = kv / (ms * 1e-3) / 1e9
    return dict(ms=ms, wall_ms=wall_ms, gbs=gbs, kv=kv, q=q, kc=kc, vc=vc, P=P)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only (asked for --gpus {args.gpus}); "
              "the path shards by sequence or KV head with no exchange inside attention, "
              "but multi-GPU runs are not part of it.", file=sys.stderr)
        return 2
    import numpy as np
    import torch
    import paged_kv_cache_422_amd as pa
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    name = args.workload
    w = W.make_workload(name)
    if name == "mixed":
        raise SystemExit("use --workload mixed via bench_mixed (not in this build yet)")
    if name == "llama13b_shared":
        raise SystemExit("llama13b_shared is benchmarked through the tests' pool layout")
    r = bench_decode(args, torch, pa, w)
    cpu = None
    if args.cpu_budget > 0:
        gbs_cpu, n_seq, wall, cores = cpu_oracle_sample(w, r["q"], r["kc"], r["vc"], args.cpu_budget)
        cpu = {"value": round(gbs_cpu, 6), "unit": "GB/s", "cores": cores, "kind": "oracle",
               "sample": f"{n_seq} sequence decodes (all heads; the workload's {w.num_seqs} "
                         f"sequences in order, repeated) in {wall:.1f} s, fp64 numpy"}
    line = {
        "metric": "paged-decode KV GB/s (% of HBM peak) + us/step, batch 64 LLaMA-7B shape",
        "value": round(r["gbs"], 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["ms"], 5),
        "us_per_step": round(r["ms"] * 1e3, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {
            "workload": f"{name} paged decode: {w.num_seqs} seqs, {w.num_q_heads} q heads / "
                        f"{w.num_kv_heads} kv heads, D {w.head_dim}, block 16, {w.dtype}",
            "num_seqs": w.num_seqs,
            "kv_bytes_per_step": r["kv"],
            "partition_size": r["P"] or pa.default_partition_size(w.num_q_heads, w.num_kv_heads, w.head_dim),
            "parallelism": "none (1 GPU)",
        },
        "roofline": {
            "bound": "hbm",
            "achieved": round(r["gbs"], 2),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(r["gbs"] / HBM_PEAK_GBS, 4),
            "traffic": None,
            "kernel": "pa_decode step (decode_partition_kernel + decode_merge_kernel)",
        },
        "cpu_baseline": cpu,
        "wall_ms_per_step": round(r["wall_ms"], 5),
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
