"""Benchmark of the fused GDN speculative-decode update on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload mtp_b128_bf16]

One step = one launch of the whole hot path (rewind, gating, L2 norms, the
serial recurrence over the draft tokens, every slot store, the gated-RMSNorm
epilogue) over one batch of synthetic inputs already resident in HBM.  Steps
run back to back on torch's current stream and cycle through the state pools
of --layers GDN layers (4 by default), as a decode step walks a model's
layers: the pools together are several times the 256 MB Infinity Cache, so a
step cannot find the slots it rewrites still cached from the step before.
Every pool is updated in place.

Prints one JSON line: draft tokens/s over the timed wall-clock region, the
kernel's achieved algorithmic HBM bandwidth against the 8 TB/s peak (HIP
events around every timed launch, on the launch stream), the HBM traffic that
rocprofv3 counters recorded for the same kernel build (if the recording
matches the current kernel source), and the CPU oracle timed on a bounded
sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E, AMD's published figure
DEFAULT_WORKLOAD = "mtp_b128_bf16"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "speculative_decode_amd", "csrc", f)
                  for f in ("gdn_kernels.hip", "gdn_host.cpp", "gdn_internal.h")]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str):
    """Per-launch HBM bytes from rocprofv3 FETCH_SIZE / WRITE_SIZE runs, if
    they were taken on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get(workload)
    if not entry or entry.get("kernel_source_hash") != kernel_source_hash():
        return None
    return entry.get("bytes_per_launch")


def cpu_baseline(batch, n_seqs: int):
    """The oracle, as it is, on the first n_seqs sequences of the workload."""
    import numpy as np
    import torch

    import oracle

    cu = batch.cu_seqlens.tolist()
    rows = list(range(cu[0], cu[n_seqs]))
    slots = set()
    for bi in range(n_seqs):
        acc = int(batch.num_accepted_tokens[bi])
        slots.add(int(batch.spec_state_indices[bi, max(acc - 1, 0)]))
        slots |= set(batch.spec_state_indices[bi].tolist())
    slots = sorted(slots)
    remap = {s: i for i, s in enumerate(slots)}
    si = torch.tensor([[remap[int(s)] for s in batch.spec_state_indices[bi]]
                       for bi in range(n_seqs)], dtype=torch.int32)
    sub = [x[rows] for x in (batch.q, batch.k, batch.v, batch.z, batch.a, batch.b)]
    pool = batch.pool[slots]
    t0 = time.perf_counter()
    oracle.spec_update(*sub, batch.A_log, batch.dt_bias, batch.norm_weight, pool,
                       batch.cu_seqlens[: n_seqs + 1], si,
                       batch.num_accepted_tokens[:n_seqs], out_dtype=batch.out_dtype,
                       scale=batch.scale, norm_eps=batch.norm_eps)
    dt = time.perf_counter() - t0
    tokens = len(rows)
    return {"value": tokens / dt, "unit": "draft tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"first {n_seqs} of {batch.num_seqs} sequences ({tokens} draft tokens, "
                      f"all {batch.HV} v-heads) of the same workload; serial C, float64; "
                      f"{dt:.2f} s incl. fp64 marshalling"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--layers", type=int, default=4,
                    help="state pools cycled through, one per GDN layer")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="instead of the benchmark, run --steps plain device copies of MIB "
                         "MiB each (reference kernel for scaling HBM byte counters)")
    ap.add_argument("--cpu-seqs", type=int, default=128,
                    help="sequences of the workload the CPU oracle is timed on (0: skip)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only; the update shards by "
              "(sequence, value head) with no exchange, so there is no multi-GPU "
              "step to time.  Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch

    from speculative_decode_amd import ops, workloads

    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        n = args.calibrate_copy << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n, "copies": args.steps}), flush=True)
        return
    ops.load_library()
    batch = workloads.make(args.workload)
    print(f"bench: {args.workload}: {workloads.DESCRIPTIONS[args.workload]}", file=sys.stderr,
          flush=True)
    kw = ops.batch_args(batch, dev)
    kw["out"] = torch.zeros((batch.n_tok, batch.HV, batch.V), dtype=batch.out_dtype, device=dev)
    pools = [kw["state"]] + [kw["state"].clone() for _ in range(args.layers - 1)]
    tokens = batch.draft_tokens()
    alg_bytes = batch.algorithmic_bytes()

    def step(i):
        kw["state"] = pools[i % len(pools)]
        ops.forward_core(**kw)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i, (e0, e1) in enumerate(ev):
        e0.record(stream)
        step(args.warmup + i)
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kern_ms = sorted(e0.elapsed_time(e1) for e0, e1 in ev)
    avg_ms = sum(kern_ms) / len(kern_ms)
    med_ms = kern_ms[len(kern_ms) // 2]
    print(f"bench: kernel avg {avg_ms * 1e3:.1f} us, median {med_ms * 1e3:.1f} us, "
          f"p10 {kern_ms[len(kern_ms) // 10] * 1e3:.1f} us, "
          f"p90 {kern_ms[(9 * len(kern_ms)) // 10] * 1e3:.1f} us", file=sys.stderr, flush=True)

    achieved = alg_bytes / (avg_ms * 1e-3) / 1e9
    traffic = recorded_traffic(args.workload)
    ms_per_step = wall * 1e3 / args.steps
    cpu = cpu_baseline(batch, min(args.cpu_seqs, batch.num_seqs)) if args.cpu_seqs > 0 else None
    dtypes = {torch.float32: "f32", torch.bfloat16: "bf16", torch.float16: "f16"}
    line = {
        "metric": "draft tokens/sec and achieved HBM GB/s (% of peak), B=128 T=8 BF16 state",
        "value": tokens * args.steps / wall,
        "unit": "draft tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {workloads.DESCRIPTIONS[args.workload]}",
                   "sequences": batch.num_seqs, "draft_tokens_per_step": tokens,
                   "HK": batch.HK, "HV": batch.HV, "K": batch.K, "V": batch.V,
                   "act_dtype": dtypes[batch.q.dtype], "state_dtype": dtypes[batch.pool.dtype],
                   "algorithmic_bytes_per_step": alg_bytes, "layers_cycled": len(pools),
                   "pool_bytes_per_layer": batch.pool.numel() * batch.pool.element_size()},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic,
                     "kernel_avg_us": avg_ms * 1e3, "kernel_median_us": med_ms * 1e3},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
