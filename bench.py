"""Benchmark of the fused GDN speculative-decode update on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload mtp_b128_bf16]
    python bench.py --path conv [--workload conv_mtp_b128]

One step = one launch of the whole hot path (rewind, gating, L2 norms, the
serial recurrence over the draft tokens, every slot store, the gated-RMSNorm
epilogue) over one batch of synthetic inputs already resident in HBM.  Steps
run back to back on torch's current stream and cycle through the state pools
of --layers GDN layers (by default 4, or more for small pools so that they
total at least 2 GiB), as a decode step walks a model's layers: the pools
together are several times the 256 MB Infinity Cache, so a
step cannot find the slots it rewrites still cached from the step before.
Every pool is updated in place.

Prints one JSON line: draft tokens/s over the timed region (HIP events around
all timed steps, which the host has enqueued ahead of the GPU), the
kernel's achieved algorithmic HBM bandwidth against the 8 TB/s peak (the
average launch duration from those events, on the launch stream; a second
pass with an event pair around every launch gives the percentiles), the HBM
traffic that
rocprofv3 counters recorded for the same kernel build (if the recording
matches the current kernel source), and the CPU oracle timed on a bounded
sample of the same workload.

--path conv times the conv update with rewind that precedes the recurrent
update instead (the same JSON fields), cycling each layer's own buffer,
inputs and outputs over 32 layers by default so that nothing it reads is
still cached from the previous use of that layer.
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
PEAK_FP32_TFLOPS = 157.3       # MI355X dense FP32 (matrix cores; also packed vector), AMD's published figure
DEFAULT_WORKLOAD = {"gdn": "mtp_b128_bf16", "conv": "conv_mtp_b128",
                    "prefill": "prefill_b16_l2048"}
DEFAULT_LAYERS = {"gdn": 4, "conv": 32, "prefill": 2}
# The state pools cycled by the gdn path must together be several times the
# 256 MB Infinity Cache, else a step's rewind reads find slots written a few
# steps earlier still cached: at least 4 pools and at least 2 GiB in all.
MIN_CYCLED_POOL_BYTES = 2 << 30
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
_CSRC = os.path.join(ROOT, "speculative_decode_amd", "csrc")
KERNEL_SOURCES = {
    "gdn": ["gdn_kernels.hip", "gdn_host.cpp", "lane_ops.h"],
    "conv": ["conv_kernels.hip", "conv_host.cpp"],
    "prefill": ["prefill_kernels.hip", "gdn_host.cpp", "lane_ops.h"],
}
SHARED_SOURCES = ["gdn_internal.h", "dtype_cvt.h"]


def pools_to_cycle(pool_bytes: int, requested=None) -> int:
    """Layers (state pools) the gdn path cycles: as requested, else at least
    four and at least MIN_CYCLED_POOL_BYTES in all."""
    if requested:
        return requested
    return max(DEFAULT_LAYERS["gdn"], -(-MIN_CYCLED_POOL_BYTES // pool_bytes))


def kernel_source_hash(path: str = "gdn") -> str:
    """Hash of the sources that build the kernel of ``path``."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[path] + SHARED_SOURCES:
        with open(os.path.join(_CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded_traffic(workload: str, path: str = "gdn"):
    """Per-launch HBM bytes from rocprofv3 FETCH_SIZE / WRITE_SIZE runs, if
    they were taken on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get(workload)
    if not entry or entry.get("kernel_source_hash") != kernel_source_hash(path):
        return None
    return entry.get("bytes_per_launch")


def host_info() -> dict:
    """The host the CPU baselines ran on: usable cores and the CPU model."""
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"nproc": len(os.sched_getaffinity(0)), "cpu_model": model}


def _oracle_parts(batch, lo: int, hi: int):
    """Prepared oracle calls (marshalled, not run) for spec sequences lo..hi-1
    of the workload, on their own rows and a pool of just the slots they
    touch; returns (calls, draft tokens)."""
    import torch

    import oracle

    cu = batch.cu_seqlens.tolist()
    g = list(range(cu[lo], cu[hi]))
    rows = [int(batch.spec_token_indx[x]) for x in g] if batch.spec_token_indx is not None else g
    si = batch.spec_state_indices[lo:hi].tolist()
    slots = sorted({s for r in si for s in r})
    remap = {s: i for i, s in enumerate(slots)}
    ridx = torch.tensor(rows, dtype=torch.long)
    sub = [x[ridx] for x in (batch.q, batch.k, batch.v, batch.z, batch.a, batch.b)]
    call = oracle.prepare_spec_update(
        *sub, batch.A_log, batch.dt_bias, batch.norm_weight, batch.pool[slots],
        torch.tensor([c - cu[lo] for c in cu[lo:hi + 1]], dtype=torch.int32),
        torch.tensor([[remap[s] for s in r] for r in si], dtype=torch.int32),
        batch.num_accepted_tokens[lo:hi], out_dtype=batch.out_dtype, scale=batch.scale,
        norm_eps=batch.norm_eps)
    return [call], len(rows)


def _oracle_single_parts(batch, lo: int, hi: int):
    """Prepared oracle calls for single-token entries lo..hi-1 (padding
    skipped), on their own rows and slots; returns (calls, tokens)."""
    import torch

    import oracle

    ent = [i for i in range(lo, hi) if int(batch.state_indices[i]) >= 0]
    if not ent:
        return [], 0
    tix = batch.non_spec_token_indx
    rows = [int(tix[i]) if tix is not None else i for i in ent]
    slots = [int(batch.state_indices[i]) for i in ent]
    ridx = torch.tensor(rows, dtype=torch.long)
    sub = [x[ridx] for x in (batch.q, batch.k, batch.v, batch.z, batch.a, batch.b)]
    call = oracle.prepare_decode_update(
        *sub, batch.A_log, batch.dt_bias, batch.norm_weight, batch.pool[slots],
        torch.arange(len(ent), dtype=torch.int32), out_dtype=batch.out_dtype,
        scale=batch.scale, norm_eps=batch.norm_eps)
    return [call], len(ent)


def _split(n: int, parts: int):
    parts = max(1, min(parts, n)) if n else 1
    return [(n * i // parts, n * (i + 1) // parts) for i in range(parts)]


def cpu_baseline(batch, n_seqs: int, threads: int = 1):
    """The oracle, as it is, on a bounded sample of the workload: its first
    n_seqs spec sequences and first n_seqs single-token entries.  The
    marshalling into float64 is done before the timer starts: only the C
    calls are timed.  With threads > 1 the sample is split into that many
    contiguous parts run at once on host threads (one oracle call per part;
    ctypes releases the interpreter lock while the C code runs)."""
    import time as _t
    from concurrent.futures import ThreadPoolExecutor

    ns = min(n_seqs, batch.num_seqs)
    nn = min(n_seqs, batch.num_non_spec)
    calls, tokens = [], 0
    for lo, hi in _split(ns, threads) if ns else []:
        c, t = _oracle_parts(batch, lo, hi)
        calls += c
        tokens += t
    for lo, hi in _split(nn, threads) if nn else []:
        c, t = _oracle_single_parts(batch, lo, hi)
        calls += c
        tokens += t
    t0 = _t.perf_counter()
    if threads > 1:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(lambda c: c.run(), calls))
    else:
        for c in calls:
            c.run()
    dt = _t.perf_counter() - t0
    what = []
    if ns:
        what.append(f"first {ns} of {batch.num_seqs} spec sequences")
    if nn:
        what.append(f"first {nn} of {batch.num_non_spec} single-token entries")
    how = (f"in {len(calls)} parts on {threads} host threads" if threads > 1
           else "serial C, float64")
    return {"value": tokens / dt, "unit": "draft tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{' and '.join(what)} ({tokens} draft tokens, all {batch.HV} v-heads) "
                      f"of the same workload; {how}; {dt:.2f} s of C calls (float64 "
                      f"marshalling outside the timer)", **host_info()}


def conv_cpu_baseline(batch):
    """The conv oracle, as it is, on the whole workload (the C call timed)."""
    import oracle

    call = oracle.prepare_conv_spec_update(
        batch.x, batch.weight, batch.bias, batch.cache, batch.cu_seqlens, batch.conv_indices,
        batch.num_accepted_tokens, token_indx=batch.token_indx, out_dtype=batch.out_dtype,
        activation=batch.activation)
    t0 = time.perf_counter()
    call.run()
    dt = time.perf_counter() - t0
    tokens = batch.draft_tokens()
    return {"value": tokens / dt, "unit": "draft tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"all {batch.num_seqs} sequences ({tokens} draft tokens, "
                      f"{batch.channels} channels) of the same workload; serial C, float64; "
                      f"{dt:.2f} s of the C call (marshalling outside the timer)",
            **host_info()}


def time_steps(step, steps: int, warmup: int, stream):
    """Warm up, then time ``steps`` back-to-back steps on ``stream``, twice.

    In both passes the host enqueues every timed step while the GPU is held
    busy by a spin kernel queued just before the timed region, so the GPU
    runs the steps back to back whatever the per-call host cost.  Pass 1
    brackets every launch with its own pair of HIP events (percentiles);
    pass 2 records one pair around all of them, so the average launch
    duration it gives carries no per-launch event overhead -- which matters
    for a kernel of a few microseconds.  Returns (pass-2 GPU ms for all
    steps, sorted pass-1 per-step ms, host wall seconds of pass 2, host
    seconds per bare step call).
    """
    import torch

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # host cost of one bare call of the binding (marshalling + enqueue)
    t = time.perf_counter()
    for i in range(16):
        step(i)
    host_call_s = (time.perf_counter() - t) / 16
    torch.cuda.synchronize()
    # host cost of one step (call + two event records), to size the spin
    e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    t = time.perf_counter()
    for i in range(8):
        e[0].record(stream)
        step(i)
        e[1].record(stream)
    host_s = (time.perf_counter() - t) / 8
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    torch.cuda._sleep(1 << 20)
    c1.record(stream)
    torch.cuda.synchronize()
    cycles_per_ms = (1 << 20) / max(c0.elapsed_time(c1), 1e-3)
    spin_cycles = int((2.0 * steps * host_s * 1e3 + 5.0) * cycles_per_ms)

    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    torch.cuda._sleep(spin_cycles)
    for i, (e0, e1) in enumerate(ev):
        e0.record(stream)
        step(warmup + i)
        e1.record(stream)
    torch.cuda.synchronize()
    per_launch = sorted(e0.elapsed_time(e1) for e0, e1 in ev)

    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    torch.cuda._sleep(spin_cycles)
    start.record(stream)
    for i in range(steps):
        step(warmup + steps + i)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(end), per_launch, wall, host_call_s


def timing_fields(gpu_ms, kern_ms, steps):
    """Roofline timing fields: the average launch duration of pass 2 and
    the per-launch event statistics of pass 1."""
    n = len(kern_ms)
    return {"kernel_avg_us": gpu_ms / steps * 1e3,
            "event_pair_avg_us": sum(kern_ms) / n * 1e3,
            "event_pair_median_us": kern_ms[n // 2] * 1e3,
            "event_pair_p10_us": kern_ms[n // 10] * 1e3,
            "event_pair_p90_us": kern_ms[(9 * n) // 10] * 1e3}


def traffic_ceilings(kw, pools, alg_bytes, args, stream, dev):
    """What the memory system delivers for the timed launch's traffic: the
    same launches with no arithmetic (gdn_traffic_pattern: same grid, unit
    mapping and metadata, the same bytes moved, the same pools cycled), at
    the kernel's blocks per CU and at 1, 2, 3 and 4, the fastest taken as the
    ceiling; and a plain device copy of the same byte count (half read, half
    written), with buffers cycled over at least 2 GiB.  All are timed like
    the kernel.  The pattern launches overwrite the pools' written slots with
    copies of the rewind tiles, so they run after the kernel's timing."""
    import torch

    from speculative_decode_amd import ops

    pk = dict(kw)
    pk["out"] = torch.empty_like(kw["out"])
    shapes = {}
    for bpc in (0, 1, 2, 3, 4):
        def pattern(i):
            pk["state"] = pools[i % len(pools)]
            ops.traffic_pattern(**pk, blocks_per_cu=bpc)

        shapes[bpc], _, _, _ = time_steps(pattern, args.steps, args.warmup, stream)
    p_ms = min(shapes.values())
    n = max(1, alg_bytes // 2)
    pairs = max(2, -(-MIN_CYCLED_POOL_BYTES // (2 * n)))
    bufs = [(torch.empty(n, dtype=torch.uint8, device=dev).fill_(1),
             torch.empty(n, dtype=torch.uint8, device=dev)) for _ in range(pairs)]

    def copy(i):
        src, dst = bufs[i % pairs]
        dst.copy_(src)

    c_ms, _, _, _ = time_steps(copy, args.steps, args.warmup, stream)
    del bufs
    p_s, c_s = p_ms / args.steps * 1e-3, c_ms / args.steps * 1e-3
    return {"ceiling_gbs": alg_bytes / p_s / 1e9, "ceiling_avg_us": p_s * 1e6,
            "ceiling_as_kernel_us": shapes[0] / args.steps * 1e3,
            "ceiling_blocks_per_cu": min(shapes, key=shapes.get),
            "copy_gbs": 2 * n / c_s / 1e9, "copy_avg_us": c_s * 1e6}


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 200; 1000 for the launch-bound tiny workload)")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--path", choices=["gdn", "conv", "prefill"], default="gdn",
                    help="gdn: the recurrent state update (default); conv: the conv update "
                         "with rewind that precedes it; prefill: the chunked prefill")
    ap.add_argument("--workload", default=None)
    ap.add_argument("--layers", type=int, default=None,
                    help="layers cycled through, each with its own state (default: for "
                         "gdn 4, or as many as make 2 GiB of pools; 32 for conv; 2 for "
                         "prefill)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="instead of the benchmark, run --steps plain device copies of MIB "
                         "MiB each (reference kernel for scaling HBM byte counters)")
    ap.add_argument("--cpu-threads", type=int,
                    default=min(16, len(os.sched_getaffinity(0))),
                    help="host threads for the multi-threaded oracle timing (gdn path)")
    ap.add_argument("--cpu-seqs", type=int, default=128,
                    help="sequences (and single-token entries) of the workload the CPU "
                         "oracle is timed on (0: skip)")
    ap.add_argument("--no-ceiling", action="store_true",
                    help="skip the traffic-pattern and copy ceilings (gdn path)")
    ap.add_argument("--issue-probe", action="store_true",
                    help="time FP32 matrix and FP32 vector instruction streams on the same "
                         "SIMDs, alone and together (gdn_issue_probe); one JSON line")
    args = ap.parse_args()
    if args.steps is None:
        args.steps = 1000 if args.workload == "tiny" else 200

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
    if args.issue_probe:
        return issue_probe(dev)
    args.workload = args.workload or DEFAULT_WORKLOAD[args.path]
    layers_given = args.layers
    args.layers = args.layers or DEFAULT_LAYERS[args.path]
    if args.path == "conv":
        return bench_conv(args, dev)
    if args.path == "prefill":
        return bench_prefill(args, dev)
    batch = workloads.make(args.workload)
    print(f"bench: {args.workload}: {workloads.DESCRIPTIONS[args.workload]}", file=sys.stderr,
          flush=True)
    kw = ops.batch_args(batch, dev)
    kw["out"] = torch.zeros((batch.n_tok, batch.HV, batch.V), dtype=batch.out_dtype, device=dev)
    pool_bytes = batch.pool.numel() * batch.pool.element_size()
    args.layers = pools_to_cycle(pool_bytes, layers_given)
    pools = [kw["state"]] + [kw["state"].clone() for _ in range(args.layers - 1)]
    tokens = batch.draft_tokens()
    alg_bytes = batch.algorithmic_bytes()

    def step(i):
        kw["state"] = pools[i % len(pools)]
        ops.forward_core(**kw)

    stream = torch.cuda.current_stream(dev)
    gpu_ms, kern_ms, wall, host_call_s = time_steps(step, args.steps, args.warmup, stream)
    tf = timing_fields(gpu_ms, kern_ms, args.steps)
    print("bench: " + ", ".join(f"{k} {v:.1f}" for k, v in tf.items()), file=sys.stderr,
          flush=True)
    avg_ms = tf["kernel_avg_us"] * 1e-3
    achieved = alg_bytes / (avg_ms * 1e-3) / 1e9
    traffic = recorded_traffic(args.workload, "gdn")
    ms_per_step = gpu_ms / args.steps
    ceiling = {}
    if not args.no_ceiling:
        ceiling = traffic_ceilings(kw, pools, alg_bytes, args, stream, dev)
        ceiling["frac_of_ceiling"] = achieved / ceiling["ceiling_gbs"]
        print("bench: " + ", ".join(f"{k} {v:.3f}" for k, v in ceiling.items()),
              file=sys.stderr, flush=True)
    cpu = cpu_all = None
    if args.cpu_seqs > 0:
        cpu = cpu_baseline(batch, args.cpu_seqs)
        cpu_all = cpu_baseline(batch, args.cpu_seqs, args.cpu_threads)
    dtypes = {torch.float32: "f32", torch.bfloat16: "bf16", torch.float16: "f16",
              torch.float8_e4m3fn: "f8e4m3"}
    line = {
        "metric": "draft tokens/sec and achieved HBM GB/s (% of peak), B=128 T=8 BF16 state",
        "value": tokens * args.steps / (gpu_ms * 1e-3),
        "unit": "draft tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "host_wall_s": wall,
        "host_us_per_call": host_call_s * 1e6,
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
                   "pool_bytes_per_layer": pool_bytes},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic, **tf, **ceiling},
        "cpu_baseline": cpu,
        "cpu_baseline_threads": cpu_all,
    }
    print(json.dumps(line), flush=True)


def bench_conv(args, dev):
    """The conv update with rewind at its full shape; one JSON line."""
    import torch

    from speculative_decode_amd import ops, workloads

    batch = workloads.make_conv(args.workload)
    print(f"bench: {args.workload}: {workloads.CONV_DESCRIPTIONS[args.workload]}",
          file=sys.stderr, flush=True)
    kw = ops.conv_batch_args(batch, dev)
    layers = []
    for i in range(args.layers):
        lk = dict(kw)
        if i:
            lk["cache"] = kw["cache"].clone()
            lk["x"] = kw["x"].clone()
        lk["out"] = torch.zeros(batch.x.shape, dtype=batch.out_dtype, device=dev)
        layers.append(lk)

    def step(i):
        ops.conv_spec_update(**layers[i % len(layers)])

    gpu_ms, kern_ms, wall, host_call_s = time_steps(step, args.steps, args.warmup,
                                       torch.cuda.current_stream(dev))
    tf = timing_fields(gpu_ms, kern_ms, args.steps)
    print("bench: " + ", ".join(f"{k} {v:.2f}" for k, v in tf.items()), file=sys.stderr,
          flush=True)
    avg_ms = tf["kernel_avg_us"] * 1e-3
    tokens = batch.draft_tokens()
    alg_bytes = batch.algorithmic_bytes()
    achieved = alg_bytes / (avg_ms * 1e-3) / 1e9
    dtypes = {torch.float32: "f32", torch.bfloat16: "bf16", torch.float16: "f16",
              torch.float8_e4m3fn: "f8e4m3"}
    line = {
        "metric": "conv update with rewind: draft tokens/sec and achieved HBM GB/s "
                  "(% of peak), B=128 T=8",
        "value": tokens * args.steps / (gpu_ms * 1e-3),
        "unit": "draft tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": gpu_ms / args.steps,
        "host_wall_s": wall,
        "host_us_per_call": host_call_s * 1e6,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: {workloads.CONV_DESCRIPTIONS[args.workload]}",
                   "sequences": batch.num_seqs, "draft_tokens_per_step": tokens,
                   "channels": batch.channels, "width": batch.width,
                   "state_len": batch.state_len, "x_dtype": dtypes[batch.x.dtype],
                   "algorithmic_bytes_per_step": alg_bytes, "layers_cycled": len(layers)},
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS,
                     "traffic": recorded_traffic(args.workload, "conv"), **tf},
        "cpu_baseline": conv_cpu_baseline(batch) if args.cpu_seqs > 0 else None,
    }
    print(json.dumps(line), flush=True)


def prefill_cpu_baseline(batch):
    """The prefill oracle, as it is, on the first sequence of the workload
    (every head): a bounded sample of the same work (the C call timed)."""
    import oracle

    L0 = int(batch.cu_seqlens[1])
    call = oracle.prepare_prefill_update(
        batch.q[:L0], batch.k[:L0], batch.v[:L0], batch.z[:L0], batch.a[:L0], batch.b[:L0],
        batch.A_log, batch.dt_bias, batch.norm_weight, batch.pool, batch.cu_seqlens[:2],
        batch.state_indices[:1],
        has_initial_state=None if batch.has_initial_state is None
        else batch.has_initial_state[:1],
        chunk_size=batch.chunk_size, out_dtype=batch.out_dtype)
    t0 = time.perf_counter()
    call.run()
    dt = time.perf_counter() - t0
    return {"value": L0 / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"the first of {batch.num_seqs} sequences ({L0} tokens, all "
                      f"{batch.HV} v-heads) of the same workload; serial C, float64; "
                      f"{dt:.2f} s of the C call (marshalling outside the timer)",
            **host_info()}


def issue_probe(dev, blocks=256, n_mfma=4000, n_valu=16000, reps=5):
    """Whether a SIMD runs FP32 matrix and FP32 vector instructions of two
    of its waves at the same time (gdn_issue_probe): one 512-thread block per
    CU, waves 0-3 two chains of v_mfma_f32_32x32x2f32, waves 4-7 eight FP32
    FMA chains, timed alone and together.  If "both" takes the sum of
    the two, the SIMD issues them one after the other, and a kernel that
    mixes them pays for both."""
    import torch

    from speculative_decode_amd import ops

    out = torch.empty(blocks * 512, dtype=torch.float32, device=dev)
    us = {}
    for mode, name in ((1, "mfma_only_us"), (2, "valu_only_us"), (3, "both_us")):
        ops.issue_probe(out, mode, n_mfma, n_valu)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            ops.issue_probe(out, mode, n_mfma, n_valu)
        e1.record()
        torch.cuda.synchronize()
        us[name] = e0.elapsed_time(e1) * 1e3 / reps
    mfma_flop = 4 * blocks * 2 * n_mfma * 32 * 32 * 2 * 2
    valu_flop = 4 * blocks * n_valu * 64 * 8 * 2
    line = {"probe": "FP32 matrix and vector instructions of two waves per SIMD",
            "blocks": blocks, "n_mfma": n_mfma, "n_valu": n_valu, **us,
            "sum_of_alone_us": us["mfma_only_us"] + us["valu_only_us"],
            "mfma_tflops_alone": mfma_flop / us["mfma_only_us"] / 1e6,
            "valu_tflops_alone": valu_flop / us["valu_only_us"] / 1e6,
            # per SIMD, at the 2.4 GHz the peak figures assume
            "mfma_cycles_each": us["mfma_only_us"] * 2400 / (2 * n_mfma),
            "valu_cycles_each": us["valu_only_us"] * 2400 / (8 * n_valu)}
    print(json.dumps(line), flush=True)


def bench_prefill(args, dev):
    """The chunked prefill at its full shape; one JSON line.  Bound by the
    FP32 vector ALU: the roofline is flops against the FP32 peak."""
    import torch

    from speculative_decode_amd import ops, workloads

    batch = workloads.make_prefill(args.workload)
    print(f"bench: {args.workload}: {workloads.PREFILL_DESCRIPTIONS[args.workload]}",
          file=sys.stderr, flush=True)
    kw = ops.prefill_batch_args(batch, dev)
    layers = []
    for i in range(args.layers):
        lk = dict(kw)
        if i:
            for name in ("q", "k", "v", "z", "a", "b", "state"):
                lk[name] = kw[name].clone()
        lk["out"] = torch.zeros((batch.n_tok, batch.HV, batch.V), dtype=batch.out_dtype,
                                device=dev)
        layers.append(lk)

    def step(i):
        ops.prefill_update(**layers[i % len(layers)])

    gpu_ms, kern_ms, wall, host_call_s = time_steps(step, args.steps, args.warmup,
                                       torch.cuda.current_stream(dev))
    tf = timing_fields(gpu_ms, kern_ms, args.steps)
    print("bench: " + ", ".join(f"{k} {v:.1f}" for k, v in tf.items()), file=sys.stderr,
          flush=True)
    avg_s = tf["kernel_avg_us"] * 1e-6
    flops = batch.flops()
    tokens = batch.tokens()
    achieved = flops / avg_s / 1e12
    line = {
        "metric": "chunked prefill: tokens/sec and achieved FP32 TFLOP/s (% of peak)",
        "value": tokens * args.steps / (gpu_ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": gpu_ms / args.steps,
        "host_wall_s": wall,
        "host_us_per_call": host_call_s * 1e6,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": f"{args.workload}: "
                               f"{workloads.PREFILL_DESCRIPTIONS[args.workload]}",
                   "sequences": batch.num_seqs, "tokens_per_step": tokens,
                   "HK": batch.HK, "HV": batch.HV, "chunk_size": batch.chunk_size,
                   "flops_per_step": flops,
                   "algorithmic_bytes_per_step": batch.algorithmic_bytes(),
                   "achieved_hbm_gbs": batch.algorithmic_bytes() / avg_s / 1e9,
                   "layers_cycled": len(layers)},
        "roofline": {"bound": "mfma", "achieved": achieved, "peak": PEAK_FP32_TFLOPS,
                     "unit": "TFLOP/s", "frac": achieved / PEAK_FP32_TFLOPS,
                     "traffic": recorded_traffic(args.workload, "prefill"), **tf},
        "cpu_baseline": prefill_cpu_baseline(batch) if args.cpu_seqs > 0 else None,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
