#!/usr/bin/env python3
"""Paged decode benchmark on one MI355X.

One step = the whole hot path over one batch: store every sequence's new token
in its last block, then attend over the whole context.  For fp16 pools that is one
pa_decode_append (the stream kernel, whose persistent waves each take an equal share of
the batch's tiles, weighed for piece boundaries, and take the new tokens from their input
rows, then the log-sum-exp reduce, which also stores the new tokens); for E4M3 and fp32
pools it is pa_cache_write(_fp8), then pa_decode(_fp8) (--step chooses).  The shared-prefix
batch steps with pa_cache_write + pa_decode_shared, which reads each group's prompt blocks
once (--step fused: pa_decode_append, every sample reading the prompt).
Default workload: a Llama-3-8B-shaped decode layer (64 sequences, 32 q / 8 kv
heads, head_dim 128, block 16, context lengths uniform in [512, 4096], fp16,
blocks scattered over a 1.2x pool).  Inputs are resident in HBM before timing.

`value` is the step rate over --steps back-to-back steps.  Each call (the dominant stream
kernel alone, the whole decode call, the cache write) is also timed launch by launch after
a 1 GiB read that leaves no cache holding the pool: the median of those cold launches is
the primary per-call figure (min and mean beside it), the back-to-back average is the
warm one.  The CPU baseline is the oracle's decode on every host core of the process.

Prints one JSON line on stdout; progress goes to stderr.
"""

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
KERNEL_SRC = os.path.join(ROOT, "paged_kv_cache_167_amd", "csrc", "pa_kernels.hip")
PROFILES = os.path.join(ROOT, "profiles")


def stream_kernel_name(is_f16):
    """The first-pass kernel that pa_decode launches for this element type."""
    return "pa_stream_mfma_kernel" if is_f16 else "pa_stream_kernel"


def traffic_file(kernel, config):
    return os.path.join(PROFILES, f"{kernel}_{config}_traffic.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    # 200 back-to-back steps: the host's start and stop latency is under 1 % of the timed span
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up steps (default 10; 200 for the prefill workloads, whose "
                         "launch times keep drifting while the clocks settle under matrix load)")
    ap.add_argument("--config", default="llama3_8b", choices=ALL_CONFIGS + ["all"],
                    help="workload; 'all' runs every one in turn, one JSON line each")
    ap.add_argument("--partition", type=int, default=0,
                    help="partition size in tokens (0: one wave per resident slot; >0: more "
                         "waves, each taking at most about that many tokens)")
    ap.add_argument("--cold-iters", type=int, default=50,
                    help="launches of each timed call (the stream kernel, pa_decode, pa_cache_write), "
                         "each after reading 1 GiB so that no cache holds the pool; their median "
                         "is the primary figure")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="decode workloads: replay one captured HIP graph of the step instead of "
                         "launching every timed step from the host (slower on ROCm 7)")
    ap.add_argument("--step", choices=["auto", "fused", "unfused", "shared"], default="auto",
                    help="decode workloads: 'fused' = one pa_decode_append (pa_decode_fp8_append) "
                         "per step; 'unfused' = pa_cache_write(_fp8), then pa_decode(_fp8); "
                         "'shared' (shared_prefix, fp16) = pa_cache_write, then pa_decode_shared, "
                         "which streams each prompt's shared blocks once for all its samples; "
                         "'auto' = shared for shared_prefix, fused for other fp16 pools and unfused "
                         "for E4M3 (and fp32) pools, the faster form of each on MI355X")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="first run one device-to-device copy of this many MiB (a kernel of "
                         "known traffic that scales the HBM byte counters)")
    args = ap.parse_args()
    args.warmup_arg = args.warmup
    return args


ALL_CONFIGS = ["tiny_fp32", "llama3_8b", "llama2_70b", "shared_prefix", "long_context_b8",
               "long_context_b16", "long_context_b32", "llama3_8b_fp8", "llama2_70b_fp8",
               "long_context_b16_fp8", "prefill_llama3_8b", "prefill_llama2_70b",
               "copy_blocks_device", "swap_out_host", "paging_tax_llama3_8b",
               "paging_tax_long_context"]
PAGING_TAX = ("paging_tax_llama3_8b", "paging_tax_long_context")
PREFILL = ("prefill_llama3_8b", "prefill_llama2_70b")
BLOCK_COPIES = ("copy_blocks_device", "swap_out_host")
HOST_LINK_GBS = 64.0  # PCIe 5.0 x16, one direction: the host link assumed for swap
PREFILL_WARMUP = 200  # ~50 ms of matrix work: launch times settle within about 100 launches
MFMA_F16_PEAK_TFLOPS = 2500.0  # MI355X dense fp16 matrix peak, published
WORKLOAD_NAMES = {
    "tiny_fp32": "tiny fp32 decode (4 sequences, ctx 1..250)",
    "llama3_8b": "Llama-3-8B-shaped decode layer",
    "llama2_70b": "Llama-2-70B-shaped 8K-context decode layer",
    "shared_prefix": "parallel sampling with shared prompt blocks",
    "long_context_b8": "32K-128K context decode, block size 8",
    "long_context_b16": "32K-128K context decode, block size 16",
    "long_context_b32": "32K-128K context decode, block size 32",
    "llama3_8b_fp8": "Llama-3-8B-shaped decode layer, FP8 E4M3 KV cache",
    "llama2_70b_fp8": "Llama-2-70B-shaped 8K-context decode layer, FP8 E4M3 KV cache",
    "long_context_b16_fp8": "32K-128K context decode, block size 16, FP8 E4M3 KV cache",
    "prefill_llama3_8b": "chunked prefill, Llama-3-8B shape: 8 x 512-token chunks after 1K-3.5K cached tokens",
    "prefill_llama2_70b": "whole-prompt prefill, Llama-2-70B shape: 4 prompts of 2048 tokens",
    "copy_blocks_device": "copy-on-write of 4096 blocks within one device pool (8 kv heads x 16 x 128, fp16)",
    "swap_out_host": "swap out of 1024 blocks from the device pools to pinned host pools (8 x 16 x 128, fp16)",
    "paging_tax_llama3_8b": "paged vs virtually contiguous decode, Llama-3-8B-shaped layer",
    "paging_tax_long_context": "paged vs virtually contiguous decode, 32K-128K contexts, block size 16",
}
FP8_SUFFIX = "_fp8"


def make_case(name):
    import workloads as W
    if name.endswith(FP8_SUFFIX):  # the same tokens, stored as E4M3 codes
        name = name[:-len(FP8_SUFFIX)]
    if name.startswith("long_context_b"):
        return W.long_context(int(name.rsplit("b", 1)[1]))
    return W.CONFIGS[name]()


def kernel_sha():
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(kernel, config, partition):
    """HBM bytes per launch from rocprofv3 FETCH_SIZE / WRITE_SIZE runs, if they were taken
    on the current kernel source and the same workload; otherwise None."""
    path = traffic_file(kernel, config)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256") != kernel_sha() or t.get("config") != config or \
            t.get("partition") != partition:
        return None
    return t.get("hbm_bytes_per_launch")


def fp8_scales(case):
    """Per-tensor E4M3 scales: the largest |k| (|v|) of the workload maps to 448."""
    import numpy as np
    f = lambda a, b: float(np.float32(max(np.abs(a.astype(np.float32)).max(initial=0.0),  # noqa: E731
                                          np.abs(b.astype(np.float32)).max(initial=0.0)) / 448.0))
    return f(case.prefix_k, case.new_k), f(case.prefix_v, case.new_v)


def host_cores():
    """Host cores this process may run on (its affinity mask), read at run time."""
    return len(os.sched_getaffinity(0))


def cpu_baseline(case, fp8=False):
    """The oracle, as it stands, on the same workload: its decode (the pools, new tokens
    included, are prepared outside the timed region), on every host core of this process."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import pa_oracle as O
    cores = host_cores()
    log(f"cpu baseline: building the oracle's pools (not timed); {cores} host cores")
    if fp8:
        ks, vs = fp8_scales(case)
        empty = np.full(case.empty_pool().shape, 0x7F, dtype=np.uint8)
        kc, vc = O.cache_write_fp8(case.prefix_k, case.prefix_v, case.prefix_slots, empty,
                                   empty.copy(), case.block_size, ks, vs)
        kc, vc = O.cache_write_fp8(case.new_k, case.new_v, case.new_slots, kc, vc, case.block_size,
                                   ks, vs)
    else:
        kc, vc = O.cache_write(case.prefix_k, case.prefix_v, case.prefix_slots, case.empty_pool(),
                               case.empty_pool(), case.block_size)
        kc, vc = O.cache_write(case.new_k, case.new_v, case.new_slots, kc, vc, case.block_size)
    elt = 1 if fp8 else case.elt_bytes
    kv_all = int(case.context_lens.astype("int64").sum()) * case.num_kv_heads * case.head_dim * 2
    n = case.num_seqs
    if kv_all * case.elt_bytes > 1.5e9:  # keep the CPU leg to tens of seconds: a prefix of the batch
        n = max(1, int(n * 1.5e9 / (kv_all * case.elt_bytes)))
    reps = 0
    with threadpool_limits(limits=cores):
        t0 = time.perf_counter()
        while reps == 0 or time.perf_counter() - t0 < 10.0:  # about 10 s of CPU work
            if fp8:
                O.decode_fp8(case.q[:n], kc, vc, ks, vs, case.block_tables[:n], case.context_lens[:n],
                             case.scale, case.block_size, case.num_kv_heads)
            else:
                O.decode(case.q[:n], kc, vc, case.block_tables[:n], case.context_lens[:n], case.scale,
                         case.block_size, case.num_kv_heads)
            reps += 1
        dt = (time.perf_counter() - t0) / reps
    kv = int(case.context_lens[:n].astype("int64").sum()) * case.num_kv_heads * case.head_dim * \
        2 * elt
    return {"value": kv / dt / 1e9, "unit": "GB/s", "cores": cores, "kind": "oracle",
            "seconds_per_call": dt, "calls": reps, "seqs_per_s": n / dt,
            "sample": f"{n} of {case.num_seqs} sequences, {reps} decode calls of about 10 s in total "
                      f"(pools with the new tokens built beforehand, untimed), numpy float64, BLAS on "
                      f"{cores} threads (the process's host cores)"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(decode shards by sequence or by kv head with no exchange between GPUs)",
              file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    import workloads
    workloads.set_progress(log)
    for name in (ALL_CONFIGS if args.config == "all" else [args.config]):
        args = argparse.Namespace(**{**vars(args), "warmup": args.warmup_arg})
        if args.warmup is None:
            args.warmup = PREFILL_WARMUP if name in PREFILL else 10
        if name in PREFILL:
            result = run_prefill(args, name)
        elif name in BLOCK_COPIES:
            result = run_block_copies(args, name)
        elif name in PAGING_TAX:
            result = run_paging_tax(args, name)
        else:
            result = run_one(args, name)
        print(json.dumps(result), flush=True)
        torch.cuda.empty_cache()


def run_one(args, config):
    """Measure one workload; returns the result line as a dict."""
    import numpy as np
    import torch

    import paged_kv_cache_167_amd as P
    dev = torch.device("cuda:0")
    partition = args.partition

    fp8 = config.endswith(FP8_SUFFIX)
    log(f"generating workload {config}")
    t_gen = time.time()
    case = make_case(config)
    elt = 1 if fp8 else case.elt_bytes  # bytes per stored K/V element
    kv_bytes = int(case.context_lens.astype(np.int64).sum()) * case.num_kv_heads * \
        case.head_dim * 2 * elt
    log(f"  {time.time() - t_gen:.1f} s; {case.num_seqs} seqs, kv bytes/step {kv_bytes/1e9:.3f} GB")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    q, tables, ctx = t(case.q), t(case.block_tables), t(case.context_lens)
    shape = (case.num_blocks, case.num_kv_heads, case.block_size, case.head_dim)
    pk, pv, ps = t(case.prefix_k), t(case.prefix_v), t(case.prefix_slots)
    if fp8:
        k_scale, v_scale = fp8_scales(case)
        k_cache = torch.full(shape, 0x7F, dtype=torch.uint8, device=dev)  # unwritten: NaN code
        v_cache = torch.full(shape, 0x7F, dtype=torch.uint8, device=dev)
        P.pa_cache_write_fp8(pk, pv, ps, k_cache, v_cache, k_scale, v_scale)
    else:
        tdt = torch.float16 if case.dtype == np.float16 else torch.float32
        k_cache = torch.full(shape, float("nan"), dtype=tdt, device=dev)
        v_cache = torch.full(shape, float("nan"), dtype=tdt, device=dev)
        P.pa_cache_write(pk, pv, ps, k_cache, v_cache)
    del pk, pv, ps
    new_k, new_v, new_slots = t(case.new_k), t(case.new_v), t(case.new_slots)
    out = torch.empty_like(q)
    mcl = case.max_context_len
    # fused step: one pa_decode_append (pa_decode_fp8_append), which stores each new token at
    # the slot its table gives position ctx - 1 (the workloads put it exactly there) and
    # attends.  By default for fp16 pools only: for E4M3 pools the fused stream kernel's
    # operand substitution costs as much as the separate store launch saves.
    shared = config == "shared_prefix" and not fp8 and case.dtype == np.float16 and \
        args.step in ("auto", "shared")
    fused = not shared and case.dtype == np.float16 and (args.step == "fused" or (args.step == "auto" and not fp8))
    if fused:
        last = case.context_lens.astype(np.int64) - 1
        table_slots = case.block_tables[np.arange(case.num_seqs), last // case.block_size].astype(np.int64) * \
            case.block_size + last % case.block_size
        assert np.array_equal(table_slots, case.new_slots), "new tokens off their table slots"

    ws_bytes = P.pa_decode_workspace_bytes(case.num_seqs, case.num_q_heads, case.num_kv_heads,
                                           case.head_dim, mcl, partition)
    if shared:
        import workloads as W
        groups = [t(a) for a in W.shared_prefix_groups(case)]
        ws_bytes = P.pa_decode_shared_workspace_bytes(case.num_seqs, int(groups[1].shape[0]), case.num_q_heads,
                                                      case.num_kv_heads, case.head_dim)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    if args.calibrate_copy_mib > 0:
        src = torch.ones(args.calibrate_copy_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cur = [stream]  # the stream the step launches on (a capture stream while a graph records it)

    def write_only():
        if fp8:
            P.pa_cache_write_fp8(new_k, new_v, new_slots, k_cache, v_cache, k_scale, v_scale,
                                 stream=cur[0])
        else:
            P.pa_cache_write(new_k, new_v, new_slots, k_cache, v_cache, stream=cur[0])

    def decode_only():
        if shared:
            P.pa_decode_shared(out, q, k_cache, v_cache, tables, ctx, *groups, case.scale, case.block_size,
                               case.num_kv_heads, max_context_len=mcl, workspace=ws, stream=cur[0])
        elif fused and fp8:
            P.pa_decode_fp8_append(out, q, new_k, new_v, k_cache, v_cache, tables, ctx, case.scale,
                                   k_scale, v_scale, case.block_size, case.num_kv_heads,
                                   max_context_len=mcl, partition_size=partition, workspace=ws,
                                   stream=cur[0])
        elif fused:
            P.pa_decode_append(out, q, new_k, new_v, k_cache, v_cache, tables, ctx, case.scale,
                               case.block_size, case.num_kv_heads, max_context_len=mcl,
                               partition_size=partition, workspace=ws, stream=cur[0])
        elif fp8:
            P.pa_decode_fp8(out, q, k_cache, v_cache, tables, ctx, case.scale, k_scale, v_scale,
                            case.block_size, case.num_kv_heads, max_context_len=mcl,
                            partition_size=partition, workspace=ws, stream=cur[0])
        else:
            P.pa_decode(out, q, k_cache, v_cache, tables, ctx, case.scale, case.block_size,
                        case.num_kv_heads, max_context_len=mcl, partition_size=partition,
                        workspace=ws, stream=cur[0])

    def step():
        if not fused:
            write_only()
        decode_only()

    def stream_kernel():  # the first of the step's two attention launches, on its own
        if shared:
            P.pa_decode_shared_partitions(out, q, k_cache, v_cache, tables, ctx, *groups, case.scale,
                                          case.block_size, case.num_kv_heads, max_context_len=mcl,
                                          workspace=ws, stream=stream)
        elif fused and fp8:
            P.pa_decode_fp8_append_partitions(out, q, new_k, new_v, k_cache, v_cache, tables, ctx,
                                              case.scale, k_scale, v_scale, case.block_size,
                                              case.num_kv_heads, max_context_len=mcl,
                                              partition_size=partition, workspace=ws,
                                              stream=stream)
        elif fused:
            P.pa_decode_append_partitions(out, q, new_k, new_v, k_cache, v_cache, tables, ctx,
                                          case.scale, case.block_size, case.num_kv_heads,
                                          max_context_len=mcl, partition_size=partition,
                                          workspace=ws, stream=stream)
        elif fp8:
            P.pa_decode_fp8_partitions(out, q, k_cache, v_cache, tables, ctx, case.scale, k_scale,
                                       v_scale, case.block_size, case.num_kv_heads,
                                       max_context_len=mcl, partition_size=partition,
                                       workspace=ws, stream=stream)
        else:
            P.pa_decode_partitions(out, q, k_cache, v_cache, tables, ctx, case.scale,
                                   case.block_size, case.num_kv_heads, max_context_len=mcl,
                                   partition_size=partition, workspace=ws, stream=stream)

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # a serving loop replays one captured step per iteration: the host's launch work (Python
    # marshalling, argument checks, two or three kernel launches) leaves the step
    graph = None
    if args.graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            cur[0] = torch.cuda.current_stream(dev)
            step()
        cur[0] = stream
        torch.cuda.synchronize()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()

    # the timed steps: nothing but the path's own launches between the two synchronisations
    # (an event recorded between two kernels costs several microseconds of GPU time)
    log(f"timing {args.steps} steps" + (" (graph replays)" if graph is not None else ""))
    t0 = time.perf_counter()
    for _ in range(args.steps):
        if graph is not None:
            graph.replay()
        else:
            step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    # Each call is timed two ways, both with HIP events on the launch stream:
    #  * cold (primary): one launch between two events, after reading 1 GiB so that neither L2
    #    nor the 256 MB MALL holds the pool (a read, not a write: a writing flush would leave
    #    dirty lines whose write-back competes with the timed kernel); median and min over
    #    --cold-iters launches;
    #  * warm: --steps back-to-back launches between two events, averaged.
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev) if args.cold_iters > 0 else None

    def warm_ms(fn):
        fn()
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    def cold_ms(fn):
        times = []
        for _ in range(args.cold_iters):
            flush.sum()
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            times.append(e0.elapsed_time(e1))
        return times

    timing = {}
    for key, fn in (("kernel", stream_kernel), ("decode", decode_only), ("write", write_only)):
        timing[key] = {"warm": warm_ms(fn), "cold": cold_ms(fn) if flush is not None else []}
    del flush
    step()  # leave the rows pa_decode writes in out
    torch.cuda.synchronize()

    def primary_ms(key):  # cold median, or the warm average when no cold launch was asked for
        c = timing[key]["cold"]
        return float(np.median(c)) if c else timing[key]["warm"]

    def summary(key):
        c = timing[key]["cold"]
        d = {"warm_us": round(timing[key]["warm"] * 1e3, 2)}
        if c:
            d.update({"cold_median_us": round(float(np.median(c)) * 1e3, 2),
                      "cold_min_us": round(float(np.min(c)) * 1e3, 2),
                      "cold_mean_us": round(float(np.mean(c)) * 1e3, 2), "cold_launches": len(c)})
        return d

    tokens_blocks = int(sum(-(-int(c) // case.block_size) for c in case.context_lens))
    q_bytes = case.num_seqs * case.num_q_heads * case.head_dim * case.elt_bytes
    # K/V rows, q in, out, the table entries in use and the context lengths
    alg_bytes = kv_bytes + 2 * q_bytes + tokens_blocks * 4 + case.num_seqs * 4
    unique = case.unique_kv_bytes() if config == "shared_prefix" else kv_bytes
    if shared:  # the shared kernel reads each shared block once: its bytes are the unique ones
        alg_bytes = alg_bytes - kv_bytes + unique
    kern_ms = primary_ms("kernel")
    achieved = alg_bytes / (kern_ms * 1e-3) / 1e9
    warm_achieved = alg_bytes / (timing["kernel"]["warm"] * 1e-3) / 1e9
    step_gbs = kv_bytes / (ms_per_step * 1e-3) / 1e9
    kernel = "pa_shared_mfma_kernel" if shared else stream_kernel_name(case.dtype == np.float16)
    traffic = measured_traffic(kernel, config, partition)
    # fp16 (or fp32) rows in, stored rows out
    write_bytes = 2 * case.num_seqs * case.num_kv_heads * case.head_dim * (case.elt_bytes + elt)
    dec_ms, wr_ms = primary_ms("decode"), primary_ms("write")
    gbs = lambda b, ms: b / (ms * 1e-3) / 1e9  # noqa: E731

    result = {
        "metric": "paged decode KV GB/s and % of MI355X HBM peak; sequences/s per layer",
        "value": round(step_gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if case.dtype == np.float16 else "f32",
        "data": "synthetic",
        "config": {
            "workload": WORKLOAD_NAMES[config], "name": config,
            "num_seqs": case.num_seqs, "num_q_heads": case.num_q_heads,
            "num_kv_heads": case.num_kv_heads, "head_dim": case.head_dim,
            "block_size": case.block_size, "num_blocks": case.num_blocks,
            "context_lens": f"{int(case.context_lens.min())}..{int(case.context_lens.max())}, "
                            f"sum {int(case.context_lens.sum())}",
            "partition_size": partition, "kv_bytes_per_step": kv_bytes,
            "kv_cache": "e4m3" if fp8 else ("f16" if case.dtype == np.float16 else "f32"),
            "step": "pa_cache_write + pa_decode_shared" if shared else
                    (("pa_decode_fp8_append" if fp8 else "pa_decode_append") if fused else
                     "pa_cache_write + pa_decode"),
            "graph": graph is not None,  # timed steps are replays of one captured HIP graph
            **({"kv_bytes_counted": "every sequence's whole context, a shared prefix once per member; "
                                    "pa_decode.unique_* and roofline count the distinct blocks"}
               if unique != kv_bytes else {}),
        },
        "pct_hbm_peak": round(100.0 * step_gbs / HBM_PEAK_GBS, 2),
        "seqs_per_s_per_layer": round(case.num_seqs / (ms_per_step * 1e-3), 1),
        "pa_decode": {  # the whole call (both launches); figures from the cold median
            "call": "pa_decode_shared" if shared else
                    (("pa_decode_fp8_append" if fp8 else "pa_decode_append") if fused else "pa_decode"),
            "us": round(dec_ms * 1e3, 2),
            **summary("decode"),
            "kv_gbs": round(gbs(kv_bytes, dec_ms), 1),
            "pct_hbm_peak": round(100.0 * gbs(kv_bytes, dec_ms) / HBM_PEAK_GBS, 2),
            "warm_pct_hbm_peak": round(100.0 * gbs(kv_bytes, timing["decode"]["warm"]) / HBM_PEAK_GBS, 2),
            "unique_kv_bytes": unique,
            "unique_kv_gbs": round(gbs(unique, dec_ms), 1),
            "unique_pct_hbm_peak": round(100.0 * gbs(unique, dec_ms) / HBM_PEAK_GBS, 2),
            "seqs_per_s_per_layer": round(case.num_seqs / (dec_ms * 1e-3), 1),
        },
        "pa_cache_write": {  # with pa_decode_append the step does not call it: timed alone
            "in_step": not fused,
            "us": round(wr_ms * 1e3, 2),
            **summary("write"),
            "gbs": round(gbs(write_bytes, wr_ms), 2),
            "bytes": write_bytes,
        },
        "roofline": {
            "kernel": kernel,
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "alg_bytes_per_launch": alg_bytes,
            "timing": "cold median" if timing["kernel"]["cold"] else "warm average",
            "launch_us": round(kern_ms * 1e3, 2),
            **summary("kernel"),
            "warm_achieved": round(warm_achieved, 1),
            "warm_frac": round(warm_achieved / HBM_PEAK_GBS, 4),
        },
    }
    if unique != kv_bytes and not shared:  # shared blocks: the bytes HBM must deliver are the unique ones
        alg_unique = alg_bytes - kv_bytes + unique
        result["roofline"]["unique_alg_bytes_per_launch"] = alg_unique
        result["roofline"]["unique_achieved"] = round(gbs(alg_unique, kern_ms), 1)
        result["roofline"]["unique_frac"] = round(gbs(alg_unique, kern_ms) / HBM_PEAK_GBS, 4)
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(case, fp8)
    del k_cache, v_cache, ws
    return result


def prefill_cpu_baseline(case):
    """The oracle on one sequence's chunk (about 10 s of CPU work at most), scaled to flops."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import pa_oracle as O
    kc, vc = O.cache_write(case.prefix_k, case.prefix_v, case.prefix_slots, case.empty_pool(),
                           case.empty_pool(), case.block_size)
    kc, vc = O.cache_write(case.new_k, case.new_v, case.new_slots, kc, vc, case.block_size)
    n_all = int(case.query_start[1])
    ctx = int(case.context_lens[0])
    n = n_all
    cores = host_cores()
    with threadpool_limits(limits=cores):
        while True:  # a prefix of sequence 0's chunk: rows 0 .. n-1 (the context cut after them)
            t0 = time.perf_counter()
            O.prefill(case.q[:n], kc, vc, case.block_tables[:1],
                      np.array([ctx - n_all + n], np.int32), np.array([0, n], np.int32),
                      case.scale, case.block_size, case.num_kv_heads)
            dt = time.perf_counter() - t0
            if dt < 30.0 or n <= 8:
                break
            n = max(8, int(n * 20.0 / dt))
    c0 = ctx - n_all  # cached tokens before the chunk
    flops = 4 * case.head_dim * case.num_q_heads * (n * c0 + n * (n + 1) // 2)
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "seconds": dt, "sample": f"the first {n} of sequence 0's {n_all} chunk tokens "
                                     f"(one call), numpy float64, BLAS on {cores} threads"}


def run_prefill(args, config):
    """One step = pa_cache_write of every chunk token, then pa_prefill; TFLOP/s of attention."""
    import numpy as np
    import torch

    import paged_kv_cache_167_amd as P
    import workloads as W
    dev = torch.device("cuda:0")
    log(f"generating workload {config}")
    case = W.PREFILL_CONFIGS[config]()
    flops = case.flops()
    log(f"  {case.num_seqs} seqs, {case.total_q} query tokens, {flops / 1e9:.1f} GFLOP per step")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    q, tables, ctx, qs = t(case.q), t(case.block_tables), t(case.context_lens), t(case.query_start)
    shape = (case.num_blocks, case.num_kv_heads, case.block_size, case.head_dim)
    k_cache = torch.full(shape, float("nan"), dtype=torch.float16, device=dev)
    v_cache = torch.full(shape, float("nan"), dtype=torch.float16, device=dev)
    if len(case.prefix_slots):
        P.pa_cache_write(t(case.prefix_k), t(case.prefix_v), t(case.prefix_slots), k_cache, v_cache)
    new_k, new_v, new_slots = t(case.new_k), t(case.new_v), t(case.new_slots)
    out = torch.empty_like(q)
    stream = torch.cuda.current_stream(dev)
    mql, mcl = case.max_query_len, case.max_context_len
    if args.calibrate_copy_mib > 0:  # a copy of known size that scales the HBM byte counters
        src = torch.ones(args.calibrate_copy_mib << 18, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def write_only():
        P.pa_cache_write(new_k, new_v, new_slots, k_cache, v_cache, stream=stream)

    def prefill_only():
        P.pa_prefill(out, q, k_cache, v_cache, tables, ctx, qs, case.scale, case.block_size,
                     case.num_kv_heads, mql, max_context_len=mcl, stream=stream)

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        write_only()
        prefill_only()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        write_only()
        prefill_only()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    per = {}
    for key, fn in (("prefill", prefill_only), ("write", write_only)):
        fn()
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        per[key] = e0.elapsed_time(e1) / args.steps
    achieved = flops / (per["prefill"] * 1e-3) / 1e12
    kv = case.kv_bytes()
    result = {
        "metric": "chunked-prefill attention TFLOP/s over the paged cache",
        "value": round(flops / (ms_per_step * 1e-3) / 1e12, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": WORKLOAD_NAMES[config], "name": config, "num_seqs": case.num_seqs,
                   "num_q_heads": case.num_q_heads, "num_kv_heads": case.num_kv_heads,
                   "head_dim": case.head_dim, "block_size": case.block_size,
                   "query_tokens": case.total_q,
                   "context_lens": f"{int(case.context_lens.min())}..{int(case.context_lens.max())}",
                   "flops_per_step": flops, "kv_bytes": kv},
        "pa_prefill": {"us": round(per["prefill"] * 1e3, 2), "tflops": round(achieved, 2),
                       "query_tokens_per_s": round(case.total_q / (per["prefill"] * 1e-3), 1)},
        "pa_cache_write": {"us": round(per["write"] * 1e3, 2)},
        "roofline": {"kernel": "pa_prefill_kernel", "bound": "mfma", "achieved": round(achieved, 2),
                     "peak": MFMA_F16_PEAK_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / MFMA_F16_PEAK_TFLOPS, 4),
                     "traffic": measured_traffic("pa_prefill_kernel", config, 0),  # HBM bytes per launch
                     "alg_flops_per_launch": flops, "avg_launch_us": round(per["prefill"] * 1e3, 2)},
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = prefill_cpu_baseline(case)
    return result


def run_block_copies(args, config):
    """Block copies: copy-on-write within the device pools, or swap out to pinned host pools.
    One step = one pa_copy_blocks call over all the pairs."""
    import numpy as np
    import torch

    import paged_kv_cache_167_amd as P
    dev = torch.device("cuda:0")
    rng = np.random.default_rng(1008)
    hkv, bsz, d = 8, 16, 128
    n_pool = 8192
    device_copy = config == "copy_blocks_device"
    n_pairs = 4096 if device_copy else 1024
    k = torch.randn((n_pool, hkv, bsz, d), dtype=torch.float16, device=dev)
    v = torch.randn_like(k)
    if device_copy:  # sources in the first half, distinct destinations in the second
        pairs = np.stack([rng.integers(0, n_pool // 2, n_pairs), n_pool // 2 + rng.permutation(n_pool // 2)[:n_pairs]], 1)
        dk, dv = k, v
    else:
        pairs = np.stack([rng.permutation(n_pool)[:n_pairs], rng.permutation(n_pairs)], 1)
        dk = torch.empty((n_pairs, hkv, bsz, d), dtype=torch.float16).pin_memory()
        dv = torch.empty_like(dk).pin_memory()
    pairs_t = torch.from_numpy(pairs.astype(np.int32)).to(dev)
    stream = torch.cuda.current_stream(dev)
    block_bytes = hkv * bsz * d * 2
    moved = 2 * n_pairs * block_bytes  # K and V blocks copied

    def step():
        P.pa_copy_blocks(k, v, dk, dv, pairs_t, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    kern_ms = e0.elapsed_time(e1) / args.steps
    # device: every byte read from and written to HBM; host: every byte crosses the host link
    traffic = 2 * moved if device_copy else moved
    achieved = traffic / (kern_ms * 1e-3) / 1e9
    peak = HBM_PEAK_GBS if device_copy else HOST_LINK_GBS
    result = {
        "metric": "paged block copy GB/s (copy-on-write / swap)",
        "value": round(moved / (ms * 1e-3) / 1e9, 1), "unit": "GB/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_NAMES[config], "name": config, "pairs": n_pairs,
                   "block_bytes_per_pool": block_bytes, "bytes_copied": moved},
        "roofline": {"kernel": "pa_copy_blocks_kernel", "bound": "hbm" if device_copy else "host link",
                     "achieved": round(achieved, 1), "peak": peak, "unit": "GB/s",
                     "frac": round(achieved / peak, 4), "traffic": None,
                     "alg_bytes_per_launch": traffic, "avg_launch_us": round(kern_ms * 1e3, 2)},
    }
    if not args.no_cpu_baseline:
        from oracle import pa_oracle as O
        kc, vc = k[: n_pool // 4].cpu().numpy(), v[: n_pool // 4].cpu().numpy()
        sub = pairs[(pairs[:, 0] < n_pool // 4)]
        sub = np.stack([sub[:, 0], np.arange(len(sub)) % (n_pool // 4)], 1)
        t0 = time.perf_counter()
        O.copy_blocks(kc, vc, kc, vc, sub)
        dt = time.perf_counter() - t0
        result["cpu_baseline"] = {"value": round(2 * len(sub) * block_bytes / dt / 1e9, 3), "unit": "GB/s",
                                  "cores": 1, "kind": "oracle",
                                  "sample": f"{len(sub)} block pairs within a {n_pool // 4}-block host pool "
                                            "(numpy array copies: one thread)"}
    return result


def run_paging_tax(args, config):
    """The same decode over the same tokens, once through block tables over a scattered pool
    (pa_decode) and once over a virtually contiguous cache backed page by page through HIP
    virtual memory (pa_decode_dense): the paging tax is the time difference."""
    import numpy as np
    import torch

    import paged_kv_cache_167_amd as P
    import workloads as W
    dev = torch.device("cuda:0")
    case = W.llama3_8b() if config == "paging_tax_llama3_8b" else W.long_context(16)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)  # noqa: E731
    q, tables, ctx = t(case.q), t(case.block_tables), t(case.context_lens)
    shape = (case.num_blocks, case.num_kv_heads, case.block_size, case.head_dim)
    kc = torch.full(shape, float("nan"), dtype=torch.float16, device=dev)
    vc = torch.full(shape, float("nan"), dtype=torch.float16, device=dev)
    P.pa_cache_write(t(case.prefix_k), t(case.prefix_v), t(case.prefix_slots), kc, vc)
    P.pa_cache_write(t(case.new_k), t(case.new_v), t(case.new_slots), kc, vc)
    mcl = case.max_context_len
    out_p, out_d = torch.empty_like(q), torch.empty_like(q)
    ws = torch.empty(P.pa_decode_workspace_bytes(case.num_seqs, case.num_q_heads, case.num_kv_heads,
                                                 case.head_dim, mcl, 0), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        hot = e0.elapsed_time(e1) / args.steps
        cold = []
        for _ in range(5):
            flush.sum()
            e0.record(stream)
            fn()
            e1.record(stream)
            torch.cuda.synchronize()
            cold.append(e0.elapsed_time(e1))
        return hot, float(np.median(cold))

    ph, pc = timed(lambda: P.pa_decode(out_p, q, kc, vc, tables, ctx, case.scale, case.block_size,
                                       case.num_kv_heads, max_context_len=mcl, workspace=ws, stream=stream))
    seq = np.concatenate([np.full(int(c) - 1, s, np.int32) for s, c in enumerate(case.context_lens)])
    pos = np.concatenate([np.arange(int(c) - 1, dtype=np.int32) for c in case.context_lens])
    order = np.concatenate(case.meta["seq_rows"])
    dense = {}
    token_bytes = case.num_kv_heads * case.head_dim * 2
    for want in (256 << 10, 2 << 20, 8 << 20):  # page sizes, rounded up to whole 16-token tiles
        unit = 16 * token_bytes
        page = -(-want // unit) * unit
        try:
            kv = P.DenseKV(case.num_seqs, mcl, case.num_kv_heads, case.head_dim, page_bytes=page)
        except P.PaError as err:  # not a multiple of the allocation granularity
            dense[f"{page >> 10}K"] = {"error": str(err)}
            continue
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        try:
            kv.step(case.context_lens.tolist())  # every page mapped from scratch
        except P.PaError as err:
            dense[f"{page >> 10}K"] = {"error": str(err)}
            kv.close()
            continue
        map_ms = (time.perf_counter() - t0) * 1e3
        pages = kv.mapped_bytes // kv.page_bytes
        kv.write(t(case.prefix_k[order]), t(case.prefix_v[order]), t(seq), t(pos))
        kv.write(t(case.new_k), t(case.new_v), t(np.arange(case.num_seqs, dtype=np.int32)),
                 t((case.context_lens - 1).astype(np.int32)))
        dh, dc = timed(lambda: kv.decode(out_d, q, case.scale, workspace=ws, stream=stream))
        dense[f"{kv.page_bytes >> 10}K"] = {
            "us": round(dh * 1e3, 2), "cold_us": round(dc * 1e3, 2),
            "kv_gbs": round(case.kv_bytes() / (dh * 1e-3) / 1e9, 1), "pages_mapped": int(pages),
            "map_all_ms": round(map_ms, 3), "map_us_per_page": round(map_ms * 1e3 / max(pages, 1), 2),
            "paging_tax_pct": round(100.0 * (ph / dh - 1.0), 2),
            "outputs_bitwise_equal": bool(torch.equal(out_p, out_d))}
        kv.close()
    kv_bytes = case.kv_bytes()
    best = min((v["us"], k) for k, v in dense.items() if "us" in v) if any("us" in v for v in dense.values()) \
        else (float("nan"), None)
    dh = best[0] * 1e-3
    result = {
        "metric": "paging tax: pa_decode over block tables vs over a virtually contiguous cache",
        "value": round(100.0 * (ph / dh - 1.0), 2), "unit": "% slower paged than the best page size (warm)",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ph, 5),
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": WORKLOAD_NAMES[config], "name": config, "num_seqs": case.num_seqs,
                   "kv_bytes_per_step": kv_bytes, "block_size": case.block_size},
        "paged": {"us": round(ph * 1e3, 2), "cold_us": round(pc * 1e3, 2),
                  "kv_gbs": round(kv_bytes / (ph * 1e-3) / 1e9, 1)},
        "dense_by_page_size": dense, "best_page": best[1],
    }
    return result


if __name__ == "__main__":
    main()
