"""Benchmark of the paged decode hot path on one MI355X.

One step = one pass of the whole hot path over one batch: the new token of every sequence
goes into its slot and the decode (plus its partition merge when the plan splits) attends
over every sequence's context -- pa_write_kv followed by the decode, or with --step fused
one pa_decode_append call that does both (plain path, no shared blocks).  Block tables
come from the library's block manager before timing (allocation is host work, off the timed path).
Inputs are synthetic, seeded, and resident in HBM before the timed region starts.
Consecutive steps use two layers' K/V pools in turn (same tables), so a step never reads
K/V that the previous step left in the Infinity Cache.

Prints one JSON line: value = algorithmic KV bytes read per step / step time (GB/s),
plus decode tokens/s, a roofline entry for the decode kernel (HIP events on the launch
stream) and the CPU oracle timed on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--workload opt13b_layer]
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

HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth
COUNTER_SOURCES = os.path.join(ROOT, "paged_kv_cache_89_amd", "csrc")


def measured_traffic(workload: str, decode_path: str):
    """HBM bytes per decode call from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    summary of this workload, or None when there is none, it was taken on the other decode
    path, or the kernel sources changed since the counters were taken."""
    import hashlib

    rec = None
    for name in (f"decode_counters_{workload}.json", f"decode_counters_{workload}_{decode_path}.json"):
        path = os.path.join(ROOT, "profiles", name)
        if os.path.exists(path):
            r = json.load(open(path))
            if r.get("decode_path", "plain") == decode_path:
                rec = r
                break
    if rec is None:
        return None
    h = hashlib.sha256()
    for f in rec["kernel_sources"]:
        h.update(open(os.path.join(COUNTER_SOURCES, f), "rb").read())
    if h.hexdigest()[:16] != rec["kernel_sources_sha256_16"]:
        return None
    return int(rec["traffic_bytes_per_launch"])


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 100; 1000 for tiny_mha, whose steps take µs)")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="opt13b_layer")
    ap.add_argument("--partition-size", type=int, default=-1,
                    help="-1: the workload's setting (0 = library choice)")
    ap.add_argument("--decode-flags", type=int, default=-1,
                    help="-1: the workload's setting (PA_DECODE_SHARED_KV for shared prompts)")
    ap.add_argument("--decode-path", choices=["auto", "plain", "shared_prefix", "multi"],
                    default="auto",
                    help="auto: the shared-prefix (cascade) decode for workloads whose "
                         "sequences share prompt blocks, else the plain decode; multi: "
                         "--query-len draft tokens per sequence verified in one pass")
    ap.add_argument("--step", choices=["fused", "separate"], default="separate",
                    help="separate: pa_write_kv, then the decode; fused: the KV write and "
                         "the decode in one call (pa_decode_append; plain path, workloads "
                         "without shared blocks)")
    ap.add_argument("--query-len", type=int, default=4,
                    help="draft tokens per sequence for --decode-path multi (causal)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one device copy of 1 GiB (for hardware-counter scaling)")
    ap.add_argument("--copy-blocks", type=int, default=0, metavar="N",
                    help="also time one pa_copy_blocks launch of N block pairs (copy-on-write)")
    ap.add_argument("--swap", type=int, default=0, metavar="N",
                    help="also time pa_swap_blocks moving the blocks of the first N sequences "
                         "to pinned host memory and back, beside a DMA copy of the same bytes")
    args = ap.parse_args()
    if args.steps is None:
        args.steps = 1000 if args.workload == "tiny_mha" else 100
    return args


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this operator is built and measured on a single "
              "MI355X (no multi-GPU path); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import paged_kv_cache_89_amd as pa
    import workloads

    names = list(workloads.SPECS)
    sp = workloads.SPECS[args.workload]
    if args.step == "fused" and (sp.group_size or args.decode_path not in ("auto", "plain")):
        raise SystemExit("--step fused needs the plain decode path and no shared blocks")
    torch.cuda.set_device(0)
    seed = 8900 + names.index(args.workload)
    P = sp.partition_size if args.partition_size < 0 else args.partition_size

    # ---- inputs (untimed): lengths, block tables from the block manager, pools, new rows
    ctx, free = workloads.draw_lengths(sp, seed)
    pg, pl = workloads.prefix_groups(sp)
    bm = pa.BlockManager(sp.num_blocks, sp.block_size, free)
    tables, _ = bm.alloc_tables(ctx, sp.max_blocks, pg, pl)
    # Two layers' K/V pools that share the block tables (as every layer of a model does):
    # the timed steps alternate between them, so no step finds the K/V it reads left in the
    # 256 MB Infinity Cache by the step before (in a real model the other layers run in
    # between).  Each layer has its own e4m3 scales.
    q, kc, vc, k_scale, v_scale = workloads.device_pool(sp, seed)
    _, kc2, vc2, k_scale2, v_scale2 = workloads.device_pool(sp, seed + 1000)
    layers = [(kc, vc, k_scale, v_scale), (kc2, vc2, k_scale2, v_scale2)]
    S, Hq, Hkv, D, B = sp.num_seqs, sp.num_heads, sp.num_kv_heads, sp.head_dim, sp.block_size
    g = torch.Generator(device="cuda")
    g.manual_seed(seed + 1)
    src_t = {"f16": torch.float16, "bf16": torch.bfloat16}[sp.src_dtype]
    # new rows per step: one token per sequence (the last position), or the query_len
    # draft positions of the multi-token path
    T = args.query_len if args.decode_path == "multi" else 1
    k_new = torch.randn((S * T, Hkv, D), generator=g, device="cuda").to(src_t)
    v_new = torch.randn((S * T, Hkv, D), generator=g, device="cuda").to(src_t)
    tables_d = torch.from_numpy(tables).cuda()
    ctx_d = torch.from_numpy(ctx).cuda()
    seq_ids = torch.arange(S, dtype=torch.int32, device="cuda").repeat_interleave(T)
    positions = (ctx_d.repeat_interleave(T) - T
                 + torch.arange(T, dtype=torch.int32, device="cuda").repeat(S)).to(torch.int32)
    max_ctx = int(ctx.max())
    out = torch.empty_like(q)
    # the plain and multi-token decodes' split (the flat split for fp16/bf16 caches)
    used_P, nparts, flat_min = pa.decode_plan(S, Hq, Hkv, D, B, max_ctx, P, kc.dtype)
    ws_bytes = pa.decode_workspace_size(S, Hq, Hkv, D, B, max_ctx, P)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def write(layer):
        lk, lv, ks, vs = layers[layer]
        k_inv = 1.0 / ks if sp.kv_dtype == "e4m3" else 1.0
        v_inv = 1.0 / vs if sp.kv_dtype == "e4m3" else 1.0
        pa.write_kv(k_new, v_new, lk, lv, tables_d, seq_ids, positions, k_inv, v_inv,
                    stream=stream)

    cascade_plan = None
    path = args.decode_path
    if path == "auto":
        path = "shared_prefix" if sp.group_size else "plain"
    # the plain decode over shared prompt blocks keeps them cacheable; the shared-prefix
    # decode reads each of them once and streams everything
    flags = pa.DECODE_SHARED_KV if sp.group_size and path == "plain" else 0
    if args.decode_flags >= 0:
        flags = args.decode_flags
    kv_bytes = workloads.kv_bytes(sp, ctx)  # K+V bytes of every sequence's own context
    unique_bytes = kv_bytes                 # K+V bytes one decode pass must read
    mfma = B == 16 and Hq // Hkv >= 2        # grouped queries run on the matrix-core kernel
    kernels = (("paged_decode_gqa_mfma_kernel" if mfma else "paged_decode_kernel")
               + (" + merge_partitions_kernel" if nparts > 1 else ""))
    if path == "multi":
        qm = torch.randn((S, T, Hq, D), generator=g, device="cuda").to(q.dtype)
        outm = torch.empty_like(qm)
        ws_bytes = pa.decode_multi_workspace_size(S, T, Hq, Hkv, D, B, max_ctx, P)
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
        kernels = ("paged_decode_gqa_mfma_kernel (query_len x group columns)"
                   + (" + merge_partitions_kernel" if nparts > 1 else ""))

        def decode(layer):
            lk, lv, ks, vs = layers[layer]
            pa.decode_multi(qm, lk, lv, tables_d, ctx_d, max_ctx, sp.scale, ks, vs,
                            partition_size=P, flags=flags, out=outm, workspace=ws,
                            stream=stream)
    elif path == "shared_prefix":
        if not sp.group_size:
            raise SystemExit("--decode-path shared_prefix needs a workload with shared prompts")
        prefix_blocks = (pl // B).astype(np.int32)
        max_pb = int(prefix_blocks.max())
        pb_d = torch.from_numpy(prefix_blocks).cuda()
        ws_bytes = pa.decode_shared_prefix_workspace_size(S, Hq, Hkv, D, B, max_ctx, max_pb, P)
        ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
        # a group's shared tokens are read once, every sequence's remaining tokens once
        shared_tok = np.minimum(prefix_blocks * B, ctx.reshape(-1, sp.group_size).max(axis=1))
        own = ctx - np.minimum(np.repeat(prefix_blocks * B, sp.group_size), ctx)
        unique_bytes = workloads.kv_bytes(sp, np.concatenate([shared_tok, own]))
        cascade_plan = pa.decode_shared_prefix_plan(S, Hq, Hkv, D, B, max_ctx, max_pb, P,
                                                    pa.FP8_E4M3 if sp.kv_dtype == "e4m3" else
                                                    pa.BF16 if sp.kv_dtype == "bf16" else pa.F16)
        kernels = ("cascade_fp8_kernel (group prefixes and own tokens in one launch)"
                   if cascade_plan["decode_launches"] == 1 else
                   "paged_decode_gqa_mfma_kernel (group prefixes) + paged_decode_kernel "
                   "(own tokens)") + " + merge_partitions_kernel"

        def decode(layer):
            lk, lv, ks, vs = layers[layer]
            pa.decode_shared_prefix(q, lk, lv, tables_d, ctx_d, pb_d, sp.group_size, max_ctx,
                                    max_pb, sp.scale, ks, vs, partition_size=P,
                                    flags=flags, out=out, workspace=ws, stream=stream)
    else:
        def decode(layer):
            lk, lv, ks, vs = layers[layer]
            pa.decode(q, lk, lv, tables_d, ctx_d, max_ctx, sp.scale, ks, vs,
                      partition_size=P, flags=flags, out=out, workspace=ws, stream=stream)

    # The step: the new tokens' KV write and the decode, as two launches or as one
    # (pa_decode_append stores each sequence's new row from the unit that reads its block;
    # a new token must not land in a block another sequence reads).  The two launches are
    # the default: the fused call measured about 0.4% slower per step on the OPT-13B layer.
    fused = args.step == "fused"  # (its preconditions were checked before any GPU work)
    if fused:
        kernels = kernels.replace("paged_decode_kernel", "paged_decode_kernel (storing the new token)", 1) \
            .replace("paged_decode_gqa_mfma_kernel", "paged_decode_gqa_mfma_kernel (storing the new token)", 1)

        def decode(layer):
            lk, lv, ks, vs = layers[layer]
            k_inv = 1.0 / ks if sp.kv_dtype == "e4m3" else 1.0
            v_inv = 1.0 / vs if sp.kv_dtype == "e4m3" else 1.0
            pa.decode_append(q, k_new, v_new, lk, lv, tables_d, ctx_d, max_ctx, sp.scale, ks, vs,
                             k_inv, v_inv, partition_size=P, flags=flags, out=out, workspace=ws,
                             stream=stream)

        def write(layer):  # part of the fused call
            pass

    for i in range(args.warmup):
        write(i % 2)
        decode(i % 2)
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps, device synchronised on both sides.  No events in
    # it: recording one costs about 3 us of GPU time, so the decode launch is timed with
    # HIP events in a second pass of K steps right after.
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        write(i % 2)
        decode(i % 2)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    for i in range(args.steps):
        write(i % 2)
        ev[i][0].record(stream)
        decode(i % 2)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    dec_ms = [a.elapsed_time(b) for a, b in ev]
    dec_ms_mean = float(np.mean(dec_ms))
    value = kv_bytes / (ms_per_step * 1e-3) / 1e9
    # the flat split's chunk length, as the last decode chose it on the device (the word
    # after the partials in the workspace)
    flat_split = None
    if flat_min and path in ("plain", "multi") and not flags:
        rows = S * T * Hq
        off = rows * nparts * (D + 2) * 4
        chunk, waves = ws[off:off + 8].view(torch.int32).tolist()
        flat_split = {"min_chunk_blocks": flat_min, "chunk_blocks": chunk, "grid_waves": waves,
                      "max_partials_per_row": nparts}
    achieved = unique_bytes / (dec_ms_mean * 1e-3) / 1e9

    if args.copy_calibration:
        # A plain device copy of known size: the hardware-counter runs scale FETCH_SIZE /
        # WRITE_SIZE of the decode kernel by what the counters read for this copy.
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # Latency distribution of the decode call: as timed above (layers alternating), and
    # with one layer only, with and without a 512 MiB write before each call (evicts L2
    # and the Infinity Cache); the write is outside the events.
    def distribution(flush, reps, alternate):
        scratch = torch.empty(512 << 20, dtype=torch.uint8, device="cuda") if flush else None
        e = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(reps)]
        for i in range(reps):
            if flush:
                scratch.fill_(i & 0xFF)
            layer = i % 2 if alternate else 0
            write(layer)
            e[i][0].record(stream)
            decode(layer)
            e[i][1].record(stream)
        torch.cuda.synchronize()
        ms = np.array([a.elapsed_time(b) for a, b in e])
        return {"median_ms": round(float(np.median(ms)), 5),
                "p10_ms": round(float(np.percentile(ms, 10)), 5),
                "p90_ms": round(float(np.percentile(ms, 90)), 5),
                "median_GBps": round(unique_bytes / (float(np.median(ms)) * 1e-3) / 1e9, 2)}

    latency = {"two_layers": distribution(False, args.steps, True),
               "one_layer": distribution(False, args.steps, False),
               "one_layer_flushed_512MiB": distribution(True, args.steps, False)}

    swap = swap_leg(sp, kc, vc, tables, args.swap) if args.swap > 0 else None
    copy = copy_leg(sp, kc, vc, tables, args.copy_blocks) if args.copy_blocks > 0 else None

    cpu = None
    if not args.no_cpu_baseline:
        # the output the oracle checks: one more decode of layer 0 (whose K/V it reads)
        write(0)
        decode(0)
        torch.cuda.synchronize()
        gpu_out = (outm if path == "multi" else out).double().cpu().numpy()
        qsrc = qm if path == "multi" else q
        cpu = cpu_baseline(sp, qsrc, kc, vc, tables, ctx, k_scale, v_scale, args.cpu_seconds,
                           gpu_out, T if path == "multi" else 0)

    block_bytes = workloads.kv_bytes(sp, -(-ctx // B) * B)  # whole blocks of every context
    shared = unique_bytes != kv_bytes
    line = {
        "metric": "paged decode attention: achieved KV HBM GB/s (% of peak) + decode tokens/s",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": sp.kv_dtype,
        "data": "synthetic",
        "pct_of_hbm_peak": round(100.0 * value / HBM_PEAK_GBS, 2),
        "value_bytes": ("logical: every sequence's own context, shared prompt blocks counted "
                        "once per sequence that reads them (above the HBM peak is possible; "
                        "roofline.achieved uses the bytes the call must read)" if shared else
                        "algorithmic: sum over sequences of n * num_kv_heads * head_dim * 2 * "
                        "bytes per element, K and V read once"),
        "decode_tokens_per_s": round(S * T / (ms_per_step * 1e-3), 1),
        "config": {
            "workload": sp.name, "num_seqs": S, "num_heads": Hq, "num_kv_heads": Hkv,
            "head_dim": D, "block_size": B, "context_lens": f"U[{sp.ctx_lo},{sp.ctx_hi}]"
            + (f"+{sp.prompt_len}" if sp.prompt_len else ""), "num_blocks": sp.num_blocks,
            "q_dtype": sp.q_dtype, "kv_dtype": sp.kv_dtype,
            "partition_size": used_P if not cascade_plan and not flat_min else None,
            "num_partitions": nparts if not cascade_plan and not flat_min else None,
            "kv_bytes_per_step": kv_bytes,
            "unique_kv_bytes_per_step": unique_bytes, "seed": seed,
            "decode_flags": flags, "decode_path": path,
            "step": ("fused: pa_decode_append stores the new tokens and decodes in one call"
                     if fused else "pa_write_kv, then the decode"),
            "block_granular_kv_bytes_per_step": block_bytes,
        } | ({"query_len": T} if path == "multi" else {})
          | ({"cascade_plan": cascade_plan} if cascade_plan else {})
          | ({"flat_split": flat_split} if flat_split else {}),
        "roofline": {
            "bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic(sp.name, path),
            "kernel": kernels,
            "mean_launch_ms": round(dec_ms_mean, 5),
            "median_launch_ms": round(float(np.median(dec_ms)), 5),
        },
        "decode_latency": latency,
        "cpu_baseline": cpu,
    }
    if shared:
        line["value_unique_GBps"] = round(unique_bytes / (ms_per_step * 1e-3) / 1e9, 2)
        line["pct_of_hbm_peak_unique"] = round(100.0 * line["value_unique_GBps"] / HBM_PEAK_GBS, 2)
    if sp.name == "opt13b_layer":
        # the 40 layers of OPT-13B, attention only: one token per sequence through all of them
        line["opt13b_40_layer_tokens_per_s"] = round(S * T / (40 * ms_per_step * 1e-3), 1)
    if swap is not None:
        line["swap"] = swap
    if copy is not None:
        line["copy_blocks"] = copy
    print(json.dumps(line), flush=True)


def copy_leg(sp, kc, vc, tables, n):
    """Batched copy-on-write: one pa_copy_blocks launch duplicating n distinct blocks of the
    batch into n free blocks (K and V), timed with HIP events; GB/s = bytes read + written
    over the launch time."""
    import torch

    import paged_kv_cache_89_amd as pa

    used = np.unique(tables[tables >= 0])
    free = np.setdiff1d(np.arange(sp.num_blocks), used)
    n = int(min(n, used.size, free.size))
    rng = np.random.default_rng(7)
    pairs = np.stack([rng.choice(used, n, replace=False), rng.choice(free, n, replace=False)],
                     1).astype(np.int32)
    pd = torch.from_numpy(pairs).cuda()
    stream = torch.cuda.current_stream()
    pa.copy_blocks(kc, vc, pd, stream=stream)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    a.record(stream)
    for _ in range(reps):
        pa.copy_blocks(kc, vc, pd, stream=stream)
    b.record(stream)
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    moved = 2 * 2 * n * kc[0].numel() * kc.element_size()   # K and V, read + write
    return {"pairs": n, "bytes_read_and_written": moved, "ms": round(ms, 4),
            "GBps": round(moved / (ms * 1e-3) / 1e9, 2)}


def swap_leg(sp, kc, vc, tables, nseq):
    """Preemption by swapping: the distinct blocks of the first nseq sequences (K and V)
    moved device -> pinned host and back with pa_swap_blocks (one launch each way, reading
    or writing host memory directly over the host link), beside torch's DMA copy of the
    same number of contiguous bytes each way.  GB/s = moved bytes / mean time."""
    import torch

    import paged_kv_cache_89_amd as pa

    rows = tables[:nseq]
    ids = np.unique(rows[rows >= 0]).astype(np.int32)
    n = int(ids.size)
    hk = torch.empty((n,) + tuple(kc.shape[1:]), dtype=kc.dtype, pin_memory=True)
    hv = torch.empty_like(hk, pin_memory=True)
    out_pairs = torch.from_numpy(np.stack([ids, np.arange(n, dtype=np.int32)], 1)).cuda()
    in_pairs = torch.from_numpy(np.stack([np.arange(n, dtype=np.int32), ids], 1)).cuda()
    nbytes = 2 * n * hk[0].numel() * hk.element_size()
    dk = torch.empty(hk.shape, dtype=kc.dtype, device="cuda")
    dv = torch.empty_like(dk)
    hk2, hv2 = torch.empty_like(hk, pin_memory=True), torch.empty_like(hv, pin_memory=True)
    stream = torch.cuda.current_stream()

    def timed(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    t_out = timed(lambda: pa.swap_blocks(kc, vc, hk, hv, out_pairs, stream=stream))
    t_in = timed(lambda: pa.swap_blocks(hk, hv, kc, vc, in_pairs, stream=stream))
    t_dma_out = timed(lambda: (hk2.copy_(dk, non_blocking=True), hv2.copy_(dv, non_blocking=True)))
    t_dma_in = timed(lambda: (dk.copy_(hk2, non_blocking=True), dv.copy_(hv2, non_blocking=True)))

    def gbs(ms):
        return round(nbytes / (ms * 1e-3) / 1e9, 2)

    return {"sequences": nseq, "blocks": n, "bytes_each_way": nbytes,
            "out_GBps": gbs(t_out), "in_GBps": gbs(t_in),
            "dma_out_GBps": gbs(t_dma_out), "dma_in_GBps": gbs(t_dma_in),
            "out_ms": round(t_out, 4), "in_ms": round(t_in, 4)}


def host_cpus():
    """(CPUs this process may run on, CPUs the host reports)."""
    try:
        mine = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        mine = os.cpu_count() or 1
    return mine, os.cpu_count() or mine


def cpu_baseline(sp, q, kc, vc, tables, ctx, k_scale, v_scale, target_s, gpu_out, query_len):
    """The oracle (plain fp64 C++, unmodified) on the host cores, over a bounded sample of
    sequences (all heads of the first few) scaled to the same GB/s metric: wall time, median
    of 3 runs, with one thread per CPU this process may use (at most 16, a GPU machine's share)
    and with one thread.  The sample's oracle output also checks the GPU output of the same
    rows (parity at the benchmark's own launch configuration)."""
    import torch

    import oracle
    import workloads

    dt = {"f16": oracle.F16, "bf16": oracle.BF16, "e4m3": oracle.E4M3}
    mine, host = host_cpus()
    threads = max(1, min(mine, 16))

    def sample(nseq):
        rows = tables[:nseq]
        used = np.unique(rows[rows >= 0])
        remap = np.full(sp.num_blocks, -1, np.int32)
        remap[used] = np.arange(used.size, dtype=np.int32)
        t = np.where(rows >= 0, remap[np.maximum(rows, 0)], -1).astype(np.int32)
        idx = torch.from_numpy(used.astype(np.int64)).cuda()

        def bits(x):
            x = x.index_select(0, idx).cpu().contiguous()
            return x.numpy() if x.dtype == torch.uint8 else x.view(torch.int16).numpy().view(np.uint16)

        qb = q[:nseq].cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
        return qb, bits(kc), bits(vc), t, ctx[:nseq].copy()

    def once(inputs, nthreads):
        qb, kb, vb, t, c = inputs
        t0 = time.perf_counter()
        if query_len:
            ref = oracle.decode_multi(qb, dt[sp.q_dtype], kb, vb, dt[sp.kv_dtype], t, c,
                                      sp.num_kv_heads, sp.block_size, sp.scale, k_scale,
                                      v_scale, threads=nthreads)
        else:
            ref = oracle.decode(qb, dt[sp.q_dtype], kb, vb, dt[sp.kv_dtype], t, c,
                                sp.num_kv_heads, sp.block_size, sp.scale, k_scale, v_scale,
                                threads=nthreads)
        return time.perf_counter() - t0, ref

    def median3(inputs, nthreads):
        runs = [once(inputs, nthreads) for _ in range(3)]
        return float(np.median([r[0] for r in runs])), runs[0][1]

    probe, _ = once(sample(1), threads)
    nseq = int(max(1, min(sp.num_seqs, target_s / 3 / max(probe, 1e-3))))
    inputs = sample(nseq)
    secs, ref = median3(inputs, threads)
    # the GPU metric's bytes: each sequence's K/V once per pass (all its query tokens)
    nbytes = workloads.kv_bytes(sp, inputs[4])
    # one thread, on a sample of about a second of work per run
    n1 = int(max(1, min(nseq, 1.0 / max(probe * threads, 1e-3))))
    inputs1 = inputs if n1 == nseq else sample(n1)
    secs1, _ = median3(inputs1, 1)
    nbytes1 = workloads.kv_bytes(sp, inputs1[4])
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), "")
    except OSError:
        pass
    # parity of the GPU rows the sample covers (fp64 oracle, unrounded)
    got = gpu_out[:nseq]
    err = np.abs(got - ref)
    rn = np.abs(ref).max(axis=-1)
    row_rel = np.where(rn > 0, err.max(axis=-1) / np.where(rn > 0, rn, 1), err.max(axis=-1))
    atol = 2e-2 if sp.kv_dtype == "e4m3" else 2e-3
    return {"value": round(nbytes / secs / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle", "seconds_median_of_3": round(secs, 3),
            "single_thread_value": round(nbytes1 / secs1 / 1e9, 4),
            "single_thread_seconds_median_of_3": round(secs1, 3),
            "host_cpus": host, "cpus_available": mine, "cpu": model,
            "sample": f"{nseq} of {sp.num_seqs} sequences, all {sp.num_heads} heads"
                      + (f", {query_len} query tokens each" if query_len else "")
                      + f" ({nbytes} KV bytes per pass), fp64 C++ oracle with "
                      f"{threads} threads, median of 3 runs; single thread: {n1} sequences",
            "parity": {"rows": int(got.shape[0] * int(np.prod(got.shape[1:-1]))),
                       "max_abs_err": float(err.max()), "max_row_rel_err": float(row_rel.max()),
                       "bar_abs": atol, "bar_row_rel": None if sp.kv_dtype == "e4m3" else 1e-2}}


if __name__ == "__main__":
    main()
