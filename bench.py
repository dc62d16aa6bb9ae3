#!/usr/bin/env python3
"""Decode-step benchmark of the paged KV-cache library on one MI355X.

A step is one decode step of the whole model: for every layer, the cache-append
scatter of the step's new token (paged_kv_append), decode attention
(paged_attention_decode), and the log-sum-exp merge (paged_attention_reduce) when
the workload runs split-context partitions.  The default workload is the
Llama-2-7B attention shape: 128 sequences with lognormal lengths (P90 287),
32 layers, 32 heads, head_dim 128, block_size 32, fp16.

Inputs are seeded synthetic data already resident in HBM when timing starts.  To
keep the last-level cache (256 MB) from serving repeated reads, the step cycles
through R distinct per-layer pools with distinct data (8 for the default workload,
about 2.9 GB of K/V touched per cycle); the block tables are shared by all layers.

Prints ONE JSON line.  `value` is decode tokens/s over the whole step (sequences /
step time); the line also carries the algorithmic HBM rate of the step, the
roofline of the dominant kernel (decode attention) timed per launch with HIP
events, and the fp64 CPU oracle timed on a bounded sample on the host cores.

`--op append_tokens` and `--op copy_blocks` instead time the block-level writers
on the same workload shapes (the prefill scatter of every layer, and a
copy-on-write fork of every sequence in every layer) and print one line each,
with GB/s as the value; `--op slotted` times decode over a radix-tree batch
addressed by slotted (block, offset, length) segments.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("decode attention tokens/s and achieved HBM GB/s (% of MI355X peak), 1 GPU")
HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, vendor figure


def algorithmic_bytes(cfg, lengths, tables_entries, shared_tokens=0):
    """Bytes one layer of the step must move at minimum, split per kernel.
    shared_tokens: attended positions that are re-reads of a prefix another
    sequence of the batch already reads (its K/V rows count once)."""
    e = cfg.elem_bytes
    S, Hq, Hkv, D = cfg.num_seqs, cfg.num_q_heads, cfg.num_kv_heads, cfg.head_dim
    kv = (int(np.sum(lengths)) - shared_tokens) * 2 * Hkv * D * e   # K and V rows
    qo = 2 * S * Hq * D * e                             # q read + output write
    meta = 4 * int(tables_entries) + 4 * S              # table entries + lengths
    append = 2 * S * 2 * Hkv * D * e                    # new K/V rows read + written
    decode = kv + qo + meta
    return {"decode": decode, "append": append + 4 * S + 4 * S, "layer": decode + append}


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="c3", help="workload key (c1a c1b c2 c3 c4 c5)")
    ap.add_argument("--op", default="step",
                    choices=["step", "append_tokens", "copy_blocks", "slotted"],
                    help="step: the decode step (default, the headline line); append_tokens: "
                         "the prefill scatter of the workload's histories into every layer; "
                         "copy_blocks: copy-on-write copies of the workload's forks; slotted: "
                         "decode of a radix-tree batch addressed by slotted segments")
    ap.add_argument("--partition-size", type=int, default=None,
                    help="override the workload's split-context partition size (0 = single pass)")
    ap.add_argument("--distinct", type=int, default=None, help="override distinct layer pools")
    ap.add_argument("--separate", action="store_true",
                    help="run the append and the decode as two launches per layer "
                         "(paged_kv_append + paged_attention_decode) instead of the fused "
                         "paged_attention_append_decode")
    ap.add_argument("--no-merge", action="store_true",
                    help="for a split workload, run the split decode and the standalone merge "
                         "(paged_attention_reduce) as two launches per layer instead of "
                         "paged_attention_split_decode, which merges in the same launch")
    ap.add_argument("--order", default="long", choices=["long", "natural"],
                    help="dispatch order of the single-pass decode: long (the default) puts "
                         "the sequences longer than twice the batch mean first and the shortest "
                         "last, computed on the host from the batch's lengths "
                         "(paged_attention_decode_ordered); natural keeps the batch order")
    ap.add_argument("--no-prefix", action="store_true",
                    help="for a shared-prefix workload, run the plain fused decode instead of "
                         "paged_attention_prefix_decode")
    ap.add_argument("--prefix-partition", type=int, default=None,
                    help="prefix partition of paged_attention_prefix_decode (0 = one)")
    ap.add_argument("--graph", action="store_true",
                    help="capture one whole step (every layer's launches) in a HIP graph and "
                         "time graph replays instead of eager launches")
    ap.add_argument("--slotted-batch", default="auto", choices=["auto", "radix", "tables"],
                    help="--op slotted: the radix-tree batch (radix; the default for the "
                         "shared-prefix workload) or the workload's block tables written as "
                         "segments (tables; the default otherwise, in split mode when the "
                         "workload's partition size is set)")
    ap.add_argument("--slotted-append", default="on", choices=["on", "off"],
                    help="--op slotted, single pass: each launch also appends the step's new "
                         "K/V rows to every sequence's last position (the default), or decode "
                         "only")
    ap.add_argument("--slotted-order", default="tree", choices=["tree", "drawn"],
                    help="--op slotted, radix batch: sequences in tree order (sorted by their "
                         "node paths, so that a tile's consecutive sequences share nodes), or "
                         "in the order the workload draws them")
    ap.add_argument("--slotted-kernel", default="auto", choices=["auto", "tiles", "per_sequence"],
                    help="--op slotted, single pass: the library's choice, or force the tiled "
                         "or the per-sequence kernel (PKV_SLOTTED_TILES)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="approximate CPU time budget of the oracle samples of the --op lines "
                         "(the step's baseline runs exactly one whole step)")
    ap.add_argument("--copy-reference", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy (reference for HBM "
                         "counter scaling and copy bandwidth) and print its rate")
    ap.add_argument("--read-reference", action="store_true",
                    help="only run the read-only HBM reference (a torch sum over 2 GiB) and "
                         "print its rate")
    return ap.parse_args()


# Source files whose contents determine each kernel's memory traffic.
TRAFFIC_SOURCES = {
    "decode_g1": ["paged_kv_cache_09_amd/csrc/decode_g1.hip",
                  "paged_kv_cache_09_amd/csrc/pkv_device.h"],
    "decode_mfma": ["paged_kv_cache_09_amd/csrc/decode_mfma.hip",
                    "paged_kv_cache_09_amd/csrc/pkv_device.h"],
    "prefix": ["paged_kv_cache_09_amd/csrc/decode_mfma.hip",
               "paged_kv_cache_09_amd/csrc/pkv_device.h"],
    "slotted": ["paged_kv_cache_09_amd/csrc/decode_mfma.hip",
                "paged_kv_cache_09_amd/csrc/pkv_device.h"],
    "append_tokens": ["paged_kv_cache_09_amd/csrc/append.hip"],
    "copy_blocks": ["paged_kv_cache_09_amd/csrc/copy.hip",
                    "paged_kv_cache_09_amd/csrc/pkv_device.h"],
}


def kernel_source_hash(kind: str) -> str:
    import hashlib
    h = hashlib.sha256()
    for f in TRAFFIC_SOURCES[kind]:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(stem: str, kind: str):
    """HBM bytes per launch from the committed counter record
    profiles/<stem>_traffic.json, or None when there is none or the sources of
    that kernel (kind) changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{stem}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != kernel_source_hash(kind):
        return None
    return rec.get("hbm_bytes_per_launch")


def time_launches(fn, reps: int, warm: int = 2) -> float:
    """Average duration in ms of fn()'s launches, queued back to back between two
    events on torch's current stream (the stream the binding launches on)."""
    import torch
    for _ in range(warm):
        fn()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        fn()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def time_launches_graph(fn, reps: int) -> tuple:
    """Average duration in ms of fn()'s launches with no host time between them:
    `reps` calls are captured in one HIP graph and a replay of it is timed between
    two events on the stream it runs on.  Eager launches of short kernels leave the
    GPU idle while Python marshals the next call, which would count as kernel time.
    Falls back to eager back-to-back launches if capture fails.  Returns (ms, how)."""
    import torch
    try:
        fn()
        torch.cuda.synchronize()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            fn()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(reps):
                fn()
        graph.replay()
        torch.cuda.synchronize()
    except RuntimeError:
        return time_launches(fn, reps), "eager back-to-back launches"
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    graph.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps, "hip graph replay of back-to-back launches"


def roofline(kernel: str, nbytes: int, ms: float, traffic):
    gbps = nbytes / (ms * 1e-3) / 1e9
    return {"kernel": kernel, "bound": "hbm", "achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS,
            "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4), "traffic": traffic,
            "bytes_per_launch": int(nbytes), "avg_launch_ms": round(ms, 5)}


def copy_rate(reps: int = 10) -> dict:
    """Plain device-to-device copy of 1 GiB (read 1 GiB + write 1 GiB), timed."""
    import torch
    n = 1 << 30
    a = torch.ones(n // 2, dtype=torch.float16, device="cuda:0")
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del a, b
    torch.cuda.empty_cache()
    return {"bytes_read": n, "bytes_written": n, "ms": round(ms, 4),
            "gbps_read_plus_write": round(2 * n / ms / 1e6, 1)}


def read_rate(reps: int = 10) -> dict:
    """Read-only HBM reference: torch's row sums of a [131072, 4096] fp32 tensor
    (2 GiB, 8x the MALL; the 512 KiB of sums written are negligible), timed with
    HIP events over back-to-back reductions.  A plain library reduction, not a
    tuned probe: the fastest of the plain torch reads tried on MI355X (a flat
    sum, amax or matrix-vector product over the same bytes read at 3.5-4.0 TB/s)."""
    import torch
    n = 2 << 30
    x = torch.ones((n // 4 // 4096, 4096), dtype=torch.float32, device="cuda:0")
    for _ in range(3):
        x.sum(dim=1)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        x.sum(dim=1)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / reps
    del x
    torch.cuda.empty_cache()
    return {"bytes_read": n, "ms": round(ms, 4), "gbps_read": round(n / ms / 1e6, 1),
            "method": "torch row sums of a [131072, 4096] fp32 tensor (2 GiB read), mean of "
                      "%d back-to-back calls" % reps}


def copy_reference():
    print(json.dumps({"copy_reference": True, **copy_rate()}))


def read_reference():
    print(json.dumps({"read_reference": True, **read_rate()}))


def main():
    args = parse()
    if args.copy_reference:
        copy_reference()
        return
    if args.read_reference:
        read_reference()
        return
    if args.gpus != 1:
        print(json.dumps({"error": "bench.py drives one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    if args.op == "append_tokens":
        bench_append_tokens(args)
    elif args.op == "copy_blocks":
        bench_copy_blocks(args)
    elif args.op == "slotted":
        bench_slotted(args)
    else:
        bench_step(args)


def bench_step(args):
    import torch
    import paged_kv_cache_09_amd as pkv
    from workloads import get_config, make_workload

    cfg = get_config(args.config)
    P = cfg.bench_partition_size if args.partition_size is None else args.partition_size
    # R distinct sets of pools (and q, new rows), cycled over the layers of a step
    # and over consecutive steps, so that the K/V a launch reads is not still in the
    # 256 MB MALL from an earlier launch
    R = args.distinct or cfg.bench_distinct_layers
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    tdt = {"fp16": torch.float16, "bf16": torch.bfloat16}[cfg.dtype]
    scale = float(np.float32(1.0 / math.sqrt(cfg.head_dim)))

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(tdt)

    # ---- set-up: R distinct layers of pools, q, new rows (not timed) --------------
    t_setup = time.time()
    layers = []
    hosts = []  # the R pool sets' host inputs (the CPU baseline runs the same step)
    w0 = None
    for d in range(R):
        w = make_workload(cfg, layer=d)
        hosts.append(w)
        if w0 is None:
            w0 = w
        shape = w.pool_shape()
        kp = torch.empty(shape, dtype=tdt, device=dev)
        vp = torch.empty(shape, dtype=tdt, device=dev)
        sentinel = int(np.array([w.nan_bits], np.uint16).view(np.int16)[0])
        kp.view(torch.int16).fill_(sentinel)
        vp.view(torch.int16).fill_(sentinel)
        tabs = torch.from_numpy(w.tables).to(dev)
        if w.total_history_tokens():
            pkv.paged_kv_append_tokens(kp, vp, up(w.k_src), up(w.v_src),
                                       torch.from_numpy(w.seg_cu).to(dev),
                                       torch.from_numpy(w.seg_start).to(dev),
                                       torch.from_numpy(w.seg_tables).to(dev))
        layers.append(dict(k=kp, v=vp, q=up(w.q), kn=up(w.k_new), vn=up(w.v_new)))
        torch.cuda.synchronize()
        del tabs
    tables = torch.from_numpy(w0.tables).to(dev)
    lens = torch.from_numpy(w0.lengths).to(dev)
    S, Hq, D = cfg.num_seqs, cfg.num_q_heads, cfg.head_dim
    out = torch.empty((cfg.num_layers, S, Hq, D), dtype=tdt, device=dev)
    mp = pkv.max_partitions(cfg.max_blocks_per_seq, cfg.block_size, P) if P else 0
    part_o = torch.empty((S, Hq, mp, D), dtype=torch.float32, device=dev) if P else None
    part_lse = torch.empty((S, Hq, mp), dtype=torch.float32, device=dev) if P else None
    torch.cuda.synchronize()
    setup_s = time.time() - t_setup

    fused = not args.separate
    prefix = cfg.prefix_tokens > 0 and not args.no_prefix
    # Single-pass decode: dispatch the long sequences first (a host-side plan from
    # the lengths the caller already has; the results do not depend on the order).
    order_dev = None
    order_rule = "natural (batch order)"
    if not P and not prefix and args.order == "long":
        # The sequences above twice the batch mean go first, so that they do not
        # finish last; the shortest go last, as many as give one work-group per
        # compute unit (at most an eighth of the batch), so that the launch's last
        # partial wave of work-groups is its shortest; the rest keep batch order.
        n_host = np.asarray(w0.lengths, np.int64)
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        order = pkv.long_first_order(n_host, cfg.num_kv_heads, cus)
        n_long = int((n_host > 2 * n_host.mean()).sum())
        n_short = min(-(-cus // cfg.num_kv_heads), S // 8, S - n_long)
        order_dev = torch.from_numpy(order).to(dev)
        order_rule = ("sequences longer than twice the batch mean first (%d of %d), the %d "
                      "shortest last (longest of them first), the rest in batch order"
                      % (n_long, S, n_short))
    # split workloads merge their partitions in the decode launch itself, with one
    # zeroed arrival counter per (sequence, KV head) that every launch leaves zero
    merged = bool(P) and not args.no_merge and not prefix
    counters = torch.zeros((S, cfg.num_kv_heads), dtype=torch.int32, device=dev)
    if prefix:
        # one group: every sequence shares the workload's prefix blocks
        PP = cfg.bench_prefix_partition if args.prefix_partition is None else args.prefix_partition
        ctx = cfg.max_blocks_per_seq * cfg.block_size
        mpp = 1 if PP == 0 else -(-ctx // PP)
        pre_o = torch.empty((S, Hq, mpp, D), dtype=torch.float32, device=dev)
        pre_lse = torch.empty((S, Hq, mpp), dtype=torch.float32, device=dev)
        group_cu = torch.tensor([0, S], dtype=torch.int32, device=dev)
        prefix_lens = torch.tensor([cfg.prefix_tokens], dtype=torch.int32, device=dev)
        P = 0

    def pool(si, li):
        """The pool set of layer li in step si."""
        return layers[(si * cfg.num_layers + li) % R]

    def attend(si, li):
        """Decode of layer li in step si; in fused mode it also appends the layer's
        new rows."""
        L = pool(si, li)
        o = None if P else out[li]
        if prefix:
            pkv.paged_attention_prefix_decode(o, L["q"], L["k"], L["v"], tables, lens, group_cu,
                                              prefix_lens, pre_o, pre_lse,
                                              k_new=L["kn"] if fused else None,
                                              v_new=L["vn"] if fused else None, scale=scale,
                                              prefix_partition=PP)
        elif merged:
            pkv.paged_attention_split_decode(out[li], L["q"], L["k"], L["v"], tables, lens, P,
                                             part_o, part_lse, counters,
                                             k_new=L["kn"] if fused else None,
                                             v_new=L["vn"] if fused else None, scale=scale)
        elif order_dev is not None:
            pkv.paged_attention_decode_ordered(o, L["q"], L["k"], L["v"], tables, lens, order_dev,
                                               k_new=L["kn"] if fused else None,
                                               v_new=L["vn"] if fused else None, scale=scale)
        elif fused:
            pkv.paged_attention_append_decode(o, L["q"], L["k"], L["v"], L["kn"], L["vn"],
                                              tables, lens, scale=scale, partition_size=P,
                                              part_o=part_o, part_lse=part_lse)
        else:
            pkv.paged_attention_decode(o, L["q"], L["k"], L["v"], tables, lens, scale=scale,
                                       partition_size=P, part_o=part_o, part_lse=part_lse)

    def step(si):
        for li in range(cfg.num_layers):
            L = pool(si, li)
            if not fused:
                pkv.paged_kv_append(L["k"], L["v"], L["kn"], L["vn"], tables, lens)
            attend(si, li)
            if P and not merged:
                pkv.paged_attention_reduce(out[li], part_o, part_lse, lens, P)

    # ---- timed region ------------------------------------------------------------
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    run = lambda i: step(args.warmup + i)
    if args.graph:
        # a graph replays the launches it captured: one step, with the pools of
        # step 0 (no cycling across steps)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step(0)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step(0)
        graph.replay()
        torch.cuda.synchronize()
        run = lambda i: graph.replay()
    # one event between consecutive steps: the first and last bracket the K steps
    # (ms_per_step), the ones between give each step's own time (percentiles)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    ev[0].record()
    for i in range(args.steps):
        run(i)
        ev[i + 1].record()
    torch.cuda.synchronize()
    ms_per_step = ev[0].elapsed_time(ev[-1]) / args.steps
    step_ms = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(args.steps)])

    # ---- average duration of the dominant kernel -----------------------------------
    # The decode launches of the step (same arguments, same layer pools) run back
    # to back from a HIP graph, timed by two events on the stream they run on; the
    # elapsed time over the launch count is the kernel's average duration.  At least
    # 64 launches are captured, so that the replay's own start-up latency (a few
    # microseconds) is spread thin over short one-layer launches.
    reps = max(R, min(args.steps, 10), -(-64 // cfg.num_layers))
    rep_ctr = [0]

    def attend_all():
        # each call is one more step's launches, so a capture of `reps` calls
        # cycles through the pool sets as the timed steps do
        si = rep_ctr[0]
        rep_ctr[0] += 1
        for li in range(cfg.num_layers):
            attend(si, li)
    decode_ms, kernel_timing = time_launches_graph(attend_all, reps)
    decode_ms /= cfg.num_layers
    # leave `out` holding step 0's result: layer 0 from the first pool set, whose
    # inputs the oracle baseline uses
    step(0)
    torch.cuda.synchronize()

    assert bool(torch.isfinite(out.float()).all()), "non-finite attention output"

    # ---- accounting -------------------------------------------------------------------
    nblk = int(np.sum(-(-w0.lengths.astype(np.int64) // cfg.block_size)))
    # a shared prefix is one set of K/V rows however many sequences attend to it
    shared = (S - 1) * cfg.prefix_tokens if cfg.prefix_tokens > 0 else 0
    ab = algorithmic_bytes(cfg, w0.lengths, nblk, shared)
    logical = algorithmic_bytes(cfg, w0.lengths, nblk)
    step_bytes = ab["layer"] * cfg.num_layers
    gbps = step_bytes / (ms_per_step * 1e-3) / 1e9
    tokens_per_s = S / (ms_per_step * 1e-3)
    kernel_bytes = ab["decode"] + (ab["append"] if fused else 0)
    dec_gbps = kernel_bytes / (decode_ms * 1e-3) / 1e9

    result = {
        "metric": METRIC,
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "step_ms_p10_p50_p90": [round(float(x), 4) for x in np.percentile(step_ms, [10, 50, 90])],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded; N(0,1) x %g values, %s lengths)" % (cfg.value_scale,
                                                                      cfg.length_kind),
        "config": {
            "workload": f"{cfg.key}: {cfg.title}",
            "num_seqs": S, "layers": cfg.num_layers, "q_heads": Hq,
            "kv_heads": cfg.num_kv_heads, "head_dim": D, "block_size": cfg.block_size,
            "mean_context": round(float(np.mean(w0.lengths)), 2),
            "max_context": int(np.max(w0.lengths)),
            "pool_blocks_per_layer": int(w0.num_blocks),
            "distinct_layer_pools": R,
            "partition_size": P,
            "launches_per_layer": ((1 if fused else 2) +
                                   (1 if (P and not merged) or (prefix and PP) else 0)),
            "launch": "hip graph replay" if args.graph else "eager",
            "shared_prefix": cfg.prefix_tokens,
            "path": ("paged_attention_prefix_decode (prefix partition %d)" % PP if prefix
                     else ("paged_attention_split_decode (merged in launch)" +
                           (" with the fused append" if fused else " after paged_kv_append"))
                     if merged
                     else ("paged_attention_decode_ordered (fused append)" if fused and order_dev
                           is not None else "paged_attention_append_decode" if fused else
                           "paged_kv_append + paged_attention_decode_ordered" if order_dev
                           is not None else "paged_kv_append + paged_attention_decode") +
                     (" + paged_attention_reduce" if P else "")),
            "dispatch_order": order_rule,
            "accumulate": "fp32",
        },
        "hbm_gbps": round(gbps, 1),
        "hbm_frac_of_peak": round(gbps / HBM_PEAK_GBPS, 4),
        "step_algorithmic_bytes": step_bytes,
        "roofline": {
            "kernel": (("paged_attention_prefix_decode (prefix + suffix pass)" if PP else
                        "paged_attention_prefix_decode (one pass)") if prefix
                       else "paged_attention_split_decode (partitions merged in launch)"
                       if merged
                       else "paged_attention_decode_ordered (fused append)" if fused and
                       order_dev is not None
                       else "paged_attention_append_decode" if fused
                       else "paged_attention_decode_ordered" if order_dev is not None
                       else "paged_attention_decode"),
            "bound": "hbm",
            "achieved": round(dec_gbps, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(dec_gbps / HBM_PEAK_GBPS, 4),
            "traffic": (measured_traffic(f"prefix_{cfg.key}", "prefix") if prefix else
                        measured_traffic(f"decode_{cfg.key}",
                                         "decode_g1" if Hq == cfg.num_kv_heads else "decode_mfma")),
            "bytes_per_launch": kernel_bytes,
            "avg_launch_ms": round(decode_ms, 5),
            "timing": kernel_timing,
        },
        "logical_bytes_per_layer": logical["layer"],
        "setup_s": round(setup_s, 1),
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"], ref = cpu_baseline(hosts, cfg, scale)
        # the oracle's layer-0 output (computed by that baseline run) against the
        # GPU's layer-0 output of the last timed step
        got = out[0].float().cpu().numpy().astype(np.float64)
        err = np.abs(got - ref)
        result["parity_vs_oracle"] = {
            "layer": 0,
            "max_abs_err": float(err.max()),
            "within_tolerance": bool(np.all(err <= 1e-2 + 1e-2 * np.abs(ref))),
            "tolerance": "|gpu - oracle| <= 1e-2 + 1e-2 |oracle|, elementwise",
        }
    result["rocm"] = torch.version.hip
    # context for the roofline: what a plain 1 GiB device copy moves on this GPU, and
    # what a plain library reduction reads (both far below the 8 TB/s vendor peak)
    result["copy_1gib_gbps_read_plus_write"] = copy_rate(5)["gbps_read_plus_write"]
    rr = read_rate(5)
    result["hbm_read_reference"] = {"gbps": rr["gbps_read"], "method": rr["method"]}

    print(json.dumps(result), flush=True)


def _side_line(metric, value, unit, args, cfg, dtype, config, roof, extra=None):
    line = {"metric": metric, "value": round(value, 1), "unit": unit, "n_gpus": 1,
            "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(roof["avg_launch_ms"] *
                                                                              config["launches"], 4),
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": dtype,
            "data": "synthetic (seeded)", "config": config, "roofline": roof}
    line.update(extra or {})
    return line


def bench_append_tokens(args):
    """Prefill scatter: every layer's K/V of the workload's histories (one run per
    sequence, positions 0..n-2) written into that layer's pools, one
    paged_kv_append_tokens launch per layer.  value = algorithmic GB/s."""
    import torch
    import paged_kv_cache_09_amd as pkv
    from workloads import get_config, make_workload

    cfg = get_config(args.config)
    R = args.distinct or cfg.bench_distinct_layers
    dev = torch.device("cuda:0")
    tdt = {"fp16": torch.float16, "bf16": torch.bfloat16}[cfg.dtype]

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(tdt)

    w = make_workload(cfg, layer=0)
    T = int(w.total_history_tokens())
    layers = []
    for d in range(R):
        wd = w if d == 0 else make_workload(cfg, layer=d)
        kp = torch.zeros(wd.pool_shape(), dtype=tdt, device=dev)
        layers.append(dict(k=kp, v=torch.zeros_like(kp), ks=up(wd.k_src), vs=up(wd.v_src)))
    cu = torch.from_numpy(w.seg_cu).to(dev)
    st = torch.from_numpy(w.seg_start).to(dev)
    tb = torch.from_numpy(w.seg_tables).to(dev)
    torch.cuda.synchronize()

    def one(li):
        L = layers[li % R]
        pkv.paged_kv_append_tokens(L["k"], L["v"], L["ks"], L["vs"], cu, st, tb)

    it = iter(range(1 << 30))
    ms = time_launches(lambda: one(next(it)), args.steps * cfg.num_layers,
                       warm=args.warmup * cfg.num_layers)
    e = cfg.elem_bytes
    rows = 2 * T * cfg.num_kv_heads * cfg.head_dim * e           # K and V rows
    nblk = int(sum(-(-(int(s) + int(n)) // cfg.block_size) - int(s) // cfg.block_size
                   for s, n in zip(w.seg_start, np.diff(w.seg_cu))))
    meta = 8 * (len(w.seg_cu)) + 4 * len(w.seg_start) + 4 * nblk
    nbytes = 2 * rows + meta                                      # read + write
    roof = roofline("paged_kv_append_tokens", nbytes, ms,
                    measured_traffic(f"append_tokens_{cfg.key}", "append_tokens"))
    config = {"workload": f"{cfg.key} prefill scatter: {cfg.title}", "runs": int(len(w.seg_start)),
              "tokens_per_layer": T, "layers": cfg.num_layers, "kv_heads": cfg.num_kv_heads,
              "head_dim": cfg.head_dim, "block_size": cfg.block_size, "distinct_layer_pools": R,
              "launches": cfg.num_layers}
    line = _side_line("prefill KV scatter (paged_kv_append_tokens) GB/s, 1 GPU", roof["achieved"],
                      "GB/s", args, cfg, cfg.dtype, config, roof,
                      {"tokens_per_s": round(T / (ms * 1e-3) / cfg.num_layers, 1)})
    if not args.no_cpu_baseline:
        from oracle import oracle as O
        kp, vp = O.new_pools(w.num_blocks, cfg.num_kv_heads, cfg.block_size, cfg.head_dim, 0)
        reps, spent = 0, 0.0
        while reps == 0 or (spent < args.cpu_seconds and reps < 20):
            t = time.perf_counter()
            O.append_tokens(kp, vp, w.k_src, w.v_src, w.seg_cu, w.seg_start, w.seg_tables,
                            cfg.block_size, w.num_blocks)
            spent += time.perf_counter() - t
            reps += 1
        line["cpu_baseline"] = {"value": round(nbytes * reps / spent / 1e9, 3), "unit": "GB/s",
                                "cores": 1, "kind": "oracle",
                                "sample": f"one layer's scatter ({T} tokens), {reps} repetitions, "
                                          f"{spent:.1f} s, single-threaded C"}
    print(json.dumps(line), flush=True)


def bench_copy_blocks(args):
    """Copy-on-write: every sequence of the workload forks once, so its partly
    filled last block is copied to a fresh block in every layer (one
    paged_kv_copy_blocks launch covering all layers).  value = algorithmic GB/s."""
    import torch
    import paged_kv_cache_09_amd as pkv
    from workloads import get_config

    cfg = get_config(args.config)
    dev = torch.device("cuda:0")
    tdt = {"fp16": torch.float16, "bf16": torch.bfloat16}[cfg.dtype]
    S, L = cfg.num_seqs, cfg.num_layers
    NB = 2 * S                          # the forked blocks and their copies, per layer
    shape = (NB, cfg.num_kv_heads, cfg.block_size, cfg.head_dim)
    g = torch.Generator(device=dev)
    g.manual_seed(0)
    kps, vps = [], []
    for _ in range(L):
        for lst in (kps, vps):
            lst.append(torch.randint(-32768, 32767, shape, dtype=torch.int16, device=dev,
                                     generator=g).view(tdt))
    rng = np.random.default_rng(0)
    perm = rng.permutation(NB).astype(np.int32)
    src = torch.from_numpy(perm[:S].copy()).to(dev)
    dst = torch.from_numpy(perm[S:].copy()).to(dev)
    torch.cuda.synchronize()

    def one():
        pkv.paged_kv_copy_blocks(kps, vps, src, dst)

    ms = time_launches(one, args.steps, warm=args.warmup)
    slab = cfg.num_kv_heads * cfg.block_size * cfg.head_dim * cfg.elem_bytes
    nbytes = 2 * (S * L * 2 * slab) + 8 * S                        # read + write, pair ids
    roof = roofline("paged_kv_copy_blocks", nbytes, ms,
                    measured_traffic(f"copy_blocks_{cfg.key}", "copy_blocks"))
    config = {"workload": f"{cfg.key} fork: every sequence copies one block in all layers "
                          f"({cfg.title})", "pairs": S, "layers": L,
              "block_bytes_per_pool": slab, "pool_blocks_per_layer": NB, "launches": 1}
    line = _side_line("copy-on-write block copy (paged_kv_copy_blocks) GB/s, 1 GPU",
                      roof["achieved"], "GB/s", args, cfg, cfg.dtype, config, roof)
    if not args.no_cpu_baseline:
        from oracle import oracle as O
        Ls = min(L, 4)
        host = [np.random.default_rng(i).integers(0, 1 << 16, size=shape, dtype=np.uint16)
                for i in range(2 * Ls)]
        reps, spent = 0, 0.0
        while reps == 0 or (spent < args.cpu_seconds and reps < 20):
            t = time.perf_counter()
            for i in range(Ls):
                O.copy_blocks(host[2 * i], host[2 * i + 1], perm[:S], perm[S:])
            spent += time.perf_counter() - t
            reps += 1
        sample_bytes = 2 * (S * Ls * 2 * slab)
        line["cpu_baseline"] = {"value": round(sample_bytes * reps / spent / 1e9, 3),
                                "unit": "GB/s", "cores": 1, "kind": "oracle",
                                "sample": f"{S} pairs x {Ls} of {L} layers, {reps} repetitions, "
                                          f"{spent:.1f} s, single-threaded C"}
    print(json.dumps(line), flush=True)


def _tables_as_segments(w):
    """A workload's block tables written as slotted segments: whole blocks, then
    the partly filled last block."""
    c = w.cfg
    B = c.block_size
    nb = -(-w.lengths.astype(np.int64) // B)
    segs = np.zeros((c.num_seqs, max(1, int(nb.max())), 3), np.int32)
    for s in range(c.num_seqs):
        for j in range(nb[s]):
            segs[s, j] = (w.tables[s, j], 0, min(B, int(w.lengths[s]) - j * B))
    return segs, nb.astype(np.int32)


def tree_ordered(w):
    """The radix batch with its sequences sorted by node path (a depth-first order
    of the tree): sequences under one node become neighbours, as a scheduler that
    batches requests by prefix would submit them.  Only the order of the
    per-sequence arrays changes; every sequence keeps its nodes and rows."""
    import dataclasses
    perm = sorted(range(len(w.paths)), key=lambda s: w.paths[s])
    return dataclasses.replace(w, paths=[w.paths[s] for s in perm], q=w.q[perm],
                               segments=w.segments[perm], num_segments=w.num_segments[perm],
                               k_new=w.k_new[perm], v_new=w.v_new[perm])


def bench_slotted(args):
    """Decode over slotted (block, slot offset, length) segments, one launch per
    step, cycling through R distinct batches.  The batch is the radix tree at the
    workload's shapes (a shared 512-token root, shared short nodes packed as
    slots, a private leaf per sequence), or the workload's own block tables
    written as segments (whole blocks; in split mode with the workload's
    partition size, paged_attention_decode_slotted_split).  In single pass the
    launch also writes each sequence's new K/V rows to its last position
    (paged_attention_append_decode_slotted) unless --slotted-append off
    (paged_attention_decode_slotted).  value = sequences / step time; the
    roofline counts each node's K/V rows once (unique bytes)."""
    import torch
    import paged_kv_cache_09_amd as pkv
    from workloads import get_config, make_workload
    from workloads.slotted import make_slotted_workload

    cfg = get_config(args.config)
    kind = args.slotted_batch
    if kind == "auto":
        kind = "radix" if cfg.prefix_tokens > 0 else "tables"
    P = (cfg.bench_partition_size if args.partition_size is None else args.partition_size)
    if kind == "radix" and args.partition_size is None:
        P = 0
    R = args.distinct or (4 if kind == "radix" else cfg.bench_distinct_layers)
    if args.slotted_kernel != "auto":
        os.environ["PKV_SLOTTED_TILES"] = "1" if args.slotted_kernel == "tiles" else "0"
    append = not P and args.slotted_append == "on"
    dev = torch.device("cuda:0")
    tdt = {"fp16": torch.float16, "bf16": torch.bfloat16}[cfg.dtype]

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(tdt)

    batches = []
    for d in range(R):
        if kind == "radix":
            w = make_slotted_workload(cfg, seed_id=1000 * cfg.cfg_id + d)
            if args.slotted_order == "tree":
                w = tree_ordered(w)
            kr, vr, cu, st, tb = w.runs()
            segs, nsegs, NB = w.segments, w.num_segments, w.num_blocks
            info = dict(unique=w.unique_tokens(), logical=int(w.lengths().sum()),
                        mean=float(w.lengths().mean()), nodes=len(w.node_k), S=len(w.paths))
        else:
            w = make_workload(cfg, layer=d)
            kr, vr, cu, st, tb = w.k_src, w.v_src, w.seg_cu, w.seg_start, w.seg_tables
            segs, nsegs = _tables_as_segments(w)
            NB = w.num_blocks
            # rows that several tables share (a shared prefix) count once
            held = np.zeros(NB * cfg.block_size, bool)
            for si in range(cfg.num_seqs):
                for b, o, ln in segs[si, :nsegs[si]]:
                    held[b * cfg.block_size + o:b * cfg.block_size + o + ln] = True
            info = dict(unique=int(held.sum()), logical=int(w.lengths.sum()),
                        mean=float(w.lengths.mean()), nodes=None, S=cfg.num_seqs)
        kp = torch.zeros((NB, cfg.num_kv_heads, cfg.block_size, cfg.head_dim), dtype=tdt,
                         device=dev)
        vp = torch.zeros_like(kp)
        pkv.paged_kv_append_tokens(kp, vp, up(kr), up(vr), torch.from_numpy(cu).to(dev),
                                   torch.from_numpy(st).to(dev), torch.from_numpy(tb).to(dev))
        if kind == "tables":
            # the step's own token, so that every position holds data
            pkv.paged_kv_append(kp, vp, up(w.k_new), up(w.v_new), torch.from_numpy(w.tables).to(dev),
                                torch.from_numpy(w.lengths).to(dev))
        batches.append(dict(w=w, k=kp, v=vp, q=up(w.q), info=info, kn=up(w.k_new),
                            vn=up(w.v_new),
                            segs=torch.from_numpy(segs).to(dev),
                            ns=torch.from_numpy(nsegs).to(dev)))
    torch.cuda.synchronize()
    b0 = batches[0]
    info = b0["info"]
    S, Hq, D = info["S"], cfg.num_q_heads, cfg.head_dim
    MS = int(b0["segs"].shape[1])
    out = torch.empty((S, Hq, D), dtype=tdt, device=dev)
    scale = float(np.float32(1.0 / math.sqrt(D)))
    if P:
        mp = -(-MS * cfg.block_size // P)
        po = torch.empty((S, Hq, mp, D), dtype=torch.float32, device=dev)
        pl = torch.empty((S, Hq, mp), dtype=torch.float32, device=dev)
        ctr = torch.zeros((S, cfg.num_kv_heads), dtype=torch.int32, device=dev)
    it = iter(range(1 << 30))

    def one():
        b = batches[next(it) % R]
        if P:
            pkv.paged_attention_decode_slotted_split(out, b["q"], b["k"], b["v"], b["segs"],
                                                     b["ns"], P, po, pl, ctr, scale=scale)
        elif append:
            pkv.paged_attention_append_decode_slotted(out, b["q"], b["k"], b["v"], b["kn"],
                                                      b["vn"], b["segs"], b["ns"], scale=scale)
        else:
            pkv.paged_attention_decode_slotted(out, b["q"], b["k"], b["v"], b["segs"], b["ns"],
                                               scale=scale)

    reps = max(64, R)
    for _ in range(args.warmup):
        one()
    ms, how = time_launches_graph(one, reps)
    e, Hkv = cfg.elem_bytes, cfg.num_kv_heads
    row = 2 * Hkv * D * e                                   # K and V of one token, all heads
    nseg = int(b0["ns"].sum())
    new_rows = 2 * S * row if append else 0                # new rows read + written
    unique = info["unique"] * row + 2 * S * Hq * D * e + 12 * nseg + 4 * S + new_rows
    logical = info["logical"] * row + 2 * S * Hq * D * e + 12 * nseg + 4 * S + new_rows
    name = "slotted_split" if P else "slotted"
    roof = roofline("paged_attention_decode_slotted_split" if P else
                    "paged_attention_append_decode_slotted" if append else
                    "paged_attention_decode_slotted", unique, ms,
                    measured_traffic(f"{name}_{cfg.key}" if kind == "tables" else
                                     f"slotted_{cfg.key}", "slotted"))
    roof["timing"] = how
    what = ("radix-tree batch in slotted blocks" if kind == "radix" else
            "block tables written as slotted segments")
    config = {"workload": f"{cfg.key} {what} ({cfg.title})",
              "num_seqs": S, "q_heads": Hq, "kv_heads": Hkv, "head_dim": D,
              "block_size": cfg.block_size, "mean_context": round(info["mean"], 1),
              "unique_tokens": info["unique"], "nodes": info["nodes"],
              "max_segments": MS, "partition_size": P, "distinct_batches": R, "launches": 1,
              "append_fused": append, "kernel_choice": args.slotted_kernel,
              "batch_order": args.slotted_order if kind == "radix" else "batch"}
    line = _side_line("slotted-segment decode tokens/s and unique-byte HBM GB/s, 1 GPU",
                      S / (ms * 1e-3), "tokens/s", args, cfg, cfg.dtype, config, roof,
                      {"logical_bytes_per_launch": logical})
    if not args.no_cpu_baseline:
        from oracle import oracle as O
        w0 = b0["w"]
        if kind == "radix":
            kr, vr, cu, st, tb = w0.runs()
        else:
            kr, vr, cu, st, tb = w0.k_src, w0.v_src, w0.seg_cu, w0.seg_start, w0.seg_tables
        NB = int(b0["k"].shape[0])
        kp, vp = O.new_pools(NB, Hkv, cfg.block_size, D, 0)
        O.append_tokens(kp, vp, kr, vr, cu, st, tb, cfg.block_size, NB)
        segs, nsegs = b0["segs"].cpu().numpy(), b0["ns"].cpu().numpy()
        threads = O.max_threads(0)
        reps, spent = 0, 0.0
        while reps == 0 or (spent < args.cpu_seconds and reps < 20):
            t = time.perf_counter()
            if append:
                O.append_slotted(kp, vp, w0.k_new, w0.v_new, segs, nsegs, cfg.block_size, NB)
            O.attention_slotted(w0.q, kp, vp, segs, nsegs, Hkv, cfg.block_size, NB, scale,
                                cfg.dtype, threads)
            spent += time.perf_counter() - t
            reps += 1
        line["cpu_baseline"] = {"value": round(S * reps / spent, 3), "unit": "tokens/s",
                                "cores": threads, "kind": "oracle",
                                "sample": f"the whole batch ({S} sequences x {Hq} heads, fp64"
                                          f"{', append + attention' if append else ''}), "
                                          f"{reps} repetitions, {spent:.1f} s"}
    print(json.dumps(line), flush=True)


def _oracle_threads(O):
    """OpenMP threads for the oracle: what OpenMP would use (OMP_NUM_THREADS), never
    more than the CPUs this process may run on.  Returns (threads, affinity CPUs)."""
    affinity = len(os.sched_getaffinity(0))
    threads = max(1, min(O.max_threads(0), affinity))
    O.max_threads(threads)
    return threads, affinity


def cpu_baseline(hosts, cfg, scale):
    """The fp64 oracle on one whole step of the workload: for every layer, the
    append of its new rows and attention of every sequence and head, over the
    same R distinct pool sets the GPU cycles through (layer l uses set l % R).
    Each set's pool is built once, untimed, and freed before the next; only the
    layers' append + attention are timed.  Returns the baseline record and the
    oracle's output of layer 0.  Single-threaded figures of the tiny (c1a) and
    long-context (c4) workloads are added as context."""
    from oracle import oracle as O
    c = cfg
    R = len(hosts)
    threads, affinity = _oracle_threads(O)
    spent, ref = 0.0, None
    for d, w in enumerate(hosts):
        kp, vp = O.new_pools(w.num_blocks, c.num_kv_heads, c.block_size, c.head_dim, w.nan_bits)
        O.append_tokens(kp, vp, w.k_src, w.v_src, w.seg_cu, w.seg_start, w.seg_tables,
                        c.block_size, w.num_blocks)
        for li in range(d, c.num_layers, R):
            t = time.perf_counter()
            O.append(kp, vp, w.k_new, w.v_new, w.tables, w.lengths, c.block_size, w.num_blocks)
            out = O.attention(w.q, kp, vp, w.tables, w.lengths, c.num_kv_heads, c.block_size,
                              w.num_blocks, scale, c.dtype, threads)
            spent += time.perf_counter() - t
            if li == 0:
                ref = out
        del kp, vp
    return {
        "value": round(c.num_seqs / spent, 3),
        "unit": "tokens/s",
        "cores": threads,
        "affinity_cpus": affinity,
        "kind": "oracle",
        "sample": (f"one whole step: {c.num_layers} layer(s) of {c.num_seqs} sequences x "
                   f"{c.num_q_heads} heads (append + fp64 attention), over {R} distinct pool "
                   f"set(s), {spent:.1f} s on {threads} OpenMP threads"),
        "single_thread": single_thread_oracle(scale),
        "cpu_model": _cpu_model(),
    }, ref


def single_thread_oracle(scale):
    """The oracle on one thread for one layer of the tiny batch (c1a) and of the
    long-context batch (c4, 8 x 16,384 tokens): tokens/s and seconds."""
    from oracle import oracle as O
    from workloads import get_config, make_workload
    res = {}
    prev = O.max_threads(0)
    for key in ("c1a", "c4"):
        cfg = get_config(key)
        w = make_workload(cfg)
        kp, vp = O.new_pools(w.num_blocks, cfg.num_kv_heads, cfg.block_size, cfg.head_dim,
                             w.nan_bits)
        O.append_tokens(kp, vp, w.k_src, w.v_src, w.seg_cu, w.seg_start, w.seg_tables,
                        cfg.block_size, w.num_blocks)
        t = time.perf_counter()
        O.append(kp, vp, w.k_new, w.v_new, w.tables, w.lengths, cfg.block_size, w.num_blocks)
        O.attention(w.q, kp, vp, w.tables, w.lengths, cfg.num_kv_heads, cfg.block_size,
                    w.num_blocks, scale, cfg.dtype, 1)
        dt = time.perf_counter() - t
        res[key] = {"tokens_per_s": round(cfg.num_seqs / dt, 3), "seconds": round(dt, 3),
                    "sample": f"one layer, {cfg.num_seqs} sequences x {cfg.num_q_heads} heads"}
        del kp, vp
    O.max_threads(prev)
    return res


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    main()
