#!/usr/bin/env python3
"""Benchmark of the FP8 E4M3 paged KV hot path on one MI355X.

One step = one serving decode step over the decode workload (64 requests,
context lengths uniform in [1024, 32768], 32 query / 8 KV heads, head_dim
128, 16-token blocks, bf16 ~ N(0,1) K/V/q):
  1. the split launch: the step's 64 new K/V rows (one per request, at the
     slot of its last token) quantized and stored by the split kernel
     itself, and paged GQA decode attention of the 64 query rows over the
     whole E4M3 cache (every KV head's tile sequence cut into equal ranges,
     one wave each), then
  2. the log-sum-exp merge of the ranges.
`value` is the step's algorithmic HBM bytes / step time (GB/s), the K timed
steps running back to back with no instrumentation between their kernels.
The dominant kernel (the decode split kernel) is then timed per launch with
HIP events on the stream it runs on, in a second pass of the same K steps,
for the roofline object.

Also measured in the same run (reported under "also"): quantize+scatter
tokens/s on the 4096-token prefill chunk (fused qkv, K/V strided slices,
random slots in a 1,048,576-slot pool, 32 rotating input sets so reads come
from HBM, replayed from a HIP graph; the same chunks stored into
consecutive slots, as a prefill filling fresh blocks; and the floors of
that launch: an empty kernel, a contiguous stream of its bytes, and a probe
moving its own bytes to the same slots without arithmetic), the
cache-build bandwidth, the long-context verify decode (4 requests of
256K..1M tokens, 4 verify rows, 16/4 heads, 64-token blocks), the decode
over selected blocks (1/8 of the decode workload's blocks), chunked-prefill
attention (a 4096-token chunk after 28,672 cached tokens, its last 1024
tokens as a chunk, and the 4096-token chunk over 1/8 of the blocks), the
compressed-index scorer (8 x 256 rows x 16 and 4 heads x 65,536 keys,
MXFP4 and E4M3 keys) with its key encoders and key builder, the decode
workload over unscaled E4M3 / E5M2 caches, and the HBM ceilings of plain
probe streams (sequential, and the cache's random 2 KiB blocks) and of the
library's copy and sum kernels on the same GPU.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, 8 TB/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_split_traffic.json")
KERNEL_SOURCES = ["fp8_e4m3_paged_kv_amd/csrc/paged_decode.hip",
                  "fp8_e4m3_paged_kv_amd/csrc/attn_tile.h",
                  "fp8_e4m3_paged_kv_amd/csrc/fp8kv_device.h"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--ranges", type=int, default=0,
                    help="decode split: ranges per KV head (0 = library choice)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the prefill-chunk, long-context and index extras")
    ap.add_argument("--extras",
                    default="prefill,longctx,sparse,prefill_attn,index,unscaled,ceilings",
                    help="comma list of the extras to run (prefill, longctx, sparse, "
                         "prefill_attn, index, unscaled, ceilings; not by default: ops, "
                         "the instruction-cost probes)")
    ap.add_argument("--scales", choices=("head", "interleaved"), default="head",
                    help="scale planes: head = two [Hkv, slots] planes; interleaved = one "
                         "[Hkv, slots, 2] array holding each row's K and V scales side by side")
    ap.add_argument("--pool", choices=("head", "slot"), default="head",
                    help="code pool layout: head = [Hkv, slots, D] (each KV head's "
                         "rows of a block contiguous), slot = [slots, Hkv, D]")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB, 5 times "
                         "(the known-size reference for HBM byte counters)")
    return ap.parse_args()


def copy_calibration(mib):
    """A plain device-to-device copy of a known size: the FETCH_SIZE and
    WRITE_SIZE counters it produces give the scale from counter units to
    bytes for the kernels measured with the same counters."""
    import torch
    n = mib * (1 << 20)
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n, "launches": 5}))


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def kernel_source_hash():
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def decode_bytes(lens, Hkv, D, B, R, Hq, bs):
    """Algorithmic HBM bytes of one decode launch: K and V codes plus their
    fp32 row scales for every (token, KV head), the page-table entries, q
    and the bf16 output."""
    kv = sum(lens) * Hkv * 2 * (D + 4)
    tables = sum((n + bs - 1) // bs for n in lens) * 4
    q_out = 2 * B * R * Hq * D * 2
    return kv + tables + q_out, kv


def quant_bytes(T, Hkv, D):
    """Algorithmic bytes of quantize+scatter: bf16 K and V rows read, E4M3
    codes and fp32 scales written, one int64 slot id per token."""
    return T * Hkv * 2 * (2 * D + D + 4) + 8 * T


SETTLE_S = 0.3
POOL = "head"                  # code pool layout (set from --pool)
POOL_DESC = {"head": "head-major [Hkv, slots, D]", "slot": "slot-major [slots, Hkv, D]"}
SCALES = "head"                # scale plane layout (set from --scales)
SCALES_DESC = {"head": "head-major [Hkv, slots]",
               "interleaved": "K/V-interleaved [Hkv, slots, 2]"}


def alloc_planes(torch, S, H, dev):
    """K and V scale planes as [Hkv, slots] views (passed transposed, as
    [slots, Hkv]): two planes, or one [Hkv, slots, 2] array with each row's
    K and V scales side by side (a 16-token block's 32 scales of one head
    are then one 128-byte line)."""
    if SCALES == "interleaved":
        kv = torch.empty((H, S, 2), dtype=torch.float32, device=dev)
        return kv[:, :, 0], kv[:, :, 1]
    k = torch.empty((H, S), dtype=torch.float32, device=dev)
    return k, torch.empty_like(k)


def alloc_pool(torch, S, H, D, dev):
    """K and V code pools as [slots, Hkv, D] views (the library takes any
    slot and head strides); stored head-major ([Hkv, slots, D]: a KV head's
    rows of a block are contiguous) or slot-major ([slots, Hkv, D])."""
    if POOL == "head":
        k = torch.empty((H, S, D), dtype=torch.uint8, device=dev).permute(1, 0, 2)
        v = torch.empty((H, S, D), dtype=torch.uint8, device=dev).permute(1, 0, 2)
    else:
        k = torch.empty((S, H, D), dtype=torch.uint8, device=dev)
        v = torch.empty_like(k)
    return k, v


def settle(fn, seconds=SETTLE_S):
    """Run fn back to back for about `seconds` of wall time (untimed). After
    a phase of other work the GPU needs some tens of launches before its
    clocks and memory subsystem reach the steady state every later launch
    sees (the first ~25 decode launches after the cache build run ~8%
    slower); this brings each measured workload there before its warmup."""
    import torch
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            fn()
        torch.cuda.synchronize()


def time_events(fn, n, stream):
    import torch
    settle(fn)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    for a, b in evs:
        a.record(stream)
        fn()
        b.record(stream)
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in evs]


def traffic_entry(per_launch_alg_bytes):
    """HBM traffic of the split kernel from the committed rocprofv3
    counter summary, if it was taken on the current kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    if t.get("pool_layout") != POOL:               # counters taken on this pool layout
        return None
    if t.get("scale_layout", "head") != SCALES:    # ... and these scale planes
        return None
    return t.get("bytes_per_launch")


def cache_build(torch, fk, k, v, slots, k_cache, v_cache, k_plane, v_plane,
                stream, chunk=1 << 20):
    """Quantize+scatter every cached token in launches of up to 1M tokens; returns
    the milliseconds of one whole build. The build first runs untimed for
    a settle period (it loads the kernels and touches the freshly allocated
    cache pages), then once more timed: quantize+scatter is idempotent, so
    the timed build writes the same bytes and measures the kernel in steady
    state."""
    def build():
        for i in range(0, slots.numel(), chunk):
            fk.kv_quant_scatter(k[i:i + chunk], v[i:i + chunk], slots[i:i + chunk],
                                k_cache, v_cache, k_plane.t(), v_plane.t())
    settle(build)
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    build()
    ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1)


def cpu_model():
    """The host CPU's model name (Linux /proc/cpuinfo), or the platform's."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(case, dc, lens, max_threads=16, budget_s=30.0):
    """The oracle (as it stands) on the same decode workload: every query row
    of as many of the 64 requests as fit the CPU budget (all of them here),
    one request per task on the host cores."""
    import numpy as np
    import torch
    import oracle
    from concurrent.futures import ThreadPoolExecutor
    L = case.layout
    bs = L.block_size
    H, D = case.num_kv_heads, case.head_dim
    cores = max(1, min(max_threads, os.cpu_count() or 1))

    def host_request(b):
        nb = (lens[b] + bs - 1) // bs
        blk = L.block_tables[b, :nb].long().to(dc["k_cache"].device)
        sl = (blk[:, None] * bs + torch.arange(bs, device=blk.device)).reshape(-1)
        kc = dc["k_cache"][sl].cpu().numpy()
        vc = dc["v_cache"][sl].cpu().numpy()
        kp = dc["k_plane"][:, sl].cpu().numpy()
        vp = dc["v_plane"][:, sl].cpu().numpy()
        bt = np.arange(nb, dtype=np.int32)[None, :]
        q = case.q[b:b + 1].contiguous().view(torch.int16).numpy().view(np.uint16)
        return q, kc, vc, kp.T, vp.T, bt, np.array([lens[b]], np.int32)

    def run(args):
        q, kc, vc, ks, vs, bt, cl = args
        return oracle.paged_decode_attn(q, kc, vc, ks, vs, bt, cl, H, bs,
                                        case.softmax_scale)

    # estimate the single-core cost from the first request, then take as
    # many requests as fit the budget of single-core CPU work
    first = host_request(0)
    t0 = time.perf_counter()
    run(first)
    t_first = time.perf_counter() - t0
    per_token = t_first / max(lens[0], 1)
    n, work = 0, 0.0
    while n < len(lens) and work + per_token * lens[n] <= budget_s:
        work += per_token * lens[n]
        n += 1
    n = max(n, 1)
    inputs = [first] + [host_request(b) for b in range(1, n)]
    t0 = time.perf_counter()
    with ThreadPoolExecutor(max_workers=min(cores, n)) as ex:
        list(ex.map(run, inputs))
    wall = time.perf_counter() - t0
    tokens = sum(lens[:n])
    alg = tokens * H * 2 * (D + 4)
    return {"value": round(alg / wall / 1e9, 4), "unit": "GB/s",
            "cores": min(cores, n), "kind": "oracle",
            "cpu_model": cpu_model(),
            "single_thread": {"value": round(lens[0] * H * 2 * (D + 4) / t_first / 1e9, 4),
                              "unit": "GB/s", "seconds": round(t_first, 3),
                              "sample": f"request 0 ({lens[0]} cached tokens x {H} KV "
                                        f"heads, all {case.num_q_heads} query rows) on one core"},
            "sample": f"all {case.num_q_heads} query rows of {n} of the {len(lens)} "
                      f"decode requests ({tokens} cached tokens x {H} KV heads), "
                      f"one request per task; ~{work:.1f} s of single-core work",
            "seconds": round(wall, 2)}


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark measures one GPU only; "
                                   "run with --gpus 1"}))
        sys.exit(2)
    global POOL, SCALES
    POOL = args.pool
    SCALES = args.scales
    import torch
    import fp8_e4m3_paged_kv_amd as fk
    from fp8_e4m3_paged_kv_amd import synth

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream(dev)

    # ---------------- decode workload (resident in HBM) ----------------
    log("building the decode workload (64 requests)...")
    case = synth.decode_workload(seed=2, device=dev)
    L = case.layout
    lens = L.context_lens.tolist()
    B, R, Hq, Hkv, D, bs = 64, 1, 32, 8, 128, L.block_size
    S = L.num_slots
    k_cache, v_cache = alloc_pool(torch, S, Hkv, D, dev)
    k_plane, v_plane = alloc_planes(torch, S, Hkv, dev)
    slots_all = L.token_slots.to(dev)
    T = slots_all.numel()
    # cache build: quantize+scatter of every cached token
    build_ms = cache_build(torch, fk, case.k, case.v, slots_all, k_cache,
                           v_cache, k_plane, v_plane, stream)
    build_gbs = quant_bytes(T, Hkv, D) / (build_ms * 1e-3) / 1e9
    log(f"cache build: {T} tokens in {build_ms:.2f} ms = {build_gbs:.1f} GB/s")

    # the step's new K/V rows: the last token of each request
    last = torch.tensor([sum(lens[:b + 1]) - 1 for b in range(B)], device=dev)
    k_new = case.k[last].contiguous()
    v_new = case.v[last].contiguous()
    del case.k, case.v
    torch.cuda.empty_cache()

    q = case.q.to(dev)
    bt = L.block_tables.to(dev)
    cl = L.context_lens.to(dev)
    maxc = bt.shape[1] * bs            # the page tables' coverage (>= every length)
    nr = fk.decode_num_ranges(Hkv, args.ranges)
    ws = torch.empty(fk.decode_workspace_bytes(B, R, Hq, Hkv, D, nr),
                     dtype=torch.uint8, device=dev)
    out = torch.empty((B, R, Hq, D), dtype=torch.bfloat16, device=dev)
    kw = dict(num_kv_heads=Hkv, block_size=bs, softmax_scale=case.softmax_scale,
              max_context=maxc, num_ranges=nr)

    ev_a = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ev_b = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    rec = {"i": None}

    # the step's new K/V rows, one per request, as [B, 1, Hkv, D]: the split
    # launch quantizes them into the cache before it reads their tiles
    k_new_rows = k_new.unsqueeze(1)
    v_new_rows = v_new.unsqueeze(1)

    def step():
        i = rec["i"]
        if i is not None:
            ev_a[i].record(stream)
        fk.paged_decode_append_partials(q, k_new_rows, v_new_rows, k_cache, v_cache,
                                        k_plane.t(), v_plane.t(), bt, cl, workspace=ws, **kw)
        if i is not None:
            ev_b[i].record(stream)
        fk.paged_decode_merge(ws, out, rows=R, num_q_heads=Hq,
                              num_kv_heads=Hkv, num_ranges=nr)

    def timed_steps():
        torch.cuda.synchronize()
        t_start = torch.cuda.Event(enable_timing=True)
        t_end = torch.cuda.Event(enable_timing=True)
        t_start.record(stream)
        for _ in range(args.steps):
            step()
        t_end.record(stream)
        torch.cuda.synchronize()
        return t_start.elapsed_time(t_end)

    settle(step)
    for _ in range(args.warmup):
        step()
    # the timed region: K whole steps, no instrumentation inside (an event
    # recorded between two kernels costs the GPU a few microseconds)
    total_ms = timed_steps()
    ms_per_step = total_ms / args.steps
    # the same K steps again, now with HIP events around every split launch
    # on its stream: the dominant kernel's per-launch duration
    for i in range(args.steps):
        rec["i"] = i
        step()
    torch.cuda.synchronize()
    rec["i"] = None
    part_ms = sorted(a.elapsed_time(b) for a, b in zip(ev_a, ev_b))
    part_avg_ms = sum(part_ms) / len(part_ms)

    dec_bytes, dec_kv = decode_bytes(lens, Hkv, D, B, R, Hq, bs)
    # the appended rows: bf16 K/V read, codes and scales written (their slots
    # come from the page table the decode reads anyway)
    app_bytes = quant_bytes(B, Hkv, D) - 8 * B
    step_bytes = dec_bytes + app_bytes
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    part_bytes = dec_bytes - B * R * Hq * D * 2 + app_bytes   # the merge writes out
    achieved = part_bytes / (part_avg_ms * 1e-3) / 1e9
    log(f"decode step: {ms_per_step * 1e3:.1f} us, split kernel "
        f"{part_avg_ms * 1e3:.1f} us = {achieved:.0f} GB/s")
    traffic = traffic_entry(part_bytes)

    result = {
        "metric": "FP8 paged decode attn HBM GB/s (% peak) + quant-scatter tokens/s, 1 GPU",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "e4m3 codes (u8) + fp32 scales; bf16/fp16 MFMA, fp32 accumulate",
        "data": "synthetic (seeded N(0,1) bf16 K/V/q)",
        "config": {"workload": "decode step: 64 new tokens quantized into the cache inside "
                               "the split launch + paged GQA decode, 64 requests, "
                               "lengths U[1024,32768]",
                   "batch": B, "context_tokens": sum(lens), "num_q_heads": Hq,
                   "num_kv_heads": Hkv, "head_dim": D, "block_size": bs,
                   "decode_ranges_per_kv_head": nr,
                   "scale_planes": SCALES_DESC[SCALES],
                   "pool_layout": POOL_DESC[POOL]},
        "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic,
                     "kernel": "decode_split_kernel",
                     "alg_bytes_per_launch": part_bytes,
                     "avg_launch_us": round(part_avg_ms * 1e3, 2),
                     "timing": "HIP events around each split launch on its stream, "
                               "in a second pass of the K steps"},
        "cpu_baseline": None,
        "also": {"cache_build_GBps": round(build_gbs, 1)},
    }

    extras = set() if args.no_extras else set(args.extras.split(","))
    if "prefill" in extras:
        qs = prefill_quant_scatter(torch, fk, synth, dev, stream)
        fl = chunk_store_floors(torch, dev, stream)
        # the chunk store against a plain 2:1 stream of its bytes launched
        # the same way (graph replay, rotating buffers)
        fl["quant_scatter_prefill_floor_tokens_per_s"] = round(
            4096 / (fl["graph_floor_stream_2to1_25MB_us"] * 1e-6), 0)
        fl["quant_scatter_prefill_over_floor"] = round(
            qs["quant_scatter_prefill_us"] / fl["graph_floor_stream_2to1_25MB_us"], 3)
        # and against the probe that moves the store's own bytes to the same
        # slots without its arithmetic
        fl["quant_scatter_prefill_over_traffic_floor"] = round(
            qs["quant_scatter_prefill_us"] / qs["quant_scatter_prefill_traffic_floor_us"], 3)
        result["also"].update(qs)
        result["also"].update(fl)
    if "longctx" in extras:
        result["also"].update(longctx_decode(torch, fk, synth, dev, stream))
    if "sparse" in extras:
        result["also"].update(sparse_decode(torch, fk, synth, dev, stream, case, q, bt,
                                            k_cache, v_cache, k_plane, v_plane))
    if "prefill_attn" in extras:
        result["also"].update(prefill_attention(torch, fk, synth, dev, stream))
    if "index" in extras:
        result["also"].update(index_scorer(torch, fk, synth, dev, stream))
    if "unscaled" in extras:
        result["also"].update(unscaled_decode(torch, fk, synth, dev, stream, case, q, bt, cl))
    if "ceilings" in extras:
        result["also"].update(hbm_ceilings(torch, dev, stream))
    if "ops" in extras:
        result["also"].update(op_costs(torch, dev, stream))

    if not args.no_cpu_baseline:
        log("timing the oracle on host cores...")
        dc = {"k_cache": k_cache, "v_cache": v_cache, "k_plane": k_plane,
              "v_plane": v_plane}
        result["cpu_baseline"] = cpu_baseline(case, dc, lens)
    print(json.dumps(result), flush=True)


def prefill_quant_scatter(torch, fk, synth, dev, stream, sets=32, reps=4):
    """Quantize+scatter of the 4096-token prefill chunk, rotating 32 input
    sets (1.6 GB > the 256 MB MALL) and slot sets; timed per launch from
    graph replays (and eagerly, for reference). Beside it, the probe
    library's copy of the store's memory traffic without its arithmetic
    (the same strided reads, 128-byte code rows and 4-byte scales to the
    same slots), replayed the same way: the floor of this access pattern."""
    log("prefill-chunk quantize+scatter...")
    H, D, T, S = 8, 128, 4096, 1 << 20
    chunks = [synth.prefill_chunk(seed=100 + i, device=dev) for i in range(sets)]
    k_cache, v_cache = alloc_pool(torch, S, H, D, dev)
    k_plane, v_plane = alloc_planes(torch, S, H, dev)
    it = {"i": 0}

    def one():
        c = chunks[it["i"] % sets]
        it["i"] += 1
        fk.kv_quant_scatter(c.k_view(), c.v_view(), c.slot_ids, k_cache,
                            v_cache, k_plane.t(), v_plane.t())
    for _ in range(sets):
        one()
    ms = time_events(one, sets * reps, stream)
    avg = sum(ms) / len(ms)
    side = torch.cuda.Stream(dev)

    def graph_us(launch):
        # launch(i) for every input set, captured in one HIP graph and
        # replayed: the per-launch time without the host's launch overhead
        torch.cuda.synchronize()
        side.wait_stream(stream)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            for i in range(sets):
                launch(i)
        stream.wait_stream(side)
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(reps):
            graph.replay()
        t1.record(stream)
        torch.cuda.synchronize()
        del graph
        return t0.elapsed_time(t1) / (reps * sets) * 1e3

    def store(slots):
        return lambda i: fk.kv_quant_scatter(chunks[i].k_view(), chunks[i].v_view(), slots(i),
                                             k_cache, v_cache, k_plane.t(), v_plane.t())
    L = probes_lib()

    def traffic(slots, mode=0):
        # mode: bit 0 no code stores, bit 1 no scale stores, bit 2 dense
        # source rows (the first 16.8 MB of the set's qkv buffer)
        def launch(i):
            kv, vv = chunks[i].k_view(), chunks[i].v_view()
            src = chunks[i].qkv if mode & 4 else kv
            sl = slots(i)
            st = L.fp8kv_probe_scatter(
                src.data_ptr(), vv.data_ptr(), kv.stride(0), kv.stride(1), sl.data_ptr(), T, H,
                k_cache.data_ptr(), v_cache.data_ptr(), k_cache.stride(1), k_cache.stride(0),
                k_plane.data_ptr(), v_plane.data_ptr(), k_plane.stride(0), k_plane.stride(1), S,
                mode, side.cuda_stream)
            if st != 0:
                raise RuntimeError(f"scatter probe: status {st}")
        return launch
    # the chunks also stored into consecutive slots (a prefill filling
    # freshly allocated blocks): input set i takes slots [i*T, (i+1)*T)
    contig = [torch.arange(i * T, (i + 1) * T, device=dev) for i in range(sets)]
    g_us = graph_us(store(lambda i: chunks[i].slot_ids))
    c_us = graph_us(store(lambda i: contig[i]))
    f_us = graph_us(traffic(lambda i: chunks[i].slot_ids))
    fc_us = graph_us(traffic(lambda i: contig[i]))
    parts = {name: graph_us(traffic(lambda i: chunks[i].slot_ids, mode))
             for name, mode in (("no_scales", 2), ("no_codes", 1), ("reads_only", 3),
                                ("dense_source", 4))}
    tok_s = T / (g_us * 1e-6)
    gbs = quant_bytes(T, H, D) / (g_us * 1e-6) / 1e9
    del chunks
    torch.cuda.empty_cache()
    return {"quant_scatter_prefill_tokens_per_s": round(tok_s, 0),
            "quant_scatter_prefill_us": round(g_us, 2),
            "quant_scatter_prefill_GBps": round(gbs, 1),
            "quant_scatter_prefill_eager_us": round(avg * 1e3, 2),
            "quant_scatter_prefill_contiguous_slots_us": round(c_us, 2),
            "quant_scatter_prefill_contiguous_slots_tokens_per_s": round(T / (c_us * 1e-6), 0),
            "quant_scatter_prefill_traffic_floor_us": round(f_us, 2),
            "quant_scatter_prefill_traffic_floor_contiguous_us": round(fc_us, 2),
            **{f"quant_scatter_prefill_traffic_{k}_us": round(v, 2) for k, v in parts.items()}}


def longctx_decode(torch, fk, synth, dev, stream, reps=20):
    log("long-context verify decode (4 x 256K..1M tokens)...")
    case = synth.longctx_workload(seed=3, device=dev)
    L = case.layout
    H, D, bs = 4, 128, L.block_size
    S = L.num_slots
    k_cache, v_cache = alloc_pool(torch, S, H, D, dev)
    k_plane, v_plane = alloc_planes(torch, S, H, dev)
    slots = L.token_slots.to(dev)
    T = slots.numel()
    build_ms = cache_build(torch, fk, case.k, case.v, slots, k_cache, v_cache,
                           k_plane, v_plane, stream)
    build_gbs = quant_bytes(T, H, D) / (build_ms * 1e-3) / 1e9
    del case.k, case.v
    torch.cuda.empty_cache()
    lens = L.context_lens.tolist()
    maxc = max(lens)
    B, R, Hq = 4, 4, 16
    q = case.q.to(dev)
    bt = L.block_tables.to(dev)
    cl = L.context_lens.to(dev)
    nr = fk.decode_num_ranges(H)
    ws = torch.empty(fk.decode_workspace_bytes(B, R, Hq, H, D, nr),
                     dtype=torch.uint8, device=dev)
    out = torch.empty((B, R, Hq, D), dtype=torch.bfloat16, device=dev)
    kw = dict(num_kv_heads=H, block_size=bs, softmax_scale=case.softmax_scale,
              max_context=maxc, num_ranges=nr, workspace=ws)

    def partials():
        fk.paged_decode_partials(q, k_cache, v_cache, k_plane.t(), v_plane.t(),
                                 bt, cl, **kw)

    def full():
        fk.paged_decode_attn_fp8(q, k_cache, v_cache, k_plane.t(), v_plane.t(),
                                 bt, cl, out=out, **kw)
    for _ in range(3):
        full()
    pm = time_events(partials, reps, stream)
    fm = time_events(full, reps, stream)
    dec, kvb = decode_bytes(lens, H, D, B, R, Hq, bs)
    p_avg = sum(pm) / len(pm)
    f_avg = sum(fm) / len(fm)
    res = {"longctx_decode_us": round(f_avg * 1e3, 1),
           "longctx_decode_GBps": round(dec / (f_avg * 1e-3) / 1e9, 1),
           "longctx_split_kernel_us": round(p_avg * 1e3, 1),
           "longctx_split_kernel_GBps": round((dec - B * R * Hq * D * 2) / (p_avg * 1e-3) / 1e9, 1),
           "longctx_cache_build_GBps": round(build_gbs, 1)}
    del k_cache, v_cache, k_plane, v_plane
    torch.cuda.empty_cache()
    return res


def sparse_decode(torch, fk, synth, dev, stream, case, q, bt, k_cache, v_cache,
                  k_plane, v_plane, reps=20):
    """Decode over selected blocks on the decode workload's cache: every
    request keeps 1/8 of its blocks (drawn at random) plus its last one.
    Algorithmic bytes: the selected keys' codes and scales, the selected
    table entries and valid counts, q."""
    log("sparse decode (1/8 of the blocks of the decode workload)...")
    sel = synth.sparse_selection(case.layout, 0.125, seed=52)
    B, R, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    bs = case.layout.block_size
    sbt = sel.block_tables.to(dev)
    sbv = sel.block_valid.to(dev)
    scl = sel.context_lens.to(dev)
    nr = fk.decode_num_ranges(Hkv, 0)
    ws = torch.empty(fk.decode_workspace_bytes(B, R, Hq, Hkv, D, nr),
                     dtype=torch.uint8, device=dev)
    out = torch.empty((B, R, Hq, D), dtype=torch.bfloat16, device=dev)
    kw = dict(num_kv_heads=Hkv, block_size=bs, softmax_scale=case.softmax_scale,
              max_context=sbt.shape[1] * bs, num_ranges=nr, workspace=ws)

    def partials():
        fk.sparse_decode_partials(q, k_cache, v_cache, k_plane.t(), v_plane.t(),
                                  sbt, sbv, scl, **kw)

    def full():
        fk.sparse_decode_attn_fp8(q, k_cache, v_cache, k_plane.t(), v_plane.t(),
                                  sbt, sbv, scl, out=out, **kw)
    keys = int(sel.block_valid.clamp(0, bs).sum())
    nsel = int((sel.block_valid > 0).sum())
    alg = keys * Hkv * (2 * D + 8) + nsel * 8 + B * R * Hq * D * 2
    pm = time_events(partials, reps, stream)
    fm = time_events(full, reps, stream)
    p_avg = sum(pm) / len(pm)
    f_avg = sum(fm) / len(fm)
    return {"sparse_selected_tokens": keys,
            "sparse_decode_us": round(f_avg * 1e3, 1),
            "sparse_split_kernel_us": round(p_avg * 1e3, 1),
            "sparse_split_kernel_GBps": round(alg / (p_avg * 1e-3) / 1e9, 1)}


def unscaled_decode(torch, fk, synth, dev, stream, case, q, bt, cl, reps=20):
    """The decode workload over unscaled caches (E4M3 and E5M2 codes, no
    scale planes): cache build and split kernel. Algorithmic bytes: 2 x D
    code bytes per (token, KV head) for the split kernel, 2 x (2D + D) + 8
    per token for the build."""
    log("unscaled E4M3 / E5M2 caches on the decode workload...")
    L = case.layout
    B, R, Hq, D = q.shape
    Hkv = 8
    S = L.num_slots
    lens = L.context_lens.tolist()
    g = synth.gen(2 + 1000, dev)
    T = int(sum(lens))
    kc, vc = alloc_pool(torch, S, Hkv, D, dev)
    slots = L.token_slots.to(dev)
    nr = fk.decode_num_ranges(Hkv, 0)
    ws = torch.empty(fk.decode_workspace_bytes(B, R, Hq, Hkv, D, nr), dtype=torch.uint8,
                     device=dev)
    res = {}
    for name, cf in (("e4m3", fk.CODES_E4M3), ("e5m2", fk.CODES_E5M2)):
        # the same K/V distribution as the scaled cache, drawn in chunks
        c = 1 << 20
        build_ms = 0.0
        for i in range(0, T, c):
            n = min(c, T - i)
            k = synth.normal_bf16((n, Hkv, D), g, device=dev)
            v = synth.normal_bf16((n, Hkv, D), g, device=dev)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            fk.kv_quant_scatter_unscaled(k, v, slots[i:i + n], kc, vc, cf)
            e1.record(stream)
            torch.cuda.synchronize()
            build_ms += e0.elapsed_time(e1)
            del k, v
        kw = dict(num_kv_heads=Hkv, block_size=L.block_size, softmax_scale=case.softmax_scale,
                  max_context=bt.shape[1] * L.block_size, code_format=cf,
                  num_ranges=nr, workspace=ws)
        run = lambda: fk.paged_decode_partials_unscaled(q, kc, vc, bt, cl, **kw)
        ms = sorted(time_events(run, reps, stream))
        med = ms[len(ms) // 2]
        alg = T * Hkv * 2 * D + sum((n + L.block_size - 1) // L.block_size for n in lens) * 4 \
            + B * R * Hq * D * 2
        res[f"unscaled_{name}_split_kernel_us"] = round(med * 1e3, 1)
        res[f"unscaled_{name}_split_kernel_GBps"] = round(alg / (med * 1e-3) / 1e9, 1)
        res[f"unscaled_{name}_cache_build_GBps"] = round(
            T * Hkv * 2 * 3 * D / (build_ms * 1e-3) / 1e9, 1)
    del kc, vc, ws
    torch.cuda.empty_cache()
    return res


def probes_lib():
    """The benchmark's probe kernels (libfp8kv_probes.so, built beside the
    cache library): fp8kv_probe(kind, a, b, dst, bytes, stream) with kind 0
    read, 1 copy, 2 read a and b / write dst (2:1), 3 write, 4 empty, 5-7
    read a's 2 KiB blocks in the order of the int32 ids b (5: one block per
    wave, one pass; 6, 7: one wave per SIMD, 4 or 8 blocks per load
    group)."""
    import ctypes
    from fp8_e4m3_paged_kv_amd import build as hipbuild
    if not os.path.exists(hipbuild.PROBES_LIB):
        raise ImportError(f"{hipbuild.PROBES_LIB} is missing: run the build")
    L = ctypes.CDLL(hipbuild.PROBES_LIB)
    P = ctypes.c_void_p
    L.fp8kv_probe.argtypes = [ctypes.c_int, P, P, P, ctypes.c_size_t, P]
    L.fp8kv_probe.restype = ctypes.c_int
    I64, I32 = ctypes.c_int64, ctypes.c_int
    L.fp8kv_probe_scatter.argtypes = [P, P, I64, I64, P, I32, I32, P, P, I64, I64, P, P,
                                      I64, I64, I64, I32, P]
    L.fp8kv_probe_scatter.restype = ctypes.c_int
    L.fp8kv_probe_ops.argtypes = [I32, P, P, I32, I32, P]
    L.fp8kv_probe_ops.restype = ctypes.c_int
    return L


def probe(L, stream, kind, a=None, b=None, d=None, nbytes=0):
    st = L.fp8kv_probe(kind, None if a is None else a.data_ptr(),
                       None if b is None else b.data_ptr(),
                       None if d is None else d.data_ptr(), nbytes, stream.cuda_stream)
    if st != 0:
        raise RuntimeError(f"probe kind {kind}: status {st}")


def hbm_ceilings(torch, dev, stream, gib=2, reps=10):
    """What plain streaming kernels reach on this GPU (the probe library's
    16-byte streams over 2 GiB buffers, non-temporal loads and ordinary
    stores: read, copy, 2:1 read:write, write), and what the library's own
    copy and sum kernels reach, for reference. The paged reads fetch the
    same 2 GiB as 2 KiB blocks (one KV head's codes of a 16-token block) in
    a random order, as the decode kernels walk the cache: in one pass
    (`paged_read`), and by one wave per SIMD in groups of 8 or 16 KiB, the
    next group's loads issued before the current one is consumed
    (`paged_read_1wave_8k` / `_16k`; 8 KiB is one decode tile of K and V
    codes, and the decode kernel also loads one tile ahead)."""
    log("HBM ceilings (probe streams, library copy and read kernels)...")
    L = probes_lib()
    n = gib << 30
    a = torch.ones(n // 8, dtype=torch.int64, device=dev)
    b = torch.ones_like(a)
    d = torch.empty_like(a)
    g = torch.Generator(device=dev)
    g.manual_seed(11)
    ids = torch.randperm(n // 2048, generator=g, device=dev).to(torch.int32)
    res = {}
    for name, fn, moved in (
            ("read", lambda: probe(L, stream, 0, a=a, d=d, nbytes=n), n),
            ("copy", lambda: probe(L, stream, 1, a=a, d=d, nbytes=n), 2 * n),
            ("read2_write1", lambda: probe(L, stream, 2, a=a, b=b, d=d, nbytes=n), 3 * n),
            ("write", lambda: probe(L, stream, 3, d=d, nbytes=n), n),
            ("paged_read", lambda: probe(L, stream, 5, a=a, b=ids, d=d, nbytes=n), n),
            ("paged_read_1wave_8k", lambda: probe(L, stream, 6, a=a, b=ids, d=d, nbytes=n), n),
            ("paged_read_1wave_16k", lambda: probe(L, stream, 7, a=a, b=ids, d=d, nbytes=n), n),
            ("torch_copy", lambda: d.copy_(a), 2 * n),
            ("torch_sum", lambda: a.sum(), n)):
        settle(fn, 0.1)
        ms = sorted(time_events(fn, reps, stream))
        res[f"hbm_{name}_GBps"] = round(moved / (ms[len(ms) // 2] * 1e-3) / 1e9, 1)
    del a, b, d, ids
    torch.cuda.empty_cache()
    return res


OP_PROBES = ("exp2_f32", "exp2_f16", "fma", "mfma", "mfma_2fma", "mfma_4fma", "mfma_1exp2",
             "mfma_3fma", "mfma_wave_beside_fma_wave", "fma_wave_alone")


def op_costs(torch, dev, stream, iters=4000):
    """Instruction costs on this GPU (the probe library's fp8kv_probe_ops):
    every wave runs `iters` iterations of 8 independent chains of one
    operation (exp2 f32, exp2 f16, FMA), or of 8 independent 16x16x32 bf16
    MFMA chains with 2, 4, 3 FMAs or one exp2 per MFMA in the same wave, at
    one and two waves per SIMD; and, at two waves per SIMD, an MFMA-only
    wave beside a wave running 2 FMAs per MFMA slot on each SIMD, and that
    FMA wave alone. Reported: each kernel's time and, per SIMD, the time
    per operation (exp2 / FMA chains, the FMA wave alone) or per MFMA (the
    others)."""
    log("instruction-cost probes...")
    L = probes_lib()
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    res = {}
    for wps in (1, 2):
        blocks = cus * wps
        out = torch.zeros(blocks * 4, device=dev)
        cyc = torch.zeros(blocks * 4, dtype=torch.int64, device=dev)
        for v, name in enumerate(OP_PROBES):
            split = name in ("mfma_wave_beside_fma_wave", "fma_wave_alone")
            if split and wps != 2:
                continue

            def launch():
                st = L.fp8kv_probe_ops(v, out.data_ptr(), cyc.data_ptr(), iters, blocks,
                                       stream.cuda_stream)
                if st != 0:
                    raise RuntimeError(f"op probe {v}: status {st}")
            for _ in range(3):
                launch()
            ms = sorted(time_events(launch, 5, stream))[2]
            # operations per SIMD: wps waves x iters x 8 (the split variants:
            # one MFMA wave x 8 MFMAs, or one FMA wave x 16 FMAs, per iteration)
            ops = iters * (16 if name == "fma_wave_alone" else 8) * (1 if split else wps)
            res[f"op_{name}_w{wps}_us"] = round(ms * 1e3, 1)
            res[f"op_{name}_w{wps}_ns_per_op"] = round(ms * 1e6 / ops, 3)
    return res


def chunk_store_floors(torch, dev, stream, sets=32, reps=4):
    """Floors for the 4096-token prefill-chunk store, in its own harness
    (one HIP graph of `sets` launches, replayed): an empty kernel (the
    per-launch floor), and a 2:1 read:write stream of the chunk's bytes
    (two 8.4 MB reads, one 8.4 MB write: 25.2 MB per launch, rotating
    over `sets` buffer sets as the store rotates its inputs)."""
    log("prefill-chunk floors (empty kernel, 25 MB 2:1 stream, graph replay)...")
    L = probes_lib()
    part = 4096 * 8 * 128 * 2 // 2                        # bytes of K (or V) in bf16 / 2
    bufs = [tuple(torch.empty(part // 8, dtype=torch.int64, device=dev) for _ in range(3))
            for _ in range(sets)]
    res = {}
    side = torch.cuda.Stream(dev)
    for name, launch in (("empty", lambda i: probe(L, side, 4)),
                         ("stream_2to1_25MB", lambda i: probe(L, side, 2, a=bufs[i][0], b=bufs[i][1],
                                                              d=bufs[i][2], nbytes=part))):
        torch.cuda.synchronize()
        side.wait_stream(stream)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            for i in range(sets):
                launch(i)
        stream.wait_stream(side)
        for _ in range(2):
            graph.replay()
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record(stream)
        for _ in range(reps):
            graph.replay()
        t1.record(stream)
        torch.cuda.synchronize()
        res[f"graph_floor_{name}_us"] = round(t0.elapsed_time(t1) / (reps * sets) * 1e3, 2)
        del graph
    del bufs
    torch.cuda.empty_cache()
    return res


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16 MFMA


def prefill_attention(torch, fk, synth, dev, stream, reps=10):
    """Chunked-prefill attention: a 4096-token chunk at the end of a
    32,768-token request, Hq 32 / Hkv 8, D 128, bs 16. Useful work: for
    every chunk token i (position P + i) and query head, P + i + 1 keys
    at 4 * D flops each (QK^T and PV)."""
    log("prefill attention (4096-token chunk on a 32,768-token request)...")
    case = synth.prefill_attn_workload(seed=71, device=dev)
    L = case.layout
    H, D = case.num_kv_heads, case.head_dim
    S = L.num_slots
    k_cache, v_cache = alloc_pool(torch, S, H, D, dev)
    k_plane, v_plane = alloc_planes(torch, S, H, dev)
    slots = L.token_slots.to(dev)
    cache_build(torch, fk, case.k, case.v, slots, k_cache, v_cache, k_plane, v_plane, stream)
    del case.k, case.v
    q = case.q.to(dev)
    B, C, Hq, _ = q.shape
    ctx = int(L.context_lens[0])
    P = ctx - C
    ql = torch.full((B,), C, dtype=torch.int32, device=dev)
    bt = L.block_tables.to(dev)
    cl = L.context_lens.to(dev)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)

    def run():
        fk.prefill_attn_fp8(q, k_cache, v_cache, k_plane.t(), v_plane.t(), bt, cl, ql,
                            num_kv_heads=H, block_size=L.block_size,
                            softmax_scale=case.softmax_scale, max_context=ctx, out=out)
    settle(run)
    ms = time_events(run, reps, stream)
    avg = sum(ms) / len(ms)
    flops = (P * C + C * (C + 1) // 2) * Hq * 4 * D
    tf = flops / (avg * 1e-3) / 1e12
    res = {"prefill_attn_us": round(avg * 1e3, 1),
           "prefill_attn_TFLOPs": round(tf, 1),
           "prefill_attn_mfma_frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)}

    # a 1024-token chunk at the end of the same request: one query block per
    # CU, where the kernel splits each block's keys over two wave groups
    # (q and out as 1024-row views: the grid follows the buffers' rows)
    C1 = 1024
    ql1 = torch.full((B,), C1, dtype=torch.int32, device=dev)
    q1, out1 = q[:, :C1], out[:, :C1]

    def run_1k():
        fk.prefill_attn_fp8(q1, k_cache, v_cache, k_plane.t(), v_plane.t(), bt, cl, ql1,
                            num_kv_heads=H, block_size=L.block_size,
                            softmax_scale=case.softmax_scale, max_context=ctx, out=out1)
    settle(run_1k)
    ms = time_events(run_1k, reps, stream)
    avg = sum(ms) / len(ms)
    P1 = ctx - C1
    tf = (P1 * C1 + C1 * (C1 + 1) // 2) * Hq * 4 * D / (avg * 1e-3) / 1e12
    res.update({"prefill_attn_1k_us": round(avg * 1e3, 1),
                "prefill_attn_1k_TFLOPs": round(tf, 1),
                "prefill_attn_1k_mfma_frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)})

    # the same chunk over selected blocks: 1/8 of the blocks before the
    # chunk, then the chunk's own (every selected block full)
    log("prefill attention over selected blocks (1/8 of the context)...")
    sel = synth.prefill_selection(L, [C], 0.125, seed=72)
    sbt, sbv, scl = (t.to(dev) for t in (sel.block_tables, sel.block_valid, sel.context_lens))
    vctx = int(sel.context_lens[0])
    Pv = vctx - C

    def run_sel():
        fk.sparse_prefill_attn_fp8(q, k_cache, v_cache, k_plane.t(), v_plane.t(), sbt, sbv,
                                   scl, ql, num_kv_heads=H, block_size=L.block_size,
                                   softmax_scale=case.softmax_scale,
                                   max_context=L.block_size * sbt.shape[1], out=out)
    settle(run_sel)
    ms = time_events(run_sel, reps, stream)
    avg = sum(ms) / len(ms)
    flops = (Pv * C + C * (C + 1) // 2) * Hq * 4 * D
    tf = flops / (avg * 1e-3) / 1e12
    res.update({"sparse_prefill_selected_tokens": vctx,
                "sparse_prefill_attn_us": round(avg * 1e3, 1),
                "sparse_prefill_attn_TFLOPs": round(tf, 1),
                "sparse_prefill_attn_mfma_frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4)})
    del k_cache, v_cache, k_plane, v_plane, out
    torch.cuda.empty_cache()
    return res


def index_scorer(torch, fk, synth, dev, stream, reps=20):
    """The compressed-index workload: 8 requests x 256 query rows x 16 index
    heads x 65,536 keys (dim 128), keys stored as MXFP4 and as E4M3; the
    scorer's useful work is 2 * B * R * H * N * 128 flops (bf16 MFMA). The
    same with 4 index heads (4 rows x 4 heads per MFMA tile), where the
    537 MB of fp32 scores weigh as much as the MFMA work: its line adds the
    score bytes per second."""
    res = {}
    for H in (16, 4):
        log(f"index scorer (8 x 256 rows x {H} heads x 65,536 keys)...")
        case = synth.index_workload(seed=4, device=dev, heads=H)
        B, R, _, _ = case.q.shape
        N = case.keys.shape[1]
        flops = 2.0 * B * R * H * N * 128
        out = torch.empty((B, R, N), dtype=torch.float32, device=dev)
        tag = "" if H == 16 else f"h{H}_"
        for name, fmt, kbytes in (("mxfp4", fk.KEYS_MXFP4, 64 + 4),
                                  ("e4m3", fk.KEYS_E4M3, 128 + 4)):
            codes, scales = fk.index_keys_quantize(case.keys, fmt)
            if H == 16:
                enc = time_events(lambda: fk.index_keys_quantize(case.keys, fmt, codes, scales),
                                  reps, stream)
                e_avg = sum(enc) / len(enc)
                res[f"index_keys_{name}_GBps"] = round(
                    B * N * (256 + kbytes) / (e_avg * 1e-3) / 1e9, 1)
            settle(lambda: fk.index_score_mxfp4(case.q, case.w, fmt, codes, scales, out=out))
            ms = time_events(lambda: fk.index_score_mxfp4(case.q, case.w, fmt, codes,
                                                          scales, out=out), reps, stream)
            avg = sum(ms) / len(ms)
            tf = flops / (avg * 1e-3) / 1e12
            res[f"index_score_{tag}{name}_us"] = round(avg * 1e3, 1)
            res[f"index_score_{tag}{name}_TFLOPs"] = round(tf, 1)
            res[f"index_score_{tag}{name}_mfma_frac"] = round(tf / MFMA_BF16_PEAK_TFLOPS, 4)
            if H != 16:
                res[f"index_score_{tag}{name}_score_GBps"] = round(
                    B * R * N * 4 / (avg * 1e-3) / 1e9, 1)
            del codes, scales
        del case, out
        torch.cuda.empty_cache()
    # key builder: 4 raw bf16 keys -> one compressed key (mean, L2 norm, encode)
    raw = synth.normal_bf16((B, 4 * N, 128), synth.gen(5, dev), device=dev)
    for name, fmt, kbytes in (("mxfp4", fk.KEYS_MXFP4, 64 + 4),
                              ("e4m3", fk.KEYS_E4M3, 128 + 4)):
        codes = torch.empty((B, N, 64 if fmt == fk.KEYS_MXFP4 else 128),
                            dtype=torch.uint8, device=dev)
        scales = (torch.empty((B, N, 4), dtype=torch.uint8, device=dev)
                  if fmt == fk.KEYS_MXFP4 else torch.empty((B, N), device=dev))
        ms = time_events(lambda: fk.index_keys_build(raw, 0, N, fmt, codes, scales),
                         reps, stream)
        avg = sum(ms) / len(ms)
        res[f"index_keys_build_{name}_us"] = round(avg * 1e3, 1)
        res[f"index_keys_build_{name}_GBps"] = round(
            B * N * (4 * 256 + kbytes) / (avg * 1e-3) / 1e9, 1)
        del codes, scales
    del raw
    torch.cuda.empty_cache()
    return res


if __name__ == "__main__":
    main()
