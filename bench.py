#!/usr/bin/env python3
"""Benchmark of the paged-attention hot path on one MI355X.

A step is the whole hot path over one synthetic batch already resident in HBM: the KV
write of the step's new tokens (slot_mapping scatter) followed by paged varlen attention
over the flattened batch.  The default workload is the long-context batch (16 decodes at
32768 tokens plus one 4096-token prefill chunk at position 28672; bf16, 64 query / 8 KV
heads, head_dim 128, block size 16, 40000-block pool, values N(0,1) with 1% scaled by 10),
the largest configuration and the one that exercises both the decode and the prefill path.

Prints ONE JSON line.  `value` is the step's attained fraction of the MI355X roofline, in
percent: max(bytes / 8 TB/s, flops / 2.5 PFLOP/s) over the step's algorithmic work, divided
by the measured step time.  The decode and prefill halves of the metric are reported beside
it (decode KV GB/s of the small-tile kernel, prefill TFLOP/s of the prefill kernel), and
`roofline` describes the dominant kernel, timed with HIP events on the launch stream.
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

PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0       # dense bf16 matrix cores
PEAK_F32_TFLOPS = 157.3         # fp32 vector
PREFILL_MIN_COLS = 64           # the library sends requests with more query rows x group heads
                                # than this to the prefill kernel (bf16, head_dim 128)
METRIC = "paged-attn decode KV GB/s + prefill TFLOP/s, % of MI355X peak"
# the sources of each kernel kind (its staging kernels included), plus the ones every kind
# depends on (shared formulas, launch configuration): a committed counter figure is used only
# while all of them are unchanged
KERNEL_SOURCES = {"prefill": ["attn_prefill_mfma.hip", "v16_stage.hip", "fp8_stage.hip"],
                  "small": ["attn_decode_mfma.hip"], "kv_write": ["kv_write.hip"], "merge": ["attn_valu.hip"],
                  "plan": ["plan.hip"]}
COMMON_SOURCES = ["pa_internal.h", "api.cpp"]


def eprint(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_sha(kind: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kind] + COMMON_SOURCES:
        with open(os.path.join(ROOT, "paged_kv_attention_05_amd", "csrc", name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def measured(file: str, field: str, kind: str, workload: str):
    """A per-launch figure from a committed rocprofv3 counter summary (profiles/<file>), if it
    was taken on the current sources of that kernel kind; else None."""
    path = os.path.join(ROOT, "profiles", file)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        data = json.load(f)
    entry = data.get(workload, {}).get(kind)
    if not entry or entry.get("kernel_sha") != kernel_sha(kind):
        return None
    return entry.get(field)


def measured_traffic(kind: str, workload: str):
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, scaled by a plain copy's reading)."""
    return measured("traffic.json", "hbm_bytes_per_launch", kind, workload)


def measured_mfma_busy(kind: str, workload: str):
    """Fraction of cycles the matrix cores are busy during the kind's launches
    (SQ_VALU_MFMA_BUSY_CYCLES over all SIMDs / (GRBM_GUI_ACTIVE per XCD x SIMDs))."""
    return measured("mfma.json", "mfma_busy", kind, workload)


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="long_context",
                    choices=["long_context", "decode_only", "shared_prefix", "spec_verify", "mixed_step_bf16",
                             "mixed_step_f32", "worked_batch", "small_decode", "block_copy"])
    ap.add_argument("--cpu-prefill-rows", type=int, default=256,
                    help="prefill rows in the oracle's timed sample (plus every decode row)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--window", type=int, default=0,
                    help="sliding window in tokens (0: none); the workload is otherwise unchanged")
    ap.add_argument("--graph", action="store_true",
                    help="capture the step once in a HIP graph (launches sized for the batch's max seq_len) "
                         "and time graph replays; per-kernel times still come from eager steps")
    ap.add_argument("--kv-fp8", action="store_true",
                    help="keep the pools as fp8 E4M3 codes with a float32 scale per (slot, KV head): the "
                         "pool is quantized once before the steps, each step writes its tokens through the "
                         "quantizing write and attends over the codes (bf16 batches; every request on the "
                         "small tiles)")
    ap.add_argument("--no-hbm-probe", action="store_true",
                    help="skip the probes of the achievable HBM bandwidth and matrix-core rate")
    ap.add_argument("--no-extras", action="store_true",
                    help="launch only the warm-up and timed steps (no per-step spread, sub-calls or HBM "
                         "probe), so that profiler counters see one set of launches per step")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="before the steps, copy this many MiB device-to-device once: a plain copy "
                         "of known size whose HBM counters scale the kernels' counters")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        eprint(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE {world}): "
               "the library has no multi-GPU path; the step shards by KV head or by request without "
               "any exchange, so per-GPU throughput is the single-GPU figure.")
        return 2

    import numpy as np
    import torch

    import paged_kv_attention_05_amd as pk
    import workloads
    from workloads.accounting import attention_work, write_work

    if not torch.cuda.is_available():
        eprint("bench.py needs a GPU")
        return 1
    pk.load_library()
    dev = torch.device("cuda:0")
    if args.workload == "block_copy":
        return bench_block_copy(args, torch, pk, dev)

    t0 = time.time()
    batch = workloads.CONFIGS[args.workload](poison=False)
    eprint(f"[bench] workload {args.workload}: {batch.description}; generated in {time.time() - t0:.1f}s")

    q, k, v = batch.q.to(dev), batch.k.to(dev), batch.v.to(dev)
    kc, vc = batch.k_cache.to(dev), batch.v_cache.to(dev)
    ks = vs = None
    if args.kv_fp8:
        if batch.dtype != "bf16":
            eprint("--kv-fp8 needs a bf16 workload")
            return 2
        # the whole pool through the quantizing write once (setup, not timed)
        nslots = kc.shape[0] * kc.shape[1]
        codes = [torch.empty(kc.shape, dtype=torch.uint8, device=dev) for _ in range(2)]
        scales = [torch.empty(kc.shape[:3], dtype=torch.float32, device=dev) for _ in range(2)]
        pk.paged_kv_write_fp8(kc.view(nslots, *kc.shape[2:]), vc.view(nslots, *vc.shape[2:]),
                              torch.arange(nslots, dtype=torch.int64, device=dev), *codes, *scales)
        torch.cuda.synchronize()
        kc, vc = codes
        ks, vs = scales
        del codes, scales
        torch.cuda.empty_cache()
    qsl, lens = batch.query_start_loc.to(dev), batch.seq_lens.to(dev)
    table, slots = batch.block_table.to(dev), batch.slot_mapping.to(dev)
    out = torch.empty_like(q)
    ws_bytes = pk.paged_attention_workspace_bytes(batch.num_heads, batch.num_kv_heads, batch.head_dim,
                                                  batch.block_size, batch.query_start_loc_host,
                                                  batch.seq_lens_host, q.dtype, sliding_window=args.window,
                                                  kv_fp8=args.kv_fp8)
    ws = torch.empty(max(ws_bytes, 256), dtype=torch.uint8, device=dev)

    graph_max = batch.max_seq_len if args.graph else 0
    if args.graph:
        ws_bytes = pk.paged_attention_workspace_bytes(batch.num_heads, batch.num_kv_heads, batch.head_dim,
                                                      batch.block_size, batch.query_start_loc_host, None, q.dtype,
                                                      sliding_window=args.window, graph_max_seq_len=graph_max,
                                                      kv_fp8=args.kv_fp8)
        if ws_bytes == 0:
            eprint("--graph needs every request to have at most 64 query columns (decode-like batches)")
            return 2
        ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)

    def step():
        if args.kv_fp8:
            pk.paged_kv_write_fp8(k, v, slots, kc, vc, ks, vs)
        else:
            pk.paged_kv_write(k, v, slots, kc, vc)
        pk.paged_attention_varlen(q, kc, vc, qsl, lens, table, batch.block_size, batch.scale, out,
                                  query_start_loc_host=batch.query_start_loc_host,
                                  seq_lens_host=batch.seq_lens_host, max_query_len=batch.max_query_len,
                                  max_seq_len=batch.max_seq_len, workspace=ws, sliding_window=args.window,
                                  graph_max_seq_len=graph_max, k_scale=ks, v_scale=vs)

    if args.copy_calibration_mib > 0:
        nbytes = args.copy_calibration_mib << 20
        src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        eprint(f"[bench] calibration copy: {nbytes} bytes read, {nbytes} bytes written")
        del src, dst

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # the timed steps, with no instrumentation in the stream
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(args.steps):
        step()
    end.record()
    torch.cuda.synchronize()
    ms_per_step = start.elapsed_time(end) / args.steps
    eager_ms = ms_per_step
    # per-kernel times: the same steps again, each library launch between HIP events on its
    # stream (the events add a little time to these steps, not to the ones above)
    pk.set_timing(True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kern = pk.timing_report()
    pk.set_timing(False)
    if args.graph:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        for _ in range(args.warmup):
            graph.replay()
        torch.cuda.synchronize()
        start.record()
        for _ in range(args.steps):
            graph.replay()
        end.record()
        torch.cuda.synchronize()
        ms_per_step = start.elapsed_time(end) / args.steps
        eprint(f"[bench] graph replays: {ms_per_step:.4f} ms/step (eager {eager_ms:.4f})")
    # per-step spread: the same steps again, each between its own events
    evs = [] if args.no_extras else \
        [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for e0, e1 in evs:
        e0.record()
        if args.graph:
            graph.replay()
        else:
            step()
        e1.record()
    torch.cuda.synchronize()
    per_step = sorted(e0.elapsed_time(e1) for e0, e1 in evs)
    spread = {"median_ms": per_step[len(per_step) // 2], "min_ms": per_step[0], "max_ms": per_step[-1]} \
        if per_step else None
    kern_avg = {name: (tot / cnt if cnt else 0.0) for name, (tot, cnt) in kern.items()}
    eprint(f"[bench] {args.steps} steps: {ms_per_step:.4f} ms/step; kernels (avg ms): "
           + ", ".join(f"{n}={t:.4f}" for n, t in kern_avg.items() if t))

    # algorithmic work, split the way the library routes requests
    g = batch.num_heads // batch.num_kv_heads
    prefill_capable = batch.dtype == "bf16" and batch.block_size == 16 and batch.head_dim == 128 \
        and 256 % g == 0
    is_pf = [prefill_capable and r.new * g > PREFILL_MIN_COLS and r.seq_len > 0 for r in batch.requests]
    if kern["prefill"][1] == 0:          # the library routed every request to the small tiles
        is_pf = [False] * len(is_pf)
    pf_ids = [i for i, f in enumerate(is_pf) if f]
    dec_ids = [i for i, f in enumerate(is_pf) if not f]
    fp8 = args.kv_fp8
    w_all = attention_work(batch, window=args.window, kv_fp8=fp8)
    w_dec = attention_work(batch, dec_ids, window=args.window, kv_fp8=fp8) if dec_ids else None
    w_pf = attention_work(batch, pf_ids, window=args.window, kv_fp8=fp8) if pf_ids else None
    w_write = write_work(batch, kv_fp8=fp8)
    peak_flops = PEAK_BF16_TFLOPS if batch.dtype == "bf16" else PEAK_F32_TFLOPS
    t_star = max((w_all["bytes"] + w_write["bytes"]) / (PEAK_HBM_GBPS * 1e9), w_all["flops"] / (peak_flops * 1e12))
    value = 100.0 * t_star / (ms_per_step * 1e-3)

    decode = None
    if w_dec is not None and kern_avg["small"] > 0:
        t = kern_avg["small"] * 1e-3
        gbps = w_dec["bytes"] / t / 1e9
        decode = {"kernel": ("small_tile_mfma_fp8" if fp8 else "small_tile_mfma") if batch.dtype == "bf16"
                  else "small_tile_valu",
                  "avg_ms": kern_avg["small"], "merge_avg_ms": kern_avg["merge"],
                  "algorithmic_bytes": w_dec["bytes"], "kv_bytes": w_dec["kv_bytes"],
                  "kv_gbps": gbps, "frac_hbm": gbps / PEAK_HBM_GBPS,
                  "kv_gbps_incl_merge": w_dec["bytes"] / ((kern_avg["small"] + kern_avg["merge"]) * 1e-3) / 1e9}
    prefill = None
    if w_pf is not None and kern_avg["prefill"] > 0:
        t = kern_avg["prefill"] * 1e-3
        tf = w_pf["flops"] / t / 1e12
        # (fp8 pools: the staging copy of the prefill requests' blocks and the kernel on it)
        prefill = {"kernel": "stage_fp8 + prefill_tile_mfma_fp8" if fp8 else "prefill_tile_mfma",
                   "avg_ms": kern_avg["prefill"], "algorithmic_flops": w_pf["flops"],
                   "algorithmic_bytes": w_pf["bytes"], "tflops": tf, "frac_mfma": tf / PEAK_BF16_TFLOPS}

    # dominant kernel: the one taking the most time per step
    dom = max(("prefill", "small", "kv_write"), key=lambda n: kern_avg[n])
    if dom == "prefill":
        roof = {"kernel": prefill["kernel"], "bound": "mfma", "achieved": prefill["tflops"],
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": prefill["frac_mfma"],
                "algorithmic_per_launch": w_pf["flops"], "avg_launch_ms": kern_avg["prefill"]}
    elif dom == "small":
        roof = {"kernel": decode["kernel"], "bound": "hbm", "achieved": decode["kv_gbps"], "peak": PEAK_HBM_GBPS,
                "unit": "GB/s", "frac": decode["frac_hbm"], "algorithmic_per_launch": w_dec["bytes"],
                "avg_launch_ms": kern_avg["small"]}
    else:
        gb = w_write["bytes"] / (kern_avg["kv_write"] * 1e-3) / 1e9
        roof = {"kernel": "kv_quant_fp8" if fp8 else "kv_copy16", "bound": "hbm", "achieved": gb, "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                "frac": gb / PEAK_HBM_GBPS, "algorithmic_per_launch": w_write["bytes"],
                "avg_launch_ms": kern_avg["kv_write"]}
    wl_key = args.workload + (f"_window{args.window}" if args.window else "") + ("_fp8" if fp8 else "")
    roof["traffic"] = measured_traffic(dom, wl_key)
    # matrix-core busy fraction of a matrix-core-bound kernel, from its committed counters
    roof["mfma_busy"] = measured_mfma_busy(dom, wl_key) if roof["bound"] == "mfma" else None

    # mixed batches: the decode-row and the prefill-row requests as sub-calls of their own
    # (attention only, over the pool the steps wrote)
    subcalls = None
    if dec_ids and pf_ids and not args.graph and not args.no_extras:
        subcalls = {}
        for name, ids, w_sub in (("decode", dec_ids, w_dec), ("prefill", pf_ids, w_pf)):
            sub = _subset(torch, batch, ids, q, qsl.device)
            o_sub = torch.empty_like(sub["q"])

            def call():
                pk.paged_attention_varlen(sub["q"], kc, vc, sub["qsl"], sub["lens"], sub["table"], batch.block_size,
                                          batch.scale, o_sub, query_start_loc_host=sub["qsl_host"],
                                          seq_lens_host=sub["lens_host"], sliding_window=args.window,
                                          k_scale=ks, v_scale=vs)
            for _ in range(args.warmup):
                call()
            torch.cuda.synchronize()
            start.record()
            for _ in range(args.steps):
                call()
            end.record()
            torch.cuda.synchronize()
            ms = start.elapsed_time(end) / args.steps
            subcalls[name] = {"requests": len(ids), "ms": ms, "algorithmic_bytes": w_sub["bytes"],
                              "algorithmic_flops": w_sub["flops"], "gbps": w_sub["bytes"] / (ms * 1e-3) / 1e9,
                              "tflops": w_sub["flops"] / (ms * 1e-3) / 1e12}

    hbm = None if (args.no_hbm_probe or args.no_extras) else hbm_probe(torch, pk, dev)
    mfma = None if (args.no_hbm_probe or args.no_extras) else mfma_probe(torch, pk, dev)

    cpu = None
    if not args.no_cpu_baseline:
        # the oracle's sample is chosen by request shape: every row of requests whose rows times
        # grouped heads fit 16 columns (decodes), and a spread of rows from the longer chunks
        chunk = [r.new * g > PREFILL_MIN_COLS and r.seq_len > 0 for r in batch.requests]
        cpu = cpu_baseline(batch, args.cpu_prefill_rows, [i for i, f in enumerate(chunk) if not f],
                           [i for i, f in enumerate(chunk) if f], peak_flops, args.window, fp8)

    line = {
        "metric": METRIC, "value": value, "unit": "% of MI355X peak", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": batch.dtype, "data": "synthetic",
        "config": {"workload": batch.name, "description": batch.description, "num_tokens": batch.num_tokens,
                   "num_reqs": batch.num_reqs, "num_heads": batch.num_heads, "num_kv_heads": batch.num_kv_heads,
                   "head_dim": batch.head_dim, "block_size": batch.block_size, "pool_blocks": batch.num_blocks,
                   "sliding_window": args.window, "launch": "hip_graph" if args.graph else "eager",
                   "kv_cache_dtype": "fp8_e4m3" if fp8 else batch.dtype,
                   "parallelism": "single-gpu"},
        "step_roofline_ms": t_star * 1e3,
        "step_algorithmic": {"bytes": w_all["bytes"] + w_write["bytes"], "flops": w_all["flops"]},
        "decode": decode, "prefill": prefill,
        "kv_write": {"avg_ms": kern_avg["kv_write"], "bytes": w_write["bytes"],
                     "gbps": w_write["bytes"] / (kern_avg["kv_write"] * 1e-3) / 1e9 if kern_avg["kv_write"] else None},
        "kernels_avg_ms": kern_avg,
        "eager_ms_per_step": eager_ms,
        "step_spread": spread,
        "subcalls": subcalls,
        "hbm_probe": hbm,
        "mfma_probe": mfma,
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


def bench_block_copy(args, torch, pk, dev):
    """Block copies of preemption and prefix sharing, on the pool of the long-context batch's
    shape (bf16, 8 KV heads x 128, 16-token blocks: 32 KiB per block and tensor): swap one
    32768-token request (2048 blocks of K and of V) out to pinned host memory and back into
    other blocks, and copy-on-write 1024 blocks inside the pool.  Swaps are bound by PCIe,
    copy-on-write by HBM (read + write)."""
    nb, n_swap, n_cow = 40001, 2048, 1024
    gen = torch.Generator().manual_seed(7)
    pools = [torch.randn((nb, 16, 8, 128), generator=gen).to(torch.bfloat16).to(dev) for _ in range(2)]
    perm = torch.randperm(nb - 1, generator=gen)
    out_ids, in_ids = perm[:n_swap].to(dev), perm[n_swap:2 * n_swap].to(dev)
    cow_src, cow_dst = perm[2 * n_swap:2 * n_swap + n_cow].to(dev), perm[2 * n_swap + n_cow:2 * n_swap + 2 * n_cow].to(dev)
    seq = torch.arange(n_swap, dtype=torch.int64, device=dev)
    host = [torch.empty((n_swap, 16, 8, 128), dtype=torch.bfloat16).pin_memory() for _ in range(2)]
    block_bytes = 16 * 8 * 128 * 2

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(args.steps):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) / args.steps

    ms_out = timed(lambda: [pk.paged_copy_blocks(p, h, out_ids, seq) for p, h in zip(pools, host)])
    ms_in = timed(lambda: [pk.paged_copy_blocks(h, p, seq, in_ids) for p, h in zip(pools, host)])
    ms_cow = timed(lambda: [pk.paged_copy_blocks(p, p, cow_src, cow_dst) for p in pools])
    swap_bytes = 2 * n_swap * block_bytes
    cow_bytes = 2 * n_cow * block_bytes * 2                      # read + write
    cow_gbps = cow_bytes / (ms_cow * 1e-3) / 1e9
    line = {"metric": "block copy GB/s (copy-on-write in HBM, swap over PCIe)", "value": cow_gbps, "unit": "GB/s",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_cow, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
            "config": {"workload": "block_copy", "pool_blocks": nb, "block_bytes_per_tensor": block_bytes,
                       "swap_blocks": n_swap, "cow_pairs": n_cow, "tensors": 2, "parallelism": "single-gpu"},
            "copy_on_write": {"ms": ms_cow, "hbm_bytes": cow_bytes, "gbps": cow_gbps},
            "swap_out_to_pinned_host": {"ms": ms_out, "bytes": swap_bytes, "gbps": swap_bytes / (ms_out * 1e-3) / 1e9},
            "swap_in_from_pinned_host": {"ms": ms_in, "bytes": swap_bytes, "gbps": swap_bytes / (ms_in * 1e-3) / 1e9},
            "roofline": {"kernel": "copy_blocks16", "bound": "hbm", "achieved": cow_gbps, "peak": PEAK_HBM_GBPS,
                         "unit": "GB/s", "frac": cow_gbps / PEAK_HBM_GBPS, "traffic": None},
            "cpu_baseline": None}
    print(json.dumps(line), flush=True)
    return 0


def _subset(torch, batch, ids, q, dev):
    """Device tensors of the requests `ids` alone: their rows of q, query_start_loc, seq_lens
    and block-table rows."""
    qh = batch.query_start_loc_host
    rows = torch.cat([torch.arange(qh[r], qh[r + 1]) for r in ids]).to(dev)
    starts = [0]
    for r in ids:
        starts.append(starts[-1] + qh[r + 1] - qh[r])
    lens = [batch.seq_lens_host[r] for r in ids]
    return {"q": q.index_select(0, rows).contiguous(),
            "qsl": torch.tensor(starts, dtype=torch.int32, device=dev),
            "lens": torch.tensor(lens, dtype=torch.int32, device=dev),
            "table": batch.block_table[ids].contiguous().to(dev), "qsl_host": starts, "lens_host": lens}


def hbm_probe(torch, pk, dev, gib=4):
    """Achievable HBM rates beside the 8 TB/s specification: the library's streaming-read
    probe over `gib` GiB (best over a sweep of grid sizes, best of 5 each) and a torch
    device-to-device copy of the same size (read + write)."""
    n = (gib << 30) // 4
    x = torch.ones(n, dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def best(fn):
        fn()
        times = []
        for _ in range(5):
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize()
            times.append(a.elapsed_time(b))
        return min(times)
    nbytes = n * 4
    reads = {grid: nbytes / (best(lambda: pk.hbm_read_probe(x, sink, grid)) * 1e-3) / 1e9
             for grid in (1024, 2048, 4096, 8192)}
    copy_ms = best(lambda: y.copy_(x))
    del x, y
    torch.cuda.empty_cache()
    top = max(reads, key=reads.get)
    return {"bytes": nbytes, "read_gbps": reads[top], "read_grid": top,
            "read_gbps_by_grid": {str(k): v for k, v in reads.items()},
            "copy_gbps_read_plus_write": 2 * nbytes / (copy_ms * 1e-3) / 1e9,
            "how": "paged_hbm_read_probe (nontemporal 16-byte loads, 256 threads per workgroup) over 4 GiB, "
                   "and torch copy_ of 4 GiB; best of 5"}


def mfma_probe(torch, pk, dev, iters=4096):
    """Matrix-core rate the chip sustains beside the 2.5 PFLOP/s specification: the library's
    probe of back-to-back bf16 32x32x16 products with no memory traffic (best over two grid
    sizes, best of 5 each), on small-integer operands and on random ones like attention's
    (the chip clocks down under the latter)."""
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    out = {}
    for label, rnd in (("integer_operands", False), ("random_operands", True)):
        rates = {}
        for grid in (1024, 2048):
            flops = pk.mfma_probe(iters, grid, sink, random_operands=rnd)
            times = []
            for _ in range(5):
                a.record()
                pk.mfma_probe(iters, grid, sink, random_operands=rnd)
                b.record()
                torch.cuda.synchronize()
                times.append(a.elapsed_time(b))
            rates[grid] = flops / (min(times) * 1e-3) / 1e12
        top = max(rates, key=rates.get)
        out[label] = {"tflops": rates[top], "grid": top, "tflops_by_grid": {str(k): v for k, v in rates.items()}}
    out["tflops"] = out["integer_operands"]["tflops"]
    out["how"] = (f"paged_mfma_probe: 512-thread workgroups, {iters} rounds of 8 independent 32x32x16 bf16 "
                  "products per wave, no memory traffic, operands small integers or random bf16; best of 5")
    return out


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(batch, n_prefill_rows, dec_ids, pf_ids, peak_flops, window=0, kv_fp8=False):
    """The oracle (float64 C, OpenMP) timed on the host on a bounded sample of the same step:
    the full KV write, then attention for every decode row and `n_prefill_rows` prefill rows
    spread evenly over the chunk.  Reported in the metric's unit (the sample's roofline time
    at MI355X peak over the oracle's time), with the raw rates beside it.  kv_fp8: the pool
    is quantized by the oracle's write before the clock starts; the timed write quantizes."""
    import numpy as np
    import torch

    import oracle
    from tests._util import to_np

    mask = np.zeros(batch.num_tokens, np.uint8)
    flops = 0.0
    touched = set()
    qsl = batch.query_start_loc_host
    if kv_fp8 and len(dec_ids) > 64:          # the oracle's fp8 gather is slower: 64 decodes, evenly spaced
        dec_ids = [dec_ids[i] for i in np.linspace(0, len(dec_ids) - 1, 64).round().astype(int)]
    for r in dec_ids:
        mask[qsl[r]:qsl[r + 1]] = 1
    pf_rows = [i for r in pf_ids for i in range(qsl[r], qsl[r + 1])]
    if pf_rows and n_prefill_rows > 0:
        pick = np.linspace(0, len(pf_rows) - 1, min(n_prefill_rows, len(pf_rows))).round().astype(int)
        mask[np.array(pf_rows)[pick]] = 1
    for r, req in enumerate(batch.requests):
        rows = np.nonzero(mask[qsl[r]:qsl[r + 1]])[0]
        if len(rows):
            touched.add(r)
            seen = req.computed + rows + 1
            if window > 0:
                seen = np.minimum(seen, window)
            flops += 4.0 * batch.num_heads * batch.head_dim * float(np.sum(seen))
    from workloads.accounting import attention_work
    kv = attention_work(batch, sorted(touched), window=window, kv_fp8=kv_fp8)["kv_bytes"] if touched else 0.0
    nbytes = kv + int(mask.sum()) * batch.num_heads * batch.head_dim * 2 * (2 if batch.dtype == "bf16" else 4)
    q, k, v = to_np(batch.q), to_np(batch.k), to_np(batch.v)
    cores = int(os.environ.get("OMP_NUM_THREADS") or len(os.sched_getaffinity(0)))
    if kv_fp8:
        # quantize the context slots the sampled requests read (the step's write adds the rest)
        shape = tuple(batch.k_cache.shape)
        bs = batch.block_size
        ctx = np.unique(np.concatenate([np.asarray(batch.requests[r].blocks, np.int64)[np.arange(
            batch.requests[r].computed) // bs] * bs + np.arange(batch.requests[r].computed) % bs
            for r in sorted(touched)] + [np.zeros(0, np.int64)]))
        kc, vc = np.zeros(shape, np.uint8), np.zeros(shape, np.uint8)
        ks, vs = np.zeros(shape[:3], np.float32), np.zeros(shape[:3], np.float32)
        flat = lambda t: to_np(t.reshape(-1, *shape[2:])[torch.from_numpy(ctx)])
        oracle.kv_write_fp8(flat(batch.k_cache), flat(batch.v_cache), ctx, kc, vc, ks, vs, batch.dtype)
    else:
        kc, vc = to_np(batch.k_cache).copy(), to_np(batch.v_cache).copy()
        ks = vs = None
    t0 = time.perf_counter()
    if kv_fp8:
        oracle.kv_write_fp8(k, v, batch.slot_mapping.numpy(), kc, vc, ks, vs, batch.dtype)
    else:
        oracle.kv_write(k, v, batch.slot_mapping.numpy(), kc, vc, batch.dtype, batch.dtype)
    oracle.paged_attention(q, kc, vc, batch.query_start_loc.numpy(), batch.seq_lens.numpy(),
                           batch.block_table.numpy(), batch.scale, batch.dtype, row_mask=mask, window=window,
                           k_scale=ks, v_scale=vs)
    secs = time.perf_counter() - t0
    t_star = max(nbytes / (PEAK_HBM_GBPS * 1e9), flops / (peak_flops * 1e12))
    eprint(f"[bench] oracle sample: {int(mask.sum())} rows in {secs:.2f}s on {cores} threads")
    return {"value": 100.0 * t_star / secs, "unit": "% of MI355X peak", "cores": cores, "kind": "oracle",
            "cpu_model": _cpu_model(),
            "seconds": secs, "flops_per_s": flops / secs, "kv_bytes_per_s": kv / secs,
            "sample": f"KV write of all {batch.num_tokens} tokens + attention of {int(mask.sum())} of "
                      f"{batch.num_tokens} rows ({len(dec_ids)} decode requests, {min(n_prefill_rows, len(pf_rows))} prefill "
                      f"rows evenly spaced), {batch.name}" + (" on fp8 E4M3 pools" if kv_fp8 else "")}


if __name__ == "__main__":
    sys.exit(main())
