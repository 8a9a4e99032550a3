#!/usr/bin/env python3
"""Hybrid-block decode benchmark of libhysparse on one MI355X.

A step is one pass of the whole hot path over one batch: the full-attention
layer with token selection (hs_full_attn_select) followed by the block's sparse
layers (hs_sparse_attn, each with its own queries, reusing the cache and the
indices).  Default workload: 32 sequences x 131072 cached rows, bf16 MQA cache,
32 query heads, 1 full + 5 sparse layers (the 128K decode configuration).

Prints ONE JSON line on stdout; progress goes to stderr.
  value        queries/s = B * n_q / median step time (HIP events, inputs resident in HBM)
  roofline     the dominant kernel's algorithmic bytes / its average launch time,
               measured with HIP events on the library's stream over a timed region
  cpu_baseline the float64 CPU oracle timed on this host on a bounded sample
"""

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "hybrid-block decode queries/s + achieved HBM GB/s at 128K–1M ctx, 1 GPU"

# HBM bytes per launch of the dense split-K pass at the default workload, from two
# rocprofv3 --pmc runs (FETCH_SIZE x 2.0 + WRITE_SIZE x 1.0, the factors read off a
# plain 1 GiB copy), keyed by a digest of the kernel sources they were taken on.
KNOWN_TRAFFIC = {"aafa7c0aec7a7cdf": 2305907712}
KERNEL_SOURCES = ["long_context_split_amd/csrc/hs_wave.hip", "long_context_split_amd/csrc/hs_mfma.hpp",
                  "long_context_split_amd/csrc/hs_common.hpp", "long_context_split_amd/csrc/hs_internal.hpp"]


def kernel_digest():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    return h.hexdigest()[:16]
HBM_PEAK_GBPS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=2, choices=[2, 3, 5],
                    help="2: 32 x 128K bf16 (default); 3: 1 x 1M FP8 E4M3, 64 heads, 4 query tokens; "
                         "5: ragged 8 x 64K-512K, 4 blocks")
    ap.add_argument("--L", type=int, default=None, help="context length override (sweeps)")
    ap.add_argument("--B", type=int, default=None, help="batch override (sweeps)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="CPU oracle time budget")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--flush", choices=["read", "write", "none"], default="read",
                    help="evict the 256 MB Infinity Cache between steps by reading (default) or writing 1 GiB")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of a HIP-graph replay")
    ap.add_argument("--no-bridge", action="store_true", help="skip the KV Bridging measurement")
    ap.add_argument("--no-swa", action="store_true", help="skip the sliding-window attention measurement")
    ap.add_argument("--swa-window", type=int, default=128, help="window of the sliding-window measurement")
    ap.add_argument("--select-block", type=int, default=0, choices=[0, 64],
                    help="64: the block-level selection variant (whole 64-token blocks)")
    ap.add_argument("--bridge-iters", type=int, default=10)
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a 1 GiB device-to-device copy (known bytes, for scaling HBM counters)")
    ap.add_argument("--no-probe", action="store_true", help="skip the streaming read probe (measured peak)")
    ap.add_argument("--probe-sizes", action="store_true",
                    help="also probe repeated reads of 16 MB .. 2 GiB buffers (the Infinity Cache's range)")
    ap.add_argument("--no-append-step", action="store_true",
                    help="skip the decode step timed with the KV append through the bridge ahead of it")
    ap.add_argument("--no-prefill", action="store_true", help="skip the chunked prefill measurement")
    return ap.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}, WORLD_SIZE {world}); the library has no "
              "multi-GPU mode (independent sequences would shard as pure data parallelism with no exchange)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    import synth
    from long_context_split_amd import hysparse as hs

    torch.cuda.init()
    dev = torch.device("cuda:0")
    spec = dict(synth.CONFIGS[args.config])
    n_blocks = spec.get("n_blocks", 1)
    top_k, window = synth.TOP_K, synth.WINDOW

    # ---------------------------------------------------------------- inputs (seeded, synthetic)
    t0 = time.time()
    blocks = []
    for blk in range(n_blocks):
        case = synth.decode_case(args.config, L=args.L, B=args.B, block=blk)
        if spec["kv"] == "bf16":
            k = torch.from_numpy(case["k"].view(np.int16)).to(dev).view(torch.bfloat16)
            v = torch.from_numpy(case["v"].view(np.int16)).to(dev).view(torch.bfloat16)
            kv = hs.KVCache(k, v, case["lengths"], case["row_start"])
        else:
            kv = fp8_cache(case, dev)
        qf = torch.from_numpy(case["q_full"].view(np.int16)).to(dev).view(torch.bfloat16)
        qs = [torch.from_numpy(q.view(np.int16)).to(dev).view(torch.bfloat16) for q in case["q_sparse"]]
        blocks.append(dict(case=case, kv=kv, qf=qf, qs=qs))
        log(f"block {blk}: generated and uploaded B={len(case['lengths'])} "
            f"L={int(case['lengths'].min())}..{int(case['lengths'].max())} ({time.time() - t0:.1f}s)")
    lens = blocks[0]["case"]["lengths"]
    B = len(lens)
    n_q, H = spec["n_q"], spec["H"]
    n_sparse = spec["n_sparse"]

    # outputs and workspaces, allocated once
    for bl in blocks:
        kv = bl["kv"]
        p = hs.params(H, n_q, top_k, window, select_block=args.select_block)
        bl["out"] = torch.empty((B, n_q, H, 128), dtype=torch.float32, device=dev)
        bl["lse"] = torch.empty((B, n_q, H), dtype=torch.float32, device=dev)
        bl["idx"] = torch.empty((B, n_q, 1, top_k + window), dtype=torch.int32, device=dev)
        bl["cnt"] = torch.empty((B, n_q, 1), dtype=torch.int32, device=dev)
        bl["ws_full"] = hs.workspace(hs.full_attn_select_workspace_size(kv, p), dev)
        bl["ws_sp"] = hs.workspace(hs.sparse_attn_workspace_size(kv, p), dev)
        bl["so"] = [torch.empty((B, n_q, H, 128), dtype=torch.float32, device=dev) for _ in range(n_sparse)]

    def step():
        for bl in blocks:
            kv = bl["kv"]
            hs.full_attn_select(kv, bl["qf"], top_k, window, out=bl["out"], lse=bl["lse"], sel_idx=bl["idx"],
                                sel_count=bl["cnt"], ws=bl["ws_full"], select_block=args.select_block)
            for i in range(n_sparse):
                hs.sparse_attn(kv, bl["qs"][i], bl["idx"], bl["cnt"], top_k, window, out=bl["so"][i],
                               ws=bl["ws_sp"])

    flush_buf = None if args.flush == "none" else torch.ones((1 << 30) // 4, dtype=torch.float32, device=dev)
    flush_sink = torch.empty((), dtype=torch.float32, device=dev)

    def flush(i):
        # evict the 256 MB Infinity Cache between steps (outside the step's events); reading 1 GiB
        # leaves clean lines, writing leaves dirty ones that drain during the next step
        if flush_buf is None:
            return
        if args.flush == "read":
            torch.sum(flush_buf, dim=(0,), out=flush_sink)
        else:
            flush_buf.fill_(float(i & 0xFF))

    # ---------------------------------------------------------------- warmup
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"warmup {args.warmup} steps done")
    graph = None
    if not args.eager:
        side = torch.cuda.Stream()
        with torch.cuda.stream(side):
            step()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        graph.replay()
        torch.cuda.synchronize()
        log("step captured in a HIP graph")

    # ---------------------------------------------------------------- timed region: step time
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    wall0 = time.time()
    for i in range(args.steps):
        flush(i)
        ev[i][0].record()
        if graph is not None:
            graph.replay()
        else:
            step()
        ev[i][1].record()
    torch.cuda.synchronize()
    wall = time.time() - wall0
    times = sorted(a.elapsed_time(b) for a, b in ev)
    ms = statistics.median(times)
    p10 = times[int(0.1 * (len(times) - 1))]
    p90 = times[int(0.9 * (len(times) - 1))]
    log(f"timed {args.steps} steps: median {ms:.4f} ms (p10 {p10:.4f}, p90 {p90:.4f}), wall {wall:.2f}s")

    # ---------------------------------------------------------------- timed region: per-kernel events
    hs.timing_enable(True)
    hs.timing_collect()
    torch.cuda.synchronize()
    for i in range(args.steps):
        flush(i)
        step()
    torch.cuda.synchronize()
    recs = hs.timing_collect()
    hs.timing_enable(False)
    per = {}
    for name, t in recs:
        per.setdefault(name, []).append(t)
    kern = {n: dict(launches=len(v), avg_ms=sum(v) / len(v), total_ms_per_step=sum(v) / args.steps)
            for n, v in per.items()}
    for n, d in sorted(kern.items(), key=lambda x: -x[1]["total_ms_per_step"]):
        log(f"kernel {n:22s} launches/step {d['launches'] / args.steps:4.1f} avg {d['avg_ms'] * 1e3:9.2f} us "
            f"per step {d['total_ms_per_step'] * 1e3:9.2f} us")

    # ---------------------------------------------------------------- algorithmic bytes
    fp8 = spec["kv"] == "e4m3"
    row_bytes = 2 * 128 + 8 if fp8 else 2 * 128 * 2             # K + V row (+ two fp32 scales for E4M3)
    sum_L = int(sum(int(x) for x in lens))
    union_rows = 0
    for bl in blocks:
        cnt = bl["cnt"].cpu().numpy()
        union_rows += int(cnt.max(axis=1).sum()) if n_q == 1 else int(cnt.sum())
    q_bytes = n_blocks * (1 + n_sparse) * B * n_q * H * 128 * 2
    o_bytes = n_blocks * (1 + n_sparse) * B * n_q * H * 128 * 4
    idx_bytes = n_blocks * (1 + n_sparse) * B * n_q * (top_k + window) * 4
    alg_bytes = n_blocks * sum_L * row_bytes + n_sparse * union_rows * row_bytes + q_bytes + o_bytes + idx_bytes
    eff_gbps = alg_bytes / (ms * 1e-3) / 1e9
    queries = B * n_q
    qps = queries / (ms * 1e-3)

    dom = max(kern.items(), key=lambda x: x[1]["total_ms_per_step"])[0] if kern else None
    k1_name = next((n for n in ("attn_wave_dense", "attn_rows_dense", "attn_partial_dense") if n in kern), None)
    k1 = kern.get(k1_name)
    k1_bytes = sum_L * row_bytes                                 # per launch (one block's full layer)
    # dense MFMA work of the pass: S = Q K^T and O = P V over every row, 2 * 2 * rows * L * d
    k1_flops = 4.0 * n_q * H * 128 * sum_L
    roof = None
    if k1:
        sec = k1["avg_ms"] * 1e-3
        default_workload = args.config == 2 and args.L is None and args.B is None and not args.select_block
        traffic = KNOWN_TRAFFIC.get(kernel_digest()) if default_workload else None
        t_hbm, t_mfma = k1_bytes / (HBM_PEAK_GBPS * 1e9), k1_flops / (MFMA_BF16_PEAK_TFLOPS * 1e12)
        if t_hbm >= t_mfma:
            ach = k1_bytes / sec / 1e9
            roof = {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": round(ach / HBM_PEAK_GBPS, 4)}
        else:
            ach = k1_flops / sec / 1e12
            roof = {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4),
                    "hbm_GBps": round(k1_bytes / sec / 1e9, 1)}
        roof.update({"traffic": traffic, "kernel": k1_name, "algorithmic_bytes_per_launch": k1_bytes,
                     "algorithmic_flops_per_launch": k1_flops, "avg_launch_us": round(k1["avg_ms"] * 1e3, 2),
                     "dominant_kernel_by_time": dom})

    # ---------------------------------------------------------------- measured streaming peak
    probe = None if args.no_probe else bench_probe(dev, args.probe_sizes)
    if probe and roof and roof["unit"] == "GB/s":
        roof["frac_of_measured_peak"] = round(roof["achieved"] / probe["peak_GBps"], 4)

    # ---------------------------------------------------------------- decode step with the KV append
    append_step = None
    if not args.no_append_step and spec["kv"] == "bf16" and n_q == 1 and n_blocks == 1 and not args.select_block:
        append_step = bench_append_step(dev, blocks[0], step, flush, graph is not None, args.steps, H, n_q)

    # ---------------------------------------------------------------- KV Bridging (prefill side)
    bridge = None if args.no_bridge else bench_bridge(dev, args.bridge_iters)
    prefill = None if args.no_prefill else bench_prefill(dev, args.bridge_iters)
    swa = None if args.no_swa else bench_swa(dev, args.bridge_iters, args.swa_window)
    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        log("calibration: 3 x 1 GiB device copies done")

    # ---------------------------------------------------------------- CPU oracle baseline
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(blocks[0]["case"], spec, top_k, window, args.cpu_seconds)

    line = {
        "metric": METRIC,
        "value": round(qps, 2),
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": (spec["name"] if args.L is None and args.B is None else
                         f"{spec['name']}_L{args.L or 'cfg'}_B{args.B or 'cfg'}") +
                        (f"_block{args.select_block}" if args.select_block else "") +
                        "".join(f"_{k.lower()}{v}" for k, v in sorted(os.environ.items()) if k.startswith("HS_")),
            "batch": B, "seq_len": int(lens.max()) if args.config == 2 else [int(x) for x in lens],
            "query_heads": H, "kv_heads": 1, "head_dim": 128, "q_tokens": n_q, "top_k": top_k, "window": window,
            "sparse_layers": n_sparse, "blocks": n_blocks, "kv_dtype": spec["kv"],
        },
        "achieved_hbm_GBps": round(eff_gbps, 1),
        "hbm_frac": round(eff_gbps / HBM_PEAK_GBPS, 4),
        "hbm_frac_of_measured_peak": round(eff_gbps / probe["peak_GBps"], 4) if probe else None,
        "algorithmic_bytes_per_step": alg_bytes,
        "ms_p10": round(p10, 5), "ms_p90": round(p90, 5),
        "kernels": {n: {"launches_per_step": d["launches"] / args.steps, "avg_us": round(d["avg_ms"] * 1e3, 2)}
                    for n, d in kern.items()},
        "roofline": roof,
        "cpu_baseline": cpu,
        "stream_probe": probe,
        "decode_step_with_append": append_step,
        "bridge": bridge,
        "swa": swa,
        "prefill": prefill,
        "timing": ("HIP-graph replay of the step" if graph is not None else "eager launches") +
                  "; HIP events per step" + ("" if args.flush == "none" else
                                             f"; Infinity Cache flushed between steps by a 1 GiB {args.flush}") +
                  "; kernel durations from per-launch HIP events on the library stream in a second (eager) region",
    }
    print(json.dumps(line), flush=True)


def bench_probe(dev, sizes=False):
    """The practical read ceiling: a 2 GiB buffer read with 16-byte non-temporal loads (the load the
    dense pass uses) at 256, 512 and 1024 workgroups of 512 threads, best of each over 10 reads with
    the Infinity Cache evicted in between (the buffer is 8x its size); with sizes, also repeated
    back-to-back reads of 16 MB .. 2 GiB buffers (below 256 MB they can be served by the cache)."""
    import torch
    from long_context_split_amd import hysparse as hs
    nbytes = 2 << 30
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
    sink = torch.zeros(4, dtype=torch.int32, device=dev)
    res = {}
    for nt in (True, False):
        for grid in (256, 512, 1024):
            hs.read_probe(buf, nbytes, nt, grid, sink)
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(10)]
            for a, b in evs:
                a.record()
                hs.read_probe(buf, nbytes, nt, grid, sink)
                b.record()
            torch.cuda.synchronize()
            best = min(a.elapsed_time(b) for a, b in evs)
            res[f"{'nt' if nt else 'plain'}_grid{grid}"] = round(nbytes / (best * 1e-3) / 1e9, 1)
    peak = max(v for k, v in res.items() if k.startswith("nt_"))
    out = {"what": "2 GiB streaming read, 16-byte loads, best of 10 per launch shape", "GBps": res,
           "peak_GBps": peak, "frac_of_published": round(peak / HBM_PEAK_GBPS, 4)}
    log(f"stream probe: {peak:.0f} GB/s ({peak / HBM_PEAK_GBPS:.3f} of 8 TB/s); {res}")
    if sizes:
        sweep = {}
        for mb in (16, 64, 128, 192, 256, 512, 2048):
            nb = mb << 20
            for _ in range(3):
                hs.read_probe(buf, nb, True, 256, sink)
            reps = 50 if mb < 512 else 10
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            for _ in range(reps):
                hs.read_probe(buf, nb, True, 256, sink)
            b.record()
            torch.cuda.synchronize()
            sweep[f"{mb}MB"] = round(nb * reps / (a.elapsed_time(b) * 1e-3) / 1e9, 1)
        out["repeated_reads_GBps"] = sweep
        log(f"repeated reads by buffer size: {sweep}")
    del buf
    return out


def bench_append_step(dev, bl, step, flush, use_graph, steps, H, n_q):
    """The decode step with its KV append ahead of it: each sequence's newest token (the last of its
    L_b rows) is projected from a Self-Decoder hidden state [B, 4096] into four target caches (the
    block's own bf16 cache and three others) by hs_kv_append, then the full layer and the sparse
    layers run on the grown cache; timed like the main step."""
    import ctypes
    import numpy as np
    import torch
    import synth
    from long_context_split_amd import hysparse as hs
    kv = bl["kv"]
    B = kv.batch
    D, nt = 4096, 4
    case = synth.bridge_case(4, T=B, D=D, n_targets=nt)
    x = torch.from_numpy(case["x"].view(np.int16)).to(dev).view(torch.bfloat16)
    wk = [torch.from_numpy(w.view(np.int16)).to(dev).view(torch.bfloat16) for w in case["w_k"]]
    wv = [torch.from_numpy(w.view(np.int16)).to(dev).view(torch.bfloat16) for w in case["w_v"]]
    others = [hs.KVCache(torch.empty_like(kv.k), torch.empty_like(kv.v)) for _ in range(nt - 1)]
    targets = [hs.KVCache(kv.k, kv.v)] + others
    h_rows = np.ascontiguousarray(kv.h_start + kv.h_seq.astype(np.int64) - 1)
    d_rows = torch.from_numpy(h_rows).to(dev)
    aws = hs.workspace(hs.kv_append_workspace_size(B, D, nt), dev)
    wkp = (ctypes.c_void_p * nt)(*[w.data_ptr() for w in wk])
    wvp = (ctypes.c_void_p * nt)(*[w.data_ptr() for w in wv])
    tgp = (ctypes.POINTER(hs.hs_kv_cache) * nt)(*[ctypes.pointer(t._c) for t in targets])
    hrp = h_rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))

    def full_step():
        hs.check(hs.lib.hs_kv_append(x.data_ptr(), B, D, nt, wkp, wvp, tgp, d_rows.data_ptr(), hrp, aws.data_ptr(),
                                     aws.numel(), torch.cuda.current_stream().cuda_stream))
        step()

    for _ in range(3):
        full_step()
    torch.cuda.synchronize()
    graph = None
    if use_graph:
        side = torch.cuda.Stream()
        with torch.cuda.stream(side):
            full_step()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            full_step()
        graph.replay()
        torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    for i in range(steps):
        flush(i)
        evs[i][0].record()
        if graph is not None:
            graph.replay()
        else:
            full_step()
        evs[i][1].record()
    torch.cuda.synchronize()
    ms = statistics.median(a.elapsed_time(b) for a, b in evs)
    hs.timing_enable(True)
    hs.timing_collect()
    for i in range(steps):
        flush(i)
        full_step()
    torch.cuda.synchronize()
    recs = hs.timing_collect()
    hs.timing_enable(False)
    app = [t for n, t in recs if n == "kv_append"]
    app_us = 1e3 * sum(app) / max(1, len(app))
    log(f"decode step with the KV append ahead: {ms * 1e3:.1f} us ({B * n_q / (ms * 1e-3):.0f} queries/s); "
        f"append {app_us:.1f} us")
    return {"workload": f"{B} new tokens x {D} -> {nt} targets (K,V) bf16 at each sequence's newest row, then "
                        "the full layer + sparse layers on the grown cache",
            "ms_per_step": round(ms, 5), "queries_per_s": round(B * n_q / (ms * 1e-3), 2),
            "append_us": round(app_us, 2),
            "append_bytes": nt * 2 * D * 128 * 2 + B * D * 2 + nt * 2 * B * 128 * 2}


def bench_prefill(dev, iters):
    """A 32768-token prompt prefilled in 4 chunks of 8192 (hs_prefill_chunk): per chunk, sliding-window
    attention (H = 32 on one bf16 KV head, window 128, bf16 output) over the growing Self-Decoder cache, then KV
    Bridging of its hidden states [8192, 4096] into 4 FP8 targets at rows 262144 + 8192 c."""
    import torch
    from long_context_split_amd import hysparse as hs
    T, nch, H, w, D, nt, cap, off = 8192, 4, 32, 128, 4096, 4, 1 << 20, 262144
    P = T * nch
    g = torch.Generator(device=dev)
    g.manual_seed(4321)
    k = torch.randn((P, 1, 128), generator=g, device=dev).to(torch.bfloat16)
    v = torch.randn((P, 1, 128), generator=g, device=dev).to(torch.bfloat16)
    q = torch.randn((nch, T, H, 128), generator=g, device=dev).to(torch.bfloat16)
    x = torch.randn((P, D), generator=g, device=dev).to(torch.bfloat16)
    sd = (2.0 / (D + 128)) ** 0.5
    wk = [(torch.randn((D, 128), generator=g, device=dev) * sd).to(torch.bfloat16) for _ in range(nt)]
    wv = [(torch.randn((D, 128), generator=g, device=dev) * sd).to(torch.bfloat16) for _ in range(nt)]
    tg = [hs.KVCache(torch.empty((cap, 1, 128), dtype=torch.uint8, device=dev),
                     torch.empty((cap, 1, 128), dtype=torch.uint8, device=dev), None, None,
                     torch.empty((cap, 1), dtype=torch.float32, device=dev),
                     torch.empty((cap, 1), dtype=torch.float32, device=dev)) for _ in range(nt)]
    caches = [hs.KVCache(k, v, [T * (c + 1)], [0]) for c in range(nch)]
    outs = [torch.empty((1, T, H, 128), dtype=torch.bfloat16, device=dev) for _ in range(nch)]   # bf16 attention output

    def prompt():
        for c in range(nch):
            hs.prefill_chunk(caches[c], q[c:c + 1], w, x[c * T:(c + 1) * T], wk, wv, tg, off + c * T, swa_out=outs[c])

    prompt()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for a, b in evs:
        a.record()
        prompt()
        b.record()
    torch.cuda.synchronize()
    ms = statistics.median(a.elapsed_time(b) for a, b in evs)
    flops = 2.0 * P * D * nt * 2 * 128 + 4.0 * sum(min(t + 1, w) for t in range(P)) * H * 128
    log(f"prefill {nch} x {T} tokens: {ms * 1e3:.1f} us ({P / (ms * 1e-3):.0f} tokens/s)")
    return {"workload": f"{P}-token prompt in {nch} chunks of {T}: sliding-window attention (H={H}, w={w}, bf16 "
                        f"cache, bf16 output) + KV Bridging [{T}, {D}] -> {nt} FP8 targets per chunk",
            "ms": round(ms, 4), "tokens_per_s": round(P / (ms * 1e-3), 1), "flops": flops,
            "tflops": round(flops / (ms * 1e-3) / 1e12, 1)}


def fp8_cache(case, dev):
    """An E4M3 cache (codes + per-row scales) of the case's float32 K and V rows, quantised on the GPU
    by the library's own KV Bridging with identity projections (K = X I exactly, then the per-row
    E4M3 quantiser); X is the bf16 rounding of the float32 rows."""
    import numpy as np
    import torch
    from long_context_split_amd import hysparse as hs
    n = case["k"].shape[0]
    eye = torch.eye(128, dtype=torch.bfloat16, device=dev)
    codes = [torch.empty((n, 1, 128), dtype=torch.uint8, device=dev) for _ in range(3)]
    scales = [torch.empty((n, 1), dtype=torch.float32, device=dev) for _ in range(3)]
    # target 0 receives K's codes (and a discarded copy as V); target 1 receives V's codes
    t_k = hs.KVCache(codes[0], codes[2], None, None, scales[0], scales[2])
    t_v = hs.KVCache(codes[2], codes[1], None, None, scales[2], scales[1])
    for src, tgt in ((case["k"], t_k), (case["v"], t_v)):
        x = torch.from_numpy(np.ascontiguousarray(src.reshape(n, 128))).to(dev).to(torch.bfloat16)
        hs.kv_bridge(x, [eye], [eye], [tgt], 0)
        torch.cuda.synchronize()
        del x
    del codes[2], scales[2]
    return hs.KVCache(codes[0], codes[1], case["lengths"], case["row_start"], scales[0], scales[1])


def bench_bridge(dev, iters):
    """KV Bridging of a 32768-token chunk: X [32768, 4096] bf16 x 4 targets x (W_k, W_v) [4096, 128],
    stored as FP8 E4M3 + per-token scale into 1M-row caches at row 262144."""
    import numpy as np
    import torch
    import synth
    from long_context_split_amd import hysparse as hs
    case = synth.bridge_case(4)
    spec = case["spec"]
    T, D, nt = case["T"], case["D"], case["n_targets"]
    x = torch.from_numpy(case["x"].view(np.int16)).to(dev).view(torch.bfloat16)
    wk = [torch.from_numpy(w.view(np.int16)).to(dev).view(torch.bfloat16) for w in case["w_k"]]
    wv = [torch.from_numpy(w.view(np.int16)).to(dev).view(torch.bfloat16) for w in case["w_v"]]
    cap = spec["capacity"]
    tg = [hs.KVCache(torch.empty((cap, 1, 128), dtype=torch.uint8, device=dev),
                     torch.empty((cap, 1, 128), dtype=torch.uint8, device=dev), None, None,
                     torch.empty((cap, 1), dtype=torch.float32, device=dev),
                     torch.empty((cap, 1), dtype=torch.float32, device=dev)) for _ in range(nt)]
    for _ in range(2):
        hs.kv_bridge(x, wk, wv, tg, spec["offset"])
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for a, b in evs:
        a.record()
        hs.kv_bridge(x, wk, wv, tg, spec["offset"])
        b.record()
    torch.cuda.synchronize()
    ms = statistics.median(a.elapsed_time(b) for a, b in evs)
    flops = 2.0 * T * D * nt * 2 * 128
    tflops = flops / (ms * 1e-3) / 1e12
    out_bytes = nt * 2 * T * (128 + 4)
    in_bytes = T * D * 2 + nt * 2 * D * 128 * 2
    log(f"bridge: {ms * 1e3:.1f} us  {tflops:.1f} TFLOP/s  ({tflops / 2500.0:.3f} of bf16 MFMA peak)")
    # context, not the product path: the same product as one plain library GEMM (torch.matmul, i.e.
    # hipBLASLt) with a bf16 output and no storage epilogue, with the weights in the layout the bridge
    # takes ([d_model, columns]) and pre-transposed ([columns, d_model])
    wcat = torch.cat([w for pair in zip(wk, wv) for w in pair], dim=1).contiguous()      # [D, nt * 2 * 128]
    wcat_t = wcat.t().contiguous()
    lib = {}
    for name, f in (("w_dm_major", lambda: torch.matmul(x, wcat)), ("w_col_major", lambda: torch.matmul(x, wcat_t.t()))):
        for _ in range(2):
            f()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
        for a, b in evs:
            a.record()
            f()
            b.record()
        torch.cuda.synchronize()
        lms = statistics.median(a.elapsed_time(b) for a, b in evs)
        lib[name] = {"us": round(lms * 1e3, 1), "tflops": round(flops / (lms * 1e-3) / 1e12, 1)}
    del wcat, wcat_t
    log(f"library GEMM (torch.matmul, bf16 out, no epilogue): {lib}")
    # decode-time append: one new token per sequence of a 32-sequence batch, same weights and targets,
    # each token to its own cache row
    nb = 32
    rows = torch.arange(nb, dtype=torch.int64) * 32768 + 1000
    xa = x[:nb].contiguous()
    for _ in range(3):
        hs.kv_append(xa, wk, wv, tg, rows)
    torch.cuda.synchronize()
    h_rows = rows.numpy()
    import ctypes
    d_rows = rows.to(dev)
    wkp = (ctypes.c_void_p * nt)(*[w.data_ptr() for w in wk])
    wvp = (ctypes.c_void_p * nt)(*[w.data_ptr() for w in wv])
    tgp = (ctypes.POINTER(hs.hs_kv_cache) * nt)(*[ctypes.pointer(t._c) for t in tg])
    hrp = h_rows.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    stream = torch.cuda.current_stream().cuda_stream
    aws = hs.workspace(hs.kv_append_workspace_size(nb, D, nt), dev)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
    for a, b in evs:
        a.record()
        hs.check(hs.lib.hs_kv_append(xa.data_ptr(), nb, D, nt, wkp, wvp, tgp, d_rows.data_ptr(), hrp,
                                     aws.data_ptr(), aws.numel(), stream))
        b.record()
    torch.cuda.synchronize()
    ms_app = statistics.median(a.elapsed_time(b) for a, b in evs)
    app_bytes = nt * 2 * D * 128 * 2 + nb * D * 2 + nt * 2 * nb * (128 + 4)
    log(f"kv append ({nb} tokens): {ms_app * 1e3:.1f} us  {app_bytes / (ms_app * 1e-3) / 1e9:.0f} GB/s")
    return {"workload": "c4_bridge_32k: X[32768,4096] bf16 x 4 targets (K,V) -> FP8 E4M3 + per-token scale",
            "ms": round(ms, 4), "tflops": round(tflops, 1), "bound": "mfma", "peak_tflops": 2500.0,
            "frac": round(tflops / 2500.0, 4), "flops": flops, "bytes": in_bytes + out_bytes,
            "library_gemm": {"what": "torch.matmul (hipBLASLt) of the same X and the 8 weight matrices "
                                     "concatenated, bf16 output, no storage epilogue; context only", **lib},
            "decode_append": {"workload": f"{nb} new tokens x 4096 -> 4 targets (K,V), FP8, scattered rows",
                              "us": round(ms_app * 1e3, 2), "bytes": app_bytes,
                              "GBps": round(app_bytes / (ms_app * 1e-3) / 1e9, 1), "bound": "hbm (weights)"}}


def bench_swa(dev, iters, w=128):
    """Self-Decoder sliding-window attention of a 32768-token prefill chunk over its own 32768-row bf16
    cache: H = 32 query heads on one KV head, window 128 (seeded normal Q, K, V)."""
    import torch
    from long_context_split_amd import hysparse as hs
    T, H = 32768, 32
    g = torch.Generator(device=dev)
    g.manual_seed(1234)
    k = torch.randn((T, 1, 128), generator=g, device=dev).to(torch.bfloat16)
    v = torch.randn((T, 1, 128), generator=g, device=dev).to(torch.bfloat16)
    q = torch.randn((1, T, H, 128), generator=g, device=dev).to(torch.bfloat16)
    kv = hs.KVCache(k, v, [T], [0])
    band = sum(min(t + 1, w) for t in range(T))
    flops = 4.0 * band * H * 128                                       # Q K^T and P V over each band

    def timed(out):
        for _ in range(2):
            hs.swa_attn(kv, q, w, out=out)
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(iters)]
        for a, b in evs:
            a.record()
            hs.swa_attn(kv, q, w, out=out)
            b.record()
        torch.cuda.synchronize()
        return statistics.median(a.elapsed_time(b) for a, b in evs)

    res = {}
    for name, dt, ob in (("f32", torch.float32, 4), ("bf16", torch.bfloat16, 2)):
        ms = timed(torch.empty((1, T, H, 128), dtype=dt, device=dev))
        nbytes = T * H * 128 * 2 + T * H * 128 * ob + 2 * T * 128 * 2  # Q in, O out, K and V once
        gbps = nbytes / (ms * 1e-3) / 1e9
        log(f"swa ({name} output): {ms * 1e3:.1f} us  {gbps:.0f} GB/s  ({gbps / HBM_PEAK_GBPS:.3f} of HBM peak)")
        res[name] = {"us": round(ms * 1e3, 2), "GBps": round(gbps, 1), "frac": round(gbps / HBM_PEAK_GBPS, 4),
                     "bytes": nbytes, "tflops": round(flops / (ms * 1e-3) / 1e12, 1)}
    return {"workload": f"swa_chunk_32k: 32768-token chunk over its 32768-row bf16 cache, H=32, n_kv=1, window {w}",
            "bound": "hbm", "peak_GBps": HBM_PEAK_GBPS, "flops": flops, **res["f32"],
            "bf16_output": res["bf16"]}


def cpu_baseline(case, spec, top_k, window, budget_s):
    """The float64 oracle, as it stands, on sequences of the same workload until the budget is spent."""
    import numpy as np
    from oracle import attention, block, bridge as obridge
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = None
    cores = len(os.sched_getaffinity(0))
    lens, starts = case["lengths"], case["row_start"]
    t0 = time.time()
    done = 0
    while True:                                 # cycle over the sequences until the budget is spent
        i = done % len(lens)
        L, r0 = int(lens[i]), int(starts[i])
        if spec["kv"] == "bf16":
            k = block.cache_values(case["k"][r0:r0 + L], "bf16")
            v = block.cache_values(case["v"][r0:r0 + L], "bf16")
        else:                                   # the oracle's own E4M3 quantiser, then its decoder
            kc, ksc = obridge.quantize_rows_e4m3(case["k"][r0:r0 + L].reshape(L, 128))
            vc, vsc = obridge.quantize_rows_e4m3(case["v"][r0:r0 + L].reshape(L, 128))
            k = block.cache_values(kc.reshape(L, 1, 128), "e4m3", ksc.reshape(L, 1))
            v = block.cache_values(vc.reshape(L, 1, 128), "e4m3", vsc.reshape(L, 1))
        q = block.cache_values(case["q_full"][i], "bf16")
        out = block.full_layer(q, k, v, top_k, window)
        for qs in case["q_sparse"]:
            attention.sparse_attention(block.cache_values(qs[i], "bf16"), k, v, out["idx"], out["cnt"])
        done += 1
        if time.time() - t0 >= budget_s:
            break
    el = time.time() - t0
    n_q = case["q_full"].shape[1]
    log(f"cpu oracle: {done} sequences in {el:.2f}s")
    return {"value": round(done * n_q / el, 3), "unit": "queries/s", "cores": blas_threads or cores,
            "host_cores_visible": cores, "kind": "oracle",
            "sample": f"{done} sequence steps, cycling over the {len(lens)} sequences of the same step "
                      f"(full layer + select + {len(case['q_sparse'])} sparse layers each), float64 NumPy",
            "seconds": round(el, 2)}


if __name__ == "__main__":
    main()
