#!/usr/bin/env python3
"""Throughput of rolling-window decode attention with exact RoPE re-basing.

One step = for each of the 36 layers: a8r_append_kv (one new token per stream,
all 64 streams in one call) then a8r_decode_attn (all 64 streams in one call),
on the 3B-class GQA shape (16 query / 2 KV heads, head_dim 128, bf16 ring,
W = 4096).  Streams start at seeded absolute positions in [0, 1e6) and ring
offsets in [0, 4096) and are pre-filled to a full window before timing; inputs
for the timed steps are pre-staged in HBM (a pool of distinct steps cycled
through).  Prints ONE JSON line.

    python bench.py [--gpus 1] [--steps 1000] [--warmup 20] [--workload qwen3b_batch64]

``--workload qwen3b_chunk8`` measures the 8-position chunk path instead;
``--prefix F`` pins an F-token prompt prefix in every (layer, stream) first;
``--workload qwen3b_single`` / ``audio8_0p1b`` time one stream (per-step
latency of the 3B-class and the Audio8-0.1B decoder shapes).
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decode-attn steps/sec + KV HBM GB/s (% roofline), 3B-class GQA, W=4096, batch 64"
HBM_PEAK_GBPS = 8000.0
BF16_DENSE_TFLOPS = 2500.0
POOL = 16
PMC_FILE = os.path.join(ROOT, "profiles", "pmc_traffic.json")
KERNEL_SRC = os.path.join(ROOT, "rolling_kv_cache_ring_amd", "csrc", "a8r_kernels.hip")


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1000)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="qwen3b_batch64",
                    choices=["qwen3b_batch64", "qwen3b_chunk8", "qwen3b_chunk12", "qwen3b_chunk16",
                             "qwen3b_single", "audio8_0p1b"])
    ap.add_argument("--path", default="fused", choices=["fused", "separate"],
                    help="step per layer as one a8r_append_decode_attn / a8r_append_chunk_attn call "
                         "(fused) or as a8r_append_kv + a8r_decode_attn / a8r_chunk_attn (separate)")
    ap.add_argument("--cache-mode", default="rotate_on_read", choices=["rotate_on_read", "rebase_on_evict"],
                    help="rebase_on_evict runs the comparison variant (keys stored rotated and re-rotated at "
                         "every eviction); the fused call then runs as append + decode")
    ap.add_argument("--prefix", type=int, default=0, metavar="F",
                    help="pin an F-token prompt prefix in every (layer, stream) before the pre-fill; "
                         "attention then covers F + W keys")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--copy-probe", action="store_true",
                    help="after the timed steps, run a plain 1 GiB device copy 5 times (counter calibration)")
    ap.add_argument("--summarize", metavar="DIR", default=None,
                    help="summarize rocprofv3 CSV output under DIR (no GPU work); see profiles/")
    ap.add_argument("--summary-command", default="", help="command line recorded in the summary")
    return ap.parse_args()


COPY_PROBE_BYTES = 1 << 30


def copy_probe(torch):
    """A plain device copy of known size: 1 GiB read + 1 GiB written per launch."""
    src = torch.empty(COPY_PROBE_BYTES // 2, dtype=torch.int16, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def summarize(args):
    """Reads rocprofv3 CSVs (kernel_stats / counter_collection) under a directory
    and prints a markdown summary; for counter runs also updates
    profiles/pmc_traffic.json with the calibrated HBM bytes per attention launch."""
    import csv
    import glob
    from collections import defaultdict
    d = args.summarize
    lines = [f"command: `{args.summary_command}`", ""]
    stats = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    for f in stats:
        rows = list(csv.DictReader(open(f)))
        lines.append("| kernel | calls | avg us | min us | max us | share |")
        lines.append("|---|---|---|---|---|---|")
        for r in rows:
            name = r["Name"]
            short = name.replace("(anonymous namespace)::", "").replace("void ", "").split("(")[0]
            lines.append(f"| `{short[:70]}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                         f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                         f"{float(r['Percentage']):.1f}% |")
    cc = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if cc:
        per = defaultdict(lambda: defaultdict(float))
        calls = defaultdict(set)
        rows_all = []
        for f in cc:
            rows_all += list(csv.DictReader(open(f)))
        is_attn = lambda n: "decode_mfma" in n or "chunk_mfma" in n or "chunk_tiled" in n or "chunk_pipe" in n
        last_attn = max([int(r["Dispatch_Id"]) for r in rows_all if is_attn(r["Kernel_Name"])] + [0])
        for r in rows_all:
            name = r["Kernel_Name"]
            if is_attn(name):
                key = "attention"
            elif "copy" in name.lower() and int(r["Dispatch_Id"]) > last_attn:
                key = "copy"        # the calibration copies run after the last attention launch
            else:
                continue
            per[key][r["Counter_Name"]] += float(r["Counter_Value"])
            calls[key].add(r["Dispatch_Id"])
        lines.append("| kernel | dispatches | counter | KiB per dispatch |")
        lines.append("|---|---|---|---|")
        avg = {}
        for key, cnt in per.items():
            for cname, v in cnt.items():
                a = v / max(1, len(calls[key]))
                avg[(key, cname)] = a
                lines.append(f"| {key} | {len(calls[key])} | {cname} | {a:.1f} |")
        rec_path = os.path.join(ROOT, "profiles", "pmc_traffic.json")
        try:
            rec = json.load(open(rec_path))
        except (OSError, ValueError):
            rec = {}
        wl = args.workload + (f"+prefix{args.prefix}" if args.prefix else "")
        entry = rec.get(wl, {})
        if entry.get("kernel_sha256_16") != kernel_hash():
            entry = {}      # counters taken on an older kernel source no longer apply
        for cname, copy_bytes in (("FETCH_SIZE", COPY_PROBE_BYTES), ("WRITE_SIZE", COPY_PROBE_BYTES)):
            if ("copy", cname) in avg and ("attention", cname) in avg:
                factor = copy_bytes / (avg[("copy", cname)] * 1024)
                entry[cname.lower() + "_factor"] = factor
                entry[cname.lower() + "_bytes"] = avg[("attention", cname)] * 1024 * factor
                lines.append(f"\n{cname}: copy probe counts {avg[('copy', cname)]:.0f} KiB for "
                             f"{copy_bytes / 1024:.0f} KiB moved -> scale factor {factor:.4f}; attention kernel "
                             f"{avg[('attention', cname)] * 1024 * factor / 1e6:.2f} MB per launch")
        entry["kernel_sha256_16"] = kernel_hash()
        entry["path"] = args.path
        if "fetch_size_bytes" in entry and "write_size_bytes" in entry:
            entry["bytes_per_launch"] = round(entry["fetch_size_bytes"] + entry["write_size_bytes"])
            lines.append(f"\nrecorded {rec_path}: {entry['bytes_per_launch'] / 1e6:.2f} MB per launch")
        rec[wl] = entry
        os.makedirs(os.path.dirname(rec_path), exist_ok=True)
        json.dump(rec, open(rec_path, "w"), indent=1, sort_keys=True)
    print("\n".join(lines))


def algorithmic_bytes(wl, live):
    """Bytes one attention launch (one layer, all streams) must move: the live
    K and V windows, the queries and the outputs."""
    e = 2
    kv = wl.n_streams * wl.n_kv_heads * live * wl.head_dim * e * 2
    q = wl.n_streams * wl.chunk * wl.n_q_heads * wl.head_dim * e
    return kv + 2 * q


def append_bytes(wl):
    return wl.n_streams * wl.chunk * wl.n_kv_heads * wl.head_dim * 2 * 2 * 2   # read + write K and V


def attention_flops(wl, live):
    # 4 * D * Hq * sum over queries of keys seen (QK^T and PV, 2 flops per MAC)
    c = wl.chunk
    keys = sum(live - c + 1 + j for j in range(c))
    return 4 * wl.head_dim * wl.n_q_heads * keys * wl.n_streams


def kernel_hash():
    with open(KERNEL_SRC, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def traffic_from_profiles(workload):
    """HBM bytes per launch measured with rocprofv3 counters, if they were taken
    on the current kernel source; else None."""
    try:
        with open(PMC_FILE) as f:
            rec = json.load(f)
        r = rec.get(workload)
        if r and r.get("kernel_sha256_16") == kernel_hash():
            return r.get("bytes_per_launch")
    except (OSError, ValueError):
        pass
    return None


def cpu_baseline(wl, seconds):
    """Time the float64 oracle on host cores on a bounded sample of the same
    workload: full-window decode (or chunk) attention for as many (layer, stream)
    pairs as fit in ``seconds``, scaled to steps/s."""
    import threadpoolctl
    import synth
    from oracle.attention import chunk_rebased
    w, hkv, hq, d, c = wl.window, wl.n_kv_heads, wl.n_q_heads, wl.head_dim, wl.chunk
    rng = np.random.default_rng(0)
    k = synth.round_bf16(rng.standard_normal((w, hkv, d)).astype(np.float32)).astype(np.float64)
    v = synth.round_bf16(rng.standard_normal((w, hkv, d)).astype(np.float32)).astype(np.float64)
    q = synth.round_bf16(rng.standard_normal((c, hq, d)).astype(np.float32)).astype(np.float64)
    info = threadpoolctl.threadpool_info()
    threads = max([i.get("num_threads", 1) for i in info] + [1])
    chunk_rebased(q, k, v)               # warm-up
    n = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < seconds:
        chunk_rebased(q, k, v)
        n += 1
    dt = time.perf_counter() - t0
    pairs_per_step = wl.n_layers * wl.n_streams
    return {
        "value": round(n / dt / pairs_per_step, 6),
        "unit": "steps/s",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"{n} (layer, stream) attention calls of the float64 numpy oracle over a full "
                   f"W={w} window ({hq}/{hkv} heads, D={d}, {c} quer{'y' if c == 1 else 'ies'}) in "
                   f"{dt:.1f} s; one step = {pairs_per_step} such calls; BLAS threads={threads}, "
                   f"host cpus={len(os.sched_getaffinity(0))}"),
    }


def main():
    args = parse()
    if args.summarize:
        summarize(args)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this path has no multi-GPU mode "
              "(streams shard across GPUs with no exchange). Run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import synth
    import rolling_kv_cache_ring_amd as a8r

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    a8r.lib()  # fails loudly if the HIP library is missing

    wl = synth.WORKLOADS[args.workload]
    B, NL, hq, hkv, d, w, c = (wl.n_streams, wl.n_layers, wl.n_q_heads, wl.n_kv_heads, wl.head_dim,
                               wl.window, wl.chunk)
    stream = torch.cuda.current_stream()
    rebase = args.cache_mode == "rebase_on_evict"
    F = args.prefix
    cfg = a8r.make_config(NL, B, hq, hkv, d, w, w, True, rebase_on_evict=rebase, prefix_capacity=F)
    cache = a8r.Cache(cfg, stream=stream.cuda_stream)

    # seeded start states; pre-fill each stream to min(P0, W) tokens ending at P0 - 1
    # (the single-stream workloads start at P0 = 0: timed from a full window, P0 = W)
    p0, r0 = synth.start_states(wl)
    if wl.n_streams == 1:
        p0, r0 = p0 + w, (r0 + w) % w
    n_pre = np.minimum(p0, w)
    cache.reset(0, p0 - n_pre, (r0 - n_pre) % w)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(0xA8)
    bf = torch.bfloat16
    if F:
        for layer in range(NL):
            pk = torch.randn((B, F, hkv, d), device="cuda", generator=gen).to(bf).view(torch.int16)
            pv = torch.randn((B, F, hkv, d), device="cuda", generator=gen).to(bf).view(torch.int16)
            cache.append_prefix(layer, 0, B, F, pk, pv)
        del pk, pv
    fill = torch.randn((B, w, hkv, d), device="cuda", generator=gen).to(bf).view(torch.int16)
    fill_v = torch.randn((B, w, hkv, d), device="cuda", generator=gen).to(bf).view(torch.int16)
    for layer in range(NL):
        for b in range(B):
            n = int(n_pre[b])
            if n:
                cache.append_kv(layer, b, 1, n, fill[b:b + 1, :n], fill_v[b:b + 1, :n],
                                want_bookkeeping=False)
    del fill, fill_v
    torch.cuda.synchronize()

    kpool = torch.randn((POOL, NL, B, c, hkv, d), device="cuda", generator=gen).to(bf).view(torch.int16)
    vpool = torch.randn((POOL, NL, B, c, hkv, d), device="cuda", generator=gen).to(bf).view(torch.int16)
    qpool = torch.randn((POOL, NL, B, c, hq, d), device="cuda", generator=gen).to(bf).view(torch.int16)
    outs = torch.empty((NL, B, c, hq, d), device="cuda", dtype=torch.int16)
    ptr = lambda t: t.data_ptr()
    k_ptrs = [[ptr(kpool[i, l]) for l in range(NL)] for i in range(POOL)]
    v_ptrs = [[ptr(vpool[i, l]) for l in range(NL)] for i in range(POOL)]
    q_ptrs = [[ptr(qpool[i, l]) for l in range(NL)] for i in range(POOL)]
    o_ptrs = [ptr(outs[l]) for l in range(NL)]
    h = cache.handle
    L = a8r.lib()

    fused = args.path == "fused" and not rebase

    def check(st):
        if st:
            raise a8r.A8RError(st, L.a8r_last_error().decode())

    def step(i):
        kp, vp, qp = k_ptrs[i % POOL], v_ptrs[i % POOL], q_ptrs[i % POOL]
        for layer in range(NL):
            if fused and c == 1:
                check(L.a8r_append_decode_attn(h, layer, 0, B, kp[layer], vp[layer], qp[layer],
                                               o_ptrs[layer], None, None))
                continue
            if fused:
                check(L.a8r_append_chunk_attn(h, layer, 0, B, c, kp[layer], vp[layer], qp[layer],
                                              o_ptrs[layer], None, None))
                continue
            check(L.a8r_append_kv(h, layer, 0, B, c, kp[layer], vp[layer], None, None))
            if c == 1:
                check(L.a8r_decode_attn(h, layer, 0, B, qp[layer], o_ptrs[layer]))
            else:
                check(L.a8r_chunk_attn(h, layer, 0, B, c, qp[layer], o_ptrs[layer]))

    def attention_only(i):
        qp = q_ptrs[i % POOL]
        for layer in range(NL):
            if c == 1:
                check(L.a8r_decode_attn(h, layer, 0, B, qp[layer], o_ptrs[layer]))
            else:
                check(L.a8r_chunk_attn(h, layer, 0, B, c, qp[layer], o_ptrs[layer]))

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    t_wall = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    ms = ev0.elapsed_time(ev1) / args.steps
    steps_per_s = 1000.0 / ms

    # average launch duration of the attention kernel.  Fused path: the timed
    # region launches nothing else (one call per layer: the fused kernel, plus
    # the split combine for a chunk), so it is the region time over its calls.
    # Separate path: a second pass launches only the attention calls (they
    # leave the cache unchanged) back to back on the same stream, bracketed by
    # one event pair.
    if fused:
        n_launch = args.steps * NL
        attn_ms = ev0.elapsed_time(ev1) / n_launch
    else:
        n_t = min(args.steps, 200)
        a0 = torch.cuda.Event(enable_timing=True)
        a1 = torch.cuda.Event(enable_timing=True)
        a0.record(stream)
        for i in range(n_t):
            attention_only(i)
        a1.record(stream)
        torch.cuda.synchronize()
        n_launch = n_t * NL
        attn_ms = a0.elapsed_time(a1) / n_launch

    live = w + F  # every stream holds a full window after pre-fill, after its prefix
    bytes_launch = algorithmic_bytes(wl, live)
    bytes_step = NL * (bytes_launch + append_bytes(wl))
    gbps_step = bytes_step * steps_per_s / 1e9
    achieved = bytes_launch / (attn_ms * 1e-3) / 1e9
    flops_launch = attention_flops(wl, live)
    traffic = traffic_from_profiles(args.workload + (f"+prefix{F}" if F else ""))

    if args.copy_probe:
        copy_probe(torch)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, args.cpu_seconds)

    line = {
        "metric": METRIC,
        "value": round(steps_per_s, 3),
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "path": "fused" if fused else "separate",
                   "cache_mode": args.cache_mode, "layers": NL, "streams": B, "q_heads": hq, "kv_heads": hkv,
                   "head_dim": d, "window": w, "positions_per_step": c, "prefix": F,
                   "start_positions": ("W (a full window)" if B == 1 else "seeded U[0,1e6)" if c == 1
                                       else "seeded U[2^24-W,2^24)")},
        "kv_gbps": round(gbps_step, 1),
        "hbm_frac_step": round(gbps_step / HBM_PEAK_GBPS, 4),
        "bytes_per_step": bytes_step,
        "roofline": {
            "bound": "hbm",
            "kernel": ("a8r_append_decode_attn (decode_mfma, fused append)" if fused and c == 1 else
                       "a8r_append_chunk_attn (chunk_pipe, fused append, + combine_kernel)" if fused else
                       "a8r_decode_attn" if c == 1 else "a8r_chunk_attn (chunk_pipe + combine_kernel)"),
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "bytes_per_launch": bytes_launch,
            "avg_launch_ms": round(attn_ms, 5),
            "launches_timed": n_launch,
            "mfma_tflops": round(flops_launch / (attn_ms * 1e-3) / 1e12, 2),
            "mfma_frac_bf16_dense": round(flops_launch / (attn_ms * 1e-3) / 1e12 / BF16_DENSE_TFLOPS, 4),
        },
        "cpu_baseline": cpu,
        "wall_s_timed": round(wall, 3),
    }
    if rebase:
        # the variant's extra work: every eviction re-rotates the whole K window
        # (read + write), per layer and step at full windows
        line["rebase"] = {
            "k_bytes_per_layer": B * hkv * w * d * 2 * 2,
            "append_and_rebase_ms_per_layer": round(ms / NL - attn_ms, 5),
        }
    print(json.dumps(line), flush=True)
    cache.close()


if __name__ == "__main__":
    main()
