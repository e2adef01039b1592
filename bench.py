"""Benchmark of the multi-LoRA delta hot path on one MI355X.

A step is one pass of the delta path over one batch already resident in HBM.
The default run is the 70B-shape decoder layer: 1280 tokens (256 decode tokens
on 256 distinct rank-16 adapters plus a 1024-token prefill request), the seven
projections of Llama-3-70B (q, o 8192 -> 8192; k, v 8192 -> 1024; gate, up
8192 -> 28672; down 28672 -> 8192), each step the SGMV delta (shrink + expand)
of all seven.  Its line nests the decode batch (256 tokens, one per request,
128 resident rank-16 adapters, 4096 -> 4096, one fused launch) and the
heterogeneous-rank paged batch (4096 tokens, 64 Zipf-length requests, ranks
8..64, 8192 -> 8192, 16-row pages in a shuffled pool), each measured the same
way with its own roofline and CPU baseline.  ``--config N`` runs one workload
alone.

Cold caches.  Every kernel's bytes come from HBM: steps rotate over device
replicas of the inputs and adapter rows (clones at other addresses) whose
per-kernel footprint summed over the rotation exceeds twice the 256 MB
last-level (Infinity) cache.

Metric: delta tokens/s (whole job) plus achieved HBM GB/s of the dominant
kernel against the 8 TB/s peak.  The timed region replays the K steps as one
HIP graph, bracketed by device synchronisation.  Per-kernel durations come
from HIP events on the launch stream around a graph of K back-to-back launches
of that kernel rotating over the replicas (span / K, mean of three replays):
events around single launches would add microseconds of event latency to
kernels that last a few.  The fp64 CPU oracle is timed beside it on a bounded
sample, on one thread and on all the cores the process may use.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--config N]
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
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16, published
LLC_BYTES = 256 * 2**20        # Infinity Cache
METRIC = "LoRA delta tokens/sec per layer + achieved HBM GB/s (% of MI355X peak)"
KERNEL_SOURCES = [os.path.join(ROOT, "segmented_gather_gemm_segments_amd", "csrc", f)
                  for f in ("kernels.hip", "base_gemm.hip", "host.cpp", "lora_internal.h")] + \
                 [os.path.join(ROOT, "include", "lora_sgmv.h")]
LAYER_WORKLOAD = "layer70b_1280tok_256ad_r16"
LAYER_GROUPS = (("q", "k", "v"), ("o",), ("gate", "up"), ("down",))


def kernel_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", type=int, default=0,
                    help="0 (default): the 70B layer with the decode and heterogeneous batches "
                         "nested; 1..5: one workload alone (2 decode, 3 prefill, 4 heterogeneous "
                         "paged, 5 the 70B layer)")
    ap.add_argument("--shape", default="q", help="config 3 shape: q or up")
    ap.add_argument("--wq", choices=("", "fp8", "int4"), default="",
                    help="adapter rows stored as FP8 E4M3 or INT4 with row scales (configs 2, 4)")
    ap.add_argument("--order", type=int, default=0, help="BGMV order (0 auto, 1 token, 2 adapter)")
    ap.add_argument("--path", choices=("fused", "two"), default="fused",
                    help="per-token (decode) step: one fused launch, or shrink + expand launches")
    ap.add_argument("--placement", choices=("grouped", "index"), default="grouped",
                    help="fused decode: workgroups take tokens in the batch's segment order "
                         "(host-built once per batch, shared by all layers) or in index order")
    ap.add_argument("--policy", type=int, default=0, help="SGMV path policy (0 auto, 1 gather, 2 mfma)")
    ap.add_argument("--shrink", choices=("auto", "tiled", "plain"), default="auto",
                    help="SGMV shrink: tiled (64-token tiles of x and A streamed through LDS, d_in cut "
                         "into slices whose partials a second launch adds), the one-launch shrink, or "
                         "auto: tiled where segments of at least --tile-min tokens carry most of the "
                         "shrink's bytes")
    ap.add_argument("--tile-min", type=int, default=0,
                    help="tiled shrink: segments of at least this many tokens take tile items "
                         "(0: the library default)")
    ap.add_argument("--max-splits", type=int, default=0, help="tiled shrink: at most this many d_in slices")
    ap.add_argument("--layer-streams", choices=("groups", "serial"), default="groups",
                    help="70B layer step: the deltas of q, k, v (and of gate, up), independent given the "
                         "layer's inputs, on separate HIP streams with o and down after their groups, "
                         "or all seven in one stream")
    ap.add_argument("--mfma-min", type=int, default=0,
                    help="SGMV plan: segments of at least this many tokens take the MFMA path "
                         "(0: the library default)")
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="bound on each workload's one-thread oracle time (0 disables the CPU baseline)")
    ap.add_argument("--replicas", type=int, default=0, help="0 = enough to exceed 2x the LLC")
    ap.add_argument("--expand-tile", type=int, default=0, choices=(0, 64, 128),
                    help="MFMA token tile of the expand plans (0 = the library's width table)")
    ap.add_argument("--churn", type=int, default=0, metavar="POOL_ADAPTERS",
                    help="adapter churn: decode batches over 1024 adapters through an LRU cache "
                         "whose pools hold POOL_ADAPTERS rank-16 adapters (uploads timed in)")
    ap.add_argument("--multi", action="store_true",
                    help="decode q, k, v of the 70B layer (256 tokens, 256 rank-16 adapters) as one "
                         "fused multi-projection launch vs three fused launches")
    ap.add_argument("--serial", action="store_true",
                    help="also time the adapter-serial comparator (one shrink + expand launch "
                         "per adapter sub-batch, same kernels)")
    ap.add_argument("--warm", action="store_true",
                    help="also time every kernel warm: K launches on one replica, its operands left in "
                         "cache by the previous launch (the default timings are all cold)")
    ap.add_argument("--decode-sweep", action="store_true",
                    help="the fused decode launch on decode batches of 32 .. 256 tokens (one workgroup per "
                         "token): how one workgroup's pass times against the number of workgroups")
    ap.add_argument("--floor", action="store_true",
                    help="only time bare streaming reads and a read-modify-write of given sizes "
                         "and workgroup counts (the device's floors for launches of that size)")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run torch device copies of MIB MiB (HBM counter calibration)")
    return ap.parse_args()


def workload(cfg: int, shape: str, wq: str = ""):
    from segmented_gather_gemm_segments_amd import workloads as wl
    if wq and cfg not in (2, 4):
        raise SystemExit("--wq applies to configs 2 and 4")
    if cfg == 1:
        return wl.tiny_sgmv()
    if cfg == 2:
        return wl.bgmv_decode(wq=wq)
    if cfg == 3:
        return wl.sgmv_prefill(shape=shape)
    if cfg == 4:
        return wl.hetero_paged(wq=wq)
    raise SystemExit("unknown config")


def read_traffic(kernel: str, workload_name: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel sources; otherwise None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload_name}.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    for line in open(path):
        if "=" in line and not line.startswith("#"):
            k, v = line.split("=", 1)
            vals[k.strip()] = v.strip()
    if vals.get("kernel_sources_sha256_16") != kernel_hash():
        return None
    try:
        return float(vals["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def profile_path(workload_name: str):
    path = os.path.join("profiles", f"{workload_name}.md")
    return path if os.path.exists(os.path.join(ROOT, path)) else None


def oracle_threads() -> int:
    """Threads for the all-cores oracle leg: the cores this process may run on
    (sched_getaffinity), capped by OMP_NUM_THREADS when the host sets it."""
    n = len(os.sched_getaffinity(0))
    cap = os.environ.get("OMP_NUM_THREADS", "")
    if cap.isdigit() and int(cap) > 0:
        n = min(n, int(cap))
    return max(1, n)


def cpu_baseline(parts, num_tokens: int, budget_s: float):
    """The oracle as it stands (C, fp64) on a bounded sample of the same
    workload: the first n tokens of the batch through every part of a step
    (one projection, or the seven of the layer), n sized so that the one-thread
    pass takes about budget_s; a batch whose whole pass takes less is passed
    through repeatedly, about budget_s in all.  Timed once on one thread and
    once on all the cores this process may use, with the same number of passes
    (the same per-token arithmetic, bit-identical output).  parts: list of
    (problem, oracle adapters)."""
    import oracle

    def run(n, threads, passes=1):
        used = 1
        t0 = time.perf_counter()
        for _ in range(passes):
            for p, ad in parts:
                out, used = oracle.apply_counted(p.x[:n], p.y[:n], p.ids[:n], ad, threads)
        return time.perf_counter() - t0, used, out

    probe = min(8, num_tokens)
    t_probe, _, _ = run(probe, 1)
    per_tok = max(t_probe / probe, 1e-7)
    n = int(min(num_tokens, max(probe, budget_s / per_tok)))
    passes = 1
    if n == num_tokens:
        passes = int(max(1, min(1000, budget_s // (per_tok * num_tokens))))
    t1, _, out1 = run(n, 1, passes)
    threads = oracle_threads()
    tn, used, outn = run(n, threads, passes)
    assert np.array_equal(out1, outn), "threaded oracle differs from the one-thread oracle"
    what = f"the first {n} of {num_tokens} tokens" if n < num_tokens else f"all {num_tokens} tokens"
    if len(parts) > 1:
        what += f" through all {len(parts)} projections"
    what += ", one pass" if passes == 1 else f", {passes} passes"
    return {"value": round(n * passes / tn, 2), "unit": "delta tokens/s", "cores": used, "kind": "oracle",
            "sample": f"{what}, {tn:.2f} s on {used} threads (OpenMP over tokens)",
            "affinity_cores": len(os.sched_getaffinity(0)),
            "single_thread": {"value": round(n * passes / t1, 2), "unit": "delta tokens/s", "cores": 1,
                              "sample": f"{what}, {t1:.2f} s"}}


def graph_span(torch, stream, fns, reps: int = 3, best: bool = False) -> float:
    """Seconds per launch: HIP events on `stream` around a graph of the
    launches `fns` (one each, back to back); mean (or best) of `reps` replays."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for f in fns:
            f()
    with torch.cuda.stream(stream):
        g.replay()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1) * 1e-3 / len(fns))
    return min(ts) if best else float(np.mean(ts))


def timed_graph(torch, stream, step, K: int, W: int):
    """W eager warmup steps, then the K steps as one HIP graph: one untimed
    replay, then the timed replay between device synchronisations.  Returns
    (wall seconds of the K steps, host seconds per eager step)."""
    t0 = time.perf_counter()
    for i in range(W):
        step(i)
    host_step_s = (time.perf_counter() - t0) / max(W, 1)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=stream):
        for i in range(K):
            step(i)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        graph.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        graph.replay()
    torch.cuda.synchronize()
    return time.perf_counter() - t0, host_step_s


def n_replicas(args, footprint: float, cap: int = 64) -> int:
    """Replicas whose rotation moves at least twice the LLC through a kernel
    whose one launch touches `footprint` bytes."""
    if args.replicas:
        return args.replicas
    return int(min(cap, max(2, np.ceil(2 * LLC_BYTES / max(footprint, 1.0)))))


def serial_comparator(torch, stream, steps_calls, tokens: int, one_launch_s: float, K: int):
    """Times the adapter-serial comparator: steps_calls[i] is the list of
    launches of step i (replayed as one graph of K steps, like the main path).
    Returns its record, with the one-launch path's speed-up over it."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for i in range(K):
            for f in steps_calls[i % len(steps_calls)]:
                f()
    with torch.cuda.stream(stream):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    with torch.cuda.stream(stream):
        g.replay()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launches = len(steps_calls[0])
    return {"kind": "adapter-serial (one shrink + expand launch per adapter sub-batch)",
            "launches_per_step": launches, "ms_per_step": round(wall / K * 1e3, 5),
            "value": round(tokens * K / wall, 1), "unit": "delta tokens/s",
            "one_launch_speedup": round((wall / K) / one_launch_s, 3), "steps": K}




def bench_churn(args, torch):
    """Decode steps under adapter churn: each step makes its batch's adapters
    resident through the LRU cache (uploads from pinned host copies on the
    cache's copy stream) and runs the fused delta.  Timed eagerly, since a
    step has host logic; the same steps are also timed with a host
    synchronisation after each (no overlap of uploads with compute)."""
    from segmented_gather_gemm_segments_amd import binding as B
    from segmented_gather_gemm_segments_amd import workloads as wl
    num_ids, tokens, d, pr = 1024, 256, 4096, 16
    K, W = args.steps, args.warmup
    uni, seq = wl.churn(num_ids=num_ids, batches=W + K, tokens=tokens, d_in=d, d_out=d,
                        wq=args.wq)
    dev = torch.device("cuda:0")
    wf = {"": B.LORA_WFMT_PLAIN, "fp8": B.LORA_WFMT_FP8_E4M3, "int4": B.LORA_WFMT_INT4}[args.wq]
    n_pages = args.churn * ((16 + pr - 1) // pr)

    def pool(seed):
        if wf == B.LORA_WFMT_PLAIN:
            st = torch.empty((n_pages, pr, d), dtype=torch.bfloat16, device=dev)
            return B.Pool(st, pr, shuffle_seed=seed)
        w = d // 2 if wf == B.LORA_WFMT_INT4 else d
        st = torch.empty((n_pages, pr, w), dtype=torch.uint8, device=dev)
        sc = torch.empty((n_pages * pr,), dtype=torch.float32, device=dev)
        return B.Pool(st, pr, shuffle_seed=seed, weight_format=wf, scales=sc)

    def pinned(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).pin_memory()

    hosts = [(pinned(uni.a_rows[a]), pinned(uni.bt_rows[a]),
              pinned(uni.a_scales[a]) if args.wq else None,
              pinned(uni.bt_scales[a]) if args.wq else None) for a in range(num_ids)]
    stream = torch.cuda.Stream()
    dev_batches = []
    with torch.cuda.stream(stream):
        for ids, x, y in seq:
            perm, _, _ = B.lora_segments_build(ids, num_ids)
            dev_batches.append((ids, torch.from_numpy(ids).to(dev),
                                torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16),
                                torch.from_numpy(y.view(np.int16)).to(dev).view(torch.bfloat16),
                                torch.from_numpy(perm).to(dev)))
    torch.cuda.synchronize()

    def run(steps, sync_each):
        pa, pb = pool(11), pool(12)
        mp = (16 + pr - 1) // pr
        pt_a = torch.empty((num_ids, mp), dtype=torch.int32, device=dev)
        pt_b = torch.empty((num_ids, mp), dtype=torch.int32, device=dev)
        rank = torch.empty(num_ids, dtype=torch.int32, device=dev)
        cache = B.Cache(pa, pb, num_ids, 16, pt_a, pt_b, rank)
        for a in range(num_ids):
            cache.register(a, int(uni.ranks[a]), *hosts[a])
        w = cache.weights(B.LORA_BF16, d, d, wf)
        calls = []
        for ids, ids_d, x_d, y_d, perm_d in dev_batches:
            calls.append((ids, B.prepare_bgmv_fused(w, ids_d, x_d, y_d, None, B.LORA_BGMV_AUTO,
                                                    stream=stream, token_order=perm_d)))
        for ids, fu in calls[:W]:
            cache.prepare(ids, stream=stream)
            fu()
        torch.cuda.synchronize()
        s0 = cache.stats()
        t0 = time.perf_counter()
        for ids, fu in calls[W:W + steps]:
            cache.prepare(ids, stream=stream)
            fu()
            if sync_each:
                stream.synchronize()
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        s1 = cache.stats()
        cache.close()
        return wall, {k: s1[k] - s0[k] for k in ("hits", "misses", "evictions", "bytes_uploaded")}, s1

    wall, dlt, final = run(K, False)
    wall_sync, _, _ = run(K, True)
    tokens_k = int(sum(int(np.sum(ids >= 0)) for ids, *_ in dev_batches[W:W + K]))
    out = {
        "metric": "LoRA delta tokens/sec per layer under adapter churn",
        "value": round(tokens_k / wall, 1), "unit": "delta tokens/s", "n_gpus": 1, "steps": K,
        "warmup": W, "ms_per_step": round(wall / K * 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded; random-init adapters; Zipf(1.1) adapter popularity)",
        "config": {"workload": uni.name.replace("_" + str(tokens) + "tok", f"_{tokens}tok_pool{args.churn}"),
                   "adapters": num_ids, "pool_adapters": args.churn, "tokens": tokens, "rank": 16,
                   "d_in": d, "d_out": d, "adapter_rows": args.wq or "bf16",
                   "timed": "eager steps: lora_cache_prepare + fused delta", "parallelism": "single GPU"},
        "churn": {"hit_rate": round(dlt["hits"] / max(1, dlt["hits"] + dlt["misses"]), 4),
                  "misses_per_step": round(dlt["misses"] / K, 2),
                  "evictions_per_step": round(dlt["evictions"] / K, 2),
                  "mb_uploaded_per_step": round(dlt["bytes_uploaded"] / K / 1e6, 3),
                  "upload_gbs_effective": round(dlt["bytes_uploaded"] / wall / 1e9, 2),
                  "ms_per_step_sync_each_step": round(wall_sync / K * 1e3, 5),
                  "resident_adapters": final["resident"], "scattered_adapters": final["scattered"]},
        "kernel_sources_sha256_16": kernel_hash(),
    }
    print(json.dumps(out), flush=True)


def bench_multi(args, torch):
    """Decode deltas of the q, k and v projections of the 70B-shape layer (256
    tokens on a permutation of 256 rank-16 adapters, 8192 -> 8192 / 1024 /
    1024): one lora_bgmv_fused_multi launch per step against three
    lora_bgmv_fused launches, both in segment order, both graph-replayed over
    cache-defeating replicas."""
    from segmented_gather_gemm_segments_amd import accounting as acc
    from segmented_gather_gemm_segments_amd import binding as B
    from segmented_gather_gemm_segments_amd import runner as R
    from segmented_gather_gemm_segments_amd import workloads as wl
    names = ["q", "k", "v"]
    small = {}
    for nt in (32,):
        b2 = [wl.layer_projection(n, decode=nt, prefill=0, with_base=False) for n in names]
        for p in b2[1:]:
            p.x = b2[0].x
        st2 = torch.cuda.Stream()
        reps2 = []
        for _ in range(8):
            dps = [R.DeviceProblem(p) for p in b2]
            order = dps[0].segments()[3]
            ys = [dp.y0.clone() for dp in dps]
            reps2.append((B.prepare_bgmv_fused_multi([dp.weights for dp in dps], dps[0].ids, dps[0].x, ys,
                                                     stream=st2, token_order=order),
                          [B.prepare_bgmv_fused(dp.weights, dps[0].ids, dps[0].x, y, None,
                                                B.LORA_BGMV_AUTO, stream=st2, token_order=order)
                           for dp, y in zip(dps, ys)]))
        torch.cuda.synchronize()
        tm = graph_span(torch, st2, [reps2[i % 8][0] for i in range(args.steps)], 3)
        t3 = graph_span(torch, st2, [f for i in range(args.steps) for f in reps2[i % 8][1]], 3) * 3
        small[str(nt)] = {"us_one_launch": round(tm * 1e6, 3), "us_three_launches": round(t3 * 1e6, 3),
                          "speedup": round(t3 / tm, 3)}
        del reps2
    base = [wl.layer_projection(n, decode=256, prefill=0, with_base=False) for n in names]
    for p in base[1:]:
        p.x = base[0].x
    stream = torch.cuda.Stream()
    per_rep = sum(p.x.nbytes / 3 + p.y.nbytes + sum(a.nbytes + b.nbytes for a, b in zip(p.a_rows, p.bt_rows))
                  for p in base)
    n_rep = args.replicas or min(32, max(2, int(np.ceil(2 * LLC_BYTES / per_rep))))
    reps = []
    for _ in range(n_rep):
        dps = [R.DeviceProblem(p) for p in base]
        for dp in dps[1:]:
            dp.x = dps[0].x
        order = dps[0].segments()[3]
        ys = [dp.y0.clone() for dp in dps]
        multi = B.prepare_bgmv_fused_multi([dp.weights for dp in dps], dps[0].ids, dps[0].x, ys,
                                           stream=stream, token_order=order)
        singles = [B.prepare_bgmv_fused(dp.weights, dps[0].ids, dps[0].x, y, None, B.LORA_BGMV_AUTO,
                                        stream=stream, token_order=order) for dp, y in zip(dps, ys)]
        reps.append((multi, singles))
    torch.cuda.synchronize()
    K = args.steps
    t_multi = graph_span(torch, stream, [reps[i % n_rep][0] for i in range(K)], 3)
    t_three = graph_span(torch, stream, [f for i in range(K) for f in reps[i % n_rep][1]], 3) * 3
    tokens = int(np.sum(base[0].ids >= 0))
    nbytes = sum(acc.fused_bytes(p.ids, p.ranks, p.d_in, p.d_out, 2) for p in base) - 2 * tokens * base[0].d_in * 2
    out = {
        "metric": "LoRA delta tokens/sec per layer (q, k, v decode deltas)",
        "value": round(tokens / t_multi, 1), "unit": "delta tokens/s", "n_gpus": 1, "steps": K,
        "warmup": args.warmup, "ms_per_step": round(t_multi * 1e3, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded; random-init adapters)",
        "config": {"workload": "layer70b_qkv_decode_256tok_256ad_r16", "projections": names,
                   "replicas": n_rep, "timed": "HIP graph of K steps, per-step span",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(nbytes / t_multi / 1e9, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(nbytes / t_multi / 1e9 / HBM_PEAK_GBS, 4), "traffic": None,
                     "kernel": "bgmv_fused_multi", "algorithmic_bytes_per_launch": int(nbytes),
                     "avg_launch_us": round(t_multi * 1e6, 3)},
        "multi_projection": {"256": {"us_one_launch": round(t_multi * 1e6, 3),
                                     "us_three_launches": round(t_three * 1e6, 3),
                                     "speedup": round(t_three / t_multi, 3)}, **small},
        "kernel_sources_sha256_16": kernel_hash(),
    }
    print(json.dumps(out), flush=True)



def run_config(args, torch, cfg: int, shape: str = "q", wq: str = ""):
    """One of configs 1..4: K steps of shrink + expand (or the fused decode
    launch) over cache-defeating replicas.  Returns the record."""
    from segmented_gather_gemm_segments_amd import accounting as acc
    from segmented_gather_gemm_segments_amd import binding as B
    from segmented_gather_gemm_segments_amd import runner as R

    p = workload(cfg, shape, wq)
    elem = 2 if p.dtype == "bf16" else 4
    mode = "bgmv" if p.mode == "bgmv" else "sgmv"
    fused = mode == "bgmv" and args.path == "fused"
    stream = torch.cuda.Stream()          # default priority; every launch goes here
    nbytes = {"shrink": acc.shrink_bytes(p.ids, p.ranks, p.d_in, elem, p.wq),
              "expand": acc.expand_bytes(p.ids, p.ranks, p.d_out, elem, p.wq),
              "fused": acc.fused_bytes(p.ids, p.ranks, p.d_in, p.d_out, elem, p.wq)}
    footprint = nbytes["fused"] if fused else min(nbytes["shrink"], nbytes["expand"])
    n_rep = n_replicas(args, footprint)
    one = R.DeviceProblem(p)
    reps = [one] + [one.replica() for _ in range(n_rep - 1)]
    mfma_min = args.mfma_min or B.LORA_DEFAULT_MFMA_MIN_TOKENS
    tiled = mode == "sgmv" and (args.shrink == "tiled" or (args.shrink == "auto" and one.tiled_pays(args.tile_min)))
    calls = []
    for dp in reps:
        y, v = dp.y0.clone(), dp.new_v()
        if mode == "bgmv":
            sh, ex = B.prepare_bgmv(dp.weights, dp.ids, dp.x, v, y, args.order, stream=stream)
            tord = dp.segments()[3] if args.placement == "grouped" else None
            fu = B.prepare_bgmv_fused(dp.weights, dp.ids, dp.x, y, None, args.order, stream=stream,
                                      token_order=tord)
            calls.append((sh, ex, fu))
        else:
            _, _, _, perm_d = dp.segments()
            if not hasattr(one, "_bench_plans"):
                one._bench_plans = (dp.plan(B.LORA_PHASE_SHRINK, args.policy, mfma_min),
                                    dp.plan(B.LORA_PHASE_EXPAND, args.policy, mfma_min, args.expand_tile),
                                    dp.plan_tiled(args.policy, args.tile_min, args.max_splits) if tiled else None)
            sp, ep, tp = one._bench_plans
            if tiled:
                calls.append(B.prepare_sgmv_tiled(dp.weights, perm_d, tp[0], tp[1], tp[2], ep, dp.x, v, y,
                                                  stream=stream))
            else:
                calls.append(B.prepare_sgmv(dp.weights, perm_d, sp, ep, dp.x, v, y, stream=stream))
    torch.cuda.synchronize()

    def step(i):
        c = calls[i % n_rep]
        if fused:
            c[2]()
        else:
            c[0]()
            c[1]()

    K = args.steps
    wall, host_step_s = timed_graph(torch, stream, step, K, args.warmup)

    # per-launch durations: graphs of K back-to-back launches of one kernel
    # rotating over the replicas (the same launches as in the timed steps)
    def span(which):
        return np.array([graph_span(torch, stream, [calls[i % n_rep][which] for i in range(K)], 1)
                         for _ in range(3)])

    phases = ["shrink", "expand"] + (["fused"] if mode == "bgmv" else [])
    timed = {k: span(i) for i, k in enumerate(phases)}
    # warm (--warm): K launches on replica 0 only (operands left in cache by the last)
    warm = {k: graph_span(torch, stream, [calls[0][i]] * K, 3) if args.warm else float("nan")
            for i, k in enumerate(phases)}
    flops = {"shrink": acc.shrink_flops(p.ids, p.ranks, p.d_in),
             "expand": acc.expand_flops(p.ids, p.ranks, p.d_out)}
    flops["fused"] = flops["shrink"] + flops["expand"]
    kern = {}
    for name, t in timed.items():
        kern[name] = {"avg_us": float(t.mean() * 1e6), "min_us": float(t.min() * 1e6),
                      "max_us": float(t.max() * 1e6), "bytes": nbytes[name],
                      "gbs": nbytes[name] / t.mean() / 1e9,
                      "frac_of_peak": nbytes[name] / t.mean() / 1e9 / HBM_PEAK_GBS,
                      "tflops": flops[name] / t.mean() / 1e12}
        if args.warm:
            kern[name]["warm_us"] = float(warm[name] * 1e6)
    tokens = int(np.sum(p.ids >= 0))
    dom = "fused" if fused else max(("shrink", "expand"), key=lambda k: kern[k]["avg_us"])
    kname = f"{mode}_{dom}"
    achieved = kern[dom]["gbs"]
    out = {
        "metric": METRIC,
        "value": round(tokens * K / wall, 1),
        "unit": "delta tokens/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(wall / K * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": p.dtype, "data": "synthetic (seeded; random-init adapters)",
        "config": {"workload": p.name, "tokens": p.num_tokens, "adapters": p.num_adapters,
                   "ranks": sorted(set(int(r) for r in p.ranks)), "d_in": p.d_in, "d_out": p.d_out,
                   "adapter_rows": p.wq or p.dtype, "layout": one.layout,
                   "mode": mode, "path": ("fused" if fused else "shrink+expand"),
                   "placement": (args.placement if fused else None),
                   "mfma_min_tokens": (mfma_min if mode == "sgmv" else None),
                   "expand_tile": ((args.expand_tile or "width table") if mode == "sgmv" else None),
                   "shrink": ((f"tiled: 64-token tiles, {one._bench_plans[2][1]} d_in slices" if tiled
                               else "one launch") if mode == "sgmv" else None),
                   "replicas": n_rep, "timed": "HIP graph replay of the K steps",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": read_traffic(kname, p.name), "kernel": kname,
                     "algorithmic_bytes_per_launch": kern[dom]["bytes"],
                     "avg_launch_us": round(kern[dom]["avg_us"], 3), "profile": profile_path(p.name)},
        # the long segments' matrix-core use (reported, not targeted: the path
        # is HBM-bound, and algorithmic flops / dense peak stays a few percent)
        "mfma_utilisation": ({k: round(kern[k]["tflops"] / MFMA_BF16_PEAK_TFLOPS, 5)
                              for k in ("shrink", "expand")} | {"peak_tflops": MFMA_BF16_PEAK_TFLOPS}
                             if mode == "sgmv" and p.dtype == "bf16" else None),
        "kernels": {k: {kk: (round(vv, 4) if isinstance(vv, float) else vv) for kk, vv in d.items()}
                    for k, d in kern.items()},
        "gpu_tokens_per_s_kernel_time": round(
            tokens / (kern["fused"]["avg_us"] * 1e-6 if fused
                      else (timed["shrink"].mean() + timed["expand"].mean())), 1),
        "host_ms_per_step_eager": round(host_step_s * 1e3, 5),
        "kernel_sources_sha256_16": kernel_hash(),
    }
    if args.serial:
        Ks = min(K, 50)
        steps_calls = []
        for dp in reps[: min(n_rep, Ks)]:
            y, v = dp.y0.clone(), dp.new_v()
            steps_calls.append([f for pair in dp.serial_calls(y, v, stream) for f in pair])
        out["comparator"] = serial_comparator(torch, stream, steps_calls, tokens, wall / K, Ks)
    if args.cpu_seconds > 0:
        import oracle
        if p.wq:
            ad = oracle.Adapters.from_quantized(p.wq, p.a_rows, p.a_scales, p.bt_rows, p.bt_scales)
        else:
            ad = oracle.Adapters.from_stacks(p.a_rows, p.bt_rows)
        out["cpu_baseline"] = cpu_baseline([(p, ad)], p.num_tokens, args.cpu_seconds)
    del calls, reps, one
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def run_layer(args, torch):
    """The 70B-shape decoder layer: a step is the SGMV delta (segmented mode,
    automatic paths) of all seven projections; each projection's base GEMM
    y = x W^T is timed beside it for the LoRA overhead fraction.  Each
    projection rotates over its own replicas (x, y, v and adapter rows), so
    that every kernel of a step reads cold bytes."""
    from segmented_gather_gemm_segments_amd import accounting as acc
    from segmented_gather_gemm_segments_amd import binding as B
    from segmented_gather_gemm_segments_amd import runner as R
    from segmented_gather_gemm_segments_amd import workloads as wl

    stream = torch.cuda.Stream()
    mfma_min = args.mfma_min or B.LORA_DEFAULT_MFMA_MIN_TOKENS
    # a layer's dependency groups: the deltas inside a group are independent
    # (q, k and v read the same input, as do gate and up); with
    # --layer-streams groups each member runs on its own stream (all at the
    # default priority) and the group joins before the next one starts
    groups = LAYER_GROUPS if args.layer_streams == "groups" else tuple((n,) for n, _, _ in wl.LAYER_70B)
    lane_of = {n: j for g in groups for j, n in enumerate(g)}
    lanes = [stream] + [torch.cuda.Stream() for _ in range(max(len(g) for g in groups) - 1)]
    projs = []
    for name, _, _ in wl.LAYER_70B:
        p = wl.layer_projection(name)
        ls = lanes[lane_of[name]]
        dp = R.DeviceProblem(p)
        y_base = torch.empty((p.num_tokens, p.d_out), dtype=torch.bfloat16, device="cuda")
        base = B.prepare_base_gemm(dp.x, dp.w, y_base, workspace=dp.base_workspace(), stream=stream)
        with torch.cuda.stream(stream):
            base()
        _, _, _, perm_d = dp.segments()
        sp = dp.plan(B.LORA_PHASE_SHRINK, args.policy, mfma_min)
        ep = dp.plan(B.LORA_PHASE_EXPAND, args.policy, mfma_min, args.expand_tile)
        use_tiled = args.shrink == "tiled" or (args.shrink == "auto" and dp.tiled_pays(args.tile_min))
        tp = dp.plan_tiled(args.policy, args.tile_min, args.max_splits) if use_tiled else None
        sb = acc.shrink_bytes(p.ids, p.ranks, p.d_in, 2)
        eb = acc.expand_bytes(p.ids, p.ranks, p.d_out, 2)
        n_rep = n_replicas(args, min(sb, eb), cap=48)
        torch.cuda.synchronize()
        calls = []
        for i in range(n_rep):
            rp = dp if i == 0 else dp.replica()
            y = y_base.clone()
            if tp is not None:
                calls.append(B.prepare_sgmv_tiled(rp.weights, perm_d, tp[0], tp[1], tp[2], ep, rp.x, rp.new_v(),
                                                  y, stream=ls))
            else:
                calls.append(B.prepare_sgmv(rp.weights, perm_d, sp, ep, rp.x, rp.new_v(), y, stream=ls))
        p.extra.pop("w", None)   # the host copy of W is no longer needed
        projs.append({"name": name, "p": p, "dp": dp, "base": base, "calls": calls, "n_rep": n_rep, "lane": ls,
                      "sb": sb, "eb": eb, "bf": acc.base_gemm_flops(p.num_tokens, p.d_out, p.d_in),
                      "y_base": y_base, "plans": (sp, ep),
                      "shrink": (f"tiled ({tp[1]} d_in slices)" if tp is not None else "one launch")})
    torch.cuda.synchronize()
    K = args.steps

    by_name = {q["name"]: q for q in projs}

    def step(i):
        for g in groups:
            members = [by_name[n] for n in g]
            if len(members) > 1:
                fork = torch.cuda.Event()
                fork.record(stream)
                for q in members[1:]:
                    q["lane"].wait_event(fork)
            for q in members:
                c = q["calls"][i % q["n_rep"]]
                c[0]()
                c[1]()
            for q in members[1:]:
                done = torch.cuda.Event()
                done.record(q["lane"])
                stream.wait_event(done)

    wall, host_step_s = timed_graph(torch, stream, step, K, args.warmup)

    # per-kernel durations over each projection's rotation; the base GEMMs as
    # the layer's sequence of seven (each cold: the others stream 1.7 GB of W
    # between two uses of one), and one by one (k/v's W then stays cached)
    per, tot = {}, {"shrink": 0.0, "expand": 0.0}
    for q in projs:
        t = {ph: float(np.mean([graph_span(torch, q["lane"], [q["calls"][i % q["n_rep"]][k] for i in range(K)], 1)
                                for _ in range(3)]))
             for k, ph in enumerate(("shrink", "expand"))}
        tb = graph_span(torch, stream, [q["base"]] * 5, 3)
        tw = ({ph: graph_span(torch, q["lane"], [q["calls"][0][k]] * K, 3) for k, ph in enumerate(("shrink", "expand"))}
              if args.warm else None)
        p = q["p"]
        per[q["name"]] = {"d_in": p.d_in, "d_out": p.d_out, "replicas": q["n_rep"], "shrink": q["shrink"],
                          "shrink_us": round(t["shrink"] * 1e6, 3),
                          "shrink_gbs": round(q["sb"] / t["shrink"] / 1e9, 1),
                          "expand_us": round(t["expand"] * 1e6, 3),
                          "expand_gbs": round(q["eb"] / t["expand"] / 1e9, 1),
                          **({"shrink_us_warm": round(tw["shrink"] * 1e6, 3),
                              "expand_us_warm": round(tw["expand"] * 1e6, 3)} if tw else {}),
                          "base_us_alone": round(tb * 1e6, 2),
                          "base_tflops_alone": round(q["bf"] / tb / 1e12, 1)}
        q["t"] = t
        tot["shrink"] += t["shrink"]
        tot["expand"] += t["expand"]
    base_layer = graph_span(torch, stream, [q["base"] for _ in range(3) for q in projs], 3) * len(projs)
    tokens = projs[0]["p"].num_tokens
    delta = tot["shrink"] + tot["expand"]
    # dominant kernel: the phase with the larger summed time; achieved = its
    # bytes per launch / its time per launch, averaged over the seven launches
    dk = max(("shrink", "expand"), key=lambda k: tot[k])
    dbytes = sum(q["sb" if dk == "shrink" else "eb"] for q in projs)
    achieved = dbytes / tot[dk] / 1e9
    base_flops = sum(q["bf"] for q in projs)
    out = {
        "metric": METRIC,
        "value": round(tokens * K / wall, 1),
        "unit": "delta tokens/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(wall / K * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic (seeded; random-init adapters and base weights)",
        "config": {"workload": LAYER_WORKLOAD, "tokens": tokens, "adapters": 256, "ranks": [16],
                   "projections": [q["name"] for q in projs], "mode": "sgmv",
                   "mfma_min_tokens": mfma_min,
                   "expand_tile": args.expand_tile or "width table",
                   "shrink": sorted(set(q["shrink"] for q in projs)),
                   "timed": "HIP graph replay of K layer deltas (7 projections x shrink + expand)",
                   "streams": " then ".join("|".join(g) for g in groups),
                   "parallelism": "single GPU"},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": read_traffic(f"sgmv_{dk}", LAYER_WORKLOAD),
                     "kernel": f"sgmv_{dk} (its 7 launches of a layer step, averaged)",
                     "algorithmic_bytes_per_launch": int(round(dbytes / len(projs))),
                     "avg_launch_us": round(tot[dk] / len(projs) * 1e6, 3),
                     "profile": profile_path(LAYER_WORKLOAD)},
        "base_roofline": {"bound": "mfma", "achieved": round(base_flops / base_layer / 1e12, 1),
                          "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                          "frac": round(base_flops / base_layer / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4)},
        "layer": {"base_us": round(base_layer * 1e6, 2), "delta_us_kernels": round(delta * 1e6, 2),
                  "delta_us_step": round(wall / K * 1e6, 2),
                  "lora_overhead_fraction": round(delta / base_layer, 4),
                  "delta_tokens_per_s_kernel_time": round(tokens / delta, 1),
                  "delta_bytes": int(sum(q["sb"] + q["eb"] for q in projs)),
                  "delta_gbs_step": round(sum(q["sb"] + q["eb"] for q in projs) / (wall / K) / 1e9, 1),
                  "projections": per},
        "host_ms_per_step_eager": round(host_step_s * 1e3, 5),
        "kernel_sources_sha256_16": kernel_hash(),
    }
    if args.serial:
        Ks = min(K, 5)
        scalls = []
        for q in projs:
            dp = q["dp"]
            scalls += [f for pair in dp.serial_calls(q["y_base"].clone(), dp.new_v(), stream) for f in pair]
        out["comparator"] = serial_comparator(torch, stream, [scalls], tokens, wall / K, Ks)
    if args.cpu_seconds > 0:
        import oracle
        parts = [(q["p"], oracle.Adapters.from_stacks(q["p"].a_rows, q["p"].bt_rows)) for q in projs]
        out["cpu_baseline"] = cpu_baseline(parts, tokens, args.cpu_seconds)
    del projs
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return out


def run_decode_sweep(args, torch):
    """The fused decode launch (grouped placement, cold replicas) on the decode
    batch's shape with 32 .. 256 tokens over 128 adapters: with one workgroup
    per token, the time at few tokens is one workgroup's own pass."""
    from segmented_gather_gemm_segments_amd import accounting as acc
    from segmented_gather_gemm_segments_amd import binding as B
    from segmented_gather_gemm_segments_amd import runner as R
    from segmented_gather_gemm_segments_amd import workloads as wl

    stream = torch.cuda.Stream()
    K = args.steps
    rows = []
    for n in (32, 64, 128, 192, 256):
        p = wl.bgmv_decode(num_tokens=n)
        nb = acc.fused_bytes(p.ids, p.ranks, p.d_in, p.d_out, 2, p.wq)
        n_rep = n_replicas(args, nb)
        one = R.DeviceProblem(p)
        reps = [one] + [one.replica() for _ in range(n_rep - 1)]
        calls = [B.prepare_bgmv_fused(dp.weights, dp.ids, dp.x, dp.y0.clone(), None, B.LORA_BGMV_AUTO,
                                      stream=stream, token_order=dp.segments()[3]) for dp in reps]
        torch.cuda.synchronize()
        t = graph_span(torch, stream, [calls[i % n_rep] for i in range(K)], 3)
        rows.append({"tokens": n, "adapters_used": int(np.unique(p.ids).size), "us": round(t * 1e6, 3),
                     "algorithmic_bytes": int(nb), "replicas": n_rep})
        del reps, calls, one
        torch.cuda.empty_cache()
    print(json.dumps({"decode_sweep": rows, "steps": K, "kernel_sources_sha256_16": kernel_hash()}), flush=True)


def run_floor(args, torch):
    """Bare streaming reads (the library's probe kernel) and a torch
    read-modify-write, each rotating over buffers totalling more than twice the
    LLC: the floor that a launch moving that many bytes with that many
    workgroups cannot beat on this device."""
    from segmented_gather_gemm_segments_amd import binding as B
    stream = torch.cuda.Stream()
    K = args.steps
    rows = [("empty launch (256 workgroups x 16 B)", 16, 256, 256, False),
            ("17 MB read, 2048 workgroups x 256 threads", 17 * 10**6 // 2048 // 16 * 16, 2048, 256, False),
            ("36 MB read, 2048 workgroups x 256 threads", 36 * 10**6 // 2048 // 16 * 16, 2048, 256, False),
            ("36 MB read, 2048 workgroups x 256 threads, non-temporal loads",
             36 * 10**6 // 2048 // 16 * 16, 2048, 256, True),
            ("36 MB read, 256 workgroups x 512 threads", 36 * 10**6 // 256 // 16 * 16, 256, 512, False),
            ("64 MB read, 2048 workgroups x 256 threads", 64 * 10**6 // 2048 // 16 * 16, 2048, 256, False),
            ("96 MB read, 2048 workgroups x 256 threads", 96 * 10**6 // 2048 // 16 * 16, 2048, 256, False),
            ("96 MB read, 2048 workgroups x 256 threads, non-temporal loads",
             96 * 10**6 // 2048 // 16 * 16, 2048, 256, True),
            ("256 MB read, 4096 workgroups x 256 threads", 256 * 10**6 // 4096 // 16 * 16, 4096, 256, False),
            ("256 MB read, 4096 workgroups x 256 threads, non-temporal loads",
             256 * 10**6 // 4096 // 16 * 16, 4096, 256, True),
            ("256 workgroups x 34 rows of 8 KiB (71 MB, the decode shape, rows distinct)", 34 * 8192, 256, 512,
             False),
            ("111 workgroups x 34 rows of 8 KiB (31 MB)", 34 * 8192, 111, 512, False)]
    sink = torch.zeros(8192, dtype=torch.int32, device="cuda")
    table = []
    for label, bpg, groups, threads, nt in rows:
        size = bpg * groups
        n_rep = int(min(64, max(2, np.ceil(2 * LLC_BYTES / max(size, 1)))))
        buf = torch.empty(size * n_rep // 2 + 16, dtype=torch.int16, device="cuda")
        buf.fill_(1)
        fns = [B.prepare_probe_stream_read(buf[(i * size) // 2:], bpg, groups, threads, sink, stream, nt)
               for i in range(n_rep)]
        t = graph_span(torch, stream, [fns[i % n_rep] for i in range(K)], 3)
        table.append({"launch": label, "bytes": size, "us": round(t * 1e6, 3),
                      "gbs": round(size / t / 1e9, 1), "frac_of_peak": round(size / t / 1e9 / HBM_PEAK_GBS, 4)})
        del buf, fns
    # a device-scope release per workgroup (what a reduction across the
    # workgroups of one launch needs), against the same launch without it
    for pairs in (128, 256):
        part = torch.empty(2 * pairs * 64, dtype=torch.float32, device="cuda")
        out = torch.empty(pairs * 64, dtype=torch.float32, device="cuda")
        cnt = torch.zeros(pairs, dtype=torch.int32, device="cuda")
        t = {}
        for fence in (False, True):
            fn = B.prepare_probe_release(pairs, fence, part, cnt, out, stream)
            t[fence] = graph_span(torch, stream, [fn] * K, 3)
        table.append({"launch": f"{2 * pairs} workgroups, each a device-scope release and an atomic "
                                f"(the last of each pair adds both)", "bytes": 0, "us": round(t[True] * 1e6, 3),
                      "us_without_release": round(t[False] * 1e6, 3),
                      "us_per_release": round((t[True] - t[False]) * 1e6 / (2 * pairs), 4)})
        del part, out, cnt
    for mib in (64, 224):
        n = mib * 2**20 // 2
        n_rep = int(max(2, np.ceil(2 * LLC_BYTES / (2 * n))))
        ts = [torch.zeros(n, dtype=torch.bfloat16, device="cuda") for _ in range(n_rep)]
        fns = [(lambda t=t: t.add_(1.0)) for t in ts]
        t = graph_span(torch, stream, [fns[i % n_rep] for i in range(K)], 3)
        table.append({"launch": f"read-modify-write of {mib} MiB bf16 (torch in-place add)",
                      "bytes": 4 * n, "us": round(t * 1e6, 3), "gbs": round(4 * n / t / 1e9, 1),
                      "frac_of_peak": round(4 * n / t / 1e9 / HBM_PEAK_GBS, 4)})
        del ts, fns
    print(json.dumps({"floor": table, "steps": K, "peak_gbs": HBM_PEAK_GBS}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the multi-GPU "
              "sharding of this path is a design note, not a built path.", file=sys.stderr)
        sys.exit(2)
    import torch

    if args.calibrate_copy > 0:
        # a plain copy of known size: FETCH_SIZE and WRITE_SIZE of these
        # dispatches should each read MIB MiB
        n = args.calibrate_copy * 2**20
        src = torch.empty(n, dtype=torch.uint8, device="cuda")
        dst = torch.empty(n, dtype=torch.uint8, device="cuda")
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_mib": args.calibrate_copy, "dispatches": 5}), flush=True)
        return

    from segmented_gather_gemm_segments_amd import binding as B

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    B.lib()
    if args.floor:
        return run_floor(args, torch)
    if args.decode_sweep:
        return run_decode_sweep(args, torch)
    if args.churn > 0:
        return bench_churn(args, torch)
    if args.multi:
        return bench_multi(args, torch)
    if args.config == 5:
        out = run_layer(args, torch)
    elif args.config:
        out = run_config(args, torch, args.config, args.shape, args.wq)
    else:
        # the default line: the 70B layer, with the decode batch and the
        # heterogeneous paged batch nested (their own rooflines and baselines)
        print("[bench] 70B layer", file=sys.stderr, flush=True)
        out = run_layer(args, torch)
        out["configs"] = {}
        for cfg in (2, 4):
            print(f"[bench] config {cfg}", file=sys.stderr, flush=True)
            out["configs"][str(cfg)] = run_config(args, torch, cfg)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
