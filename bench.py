#!/usr/bin/env python3
"""Throughput of the paged-attention hot path on one MI355X.

Headline (the JSON line's ``value``): one decode step of an E2B-like stack --
35 layers (28 sliding, D 256, W 512; 7 full, D 512), Hq 8, Hkv 1, layers 15-34
KV-shared (15 slabs), batch 64, cached lengths uniform in [512, 4096], page size
16 over a permuted pool.  A step stores the new token's K/V on the 15 owning
layers (shared layers store nothing) and runs decode on all 35 layers; it is
the library's decode step (pakv_decode_step), captured once per batch-size
bucket into a HIP graph and replayed, as a serving engine does.  ``value`` =
algorithmic decode bytes per step (visible K/V rows once per sequence and KV
head, plus Q and O) / step time, in GB/s.

Also on the same line:
* ``roofline``: the kernel with the largest total time in the step, its
  algorithmic bytes per launch over its mean launch duration, measured with
  HIP events the library records around each launch (pakv_set_timing_events),
  against 8 TB/s;
* ``cold``: the same layer calls one at a time with the caches flushed (a
  1 GiB fill) between repetitions: sum of algorithmic bytes over sum of the
  median kernel times;
* ``decode_26b``: the 26B-A4B-like decode step (30 layers: 25 sliding D 256
  W 1024 Hq 16 Hkv 8 on a window pool, 5 full D 512 Hq 16 Hkv 2 K=V layers
  storing keys only; batch 48, lengths uniform in [2048, 16384]);
* ``decode_int8_long``: the int8 long-context step (batch 8 x 131,072; one
  full D 512 and one sliding D 256 W 1024 layer, both int8 per-token-head);
* ``extend``: the chunked-prefill stack on the E2B-like layers (4 sequences,
  cached prefixes 0 / 1024 / 2048 / 4096, 2048-token chunks stored through
  paged_kv_store on the owning layers), in TFLOP/s of visible (query, key)
  pairs (4 * D flops per pair and query head), against 2.5 PFLOP/s dense bf16;
* ``cpu_baseline``: the float64 CPU oracle timed on a bounded sample of the
  headline decode workload, same byte count per unit.

Inputs are synthetic: seeded N(0, 1) draws rounded to bf16, generated on the
device with torch's generator (data generation is not timed).  Only --gpus 1
is supported.
"""

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
METRIC = "paged-attn decode GB/s (% HBM peak); extend TFLOP/s (% bf16 MFMA peak)"
LADDER = [1, 2, 4, 8, 16, 32, 48, 64]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--extend-steps", type=int, default=3)
    ap.add_argument("--cold-reps", type=int, default=20, help="timed repetitions per call of the cold figures")
    ap.add_argument("--no-extend", action="store_true")
    ap.add_argument("--no-other-decode", action="store_true",
                    help="skip the 26B-like and the int8 and fp8 long-context steps")
    ap.add_argument("--no-cold", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="rough budget of the CPU oracle sample")
    ap.add_argument("--eager", action="store_true", help="launch the decode steps eagerly instead of from graphs")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (a known-size reference for HBM byte counters)")
    ap.add_argument("--only", choices=["e2b", "26b", "int8", "fp8", "extend", "extend_int8"], default=None,
                    help="run one workload only (profiling runs)")
    ap.add_argument("--no-ladder", action="store_true",
                    help="skip the per-batch-bucket step times (profiling runs: every dispatch is then one of "
                         "the full batch)")
    return ap.parse_args()


# ------------------------------------------------------------------ helpers

def i32(torch, x):
    return torch.tensor(np.asarray(x, dtype=np.int32), dtype=torch.int32, device="cuda")


def source_hash(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "full_attention_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def load_traffic(kernel, workload, src_hash):
    """HBM bytes per launch from the committed rocprofv3 --pmc summaries
    (profiles/*_traffic.md), if taken on the current kernel source; else None."""
    pdir = os.path.join(ROOT, "profiles")
    if not os.path.isdir(pdir):
        return None
    for name in sorted(os.listdir(pdir)):
        if not name.endswith("_traffic.md"):
            continue
        for line in open(os.path.join(pdir, name)):
            if not line.startswith("traffic-record "):
                continue
            fields = dict(re.findall(r"(\w+)=(.*?)(?= \w+=|$)", line.strip()[len("traffic-record "):]))
            if (fields.get("kernel") == kernel and fields.get("workload") == workload
                    and fields.get("source_hash") == src_hash):
                return int(fields["hbm_bytes_per_launch"])
    return None


DECODE_SOURCES = ("kernels_decode.hip", "device_common.h", "async_copy.h", "pakv_internal.h")
EXTEND_SOURCES = ("kernels_extend.hip", "device_common.h", "async_copy.h", "pakv_internal.h")
EXTEND_WL = "E2B-like extend, 35 layers, 4 sequences"
E2B_WL = "E2B-like decode, 35 layers, batch 64"
MOE_WL = "26B-like decode, 30 layers, batch 48"
INT8_WL = "int8 long decode, batch 8 x 131072"
FP8_WL = "fp8 long decode, batch 8 x 131072"


class Timing:
    """Event pairs handed to the library's timing hook."""

    def __init__(self, torch, pakv, n_pairs):
        import ctypes
        self.torch, self.pakv = torch, pakv
        self.events = [torch.cuda.Event(enable_timing=True) for _ in range(2 * n_pairs)]
        for e in self.events:        # torch creates the HIP event on first record
            e.record()
        torch.cuda.synchronize()
        self.handles = (ctypes.c_void_p * len(self.events))(*[e.cuda_event for e in self.events])

    def arm(self, mask):
        self.pakv.set_timing_events(self.handles, mask)

    def disarm(self):
        used = self.pakv.timing_pairs_used()
        self.pakv.set_timing_events(None, 0)
        return used

    def durations_ms(self, n):
        return [self.events[2 * i].elapsed_time(self.events[2 * i + 1]) for i in range(n)]


def fmt_of(spec):
    return "keqv" if spec.k_eq_v else spec.kv_dtype


# ------------------------------------------------------------------ decode workloads

def setup_decode(torch, wl, window_pool=False, ladder=LADDER):
    """Cache, cached rows, step buffers and the captured step of a decode
    workload: every owner stores its new row inside the step."""
    from full_attention_amd import pakv
    from full_attention_amd.cache import PagedKVCache
    from workloads import DeviceDraws, make_page_pool

    B = wl.num_seqs
    L = np.array(wl.cached_lens, dtype=np.int64)          # cached before the step
    kv_len = L + 1                                         # the new token is stored first
    rng = np.random.default_rng(wl.seed)
    max_kv = int(kv_len.max())
    max_pages = (max_kv + 15) // 16
    if window_pool:
        W = max(s.window for s in wl.layers)
        n_full = int(((kv_len + 15) // 16).sum()) + 4
        n_win = B * ((W + 15) // 16 + 1) + 4
        fpool = pakv.PagePool(n_full, B, max_pages, 0)
        wpool = pakv.PagePool(n_win, B, max_pages, W)
        for b in range(B):
            fpool.reserve(b, int(kv_len[b]) - 1, int(kv_len[b]))
            wpool.reserve(b, int(kv_len[b]) - 1, int(kv_len[b]))
        cache = PagedKVCache(wl.layers, wl.first_shared, {"full": n_full, "sliding": n_win})
        cache.set_page_table(fpool.table(), "full")
        cache.set_page_table(wpool.table(), "sliding")
        pool_note = f"full pool {n_full} pages, window pool {n_win} pages (its own page table)"
    else:
        pool = make_page_pool(rng, kv_len)
        cache = PagedKVCache(wl.layers, wl.first_shared, pool.num_pages)
        cache.set_page_table(pool.page_table)
        pool_note = f"one permuted pool of {pool.num_pages} pages"
    draws = DeviceDraws(wl.seed)
    layers = wl.layers
    owners = [l for l in range(len(layers)) if cache.sources[l] == l]
    # cached rows: full layers hold every position; sliding layers only the
    # positions the step's query can see (the rest keep the NaN sentinel)
    for l in owners:
        s = layers[l]
        lo = np.maximum(0, kv_len - s.window) if s.window else np.zeros(B, np.int64)
        counts = L - lo
        cu = np.concatenate([[0], np.cumsum(counts)])
        k = draws.bf16((int(cu[-1]), s.num_kv_heads, s.head_dim))
        v = None if s.k_eq_v else draws.bf16((int(cu[-1]), s.num_kv_heads, s.head_dim))
        cache.store(l, i32(torch, cu), i32(torch, lo), k, v)
        del k, v
    new_k, new_v, q, out = {}, {}, [], []
    for l, s in enumerate(layers):
        if l in owners:
            new_k[l] = draws.bf16((B, s.num_kv_heads, s.head_dim))
            new_v[l] = None if s.k_eq_v else draws.bf16((B, s.num_kv_heads, s.head_dim))
        q.append(draws.bf16((B, s.num_q_heads, s.head_dim)))
        out.append(torch.empty_like(q[-1]))
    kv_t = i32(torch, kv_len)
    torch.cuda.synchronize()
    io = [(l, q[l], out[l], new_k.get(l), new_v.get(l)) for l in range(len(layers))]
    step = cache.capture_decode_step(kv_t, max_kv, io, [b for b in ladder if b <= B] + ([B] if B not in ladder else []))
    st = dict(wl=wl, cache=cache, layers=layers, owners=owners, B=B, L=L, kv_len=kv_len, kv_t=kv_t,
              max_kv_len=max_kv, new_k=new_k, new_v=new_v, q=q, out=out, step=step, pool_note=pool_note,
              cu_new=i32(torch, np.arange(B + 1)), pos_new=i32(torch, L))
    # eager calls: one workspace for every layer, one plan per kind of layer
    need = max(cache.workspace(l, B, max_kv)[1] for l in range(len(layers)))
    cache._workspace = torch.zeros(need, dtype=torch.uint8, device="cuda")
    st["plans"] = {}
    for l in range(len(layers)):
        key = cache.plan_key(l)
        if key not in st["plans"]:
            st["plans"][key] = (l, cache.decode_plan(l, kv_t, max_kv))
    torch.cuda.synchronize()
    return st


def eager_plans(st):
    from full_attention_amd import pakv as pakv_mod
    cache = st["cache"]
    for key, (layer, buf) in st["plans"].items():
        pakv_mod.decode_plan(cache.map, layer, cache.pages_of(layer), st["kv_t"], st["B"], st["max_kv_len"], buf,
                             buf.numel())


def eager_layer(st, l):
    """Layer l's part of the step, as the captured step runs it."""
    cache = st["cache"]
    s = st["layers"][l]
    plan = st["plans"][cache.plan_key(l)][1]
    if l in st["new_k"] and s.kv_dtype == "bf16" and not s.k_eq_v:
        cache.decode_append(l, plan, st["new_k"][l], st["new_v"][l], st["q"][l], st["max_kv_len"],
                            out=st["out"][l])
        return
    if l in st["new_k"]:
        cache.store(l, st["cu_new"], st["pos_new"], st["new_k"][l], st["new_v"][l])
    cache.decode(l, st["kv_t"], st["q"][l], st["max_kv_len"], out=st["out"][l], plan=plan)


def eager_step(st):
    eager_plans(st)
    for l in range(len(st["layers"])):
        eager_layer(st, l)


def decode_bytes(st):
    """Algorithmic bytes per layer: each visible K/V row once per (sequence, KV
    head) -- K only for a K=V layer, codes plus scales for 8-bit ones -- plus
    Q read and O written."""
    per_layer = []
    for s in st["layers"]:
        vis = np.minimum(st["kv_len"], s.window) if s.window else st["kv_len"]
        row = 2 * s.head_dim if s.kv_dtype == "bf16" else s.head_dim + 4
        kv = int(vis.sum()) * s.num_kv_heads * (1 if s.k_eq_v else 2) * row
        qo = 2 * st["B"] * s.num_q_heads * s.head_dim * 2
        per_layer.append(kv + qo)
    return per_layer


def time_step(torch, st, steps, warmup, eager):
    run = (lambda: eager_step(st)) if eager else (lambda: st["step"].run(st["B"]))
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        run()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps


def host_ahead(torch, step):
    """A spin kernel to enqueue before an eager step so that the GPU reaches
    the step only after the host has queued all of it: then each launch starts
    as the previous one ends, as in a graph replay.  (The start event of
    hipExtLaunchKernelGGL completes when the GPU reaches it; on an idle GPU
    that is before the host has submitted the kernel itself, and the host's
    submission time would be counted as kernel time.)  Returns a callable."""
    step()                                   # warm: first-call costs stay out of the estimate
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    step()
    host_ms = (time.perf_counter() - t0) * 1e3
    torch.cuda.synchronize()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    cycles = 1 << 20
    start.record()
    torch.cuda._sleep(cycles)
    stop.record()
    torch.cuda.synchronize()
    per_ms = cycles / max(start.elapsed_time(stop), 1e-3)
    n = int(per_ms * (2.0 * host_ms + 0.5))
    return lambda: torch.cuda._sleep(n)


def kernel_durations(torch, pakv, step, n_launch_per_step, mask, steps):
    """Mean duration (ms) of each selected launch in a step, over `steps`
    eager steps.  The library launches each selected kernel through
    hipExtLaunchKernelGGL with a caller event pair, so the dispatch itself
    records start and stop; each step is queued behind a spin kernel
    (host_ahead) so that host-side launch time is not counted either."""
    ahead = host_ahead(torch, step)
    timing = Timing(torch, pakv, n_launch_per_step * steps)
    torch.cuda.synchronize()
    timing.arm(mask)
    try:
        for _ in range(steps):
            ahead()
            step()
    finally:
        used = timing.disarm()
    torch.cuda.synchronize()
    assert used == n_launch_per_step * steps, (used, n_launch_per_step, steps)
    d = np.array(timing.durations_ms(used)).reshape(steps, n_launch_per_step)
    return d.mean(axis=0), "hipExtLaunchKernelGGL events, eager steps queued ahead of the GPU"


def cold_calls(torch, pakv, calls, mask, reps):
    """Each call alone with the caches flushed before it (an eager 1 GiB fill,
    outside the events): 5 untimed repetitions, then `reps` timed ones; the
    median kernel time per call (ms)."""
    flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    timing = Timing(torch, pakv, 1)
    med = []
    for fn in calls:
        d = []
        for r in range(5 + reps):
            flush.fill_(r & 0xff)
            timing.arm(mask)
            try:
                fn()
            finally:
                used = timing.disarm()
            torch.cuda.synchronize()
            assert used == 1
            if r >= 5:
                d.append(timing.durations_ms(1)[0])
        med.append(float(np.median(d)))
    del flush
    return med


def batch_ladder(torch, st, reps=30):
    """The captured step replayed for the first B sequences, for each batch
    bucket B of the ladder up to the workload's batch: milliseconds per step
    (latency of smaller batches; the headline is the full batch)."""
    out = {}
    for b in [x for x in LADDER if x <= st["B"]]:
        for _ in range(5):
            st["step"].run(b)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(reps):
            st["step"].run(b)
        torch.cuda.synchronize()
        out[str(b)] = round((time.perf_counter() - t0) * 1e3 / reps, 4)
    return out


def decode_report(torch, pakv, st, args, wl_name, config):
    """The JSON object of one decode workload: warm step, roofline of the
    dominant kernel, cold per-call aggregate."""
    nl = len(st["layers"])
    ms_step = time_step(torch, st, args.steps, args.warmup, args.eager)
    per_layer = decode_bytes(st)
    step_bytes = sum(per_layer)
    value = step_bytes / (ms_step * 1e-3) / 1e9
    ksteps = max(1, min(args.steps, 10))
    mean_ms, method = kernel_durations(torch, pakv, lambda: eager_step(st), nl, pakv.TIME_DECODE, ksteps)
    groups = {}
    for l, s in enumerate(st["layers"]):
        key = f"decode_kernel<{s.head_dim},{fmt_of(s)}>"
        g = groups.setdefault(key, {"ms": 0.0, "launches": 0, "bytes": 0})
        g["ms"] += float(mean_ms[l])
        g["launches"] += 1
        g["bytes"] += per_layer[l]
    dom_name, dom = max(groups.items(), key=lambda kv: kv[1]["ms"])
    achieved = dom["bytes"] / dom["launches"] / (dom["ms"] / dom["launches"] * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": load_traffic(dom_name, wl_name, source_hash(*DECODE_SOURCES)),
                "kernel": dom_name, "launches_per_step": dom["launches"],
                "mean_launch_us": round(dom["ms"] / dom["launches"] * 1e3, 2), "timing": method,
                "algorithmic_bytes_per_launch": int(dom["bytes"] / dom["launches"]),
                "per_kernel_us_per_step": {k: round(v["ms"] * 1e3, 1) for k, v in groups.items()}}
    rep = {"value": round(value, 1), "unit": "GB/s", "ms_per_step": round(ms_step, 4),
           "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
           "config": dict(config, workload=config["workload"], algorithmic_bytes_per_step=int(step_bytes),
                          launch="eager" if args.eager else "HIP graph replay (pakv_decode_step)"),
           "roofline": roofline}
    if not args.eager and not args.no_ladder:
        rep["ms_per_step_by_batch"] = batch_ladder(torch, st)
    if not args.no_cold:
        eager_plans(st)
        med = cold_calls(torch, pakv, [lambda l=l: eager_layer(st, l) for l in range(nl)], pakv.TIME_DECODE,
                         args.cold_reps)
        cold = step_bytes / (sum(med) * 1e-3) / 1e9
        dom_layers = [l for l, s in enumerate(st["layers"]) if f"decode_kernel<{s.head_dim},{fmt_of(s)}>" == dom_name]
        dk = sum(per_layer[l] for l in dom_layers) / (sum(med[l] for l in dom_layers) * 1e-3) / 1e9
        rep["cold"] = {"value": round(cold, 1), "unit": "GB/s", "frac": round(cold / HBM_PEAK_GBS, 4),
                       "dominant_kernel_frac": round(dk / HBM_PEAK_GBS, 4),
                       "sum_median_us": round(sum(med) * 1e3, 1),
                       "method": f"each layer's decode call alone, caches flushed by a 1 GiB fill before each of "
                                 f"5 + {args.cold_reps} repetitions; sum of algorithmic bytes / sum of median "
                                 f"kernel times"}
    return rep


# ------------------------------------------------------------------ extend workload

def setup_extend(torch, kv_dtype="bf16"):
    """The E2B-like extend stack; kv_dtype other than bf16 gives every layer
    that slab format, and its extend calls go through the staged path."""
    import dataclasses
    from full_attention_amd.cache import PagedKVCache
    from workloads import DeviceDraws, e2b_extend_workload, make_page_pool

    wl = e2b_extend_workload()
    if kv_dtype != "bf16":
        wl = dataclasses.replace(wl, layers=[dataclasses.replace(s, kv_dtype=kv_dtype) for s in wl.layers])
    P = np.array(wl.cached_lens, dtype=np.int64)
    n = np.array(wl.extend_lens, dtype=np.int64)
    B = len(P)
    rng = np.random.default_rng(wl.seed)
    pool = make_page_pool(rng, P + n)
    cache = PagedKVCache(wl.layers, wl.first_shared, pool.num_pages, sentinel=True)
    cache.set_page_table(pool.page_table)
    draws = DeviceDraws(wl.seed)
    layers = wl.layers
    owners = [l for l in range(len(layers)) if cache.sources[l] == l]
    cu_n = np.concatenate([[0], np.cumsum(n)])
    chunk_k, chunk_v, q, out = {}, {}, [], []
    for l in owners:
        s = layers[l]
        lo = np.maximum(0, P - s.window + 1) if s.window else np.zeros(B, np.int64)
        counts = P - lo
        if counts.sum() > 0:
            cu = np.concatenate([[0], np.cumsum(counts)])
            k = draws.bf16((int(cu[-1]), s.num_kv_heads, s.head_dim))
            v = draws.bf16((int(cu[-1]), s.num_kv_heads, s.head_dim))
            cache.store(l, i32(torch, cu), i32(torch, lo), k, v)
        chunk_k[l] = draws.bf16((int(cu_n[-1]), s.num_kv_heads, s.head_dim))
        chunk_v[l] = draws.bf16((int(cu_n[-1]), s.num_kv_heads, s.head_dim))
    for s in layers:
        q.append(draws.bf16((int(cu_n[-1]), s.num_q_heads, s.head_dim)))
        out.append(torch.empty_like(q[-1]))
    # staged: one workspace per source layer; a KV-shared layer reuses what
    # its source's call staged (same slab, pages and lengths)
    stage_ws = {}
    if kv_dtype != "bf16":
        for l in owners:
            need = cache.staging_bytes(l, B, int(n.max()), int((P + n).max()))
            stage_ws[l] = torch.empty(need, dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    return dict(wl=wl, cache=cache, layers=layers, owners=owners, B=B, P=P, n=n, staged=kv_dtype != "bf16",
                stage_ws=stage_ws,
                cu_t=i32(torch, cu_n), P_t=i32(torch, P), chunk_k=chunk_k, chunk_v=chunk_v, q=q, out=out,
                max_q=int(n.max()), max_kv=int((P + n).max()))


def extend_layer(st, l):
    if st["staged"]:
        src = st["cache"].sources[l]
        st["cache"].extend_staged(l, st["cu_t"], st["P_t"], st["q"][l], st["max_q"], st["max_kv"], out=st["out"][l],
                                  workspace=st["stage_ws"][src], stage=src == l)
    else:
        st["cache"].extend(l, st["cu_t"], st["P_t"], st["q"][l], st["max_q"], st["max_kv"], out=st["out"][l])


def extend_step(st):
    cache = st["cache"]
    for l in range(len(st["layers"])):
        if l in st["chunk_k"]:
            cache.store(l, st["cu_t"], st["P_t"], st["chunk_k"][l], st["chunk_v"][l])
        extend_layer(st, l)


def extend_flops(st):
    """Per layer: 4 * D * Hq flops per visible (query, key) pair."""
    out = []
    for s in st["layers"]:
        pairs = 0
        for p, n in zip(st["P"], st["n"]):
            pos = np.arange(p, p + n)
            vis = pos + 1 if not s.window else np.minimum(pos + 1, s.window)
            pairs += int(vis.sum())
        out.append(4 * s.head_dim * s.num_q_heads * pairs)
    return out


def extend_report(torch, pakv, args, kv_dtype="bf16"):
    ex = setup_extend(torch, kv_dtype)
    tag = ",staged" if ex["staged"] else ""
    nl = len(ex["layers"])
    extend_step(ex)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.extend_steps):
        extend_step(ex)
    torch.cuda.synchronize()
    ms_ex = (time.perf_counter() - t0) * 1e3 / args.extend_steps
    flops = extend_flops(ex)
    tflops = sum(flops) / (ms_ex * 1e-3) / 1e12
    mean_ex, emethod = kernel_durations(torch, pakv, lambda: extend_step(ex), nl, pakv.TIME_EXTEND, 1)
    eg = {}
    for l, s in enumerate(ex["layers"]):
        key = f"extend_kernel<{s.head_dim}{tag}>"
        g = eg.setdefault(key, {"ms": 0.0, "launches": 0, "flops": 0})
        g["ms"] += float(mean_ex[l])
        g["launches"] += 1
        g["flops"] += flops[l]
    en, e = max(eg.items(), key=lambda kv: kv[1]["ms"])
    ach = e["flops"] / (e["ms"] * 1e-3) / 1e12
    rep = {"value": round(tflops, 2), "unit": "TFLOP/s", "ms_per_step": round(ms_ex, 3),
           "frac_of_mfma_peak": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
           "config": {"workload": EXTEND_WL + ", prefixes 0/1024/2048/4096, "
                                  "2048-token chunks stored on the 15 owners"
                                  + (f", {kv_dtype} per-token-head KV on every layer, extend staged"
                                     if ex["staged"] else ""), "flops_per_step": int(sum(flops)),
                      "launch": "eager (store then extend per layer)"
                                + (": staging pass + bf16 MFMA kernel per extend call" if ex["staged"] else "")},
           "roofline": {"bound": "mfma", "achieved": round(ach, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(ach / MFMA_BF16_PEAK_TFLOPS, 4),
                        "traffic": None if ex["staged"] else load_traffic(en, EXTEND_WL,
                                                                          source_hash(*EXTEND_SOURCES)),
                        "kernel": en, "launches_per_step": e["launches"], "timing": emethod,
                        "mean_launch_us": round(e["ms"] / e["launches"] * 1e3, 1),
                        "algorithmic_flops_per_launch": int(e["flops"] / e["launches"]),
                        "per_kernel_us_per_step": {k: round(v["ms"] * 1e3, 1) for k, v in eg.items()}}}
    if ex["staged"]:
        mean_st, _ = kernel_durations(torch, pakv, lambda: extend_step(ex), len(ex["owners"]), pakv.TIME_STAGE, 1)
        rep["staging_us_per_step"] = round(float(np.sum(mean_st)) * 1e3, 1)
        rep["config"]["staging"] = "one staging pass per owner; the KV-shared layers reuse their source's"
    if not args.no_cold and not ex["staged"]:
        med = cold_calls(torch, pakv, [lambda l=l: extend_layer(ex, l) for l in range(nl)], pakv.TIME_EXTEND,
                         max(3, args.cold_reps // 4))
        cold = sum(flops) / (sum(med) * 1e-3) / 1e12
        dom_layers = [l for l, s in enumerate(ex["layers"]) if f"extend_kernel<{s.head_dim}{tag}>" == en]
        dk = sum(flops[l] for l in dom_layers) / (sum(med[l] for l in dom_layers) * 1e-3) / 1e12
        rep["cold"] = {"value": round(cold, 2), "unit": "TFLOP/s", "frac": round(cold / MFMA_BF16_PEAK_TFLOPS, 4),
                       "dominant_kernel_frac": round(dk / MFMA_BF16_PEAK_TFLOPS, 4),
                       "method": "each layer's extend call alone, caches flushed by a 1 GiB fill before each "
                                 "repetition; sum of flops / sum of median kernel times"}
    del ex
    return rep


# ------------------------------------------------------------------ CPU baseline

def cpu_baseline(st, budget_s):
    """The float64 oracle (attend over logical rows) on the decode workload,
    layer by layer and sequence by sequence in step order, until about
    budget_s seconds of oracle time (or the whole step).  Rows are fresh numpy
    draws of the same shapes (timing only; no parity is claimed from this
    leg).  Throughput counts the same algorithmic bytes as the GPU line."""
    from oracle import attend, decode_positions
    from workloads import bf16_to_f32, normal_bf16
    try:
        from threadpoolctl import threadpool_info
        blas = [(i.get("internal_api"), i.get("num_threads")) for i in threadpool_info()]
    except Exception:
        blas = []
    rng = np.random.default_rng(7)
    layers = st["layers"]
    done_bytes, spent, units = 0, 0.0, 0
    # a first pass over the step, then a second pass that repeats each unit's
    # oracle call on the same rows until about budget_s seconds in total
    for rep_pass in range(2):
        reps = 1 if rep_pass == 0 else max(0, int(np.ceil((budget_s - spent) / max(spent, 1e-3))))
        if reps == 0:
            break
        for l, s in enumerate(layers):
            for b in range(st["B"]):
                n = int(st["kv_len"][b])
                lo = max(0, n - s.window) if s.window else 0
                pos = np.arange(lo, n)
                kr = bf16_to_f32(normal_bf16(rng, (len(pos), 1, s.head_dim))).astype(np.float64)
                vr = bf16_to_f32(normal_bf16(rng, (len(pos), 1, s.head_dim))).astype(np.float64)
                qv = bf16_to_f32(normal_bf16(rng, (1, s.num_q_heads, s.head_dim))).astype(np.float64)
                for _ in range(reps):
                    t0 = time.perf_counter()
                    attend(qv, decode_positions(n), kr, vr, pos, s.window, s.sm_scale)
                    spent += time.perf_counter() - t0
                    units += 1
                    done_bytes += (len(pos) * s.num_kv_heads * 2 * 2 * s.head_dim
                                   + 2 * s.num_q_heads * s.head_dim * 2)
    cores = len(os.sched_getaffinity(0))
    threads = max([t for _, t in blas if t] or [1])
    return {"value": round(done_bytes / spent / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": (f"float64 oracle attend() on {units} (layer, sequence) decode units of the same "
                       f"workload in step order (the whole 35-layer x 64-sequence step, then each unit "
                       f"repeated on its rows up to the budget); {spent:.1f} s of oracle time; "
                       f"host affinity {cores} cores; BLAS {blas}")}


# ------------------------------------------------------------------ main

def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the path would shard by sequence, with no exchange for decode)", file=sys.stderr)
        sys.exit(2)
    import torch
    from full_attention_amd import pakv
    from workloads import e2b_decode_workload, int8_long_workload, moe26b_decode_workload

    torch.cuda.set_device(0)
    if args.calibrate_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    def progress(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    line = {"metric": METRIC, "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic (seeded N(0,1) rounded to bf16; random page permutation)"}
    st = None
    if args.only in (None, "e2b"):
        st = setup_decode(torch, e2b_decode_workload())
        progress("E2B-like decode set up")
        rep = decode_report(torch, pakv, st, args, E2B_WL, {
            "workload": E2B_WL + " (28 sliding D256 W512 + 7 full D512; Hq 8, Hkv 1; layers 15-34 KV-shared, "
                                 "15 slabs; context U[512,4096]; page 16)",
            "global_batch": st["B"], "seq_len": int(st["max_kv_len"]), "layers": len(st["layers"]),
            "step": "plan 2 kinds of layer + 15 owners store their new K/V and decode in one launch each "
                    "+ 20 shared layers decode"})
        line.update(value=rep["value"], ms_per_step=rep["ms_per_step"], config=rep["config"],
                    frac_of_hbm_peak=rep["frac_of_hbm_peak"], roofline=rep["roofline"])
        if "ms_per_step_by_batch" in rep:
            line["ms_per_step_by_batch"] = rep["ms_per_step_by_batch"]
        if "cold" in rep:
            line["cold"] = rep["cold"]
        progress(f"E2B-like decode: {rep['value']} GB/s")
    if not args.no_other_decode and args.only in (None, "26b"):
        mo = setup_decode(torch, moe26b_decode_workload(), window_pool=True)
        progress("26B-like decode set up")
        line["decode_26b"] = decode_report(torch, pakv, mo, args, MOE_WL, {
            "workload": MOE_WL + " (25 sliding D256 W1024 Hq16 Hkv8 on a window pool; 5 full D512 Hq16 Hkv2 "
                                 "K=V, keys only; context U[2048,16384]; page 16; " + mo["pool_note"] + ")",
            "global_batch": mo["B"], "seq_len": int(mo["max_kv_len"]), "layers": len(mo["layers"]),
            "step": "plan 2 kinds of layer + 25 sliding owners store and decode in one launch each + 5 K=V "
                    "owners store their key row then decode"})
        progress(f"26B-like decode: {line['decode_26b']['value']} GB/s")
        del mo
        torch.cuda.empty_cache()
    if not args.no_other_decode and args.only in (None, "int8"):
        lo = setup_decode(torch, int8_long_workload(), window_pool=True)
        progress("int8 long decode set up")
        line["decode_int8_long"] = decode_report(torch, pakv, lo, args, INT8_WL, {
            "workload": INT8_WL + " (one full D512 and one sliding D256 W1024 layer, Hq 8 Hkv 1, int8 "
                                  "per-token-head; " + lo["pool_note"] + ")",
            "global_batch": lo["B"], "seq_len": int(lo["max_kv_len"]), "layers": 2,
            "step": "plan 2 kinds of layer + 2 int8 owners store their new row then decode"})
        progress(f"int8 long decode: {line['decode_int8_long']['value']} GB/s")
        del lo
        torch.cuda.empty_cache()
    if not args.no_other_decode and args.only in (None, "fp8"):
        import dataclasses
        wl8 = int8_long_workload()
        wl8 = dataclasses.replace(wl8, layers=[dataclasses.replace(s, kv_dtype="fp8") for s in wl8.layers])
        f8 = setup_decode(torch, wl8, window_pool=True)
        progress("fp8 long decode set up")
        line["decode_fp8_long"] = decode_report(torch, pakv, f8, args, FP8_WL, {
            "workload": FP8_WL + " (the int8 long-context workload with fp8 E4M3 per-token-head KV: one full "
                                 "D512 and one sliding D256 W1024 layer, Hq 8 Hkv 1; " + f8["pool_note"] + ")",
            "global_batch": f8["B"], "seq_len": int(f8["max_kv_len"]), "layers": 2,
            "step": "plan 2 kinds of layer + 2 fp8 owners store their new row then decode"})
        progress(f"fp8 long decode: {line['decode_fp8_long']['value']} GB/s")
        del f8
        torch.cuda.empty_cache()
    if not args.no_extend and args.only in (None, "extend"):
        line["extend"] = extend_report(torch, pakv, args)
        progress(f"extend: {line['extend']['value']} TFLOP/s")
    if not args.no_extend and args.only in (None, "extend_int8"):
        torch.cuda.empty_cache()
        line["extend_int8"] = extend_report(torch, pakv, args, kv_dtype="int8")
        progress(f"int8 extend (staged): {line['extend_int8']['value']} TFLOP/s")
    if "value" not in line:                 # a single non-headline workload (profiling runs)
        key = next(k for k in ("decode_26b", "decode_int8_long", "decode_fp8_long", "extend", "extend_int8")
                   if k in line)
        line.update(value=line[key]["value"], unit=line[key]["unit"], ms_per_step=line[key]["ms_per_step"],
                    config=line[key]["config"])
    if not args.no_cpu_baseline and st is not None:
        line["cpu_baseline"] = cpu_baseline(st, args.cpu_seconds)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
