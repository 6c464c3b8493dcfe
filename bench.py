#!/usr/bin/env python3
"""Benchmark of the multi-LoRA SGMV delta hot path on one MI355X.

One step = one pass of the whole hot path over one batch: the on-device segment build
(counting sort of the tokens by adapter, work descriptors) followed by the fused delta
y += scale * (x A^T) B^T, both through the libsgmv C-ABI on one HIP stream. For bf16 batches
of at most 512 tokens the step is one call of sgmv_lora_delta_ids, whose single launch does
both (--step one, the default there); --step two times the builder launch and the delta
launch as separate calls. Inputs are synthetic and already resident in HBM when the timed
region starts.

Default workload: decode, 256 tokens (one per sequence), d_in = d_out = 4096, rank 16, a pool
of 64 adapters, bf16 with fp32 accumulation. The step cycles through several independent
copies of every buffer (pool, x, y, ids, segment arrays) whose total size is about twice the
256 MB last-level cache, so each step reads its operands from HBM rather than from that
cache.

Timing: W untimed warm-up steps, then K plain steps between two device synchronisations
(ms_per_step, value = tokens with an adapter per second), with two HIP events recorded on the
launch stream around them. The roofline takes the kernel that does the delta (including the
build it does itself in the single-launch step): its average launch duration is the timed
region's event time over K for the single launch (one kernel per step; the figure includes
the gaps between launches), and for two launches the event time of K launches of that kernel
alone, run after the timed region on the same rotating buffer sets. The roofline figure
divides the algorithmic bytes of one delta launch (x rows and y rows read and written for
every token with an adapter, each used adapter's true-rank A and B once, 12 bytes of index
per token) by that duration, against the 8 TB/s HBM peak. The builder's figure for two
launches is the timed step less the delta alone: a few microseconds of kernel, which the host
cannot launch alone as fast as the GPU runs it. The line also gives the host's time to issue
each region's launches; a warning goes to stderr if it comes near the region's own time.
A further K steps, outside the timed region, give the spread of launch durations: every
eighth launch records a pair of events in its own dispatch (start and end of the kernel, no
extra stream packets). Such launches can run longer than plain ones (the single launch by
about 1.7 us), so these samples give the p10/p50/p90 only, except with --trace, whose
per-step batches change and whose builder and delta averages come from them.

--trace (with --step two) replaces the fixed batch by seeded decode traces, one per buffer
set, in which sequences keep their adapter and join or leave the batch; --segment-cache then
builds through the grouping cache, and the line reports the builder time on steps with
unchanged and with changed ids.

The CPU baseline is the fp64 oracle (plain per-token NumPy loop) on the same batch, repeated
for about 10 s on this host.

--phase-stamps instead prints the per-phase times of the decode single launch, read from
libsgmv_stamps.so (the library built with phase stamps in that kernel).

Prints exactly one JSON line on stdout; progress goes to stderr.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "LoRA-delta tokens/s + achieved HBM GB/s (% of peak), decode bs=256 d=4096 r=16"
HBM_PEAK_GBPS = 8000.0
MALL_BYTES = 256 * 2 ** 20
PROFILES = os.path.join(ROOT, "profiles")
# sources of the fused delta kernel: byte-counter results are kept only while these match
KERNEL_SOURCES = [os.path.join(ROOT, "segmented_gather_gemv_amd", "csrc", f)
                  for f in ("delta_bf16.h", "delta_bf16_fused.hip", "delta_bf16_build.hip",
                            "common.h", "workspace.h", "segments_common.h")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


class HipEvents:
    """Raw HIP events through the runtime torch has loaded (same SONAME)."""

    def __init__(self):
        self.lib = ctypes.CDLL("libamdhip64.so.7")
        self.lib.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.lib.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        self.lib.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.lib.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.lib.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self, n):
        evs = []
        for _ in range(n):
            e = ctypes.c_void_p()
            assert self.lib.hipEventCreate(ctypes.byref(e)) == 0
            evs.append(e)
        return evs

    def record(self, e, stream):
        assert self.lib.hipEventRecord(e, stream) == 0

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.lib.hipEventDestroy(e)


def region_us(ev, stream, fn, n):
    """Mean microseconds per call of fn(i), i < n, from two HIP events recorded on `stream` (a
    torch stream, made current for the calls) around all n calls: the kernels and the gaps
    between them, with no event inside any launch. Also returns the host's time per call to
    issue them (no wait inside the loop): when that is close to the first figure, the host's
    launch rate, not the GPU, set it."""
    import torch
    h = ctypes.c_void_p(stream.cuda_stream)
    e = ev.create(2)
    with torch.cuda.stream(stream):
        ev.record(e[0], h)
        t0 = time.perf_counter()
        for i in range(n):
            fn(i)
        t1 = time.perf_counter()
        ev.record(e[1], h)
    torch.cuda.synchronize()
    t = ev.elapsed_ms(e[0], e[1]) / n * 1e3
    ev.destroy(e)
    return t, (t1 - t0) / n * 1e6


def kernel_source_sha() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def traffic_path(workload: str, one_launch: bool) -> str:
    entry = "sgmv_lora_delta_ids" if one_launch else "sgmv_lora_delta"
    return os.path.join(PROFILES, f"{entry}_{workload}_traffic.json")


def load_traffic(workload: str, one_launch: bool):
    """HBM bytes per delta launch from the committed rocprofv3 counter summary, if it was
    taken on the current kernel source; else None."""
    p = traffic_path(workload, one_launch)
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p))
    except Exception:
        return None
    if d.get("kernel_sha") != kernel_source_sha():
        return None
    return d.get("hbm_bytes_per_launch")


def _counter_per_dispatch(csv_path: str, counter: str, name_part: str):
    """Mean of a rocprofv3 --pmc counter over the dispatches of one kernel: among kernel names
    containing name_part, the one dispatched most often (counter_collection.csv has one row
    per dispatch and counter)."""
    import csv
    by_name = {}
    for row in csv.DictReader(open(csv_path)):
        if row.get("Counter_Name") == counter and name_part in row.get("Kernel_Name", ""):
            by_name.setdefault(row["Kernel_Name"], []).append(float(row["Counter_Value"]))
    if not by_name:
        raise SystemExit(f"no {counter} rows for kernels matching '{name_part}' in {csv_path}")
    vals = max(by_name.values(), key=len)
    return sum(vals) / len(vals), len(vals)


def write_traffic(args):
    """Turn four rocprofv3 counter CSVs (delta FETCH_SIZE, delta WRITE_SIZE, copy FETCH_SIZE,
    copy WRITE_SIZE) into profiles/<entry point>_<workload>_traffic.json. The counters read
    KiB per dispatch; each is scaled by bytes-moved / counter-reading of a plain device copy
    of known size measured the same way."""
    d_fetch, d_wr, c_fetch, c_wr = args.write_traffic
    copy_bytes = args.copy_mib * 2 ** 20
    f_kib, n1 = _counter_per_dispatch(d_fetch, "FETCH_SIZE", "delta_bf16_kernel")
    w_kib, n2 = _counter_per_dispatch(d_wr, "WRITE_SIZE", "delta_bf16_kernel")
    cf_kib, _ = _counter_per_dispatch(c_fetch, "FETCH_SIZE", "elementwise")
    cw_kib, _ = _counter_per_dispatch(c_wr, "WRITE_SIZE", "elementwise")
    f_scale = copy_bytes / cf_kib
    w_scale = copy_bytes / cw_kib
    out = {
        "workload": args.workload,
        "kernel": ("delta_bf16_kernel<fused, aligned, build>" if args.step == "one"
                   else "delta_bf16_kernel<fused, aligned>"),
        "kernel_sha": kernel_source_sha(),
        "fetch_kib_per_dispatch": f_kib, "write_kib_per_dispatch": w_kib,
        "dispatches": [n1, n2],
        "copy_bytes": copy_bytes, "copy_fetch_kib": cf_kib, "copy_write_kib": cw_kib,
        "fetch_bytes_per_kib": f_scale, "write_bytes_per_kib": w_scale,
        "hbm_bytes_per_launch": f_kib * f_scale + w_kib * w_scale,
    }
    path = traffic_path(args.workload, args.step == "one")
    json.dump(out, open(path, "w"), indent=1)
    print(json.dumps(out))


def calibration_copy(args):
    """A plain device copy of known size: the scale reference for the byte counters and, over
    several buffer pairs whose total exceeds the last-level cache (--copy-sets), the copy
    time of a working set that starts in HBM, for comparison with the delta kernel."""
    import torch
    n = args.copy_mib * 2 ** 20 // 2
    pairs = [(torch.ones(n, dtype=torch.bfloat16, device="cuda"),
              torch.empty(n, dtype=torch.bfloat16, device="cuda")) for _ in range(args.copy_sets)]
    torch.cuda.synchronize()
    reps = max(8, 2 * args.copy_sets)
    for i in range(reps):  # elementwise kernel: reads a, writes b, copy_mib MiB each way
        a, b = pairs[i % args.copy_sets]
        torch.mul(a, 1.0, out=b)
    torch.cuda.synchronize()
    log(f"elementwise copy of {args.copy_mib} MiB, {reps} times over {args.copy_sets} pairs")


def stream_ceiling(read_bytes: int, write_bytes: int, reps: int, ev, stream) -> dict:
    """The best time of a hand-written HIP streaming kernel (libsgmv_bench.so) that reads
    read_bytes and writes write_bytes in 16-byte lanes in one launch, over a sweep of launch
    shapes (threads per workgroup x loads in flight per thread), with the buffers rotating over
    sets larger than twice the last-level cache so every launch starts in HBM; each shape is
    timed like the delta kernel (stream events around `reps` back-to-back launches)."""
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "segmented_gather_gemv_amd", "libsgmv_bench.so"))
    lib.sgmv_bench_stream.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p,
                                      ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                      ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    rb = (read_bytes + 15) // 16 * 16
    wb = (write_bytes + 15) // 16 * 16
    n_sets = max(2, -(-2 * MALL_BYTES // (rb + wb)))
    g = torch.Generator(device="cuda").manual_seed(5)
    src = [torch.randint(0, 1 << 30, (rb // 4,), dtype=torch.int32, device="cuda", generator=g)
           for _ in range(n_sets)]
    dst = [torch.empty(max(wb // 4, 4), dtype=torch.int32, device="cuda") for _ in range(n_sets)]
    torch.cuda.synchronize()
    h = ctypes.c_void_p(stream.cuda_stream)
    rows = []
    for block in (256, 512, 1024):
        for unroll in (1, 2, 4, 8, 16):
            def launch(i):
                rc = lib.sgmv_bench_stream(src[i % n_sets].data_ptr(), rb,
                                           dst[i % n_sets].data_ptr(), wb, block, unroll,
                                           None, None, h)
                assert rc == 0, f"sgmv_bench_stream failed ({rc})"
            with torch.cuda.stream(stream):
                for i in range(2 * n_sets):
                    launch(i)
            torch.cuda.synchronize()
            us, host = region_us(ev, stream, launch, reps)
            rows.append({"block": block, "unroll": unroll, "us": round(us, 3),
                         "host_issue_us": round(host, 2)})
    best = min(rows, key=lambda r: r["us"])
    gbps = (rb + wb) / (best["us"] * 1e-6) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return {"read_bytes": rb, "write_bytes": wb, "buffer_sets": n_sets, "best": best,
            "gbps": gbps, "frac_of_peak": gbps / HBM_PEAK_GBPS, "sweep": rows}


def flush_last_level_cache(n_bytes: int = 2 * MALL_BYTES):
    """Writes n_bytes of device memory (untimed), so what setup left in the 256 MB memory-side
    cache is evicted before a timed region."""
    import torch
    buf = torch.empty(n_bytes // 4, dtype=torch.int32, device="cuda")
    buf.fill_(1)
    torch.cuda.synchronize()
    del buf


def device_clocks() -> dict:
    """Shader and memory clocks as rocm-smi reports them (current level), or an error note."""
    import subprocess
    try:
        r = subprocess.run(["rocm-smi", "--showclocks", "--json"], capture_output=True,
                           text=True, timeout=30)
        d = json.loads(r.stdout)
        card = d[sorted(d)[0]]
        keep = {k: v for k, v in card.items() if "clock" in k.lower() and
                any(c in k.lower() for c in ("sclk", "mclk", "fclk", "socclk"))}
        return keep or card
    except Exception as e:  # the tool may be missing or print no JSON
        return {"error": f"rocm-smi --showclocks: {type(e).__name__}"}


def cpu_baseline(w, seconds: float):
    """The oracle as it stands, on the same batch, repeated for about `seconds`."""
    import numpy as np
    import oracle
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max([i.get("num_threads", 1) for i in info] or [1])
    except Exception:
        threads = 1
    x = w.x.float().numpy()
    y0 = w.y0.float().numpy()
    a = w.a.float().numpy()
    b = w.b.float().numpy()
    ids = w.ids.numpy()
    rank = w.rank.numpy()
    alpha = w.alpha.numpy()
    n_tok = int((ids >= 0).sum())
    reps = 0
    t0 = time.perf_counter()
    while True:
        oracle.lora_delta(x, y0, ids, a, b, rank, alpha)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds or reps >= 1000:
            break
    one_thread = ""
    try:  # the same loop held to one BLAS thread, briefly
        import threadpoolctl
        with threadpoolctl.threadpool_limits(1):
            r1, t1 = 0, time.perf_counter()
            while True:
                oracle.lora_delta(x, y0, ids, a, b, rank, alpha)
                r1 += 1
                e1 = time.perf_counter() - t1
                if e1 >= min(3.0, seconds) or r1 >= 1000:
                    break
        one_thread = f"; with one BLAS thread {n_tok * r1 / e1:.0f} tokens/s ({r1} times)"
    except Exception:
        pass
    return {"value": n_tok * reps / el, "unit": "tokens/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{w.note}: the full batch ({n_tok} tokens with an adapter) through the "
                      f"fp64 per-token oracle, {reps} times in {el:.1f} s on "
                      f"{os.cpu_count()} visible host cores{one_thread}"}


def merge_bench(args):
    """Merged weight (sgmv_merge_adapter) on the decode shapes: W 4096 x 4096 bf16, rank 16.
    Times the merge kernel (W and W' rotating over sets larger than the last-level cache), the
    base GEMM x W^T of the decode batch (torch.matmul, the vendor GEMM library) and the unmerged
    delta of a batch whose 256 tokens all use one adapter, each from stream events around a run
    of its launches, and
    reports the merge as HBM bandwidth against the peak plus the number of steps after which
    merging pays for itself (Ascend article 4.4)."""
    import torch
    import segmented_gather_gemv_amd as sg
    import workloads

    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(device=dev)
    ev = HipEvents()
    w = workloads.get("decode")
    N, K = w.N, w.K
    e = 2
    n_sets = max(2, -(-2 * MALL_BYTES // (2 * N * K * e)))
    g = torch.Generator().manual_seed(7)
    with torch.cuda.stream(stream):
        pool = sg.sgmv_pool_pack(w.a.to(dev), w.b.to(dev), w.rank.tolist(), w.alpha.tolist())
        Ws = [(torch.randn(N, K, generator=g) * 0.02).to(torch.bfloat16).to(dev)
              for _ in range(n_sets)]
        Wo = [torch.empty_like(Ws[0]) for _ in range(n_sets)]
        x = w.x.to(dev)
        ids = torch.zeros(w.M, dtype=torch.int32, device=dev)  # one adapter for the batch
        ys = [w.y0.to(dev) for _ in range(n_sets)]
        seg = sg.sgmv_segments_alloc(w.M, w.L, 0, dev)
    torch.cuda.synchronize()
    log(f"merge bench: W {N}x{K} bf16 x {n_sets} sets, rank {int(w.rank[0])}")

    def timed(fn, reps):  # us per call
        with torch.cuda.stream(stream):
            for i in range(args.warmup):
                fn(i)
        torch.cuda.synchronize()
        t, host = region_us(ev, stream, fn, reps)
        if host > 0.9 * t:
            log(f"warning: host issue {host:.2f} us per call against {t:.2f} us: launch-bound")
        return t

    reps = max(16, min(args.steps, 200))
    merge_us = timed(lambda i: sg.sgmv_merge_adapter(Ws[i % n_sets], pool, 0,
                                                    out=Wo[i % n_sets]), reps)
    delta_us = timed(lambda i: sg.sgmv_lora_delta_ids(ids, x, pool, seg, ys[i % n_sets]), reps)
    gemm_us = timed(lambda i: torch.matmul(x, Ws[i % n_sets].t()), reps)  # base y = x W^T
    r = int(w.rank[0])
    alg = 2 * N * K * e + r * (N + K) * e
    gbps = alg / (merge_us * 1e-6) / 1e9
    log(f"merge {merge_us:.2f} us ({gbps:.0f} GB/s, {gbps / HBM_PEAK_GBPS * 100:.1f}% of peak) | "
        f"base GEMM {gemm_us:.2f} us | one-adapter delta {delta_us:.2f} us | break-even "
        f"{merge_us / delta_us:.1f} steps")
    print(json.dumps({
        "metric": "merged-weight build (sgmv_merge_adapter) HBM GB/s, W 4096x4096 bf16 r=16",
        "value": gbps, "unit": "GB/s", "n_gpus": 1, "steps": reps, "warmup": args.warmup,
        "ms_per_step": merge_us / 1e3, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "merge adapter 0 of the decode pool into a random base weight",
                   "N": N, "K": K, "rank": r, "buffer_sets": n_sets,
                   "merge_kernel_us": merge_us, "base_gemm_us_bs256": gemm_us,
                   "unmerged_delta_us_one_adapter_bs256": delta_us,
                   "break_even_steps": merge_us / delta_us,
                   "algorithmic_bytes_per_launch": alg},
        "roofline": {"bound": "hbm", "achieved": gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": gbps / HBM_PEAK_GBPS, "traffic": None},
        "cpu_baseline": None}), flush=True)


def chunk_sweep(args):
    """Chunk size against batch shape (the chunk-size rule of sgmv_chunk_size_for_batch):
    step time (segment build + fused delta) for batches of M tokens spread uniformly over n
    adapters of the decode pool (d = 4096, rank 16), at several chunk sizes, with two launches
    and, where it applies, as one sgmv_lora_delta_ids launch. Every figure comes from stream
    events around a run of launches: whole steps for the total, each kernel alone for the
    builder and delta columns."""
    import numpy as np
    import torch
    import segmented_gather_gemv_amd as sg
    import workloads

    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(device=dev)
    ev = HipEvents()
    lib = sg.library()
    specs = [(256, 1), (256, 4), (256, 16), (256, 64), (512, 1), (512, 8), (512, 64),
             (1024, 1), (1024, 8), (1024, 64), (2048, 1), (2048, 16), (4096, 1), (4096, 16),
             (8192, 1), (8192, 12), (8192, 64)]
    chunks = [0, 16, 32, 64, 128]
    if args.sweep_ranks != "16":  # a shorter grid per rank
        specs = [(256, 1), (256, 16), (512, 8), (1024, 1), (1024, 16), (2048, 16), (4096, 16),
                 (8192, 12)]
        chunks = [0, 16, 32]
    reps, sets = 40, 4
    s_handle = ctypes.c_void_p(stream.cuda_stream)
    dflt_opts = sg.LaunchOpts()
    dflt = dflt_opts.ref()
    rows = []
    for R, (M, n_ad) in [(int(r), sp) for r in args.sweep_ranks.split(",") for sp in specs]:
        w = workloads.custom(M=M, K=4096, N=4096, L=64, R=R, name="sweep", seed=M + n_ad)
        rng = np.random.default_rng(M * 100 + n_ad)
        ad = rng.choice(64, size=n_ad, replace=False)
        w.ids = torch.from_numpy(ad[rng.integers(0, n_ad, M)].astype(np.int32))
        with torch.cuda.stream(stream):
            pool = sg.sgmv_pool_pack(w.a.to(dev), w.b.to(dev), w.rank.tolist(), w.alpha.tolist())
            xs = [w.x.to(dev) for _ in range(sets)]
            ys = [w.y0.to(dev) for _ in range(sets)]
            ids = w.ids.to(dev)
        torch.cuda.synchronize()
        for C in chunks:
            segs = [sg.sgmv_segments_alloc(M, 64, C, dev) for _ in range(sets)]
            calls = []  # ctypes arguments made once: the loops below only launch
            for st in range(sets):
                sl, n_sl = sg._slices([(ys[st], 0)], pool, M)
                calls.append(((ctypes.c_void_p(ids.data_ptr()), M, 64, C, 1,
                               ctypes.byref(segs[st].desc)),
                              (ctypes.c_void_p(xs[st].data_ptr()), xs[st].stride(0), M,
                               ctypes.byref(pool.desc), ctypes.byref(segs[st].desc), sl, n_sl)))
            modes = ["two"] + (["one"] if M <= 512 else [])
            for mode in modes:
                rcs = []

                def build(i):
                    rcs.append(lib.sgmv_build_segments_ex(*calls[i % sets][0], None, s_handle))

                def delta(i):
                    bargs, dargs = calls[i % sets]
                    if mode == "one":
                        rcs.append(lib.sgmv_lora_delta_ids_ex(bargs[0], *dargs, dflt, s_handle))
                    else:
                        rcs.append(lib.sgmv_lora_delta_ex(*dargs, dflt, s_handle))

                def full(i):
                    if mode == "two":
                        build(i)
                    delta(i)

                for i in range(5):
                    full(i)
                torch.cuda.synchronize()
                t, th = region_us(ev, stream, full, reps)
                b, bh = region_us(ev, stream, build, reps) if mode == "two" else (None, 0.0)
                d, dh = region_us(ev, stream, delta, reps) if mode == "two" else (t, th)
                assert not any(rcs), f"library call failed with status {max(rcs)}"
                row = {"M": M, "adapters": n_ad, "rank": R, "chunk": C, "launches": mode,
                       "build_us": round(b, 2) if b is not None else None,
                       "delta_us": round(d, 2), "total_us": round(t, 2),
                       "host_issue_us": [round(th, 2), round(bh, 2), round(dh, 2)]}
                rows.append(row)
                log(json.dumps(row))
            del segs
    best = {}
    for r in rows:
        k = (r["rank"], r["M"], r["adapters"])
        if k not in best or r["total_us"] < best[k]["total_us"]:
            best[k] = r
    print(json.dumps({"metric": "build + delta step time by chunk size (sweep)",
                      "value": None, "unit": "us", "n_gpus": 1, "data": "synthetic",
                      "config": {"workload": "M tokens uniform over n adapters of a 64-adapter "
                                             "pool, d=4096, every adapter at rank r",
                                 "ranks": args.sweep_ranks},
                      "rows": rows,
                      "best": [best[k] for k in sorted(best)]}), flush=True)


def phase_stamps(args):
    """Per-phase times of the decode single launch from libsgmv_stamps.so, the profiling copy
    of the library whose single-launch kernel records the 100 MHz real-time counter at its
    phase points (thread 0 of every workgroup; the last point waits for the workgroup's stores).
    The stamp stores and that wait make the copy slightly slower than the library; the phases
    are what it is for. Prints one JSON line: p10/p50/p90 of every phase in ns over the
    workgroups that carry a piece, over `reps` rounds of rotating-buffer launches."""
    import ctypes

    import numpy as np
    import torch
    import segmented_gather_gemv_amd as sg
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    path = os.path.join(ROOT, "segmented_gather_gemv_amd", "libsgmv_stamps.so")
    if not os.path.exists(path):
        print("libsgmv_stamps.so is not built (segmented_gather_gemv_amd/build.py builds it)",
              file=sys.stderr)
        sys.exit(1)
    lib = ctypes.CDLL(path)
    base = sg.library()
    f = lib.sgmv_lora_delta_ids_ex
    f.argtypes, f.restype = base.sgmv_lora_delta_ids_ex.argtypes, ctypes.c_int
    lib.sgmv_phase_stamps.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    lib.sgmv_phase_stamps.restype = ctypes.c_int
    vp = ctypes.c_void_p
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(device=dev)  # default priority
    w = workloads.get("decode")
    n_sets = 24
    sets = []
    with torch.cuda.stream(stream):
        a_dev, b_dev = w.a.to(dev), w.b.to(dev)
        for _ in range(n_sets):
            pool = sg.sgmv_pool_pack(a_dev, b_dev, w.rank.tolist(), w.alpha.tolist())
            x, y, ids = w.x.to(dev), w.y0.to(dev), w.ids.to(dev)
            seg = sg.sgmv_segments_alloc(w.M, w.L, 0, dev)
            sl, n_sl = sg._slices([(y, 0)], pool, w.M)
            sets.append(dict(pool=pool, x=x, y=y, ids=ids, seg=seg, sl=sl, n_sl=n_sl))
    torch.cuda.synchronize()
    names = ["launch to ids in", "ids to tokens known", "x in, first K step multiplied",
             "partial published (B, y in)", "counter complete", "partials summed, h in LDS",
             "expand, y stores issued", "y stores complete"]
    phases = {k: [] for k in names}
    ends, spreads, n_full, starts = [], [], [], []
    reps = 8
    rows_max, slots = 8192, 16
    for rep in range(reps):
        with torch.cuda.stream(stream):
            for i in range(n_sets + 1):  # every launch overwrites the rows; the last one stays
                st = sets[(i + rep) % n_sets]
                rc = f(vp(st["ids"].data_ptr()), vp(st["x"].data_ptr()), st["x"].stride(0), w.M,
                       ctypes.byref(st["pool"].desc), ctypes.byref(st["seg"].desc), st["sl"],
                       st["n_sl"], None, vp(stream.cuda_stream))
                if rc != 0:
                    raise SystemExit(f"sgmv_lora_delta_ids_ex returned {rc}")
        torch.cuda.synchronize()
        buf = np.zeros(rows_max * slots, dtype=np.uint64)
        if lib.sgmv_phase_stamps(buf.ctypes.data_as(vp), buf.nbytes) != 0:
            raise SystemExit("sgmv_phase_stamps failed")
        st_ = buf.reshape(rows_max, slots).astype(np.int64)
        live = st_[:, 0] > 0
        full = live & (st_[:, 8] > st_[:, 0])  # workgroups that ran a piece to its end
        t0 = st_[live, 0].min()
        rows = st_[full]
        for k, nm in enumerate(names):
            phases[nm].extend(((rows[:, k + 1] - rows[:, k]) * 10.0).tolist())
        ends.append(float((rows[:, 8].max() - t0) * 10.0))
        spreads.append(float((st_[live, 0].max() - t0) * 10.0))
        starts.extend(((rows[:, 0] - t0) * 10.0).tolist())
        n_full.append(int(full.sum()))
    out = {"metric": "decode single-launch phase times (ns, p10/p50/p90 over workgroups)",
           "workload": w.note, "rounds": reps, "workgroups_with_piece": int(np.median(n_full)),
           "start_spread_ns": round(float(np.median(spreads))),
           "first_start_to_last_end_ns": round(float(np.median(ends))),
           "piece_workgroup_start_ns_p10_p50_p90_max": [
               round(float(np.percentile(starts, q))) for q in (10, 50, 90, 100)]}
    for nm in names:
        v = np.asarray(phases[nm])
        out[nm] = [round(float(np.percentile(v, q))) for q in (10, 50, 90)]
    for nm in names:
        log(f"{nm:34s} p50 {out[nm][1] / 1000:.2f} us (p10 {out[nm][0] / 1000:.2f}, "
            f"p90 {out[nm][2] / 1000:.2f})")
    print(json.dumps(out), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="decode",
                    choices=["decode", "prefill", "mixed", "qkv", "tiny"])
    ap.add_argument("--sets", type=int, default=0,
                    help="independent buffer copies cycled by the steps (0: auto)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--event-every", type=int, default=8,
                    help="steps between the sampled launches that carry dispatch events")
    ap.add_argument("--split-small", type=int, default=0,
                    help="column splits per small piece (0: library choice)")
    ap.add_argument("--split-large", type=int, default=0,
                    help="column splits per large piece (0: library choice)")
    ap.add_argument("--exchange", type=int, default=0, choices=[-1, 0, 1],
                    help="K-split exchange of small pieces: 0 library choice, 1 on, -1 off")
    ap.add_argument("--step", default="auto", choices=["auto", "one", "two"],
                    help="one: sgmv_lora_delta_ids (build inside the delta launch; bf16, "
                         "M <= 512); two: builder launch + delta launch; auto: one where it "
                         "applies")
    ap.add_argument("--graph", action="store_true",
                    help="capture the K timed steps in one HIP graph and time its replay, as a "
                         "serving loop replays its decode step (not with --trace)")
    ap.add_argument("--trace", action="store_true",
                    help="ids follow a seeded decode trace (sequences join and leave; one "
                         "trace per buffer set) instead of one fixed batch; needs --step two")
    ap.add_argument("--trace-mean-len", type=int, default=256,
                    help="mean sequence life in steps for --trace")
    ap.add_argument("--trace-admit-every", type=int, default=8,
                    help="steps between admissions of new sequences for --trace")
    ap.add_argument("--chunk-size", type=int, default=-1,
                    help="override the workload's chunk size (-1: the workload's; -2: "
                         "sgmv_chunk_size_for_batch)")
    ap.add_argument("--fold-scale", action="store_true",
                    help="pack the pools with each adapter's scale folded into B")
    ap.add_argument("--segment-cache", action="store_true",
                    help="build through sgmv_build_segments_cached (with --trace)")
    ap.add_argument("--chunk-sweep", action="store_true",
                    help="step time by chunk size over batch sizes and adapter counts")
    ap.add_argument("--sweep-ranks", default="16",
                    help="comma-separated adapter ranks for --chunk-sweep")
    ap.add_argument("--merge", action="store_true",
                    help="time the merged-weight kernel against the base GEMM + delta")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="only run a plain device copy of --copy-mib MiB (counter scale)")
    ap.add_argument("--copy-mib", type=int, default=256)
    ap.add_argument("--copy-sets", type=int, default=1,
                    help="buffer pairs the calibration copy rotates over")
    ap.add_argument("--stream-ceiling", action="store_true",
                    help="only time the streaming reference kernel with the workload's byte "
                         "mix over its launch-shape sweep")
    ap.add_argument("--no-stream-ceiling", action="store_true",
                    help="skip the streaming reference kernel in the benchmark line")
    ap.add_argument("--phase-stamps", action="store_true",
                    help="per-phase times of the decode single launch from libsgmv_stamps.so")
    ap.add_argument("--write-traffic", nargs=4, metavar="CSV",
                    help="delta FETCH, delta WRITE, copy FETCH, copy WRITE counter CSVs")
    args = ap.parse_args()
    if args.write_traffic and args.step == "auto":
        args.step = "one" if args.workload == "decode" else "two"
    if args.write_traffic:
        write_traffic(args)
        return
    if args.calibration_copy:
        calibration_copy(args)
        return
    if args.stream_ceiling:
        import torch
        import workloads
        w = workloads.get(args.workload)
        elem = 2 if w.dtype == torch.bfloat16 else 4
        ids_np = w.ids.numpy()
        alg = workloads.algorithmic_bytes(ids_np, w.rank.numpy(), w.K, w.N, elem)
        wr = int((ids_np >= 0).sum()) * w.N * elem
        stream = torch.cuda.Stream()
        res = stream_ceiling(alg - wr, wr, max(50, min(args.steps, 400)), HipEvents(), stream)
        log(json.dumps({k: v for k, v in res.items() if k != "sweep"}))
        print(json.dumps({"metric": "streaming reference kernel, the workload's byte mix",
                          "workload": args.workload, **res}), flush=True)
        return
    if args.merge:
        merge_bench(args)
        return
    if args.phase_stamps:
        phase_stamps(args)
        return
    if args.chunk_sweep:
        chunk_sweep(args)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch
    import segmented_gather_gemv_amd as sg
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(device=dev)  # default priority
    lib = sg.library()
    ev = HipEvents()

    w = workloads.get(args.workload)
    if args.chunk_size == -2:
        n_ad = int(len(set(w.ids[w.ids >= 0].tolist())))
        w.chunk_size = sg.sgmv_chunk_size_for_batch(w.M, n_ad)
    elif args.chunk_size >= 0:
        w.chunk_size = args.chunk_size
    log(f"workload: {w.note} (chunk size {w.chunk_size})")
    # the single launch takes bf16 batches of 1..512 tokens whose ranks fit one 16-rank tile
    fits_one = w.dtype == torch.bfloat16 and 1 <= w.M <= 512 and w.a.shape[1] <= 16
    if args.step == "one" and not fits_one:
        print("--step one needs a bf16 batch of 1..512 tokens with ranks <= 16", file=sys.stderr)
        sys.exit(2)
    one_launch = args.step == "one" or (args.step == "auto" and fits_one)
    if (args.trace or args.segment_cache) and (one_launch or not args.trace):
        print("--trace (and --segment-cache with it) needs --step two", file=sys.stderr)
        sys.exit(2)
    if args.graph and args.trace:
        print("--graph replays fixed batches; it does not take --trace", file=sys.stderr)
        sys.exit(2)
    elem = 2 if w.dtype == torch.bfloat16 else 4
    per_set = (w.a.numel() + w.b.numel() + w.x.numel() + w.y0.numel()) * elem
    n_sets = args.sets or max(2, min(64, -(-2 * MALL_BYTES // per_set)))
    log(f"buffer sets: {n_sets} x {per_set / 2**20:.1f} MiB")

    sets = []
    with torch.cuda.stream(stream):
        a_dev, b_dev = w.a.to(dev), w.b.to(dev)
        for i in range(n_sets):
            pool = sg.sgmv_pool_pack(a_dev, b_dev, w.rank.tolist(), w.alpha.tolist(),
                                     fold_scale=args.fold_scale)
            x = w.x.to(dev)
            y = w.y0.to(dev)
            ids = w.ids.to(dev)
            seg = sg.sgmv_segments_alloc(w.M, w.L, w.chunk_size, dev)
            outs = [(y[:, n0:n0 + n], n0) for n0, n in w.slices] if len(w.slices) > 1 else [(y, 0)]
            sl, n_sl = sg._slices(outs, pool, w.M)
            sets.append(dict(pool=pool, x=x, y=y, ids=ids, seg=seg, sl=sl, n_sl=n_sl,
                             outs=outs))
        del a_dev, b_dev
    torch.cuda.synchronize()

    # --trace: buffer set j replays its own seeded decode trace, one row per use of the set
    # (rows for the warm-up, the timed region and the sampled region)
    # sampled launches (dispatch events) in a region of their own: at least 50 of them
    every = max(1, args.event_every)
    n_samp = max(50, len(range(0, args.steps, every)))
    K_samp = n_samp * every
    rows = -(-(args.warmup + args.steps + K_samp) // n_sets)
    if args.trace:
        for j, st in enumerate(sets):
            tr = workloads.decode_trace(rows, M=w.M, L=w.L, mean_len=args.trace_mean_len,
                                        admit_every=args.trace_admit_every, seed=1000 + j)
            st["trace"] = tr
            st["trace_dev"] = tr.to(dev)
            st["cache"] = sg.sgmv_segments_cache_alloc(w.M, dev)
        torch.cuda.synchronize()

    s_handle = ctypes.c_void_p(stream.cuda_stream)
    build_fn, delta_fn = lib.sgmv_build_segments_ex, lib.sgmv_lora_delta_ex
    cached_fn = lib.sgmv_build_segments_cached_ex
    ids_fn = lib.sgmv_lora_delta_ids_ex
    K = args.steps
    # launches that record a pair of events in their own dispatch (start, end of the kernel);
    # they run in a region of their own, after the timed one
    evs = [ev.create(4) for _ in range(n_samp)]
    plain = sg.LaunchOpts(n_split_small=args.split_small, n_split_large=args.split_large,
                          exchange=args.exchange)
    opts_b = [sg.LaunchOpts(e[0], e[1]) for e in evs]
    opts_d = [sg.LaunchOpts(e[2], e[3], args.split_small, args.split_large, args.exchange)
              for e in evs]
    calls = []
    for st in sets:
        bargs = (ctypes.c_void_p(st["ids"].data_ptr()), w.M, w.L, w.chunk_size, 1,
                 ctypes.byref(st["seg"].desc))
        dargs = (ctypes.c_void_p(st["x"].data_ptr()), st["x"].stride(0), w.M,
                 ctypes.byref(st["pool"].desc), ctypes.byref(st["seg"].desc), st["sl"],
                 st["n_sl"])
        calls.append((bargs, dargs))

    def trace_row(g):
        st = sets[g % n_sets]
        return st, g // n_sets

    def step(g, sample=None, part="both"):
        """The launches of use g of buffer set g % n_sets (trace row g // n_sets); `sample`
        picks a pair of dispatch events per launch; part: "both", "build" or "delta"."""
        bargs, dargs = calls[g % n_sets]
        od = opts_d[sample].ref() if sample is not None else plain.ref()
        if one_launch:
            return ids_fn(bargs[0], *dargs, od, s_handle)
        rc = 0
        if part != "delta":
            ob = opts_b[sample].ref() if sample is not None else None
            if args.trace:
                st, r = trace_row(g)
                ids_p = ctypes.c_void_p(st["trace_dev"][r].data_ptr())
                if args.segment_cache:
                    rc = cached_fn(ids_p, *bargs[1:], ctypes.c_void_p(st["cache"].data_ptr()),
                                   ob, s_handle)
                else:
                    rc = build_fn(ids_p, *bargs[1:], ob, s_handle)
            else:
                rc = build_fn(*bargs, ob, s_handle)
        if part != "build":
            rc |= delta_fn(*dargs, od, s_handle)
        return rc

    def region(g0, n, part="both"):
        """Seconds per step over n plain steps from use g0 (stream events around them), and the
        host's issue time per step."""
        rcs = []
        t, host = region_us(ev, stream, lambda j: rcs.append(step(g0 + j, part=part)), n)
        assert not any(rcs), f"library call failed with status {max(rcs)}"
        return t / 1e6, host / 1e6

    rc = 0
    # setup: one call per buffer set, so that every set's first-use costs (address
    # translation fills for buffers the kernel has not touched yet) are paid before the warm-up;
    # a serving loop reuses one pool and its activation buffers every step
    for i in range(n_sets):
        rc |= step(i)
    torch.cuda.synchronize()
    for i in range(args.warmup):
        rc |= step(i)
    torch.cuda.synchronize()
    assert rc == 0, f"library call failed with status {rc}"
    for st in sets:
        assert int(st["seg"].info[3].item()) == sg.SGMV_OK

    # the timed region: K plain steps, host clock and stream events around them; with --graph
    # the same K steps captured once in a HIP graph, run once untimed, then replayed
    graph = None
    if args.graph:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            for i in range(K):
                rc |= step(args.warmup + i)
        with torch.cuda.stream(stream):
            graph.replay()
        torch.cuda.synchronize()
        assert rc == 0, f"library call failed with status {rc}"
    reg = ev.create(2)
    flush_last_level_cache()  # setup's residue leaves the memory-side cache
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev.record(reg[0], s_handle)
    if graph is not None:
        with torch.cuda.stream(stream):
            graph.replay()
    else:
        for i in range(K):
            rc |= step(args.warmup + i)
    t_issue = time.perf_counter()
    ev.record(reg[1], s_handle)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    assert rc == 0, f"library call failed with status {rc}"
    region_s = ev.elapsed_ms(reg[0], reg[1]) / K / 1e3
    ev.destroy(reg)

    clocks = device_clocks()  # right after the timed region
    # the sampled region: n_samp * every more steps, every `every`-th with dispatch events
    # (per-launch durations; each such launch runs longer than a plain one)
    g_samp = args.warmup + K
    samp_g = []
    for i in range(K_samp):
        j = i // every if i % every == 0 else None
        if j is not None:
            samp_g.append(g_samp + i)
        rc |= step(g_samp + i, sample=j)
    torch.cuda.synchronize()
    assert rc == 0, f"library call failed with status {rc}"
    build_ms = [0.0 if one_launch else ev.elapsed_ms(e[0], e[1]) for e in evs]
    delta_ms = [ev.elapsed_ms(e[2], e[3]) for e in evs]
    for e in evs:
        ev.destroy(e)
    n_ev = len(delta_ms)

    # the delta kernel's average from plain launches: the timed region itself for the single
    # launch, K launches of the delta alone for two (the segments of every set are built). The
    # builder is too short to time alone (the host issues its launches no faster than the GPU
    # runs them), so its figure is its share of the step: the step less the delta alone. The
    # trace's batches change per step, so there the sampled launches give both.
    host_us = {"timed_step": (t_issue - t0) / K * 1e6}
    b_avg = 0.0
    if one_launch:
        timing = {"delta": "stream events around the timed steps (one launch per step)"
                           + (", replayed from one HIP graph" if graph is not None else "")}
        d_avg = region_s
    elif args.trace:
        timing = {"delta": "dispatch events of the sampled launches",
                  "builder": "dispatch events of the sampled launches"}
        d_avg = sum(delta_ms) / n_ev / 1e3
        b_avg = sum(build_ms) / n_ev / 1e3
    else:
        timing = {"delta": "stream events around K launches of the delta kernel alone",
                  "builder": "the timed step less the delta alone (builder launch and gap)"}
        flush_last_level_cache()
        d_avg, h = region(g_samp + K_samp, K, part="delta")
        host_us["delta_alone"] = h * 1e6
        b_avg = max(region_s - d_avg, 0.0)
    for k, v in host_us.items():
        ref = region_s if k == "timed_step" else d_avg
        if v > 0.9 * ref * 1e6:
            log(f"warning: host issue {v:.2f} us per launch in the {k} region against "
                f"{ref * 1e6:.2f} us: launch-bound")

    wall = t1 - t0
    ids_np = w.ids.numpy()
    n_lora = int((ids_np >= 0).sum())
    alg_bytes = workloads.algorithmic_bytes(ids_np, w.rank.numpy(), w.K, w.N, elem)
    alg_flops = workloads.algorithmic_flops(ids_np, w.rank.numpy(), w.K, w.N)
    trace_info = None
    if args.trace:  # per-step token counts; roofline bytes averaged over the sampled steps
        def row_ids(g):
            st, r = trace_row(g)
            return st["trace"][r].numpy()

        def hit(g):
            st, r = trace_row(g)
            return r > 0 and bool((st["trace"][r] == st["trace"][r - 1]).all())

        steps_g = [args.warmup + i for i in range(K)]
        n_lora = sum(int((row_ids(g) >= 0).sum()) for g in steps_g) / K
        alg_bytes = sum(workloads.algorithmic_bytes(row_ids(g), w.rank.numpy(), w.K, w.N, elem)
                        for g in samp_g) / len(samp_g)
        alg_flops = sum(workloads.algorithmic_flops(row_ids(g), w.rank.numpy(), w.K, w.N)
                        for g in samp_g) / len(samp_g)
        hits = [hit(g) for g in samp_g]
        bh = [b for b, h in zip(build_ms, hits) if h]
        bm = [b for b, h in zip(build_ms, hits) if not h]
        trace_info = {
            "mean_len": args.trace_mean_len, "admit_every": args.trace_admit_every,
            "segment_cache": bool(args.segment_cache),
            "unchanged_step_fraction": sum(hit(g) for g in steps_g) / K,
            "builder_us_unchanged_ids": sum(bh) / len(bh) * 1e3 if bh else None,
            "builder_us_changed_ids": sum(bm) / len(bm) * 1e3 if bm else None,
        }
        log(f"trace: {trace_info}")
    srt = sorted(delta_ms)
    achieved = alg_bytes / d_avg / 1e9
    # counters were taken on the workload's own batch and chunk size
    traffic = (load_traffic(args.workload, one_launch)
               if args.chunk_size == -1 and not args.trace else None)
    kname = "build + delta kernel" if one_launch else "delta kernel"
    log(f"step {wall / K * 1e6:.2f} us | {kname} avg {d_avg * 1e6:.2f} us "
        f"(p10 {srt[n_ev // 10] * 1e3:.2f}, p50 {srt[n_ev // 2] * 1e3:.2f}, "
        f"p90 {srt[9 * n_ev // 10] * 1e3:.2f} over {n_ev} sampled launches) "
        f"| builder {'(inside)' if one_launch else f'{b_avg * 1e6:.2f} us'} "
        f"| {achieved:.0f} GB/s algorithmic "
        f"({achieved / HBM_PEAK_GBPS * 100:.1f}% of peak) | {alg_flops / d_avg / 1e12:.2f} TFLOP/s")

    result = {
        "metric": METRIC,
        "value": n_lora * K / wall,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": wall / K * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == torch.bfloat16 else "f32",
        "data": "synthetic",
        "config": {
            "workload": w.note,
            "chunk_size": w.chunk_size,
            "tokens_per_step": w.M,
            "lora_tokens_per_step": n_lora,
            "buffer_sets": n_sets,
            "step": ("segment build + fused delta in one launch (sgmv_lora_delta_ids)"
                     if one_launch else "device segment build launch + fused delta launch")
                    + (", K steps replayed from one HIP graph" if graph is not None else ""),
            "kernel_timing": timing,
            "host_issue_us": host_us,
            "delta_kernel_us": d_avg * 1e6,
            "sampled_launches": n_ev,
            "sampled_delta_kernel_us_p10_p50_p90": [srt[n_ev // 10] * 1e3, srt[n_ev // 2] * 1e3,
                                                    srt[9 * n_ev // 10] * 1e3],
            "clocks_after_timed_region": clocks,
            "device": (f"{torch.cuda.get_device_name(dev)} "
                       f"({torch.cuda.get_device_properties(dev).gcnArchName})"),
            "hip_runtime": torch.version.hip,
            "builder_kernel_us": None if one_launch else b_avg * 1e6,
            "algorithmic_bytes_per_launch": alg_bytes,
            "algorithmic_flops_per_launch": alg_flops,
        },
        "roofline": {
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBPS,
            "traffic": traffic,
        },
        "cpu_baseline": None,
    }
    if args.fold_scale:
        result["config"]["pool"] = "scale folded into B at pack time"
    if trace_info is not None:
        result["config"]["trace"] = trace_info
        result["config"]["lora_tokens_per_step"] = n_lora
        result["config"]["step"] += (" (through the grouping cache)" if args.segment_cache
                                     else "")
    del sets
    torch.cuda.empty_cache()
    if not args.no_stream_ceiling and not args.trace:
        # the same byte mix through the streaming reference kernel: the memory system's
        # ceiling for one launch that moves these bytes
        wr = int(round(n_lora)) * w.N * elem
        sc = stream_ceiling(int(alg_bytes) - wr, wr, max(50, min(K, 400)), ev, stream)
        sc["delta_kernel_frac_of_ceiling"] = sc["best"]["us"] / (d_avg * 1e6)
        result["config"]["stream_ceiling"] = {k: v for k, v in sc.items() if k != "sweep"}
        log("streaming reference sweep (block x loads per thread: us): " +
            ", ".join(f"{r['block']}x{r['unroll']}: {r['us']:.2f}" for r in sc["sweep"]))
        log(f"streaming reference, same bytes: {sc['best']['us']:.2f} us "
            f"({sc['gbps']:.0f} GB/s, {sc['frac_of_peak'] * 100:.1f}% of peak; block "
            f"{sc['best']['block']} x {sc['best']['unroll']} loads); delta kernel at "
            f"{sc['delta_kernel_frac_of_ceiling'] * 100:.1f}% of it")
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
