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

Timing: W untimed warm-up steps, then K steps between two device synchronisations
(ms_per_step, value = tokens with an adapter per second). Inside the same timed region every
eighth step's kernel launches (the single build + delta kernel, or the builder and the
delta kernel) record a pair of HIP events as part of their own dispatch on the launch stream
(start and end of the kernel, no extra stream packets); their averages give the per-launch
durations used for the roofline, which takes the kernel that does the delta (including the
build it does itself in the single-launch step).
Events on every launch would slow the host's launch path and lengthen the step. The roofline
figure divides the algorithmic bytes of one delta launch (x rows and y rows read and written
for every token with an adapter, each used adapter's true-rank A and B once, 12 bytes of
index per token) by that duration, against the 8 TB/s HBM peak.

--trace (with --step two) replaces the fixed batch by seeded decode traces, one per buffer
set, in which sequences keep their adapter and join or leave the batch; --segment-cache then
builds through the grouping cache, and the line reports the builder time on steps with
unchanged and with changed ids.

The CPU baseline is the fp64 oracle (plain per-token NumPy loop) on the same batch, repeated
for about 10 s on this host.

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

    def elapsed_ms(self, a, b):
        ms = ctypes.c_float()
        assert self.lib.hipEventElapsedTime(ctypes.byref(ms), a, b) == 0
        return ms.value

    def destroy(self, evs):
        for e in evs:
            self.lib.hipEventDestroy(e)


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
    Times the merge kernel (dispatch events, W and W' rotating over sets larger than the
    last-level cache), the base GEMM x W^T of the decode batch (torch.matmul, the vendor GEMM
    library) and the unmerged delta of a batch whose 256 tokens all use one adapter, and
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

    def timed(fn, reps):
        pairs = [ev.create(2) for _ in range(reps)]
        with torch.cuda.stream(stream):
            for i in range(args.warmup):
                fn(i, None)
            torch.cuda.synchronize()
            for i in range(reps):
                fn(i, sg.LaunchOpts(pairs[i][0], pairs[i][1]))
        torch.cuda.synchronize()
        ms = [ev.elapsed_ms(a, b) for a, b in pairs]
        for p_ in pairs:
            ev.destroy(p_)
        return sum(ms) / len(ms) * 1e3  # us

    reps = max(16, min(args.steps, 200))
    merge_us = timed(lambda i, o: sg.sgmv_merge_adapter(Ws[i % n_sets], pool, 0,
                                                       out=Wo[i % n_sets], opts=o), reps)
    delta_us = timed(lambda i, o: sg.sgmv_lora_delta_ids(ids, x, pool, seg, ys[i % n_sets],
                                                         opts=o), reps)
    # base GEMM y = x W^T through torch (events around each call on the stream)
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            torch.matmul(x, Ws[i % n_sets].t())
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        for i in range(reps):
            evs[i][0].record(stream)
            torch.matmul(x, Ws[i % n_sets].t())
            evs[i][1].record(stream)
    torch.cuda.synchronize()
    gemm_us = sum(a.elapsed_time(b) for a, b in evs) / reps * 1e3
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
    step time (segment build + fused delta, dispatch events) for batches of M tokens spread
    uniformly over n adapters of the decode pool (d = 4096, rank 16), at several chunk sizes,
    with two launches and, where it applies, as one sgmv_lora_delta_ids launch."""
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
            modes = ["two"] + (["one"] if M <= 512 else [])
            for mode in modes:
                pairs = [ev.create(4) for _ in range(reps)]
                with torch.cuda.stream(stream):
                    for i in range(-5, reps):
                        e = pairs[i] if i >= 0 else None
                        st = i % sets
                        if mode == "one":
                            o = sg.LaunchOpts(e[0], e[1]) if e else None
                            sg.sgmv_lora_delta_ids(ids, xs[st], pool, segs[st], ys[st], opts=o)
                        else:
                            sg.sgmv_build_segments(ids, 64, C, out=segs[st],
                                                   opts=sg.LaunchOpts(e[0], e[1]) if e else None)
                            sg.sgmv_lora_delta(xs[st], pool, segs[st], ys[st],
                                               opts=sg.LaunchOpts(e[2], e[3]) if e else None)
                torch.cuda.synchronize()
                b = float(np.mean([ev.elapsed_ms(p_[0], p_[1]) for p_ in pairs])) * 1e3
                d = 0.0 if mode == "one" else \
                    float(np.mean([ev.elapsed_ms(p_[2], p_[3]) for p_ in pairs])) * 1e3
                for p_ in pairs:
                    ev.destroy(p_)
                row = {"M": M, "adapters": n_ad, "rank": R, "chunk": C, "launches": mode,
                       "build_us": round(b, 2) if mode == "two" else None,
                       "delta_us": round(d, 2) if mode == "two" else round(b, 2),
                       "total_us": round(b + d, 2)}
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
                    help="timed steps between launches that carry timing events")
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
    if args.merge:
        merge_bench(args)
        return
    if args.chunk_sweep:
        chunk_sweep(args)
        return

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
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
    rows = -(-(args.warmup + args.steps) // n_sets)
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
    # per timed step: events the kernels' own dispatches record (start, end) -- no extra
    # packets in the stream
    every = max(1, args.event_every)
    sampled = list(range(0, K, every))
    evs = {i: ev.create(4) for i in sampled}
    plain = sg.LaunchOpts(n_split_small=args.split_small, n_split_large=args.split_large,
                          exchange=args.exchange)
    opts_b = {i: sg.LaunchOpts(e[0], e[1]) for i, e in evs.items()}
    opts_d = {i: sg.LaunchOpts(e[2], e[3], args.split_small, args.split_large, args.exchange)
              for i, e in evs.items()}
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

    def step(i, timed=False):
        g = i + (args.warmup if timed else 0)  # use count over warm-up and timed steps
        bargs, dargs = calls[g % n_sets] if args.trace else calls[i % n_sets]
        sample = timed and i in evs
        if one_launch:
            return ids_fn(bargs[0], *dargs, opts_d[i].ref() if sample else plain.ref(), s_handle)
        ob = opts_b[i].ref() if sample else None
        if args.trace:
            st, r = trace_row(g)
            ids_p = ctypes.c_void_p(st["trace_dev"][r].data_ptr())
            if args.segment_cache:
                rc = cached_fn(ids_p, *bargs[1:], ctypes.c_void_p(st["cache"].data_ptr()), ob,
                               s_handle)
            else:
                rc = build_fn(ids_p, *bargs[1:], ob, s_handle)
        else:
            rc = build_fn(*bargs, ob, s_handle)
        rc |= delta_fn(*dargs, opts_d[i].ref() if sample else plain.ref(), s_handle)
        return rc

    rc = 0
    for i in range(args.warmup):
        rc |= step(i)
    torch.cuda.synchronize()
    assert rc == 0, f"library call failed with status {rc}"
    for st in sets:
        assert int(st["seg"].info[3].item()) == sg.SGMV_OK

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(K):
        rc |= step(i, timed=True)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    assert rc == 0, f"library call failed with status {rc}"
    build_ms = [0.0 if one_launch else ev.elapsed_ms(e[0], e[1]) for e in evs.values()]
    delta_ms = [ev.elapsed_ms(e[2], e[3]) for e in evs.values()]
    for e in evs.values():
        ev.destroy(e)
    n_ev = len(delta_ms)

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
        samp_g = [args.warmup + i for i in sampled]
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
    d_avg = sum(delta_ms) / n_ev / 1e3  # seconds
    b_avg = sum(build_ms) / n_ev / 1e3
    srt = sorted(delta_ms)
    achieved = alg_bytes / d_avg / 1e9
    # counters were taken on the workload's own batch and chunk size
    traffic = (load_traffic(args.workload, one_launch)
               if args.chunk_size == -1 and not args.trace else None)
    kname = "build + delta kernel" if one_launch else "delta kernel"
    log(f"step {wall / K * 1e6:.2f} us | {kname} avg {d_avg * 1e6:.2f} us "
        f"(p10 {srt[n_ev // 10] * 1e3:.2f}, p50 {srt[n_ev // 2] * 1e3:.2f}, "
        f"p90 {srt[9 * n_ev // 10] * 1e3:.2f}, {n_ev} sampled launches) "
        f"| builder avg {'(inside)' if one_launch else f'{b_avg * 1e6:.2f} us'} "
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
                     if one_launch else "device segment build launch + fused delta launch"),
            "timed_launches_sampled": n_ev,
            "delta_kernel_us": d_avg * 1e6,
            "delta_kernel_us_p10_p50_p90": [srt[n_ev // 10] * 1e3, srt[n_ev // 2] * 1e3,
                                            srt[9 * n_ev // 10] * 1e3],
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
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
