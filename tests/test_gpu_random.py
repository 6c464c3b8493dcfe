"""GPU parity over seeded random configurations: shapes (odd K and N included), pool sizes,
rank mixes, chunk sizes, id distributions (uniform, skewed, runs, many ids -1) and output
slices, each drawn from its own seed.

Every case runs the device builder against the host builder (bit for bit), the fused delta
against the fp64 oracle (bf16: rel-L2 <= 5e-3 and max-abs <= 1e-2 * max|ref|; fp32: rel-L2 <=
1e-4) on the drawn base output and on a zero base (the delta alone), the unfused shrink +
expand against the oracle, and, for bf16 batches, the build-and-delta call against the two
calls (segment arrays and y bit for bit).
"""
import os

import numpy as np
import pytest
import torch

import workloads
from test_gpu_parity import DEV, check_no_adapter_rows, compare, np32, oracle_y, upload

pytestmark = pytest.mark.gpu

N_CASES = int(os.environ.get("SGMV_RANDOM_CASES", "40"))  # more for a deeper sweep


@pytest.fixture(scope="module")
def sg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import segmented_gather_gemv_amd as m
    return m


def random_case(seed):
    rng = np.random.default_rng(1000 + seed)
    M = int(rng.choice([1, 7, 16, 17, 63, 64, 65, 200, 511, 512, 513, 900, 1500]))
    K = int(rng.choice([32, 100, 256, 520, 1024, 1000]))
    N = int(rng.choice([16, 37, 128, 300, 640, 1024]))
    L = int(rng.integers(1, 300))
    R = int(rng.choice([1, 3, 8, 16, 24, 32, 48, 64]))
    ranks = sorted(set(int(v) for v in rng.integers(1, R + 1, size=rng.integers(1, 4))))
    dtype = torch.float32 if rng.random() < 0.15 else torch.bfloat16
    chunk = int(rng.choice([0, 0, 0, 1, 5, 16, 64]))
    kw = dict(M=M, K=K, N=N, L=L, R=R, ranks=ranks, dtype=dtype, chunk=chunk,
              no_lora_frac=float(rng.choice([0.0, 0.0, 0.1, 0.5])),
              w_std=0.1 if dtype == torch.float32 else 0.02)
    kind = rng.choice(["uniform", "runs", "skewed"])
    if kind == "runs" and M > 1:
        cuts = np.sort(rng.choice(np.arange(1, M), size=min(M - 1, int(rng.integers(1, 8))),
                                  replace=False))
        kw["seq_lens"] = np.diff(np.concatenate([[0], cuts, [M]])).tolist()
    n_slices = int(rng.choice([1, 1, 2, 3])) if N >= 48 else 1
    if n_slices > 1:
        edges = np.sort(rng.choice(np.arange(8, N - 8, 8), size=n_slices - 1, replace=False))
        bounds = np.concatenate([[0], edges, [N]])
        kw["slices"] = [(int(a), int(b - a)) for a, b in zip(bounds[:-1], bounds[1:])]
    w = workloads.custom(name=f"random{seed}", seed=2000 + seed, **kw)
    if kind == "skewed" and M > 1:  # most tokens on a few adapters
        hot = rng.integers(0, L, size=min(L, 3))
        ids = w.ids.numpy().copy()
        pick = rng.random(M) < 0.8
        ids[pick & (ids >= 0)] = rng.choice(hot, size=int((pick & (ids >= 0)).sum()))
        w.ids = torch.from_numpy(ids.astype(np.int32))
    return w, kind


def _apply(sg, w, x, y0, fn):
    y = y0.clone()
    views = [(y[:, n0:n0 + n].contiguous(), n0) for n0, n in w.slices]
    fn(views if len(views) > 1 else views[0][0])
    torch.cuda.synchronize()
    for t, n0 in views:
        y[:, n0:n0 + t.shape[1]] = t
    return y


@pytest.mark.parametrize("seed", range(N_CASES))
def test_random_configuration(sg, seed):
    w, kind = random_case(seed)
    what = (f"seed {seed}: M={w.M} K={w.K} N={w.N} L={w.L} R={w.R} {w.dtype} C={w.chunk_size} "
            f"{kind} slices={w.slices}")
    print(what, flush=True)
    pool, x, y0, ids = upload(w, sg)
    # builders
    dev = sg.sgmv_build_segments(ids, w.L, w.chunk_size, on_device=True)
    host = sg.sgmv_build_segments(w.ids, w.L, w.chunk_size, on_device=False).host()
    hd = dev.host()
    for k in ("sorted_token_ids", "seg_indptr", "seg_lora_ids", "large_tiles", "small_tiles"):
        assert torch.equal(hd[k], host[k]), (what, k)
    # fused delta against the oracle
    ref = oracle_y(w, np32(w.y0))
    y = _apply(sg, w, x, y0, lambda v: sg.sgmv_lora_delta(x, pool, dev, v))
    compare(np32(y), ref, w.dtype, what=what)
    check_no_adapter_rows(w, y, w.y0)
    # zero-base twin: the delta alone, which a large base output would hide
    yz = _apply(sg, w, x, torch.zeros_like(y0), lambda v: sg.sgmv_lora_delta(x, pool, dev, v))
    compare(np32(yz), oracle_y(w, np.zeros_like(np32(w.y0))), w.dtype, what=what + " zero base")
    # unfused shrink + expand against the oracle
    h = sg.sgmv_shrink(x, pool, dev)
    y2 = _apply(sg, w, x, y0, lambda v: sg.sgmv_expand(h, pool, dev, v))
    compare(np32(y2), ref, w.dtype, what=what + " unfused")
    # build and delta in one call against the two calls
    if w.dtype == torch.bfloat16:
        one = sg.sgmv_segments_alloc(w.M, w.L, w.chunk_size, DEV)
        y3 = _apply(sg, w, x, y0, lambda v: sg.sgmv_lora_delta_ids(ids, x, pool, one, v))
        ho = one.host()
        for k in ("sorted_token_ids", "seg_indptr", "seg_lora_ids", "large_tiles",
                  "small_tiles"):
            assert torch.equal(ho[k], hd[k]), (what, k)
        assert torch.equal(y3, y), what
