"""The hot path under HIP graph capture: the single launch, the two launches (builder +
delta) and the cached build are captured once on torch's capture stream and replayed several
times, with new ids and activations written into the captured buffers between replays (eager
work and synchronisations in between). Every replay must equal, bit for bit, the same calls
run eagerly on fresh segments. No call of the library records a memset.
"""
import numpy as np
import pytest
import torch

import workloads

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.fixture(scope="module")
def sg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import segmented_gather_gemv_amd as m
    return m


def _ids(M, L, seed):
    rng = np.random.default_rng(seed)
    v = rng.integers(-1, L, M).astype(np.int32)
    return torch.from_numpy(v)


def _eager(sg, w, pool, x, ids, y0, opts=None):
    y = y0.clone()
    seg = sg.sgmv_build_segments(ids, w.L, w.chunk_size)
    sg.sgmv_lora_delta(x, pool, seg, y, opts=opts)
    torch.cuda.synchronize()
    return y, seg


CASES = {
    # single launch (bf16, rank 16, M <= 512), and two launches (rank 32; M > 512)
    "one_launch": dict(M=128, K=1024, N=1024, L=16, R=16),
    "two_launch_rank32": dict(M=96, K=512, N=768, L=8, R=32, ranks=[5, 32]),
    "two_launch_m600": dict(M=600, K=512, N=256, L=20, R=16, chunk=16),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_delta_ids_replays(sg, name):
    w = workloads.custom(name=name, seed=51, **CASES[name])
    pool = sg.sgmv_pool_pack(w.a.to(DEV), w.b.to(DEV), w.rank.tolist(), w.alpha.tolist())
    x = w.x.to(DEV)
    ids = w.ids.to(DEV)
    y0 = w.y0.to(DEV)
    y = torch.empty_like(y0)
    seg = sg.sgmv_segments_alloc(w.M, w.L, w.chunk_size, DEV)
    opts = sg.LaunchOpts(n_split_small=4, exchange=1)
    # warm up outside capture (library and module loading)
    y.copy_(y0)
    sg.sgmv_lora_delta_ids(ids, x, pool, seg, y, opts=opts)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            y.copy_(y0)
            sg.sgmv_lora_delta_ids(ids, x, pool, seg, y, opts=opts)
    torch.cuda.synchronize()
    for step in range(4):
        new_ids = _ids(w.M, w.L, 100 + step)
        ids.copy_(new_ids.to(DEV))
        x.copy_((torch.randn(w.M, w.K, generator=torch.Generator().manual_seed(step))
                 .to(w.dtype)).to(DEV))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref, rseg = _eager(sg, w, pool, x, ids, y0, opts)
        assert torch.equal(y, ref), (name, step)
        hs, hr = seg.host(), rseg.host()
        for k in ("sorted_token_ids", "seg_indptr", "seg_lora_ids", "large_tiles",
                  "small_tiles"):
            assert torch.equal(hs[k], hr[k]), (name, step, k)


def test_cached_build_and_delta_replays(sg):
    """Cached build + fused delta captured together; replays alternate between unchanged ids
    (the build is skipped inside the graph) and new ids (rebuilt)."""
    w = workloads.custom(name="gcache", seed=52, M=256, K=1024, N=512, L=32, R=16)
    pool = sg.sgmv_pool_pack(w.a.to(DEV), w.b.to(DEV), w.rank.tolist(), w.alpha.tolist())
    x, ids, y0 = w.x.to(DEV), w.ids.to(DEV), w.y0.to(DEV)
    y = torch.empty_like(y0)
    seg = sg.sgmv_segments_alloc(w.M, w.L, 0, DEV)
    cache = sg.sgmv_segments_cache_alloc(w.M, DEV)
    sg.sgmv_build_segments_cached(ids, seg, cache)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            y.copy_(y0)
            sg.sgmv_build_segments_cached(ids, seg, cache)
            sg.sgmv_lora_delta(x, pool, seg, y)
    torch.cuda.synchronize()
    for step in range(5):
        if step % 2 == 1:  # new ids on odd steps, unchanged on even ones
            ids.copy_(_ids(w.M, w.L, 200 + step).to(DEV))
            torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref, _ = _eager(sg, w, pool, x, ids, y0)
        assert torch.equal(y, ref), step
