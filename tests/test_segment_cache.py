"""The grouping cache across steps (sgmv_build_segments_cached; Ascend article 4.2 and 5.3: a
sequence keeps its adapter, so the grouping changes only when sequences join or leave).

Bar: at every step of a seeded decode trace the cached call leaves the segment arrays bit-equal
to the oracle's segments of that step's ids (and to a fresh build of them); when the ids (and M, L, chunk size) equal those of the
last build made through the cache, it writes nothing (checked by poisoning the arrays); a
zeroed cache[0] forces a rebuild. Host path on the CPU; device path (three builder kernels by
batch size) and the fused delta on cached segments on the GPU.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import segmented_gather_gemv_amd as sg
import workloads
from test_abi_host import check_records

KEYS = ("sorted_token_ids", "seg_indptr", "seg_lora_ids", "large_tiles", "small_tiles",
        "num_segments", "status")


def _same(a, b):
    ha, hb = a.host(), b.host()
    for k in KEYS:
        if isinstance(ha[k], torch.Tensor):
            assert torch.equal(ha[k], hb[k]), k
        else:
            assert ha[k] == hb[k], k


def _same_as_oracle(seg, ids, L, C):
    """The arrays in seg equal the oracle's segments of these ids (bad ids read as -1, as the
    device builder treats them), and the records satisfy their invariants."""
    got = seg.host()
    clean = np.asarray(ids.cpu(), dtype=np.int64).copy()
    clean[(clean < -1) | (clean >= L)] = -1
    ref = oracle.segments(clean, L, C)
    M = clean.shape[0]
    assert np.array_equal(got["sorted_token_ids"].numpy()[:M], ref["sorted_token_ids"])
    assert np.array_equal(got["seg_indptr"].numpy(), ref["seg_indptr"])
    assert np.array_equal(got["seg_lora_ids"].numpy(), ref["seg_lora_ids"])
    assert got["num_segments"] == ref["num_segments"]
    check_records(got, ref)


def _poison(seg):
    for t in (seg.sorted_token_ids, seg.seg_indptr, seg.seg_lora_ids, seg.tiles, seg.info):
        t.fill_(-77)


def _poisoned(seg):
    return all(bool((t == -77).all()) for t in (seg.sorted_token_ids, seg.seg_indptr,
                                                 seg.seg_lora_ids, seg.tiles, seg.info))


def _trace_check(dev, M, L, C, steps, mean_len, admit_every, seed):
    trace = workloads.decode_trace(steps, M=M, L=L, mean_len=mean_len, admit_every=admit_every,
                                   seed=seed)
    on_device = dev != "cpu"
    seg = sg.sgmv_segments_alloc(M, L, C, dev)
    cache = sg.sgmv_segments_cache_alloc(M, dev)
    hits = 0
    for s in range(steps):
        ids = trace[s].to(dev)
        sg.sgmv_build_segments_cached(ids, seg, cache, on_device=on_device)
        _same_as_oracle(seg, trace[s], L, C)
        fresh = sg.sgmv_build_segments(ids, L, C, on_device=on_device)
        _same(seg, fresh)
        hits += int(s > 0 and torch.equal(trace[s], trace[s - 1]))
    return hits


# ---------------------------------------------------------------------------------------
# host path (CPU)
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("C", [0, 3, 64])
def test_host_cache_trace(C):
    hits = _trace_check("cpu", 256, 64, C, 60, 256, 4, seed=5)
    assert 0 < hits < 59  # the trace has both kinds of step


def test_decode_trace_recipe():
    """Sequences keep their adapter while alive; freed slots hold -1 until an admission step."""
    t = workloads.decode_trace(50, M=64, L=8, mean_len=6, admit_every=5, seed=3)
    assert t.shape == (50, 64) and t.dtype == torch.int32
    assert int(t.min()) >= -1 and int(t.max()) < 8
    for s in range(1, 50):
        prev, cur = t[s - 1], t[s]
        if s % 5:  # no admission: a slot either keeps its adapter or has just been freed
            assert bool(((cur == prev) | (cur == -1)).all())
        else:      # admission: every free slot takes a new sequence
            assert bool((cur >= 0).all())


def test_host_cache_hit_writes_nothing():
    ids = workloads.decode_trace(1, M=100, L=10, seed=1)[0]
    seg = sg.sgmv_segments_alloc(100, 10, 0, "cpu")
    cache = sg.sgmv_segments_cache_alloc(100, "cpu")
    sg.sgmv_build_segments_cached(ids, seg, cache, on_device=False)
    _same_as_oracle(seg, ids, 10, 0)
    _same(seg, sg.sgmv_build_segments(ids, 10, 0, on_device=False))
    _poison(seg)
    sg.sgmv_build_segments_cached(ids.clone(), seg, cache, on_device=False)
    assert _poisoned(seg)
    ids2 = ids.clone()
    ids2[17] = (int(ids2[17]) + 1) % 10
    sg.sgmv_build_segments_cached(ids2, seg, cache, on_device=False)
    _same_as_oracle(seg, ids2, 10, 0)
    _same(seg, sg.sgmv_build_segments(ids2, 10, 0, on_device=False))
    # a zeroed tag forces a rebuild of unchanged ids
    _poison(seg)
    cache[0] = 0
    sg.sgmv_build_segments_cached(ids2, seg, cache, on_device=False)
    _same_as_oracle(seg, ids2, 10, 0)
    _same(seg, sg.sgmv_build_segments(ids2, 10, 0, on_device=False))


def test_host_cache_bad_id_is_not_cached():
    ids = torch.tensor([0, 1, 7, 1], dtype=torch.int32)  # 7 >= L
    seg = sg.sgmv_segments_alloc(4, 3, 0, "cpu")
    cache = sg.sgmv_segments_cache_alloc(4, "cpu")
    for _ in range(2):
        with pytest.raises(sg.SgmvError):
            sg.sgmv_build_segments_cached(ids, seg, cache, on_device=False)
        assert int(cache[0]) == 0


def test_cache_errors():
    lib = sg.library()
    seg = sg.sgmv_segments_alloc(8, 4, 0, "cpu")
    ids = torch.zeros(8, dtype=torch.int32)
    assert lib.sgmv_build_segments_cached(ctypes.c_void_p(ids.data_ptr()), 8, 4, 0, 0,
                                          ctypes.byref(seg.desc), None, None) == sg.SGMV_EINVAL
    cache = sg.sgmv_segments_cache_alloc(8, "cpu")
    # the segments' own checks still apply (M, chunk size)
    assert lib.sgmv_build_segments_cached(ctypes.c_void_p(ids.data_ptr()), 7, 4, 0, 0,
                                          ctypes.byref(seg.desc),
                                          ctypes.c_void_p(cache.data_ptr()),
                                          None) == sg.SGMV_EINVAL
    with pytest.raises(ValueError):
        sg.sgmv_build_segments_cached(ids, seg, cache[:5], on_device=False)
    with pytest.raises(ValueError):
        sg.sgmv_build_segments_cached(ids, seg, cache, on_device=True)
    # an empty batch is a no-op with or without a cache
    seg0 = sg.sgmv_segments_alloc(0, 4, 0, "cpu")
    assert lib.sgmv_build_segments_cached(None, 0, 4, 0, 0, ctypes.byref(seg0.desc), None,
                                          None) == sg.SGMV_OK


# ---------------------------------------------------------------------------------------
# device path (GPU)
# ---------------------------------------------------------------------------------------
DEV = "cuda"


@pytest.fixture(scope="module")
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return True


# (M, L, C): one per device builder kernel (M <= 1024, mid-size, rounds of 1024 tokens)
SIZES = [(256, 64, 0), (700, 200, 5), (3000, 300, 0), (40000, 1000, 64)]


@pytest.mark.gpu
@pytest.mark.parametrize("M,L,C", SIZES)
def test_device_cache_trace(gpu, M, L, C):
    steps = 40 if M <= 3000 else 12
    print(f"device cache trace M={M} L={L} C={C}", flush=True)
    hits = _trace_check(DEV, M, L, C, steps, mean_len=M, admit_every=3, seed=M)
    assert 0 < hits < steps - 1


@pytest.mark.gpu
@pytest.mark.parametrize("M,L,C", SIZES)
def test_device_cache_hit_writes_nothing(gpu, M, L, C):
    ids = workloads.decode_trace(1, M=M, L=L, seed=11)[0].to(DEV)
    seg = sg.sgmv_segments_alloc(M, L, C, DEV)
    cache = sg.sgmv_segments_cache_alloc(M, DEV)
    sg.sgmv_build_segments_cached(ids, seg, cache)
    _same_as_oracle(seg, ids, L, C)
    _same(seg, sg.sgmv_build_segments(ids, L, C))
    _poison(seg)
    sg.sgmv_build_segments_cached(ids.clone(), seg, cache)
    torch.cuda.synchronize()
    assert _poisoned(seg)
    ids2 = ids.clone()
    ids2[M - 1] = -1 if int(ids2[M - 1]) >= 0 else 0  # the last token changes
    sg.sgmv_build_segments_cached(ids2, seg, cache)
    _same_as_oracle(seg, ids2, L, C)
    _same(seg, sg.sgmv_build_segments(ids2, L, C))
    _poison(seg)
    cache[0] = 0
    sg.sgmv_build_segments_cached(ids2, seg, cache)
    _same_as_oracle(seg, ids2, L, C)
    _same(seg, sg.sgmv_build_segments(ids2, L, C))


@pytest.mark.gpu
def test_device_cache_bad_ids_cached_with_status(gpu):
    """The device path treats a bad id as -1 and flags it; a cached hit keeps that status."""
    ids = torch.tensor([0, 1, 9, 1, -5, 2], dtype=torch.int32, device=DEV)
    seg = sg.sgmv_segments_alloc(6, 3, 0, DEV)
    cache = sg.sgmv_segments_cache_alloc(6, DEV)
    for _ in range(2):
        sg.sgmv_build_segments_cached(ids, seg, cache)
        assert int(seg.info[3]) == sg.SGMV_EBADID
        _same_as_oracle(seg, ids, 3, 0)
        _same(seg, sg.sgmv_build_segments(ids, 3, 0))


@pytest.mark.gpu
def test_fused_delta_on_cached_segments(gpu):
    """Decode steps through the cache, then the fused delta with the K-split exchange: y is
    bit-equal to the delta on freshly built segments at every step (hits leave the exchange
    control words uncleared; every call still advances them by exactly 64) and meets the
    oracle's bar."""
    from test_gpu_parity import compare, np32, upload
    w = workloads.custom(M=128, K=512, N=512, L=16, R=16, name="cache", seed=9)
    pool, x, y0, _ = upload(w, sg)
    trace = workloads.decode_trace(12, M=128, L=16, mean_len=30, admit_every=4, seed=2)
    seg = sg.sgmv_segments_alloc(128, 16, 0, DEV)
    cache = sg.sgmv_segments_cache_alloc(128, DEV)
    opts = sg.LaunchOpts(n_split_small=4, exchange=1)
    for s in range(12):
        ids = trace[s].to(DEV)
        sg.sgmv_build_segments_cached(ids, seg, cache)
        ya = y0.clone()
        sg.sgmv_lora_delta(x, pool, seg, ya, opts=opts)
        fresh = sg.sgmv_build_segments(ids, 16, 0)
        yb = y0.clone()
        sg.sgmv_lora_delta(x, pool, fresh, yb, opts=opts)
        torch.cuda.synchronize()
        assert torch.equal(ya, yb), s
        ref = oracle.lora_delta(np32(w.x), np32(w.y0), trace[s].numpy(), np32(w.a), np32(w.b),
                                w.rank.numpy(), w.alpha.numpy())
        compare(np32(ya), ref, w.dtype, what=f"cached step {s}")
