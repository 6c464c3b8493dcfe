"""GPU parity of sgmv_lora_delta_ids: segment build and fused delta in one call.

Bar: bit-exact against the two-call path (device builder, then the fused delta) with the
same launch options, for the segment arrays and for every element of y, plus the oracle bar
of the fused delta on y. The single-launch path covers bf16 batches of 1..512 tokens whose
ranks fit one 16-rank tile; larger batches, wider ranks and fp32 pools take two launches and
must agree the same way.
"""
import numpy as np
import pytest
import torch

import workloads
from test_gpu_parity import (DEV, _check_control, _xch_control, check_no_adapter_rows, compare,
                             large_counters, large_splits, np32, oracle_y, runs_parts, upload)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import segmented_gather_gemv_amd as m
    return m


def _ids_perm(M, L, seed):
    return torch.from_numpy(np.random.default_rng(seed).permutation(M) % L).to(torch.int32)


def _ids_few(M, adapters, no_lora_frac, seed):
    """Ids drawn from a few adapters, a fraction of the tokens without one (-1)."""
    rng = np.random.default_rng(seed)
    ids = rng.choice(np.asarray(adapters), size=M)
    ids[rng.random(M) < no_lora_frac] = -1
    return torch.from_numpy(ids.astype(np.int32))


# name: (custom workload arguments, ids override or None)
CASES = {
    "one_token": (dict(M=1, K=512, N=256, L=4, R=16), None),
    "small_16": (dict(M=16, K=1024, N=512, L=3, R=16, seq_lens=[16]), None),
    "large_17": (dict(M=17, K=1024, N=512, L=3, R=16, seq_lens=[17]), None),
    "max_one_adapter": (dict(M=512, K=1024, N=512, L=2, R=16, seq_lens=[512]), None),
    "max_distinct": (dict(M=512, K=256, N=256, L=512, R=16), lambda: _ids_perm(512, 512, 1)),
    "all_no_adapter": (dict(M=100, K=512, N=256, L=4, R=16, no_lora_frac=1.0), None),
    "pool_1024": (dict(M=300, K=512, N=256, L=1024, R=16, no_lora_frac=0.1), None),
    "chunked": (dict(M=300, K=1024, N=512, L=5, R=32, chunk=3, no_lora_frac=0.05), None),
    "mixed_rank": (dict(M=180, K=1536, N=768, L=30, R=64, ranks=[5, 16, 31, 64]), None),
    "unaligned": (dict(M=90, K=1000, N=300, L=20, R=24), None),
    "prefill_like": (dict(M=400, K=2048, N=768, L=6, R=64, ranks=[16, 40, 64],
                          seq_lens=[200, 17, 64, 119]), None),
    "qkv_slices": (dict(M=128, K=1024, N=512, L=8, R=16, slices=[(0, 256), (256, 128),
                                                                  (384, 128)]), None),
    # one launch at rank 16: mixed ranks below the tile, chunks, unaligned K and N, prefill
    "mixed_rank_r16": (dict(M=180, K=1536, N=768, L=30, R=16, ranks=[3, 9, 16]), None),
    "chunked_r16": (dict(M=300, K=1024, N=512, L=5, R=16, chunk=3, no_lora_frac=0.05), None),
    "chunked16_r16": (dict(M=512, K=2048, N=1024, L=3, R=16, chunk=16), None),
    "unaligned_r16": (dict(M=90, K=1000, N=300, L=20, R=16, ranks=[7, 16]), None),
    "prefill_like_r16": (dict(M=400, K=2048, N=768, L=6, R=16, ranks=[5, 16],
                              seq_lens=[200, 17, 64, 119]), None),
    # few adapters: large pieces as 16-row parts (one adapter; two adapters of different
    # ranks with ragged pieces and tokens without an adapter), at and past the largest batch
    # that runs parts
    "one_adapter_256": (dict(M=256, K=2048, N=1024, L=64, R=16),
                        lambda: torch.full((256,), 5, dtype=torch.int32)),
    "two_adapters_ragged": (dict(M=250, K=1152, N=640, L=8, R=32, ranks=[8, 32]),
                            lambda: _ids_few(250, [3, 6], 0.05, 2)),
    "parts_1024": (dict(M=1024, K=1024, N=512, L=4, R=16), None),
    # parts of chunked segments: a 40-row chunk is one large piece of three parts; a 100-row
    # chunk a full piece (four parts) and a 36-row piece (three)
    "chunked40_parts": (dict(M=400, K=1024, N=512, L=3, R=16, chunk=40), None),
    "chunked100_parts": (dict(M=500, K=1024, N=384, L=2, R=32, chunk=100,
                              no_lora_frac=0.05), None),
    "whole_1025": (dict(M=1025, K=1024, N=512, L=4, R=16), None),
    # two launches: beyond the single-launch batch size, and fp32
    "two_launch_513": (dict(M=513, K=512, N=256, L=40, R=16, no_lora_frac=0.05), None),
    "two_launch_f32": (dict(M=64, K=256, N=128, L=5, R=16, dtype=torch.float32), None),
}


def _workload(name, seed=7):
    kw, ids = CASES[name]
    w = workloads.custom(name=name, seed=seed, **kw)
    if ids is not None:
        w.ids = ids()
    return w


def _delta(sg, w, x, y0, fn, opts):
    """Apply fn(views, opts) on a copy of y0, with one view per output slice."""
    y = y0.clone()
    views = [(y[:, n0:n0 + n].contiguous(), n0) for n0, n in w.slices]
    fn(views if len(views) > 1 else views[0][0], opts)
    torch.cuda.synchronize()
    for t, n0 in views:
        y[:, n0:n0 + t.shape[1]] = t
    return y


def _poisoned(sg, w):
    seg = sg.sgmv_segments_alloc(w.M, w.L, w.chunk_size, DEV)
    for t in (seg.sorted_token_ids, seg.seg_indptr, seg.seg_lora_ids, seg.tiles, seg.info):
        t.fill_(-77)
    return seg


def _same_segments(a, b):
    ha, hb = a.host(), b.host()
    for k in ("sorted_token_ids", "seg_indptr", "seg_lora_ids", "large_tiles", "small_tiles"):
        assert torch.equal(ha[k], hb[k]), k
    assert ha["num_segments"] == hb["num_segments"]
    assert ha["status"] == hb["status"]
    return ha


def _check_control_any_slot(sg, seg, calls, pool):
    """The single launch may index small pieces' control words by adapter instead of by
    descriptor: the large counters and, among the small ones, exactly num_small_tiles of them
    advance by 64 per call; every other word stays zero."""
    ctl = _xch_control(sg, seg)
    ns = int(seg.info[2].item())
    lc = seg.desc.large_cap
    want = large_counters(sg, seg, calls, runs_parts(sg, pool, seg.desc.M))
    assert torch.equal(ctl[:lc], want), ctl[:lc, :4]
    small = ctl[lc:, 0]
    assert int((small == 64 * calls).sum()) == ns and int((small == 0).sum()) == small.numel() - ns
    assert torch.all(ctl[lc:, 1:] == 0)


def _both(sg, w, pool, x, y0, ids, opts):
    sep = sg.sgmv_build_segments(ids, w.L, w.chunk_size, on_device=True)
    ya = _delta(sg, w, x, y0, lambda y, o: sg.sgmv_lora_delta(x, pool, sep, y, opts=o), opts)
    one = _poisoned(sg, w)
    yb = _delta(sg, w, x, y0,
                lambda y, o: sg.sgmv_lora_delta_ids(ids, x, pool, one, y, opts=o), opts)
    return sep, ya, one, yb


@pytest.mark.parametrize("name", sorted(CASES))
def test_build_and_delta_match_two_calls(sg, name):
    w = _workload(name)
    pool, x, y0, ids = upload(w, sg)
    sep, ya, one, yb = _both(sg, w, pool, x, y0, ids, None)
    h = _same_segments(sep, one)
    assert h["status"] == sg.SGMV_OK
    assert torch.equal(ya, yb)
    compare(np32(yb), oracle_y(w, np32(w.y0)), w.dtype, what=name)
    check_no_adapter_rows(w, yb, w.y0)


@pytest.mark.parametrize("name", ["max_one_adapter", "mixed_rank", "prefill_like", "chunked",
                                  "unaligned", "mixed_rank_r16", "prefill_like_r16",
                                  "chunked_r16", "unaligned_r16", "one_adapter_256",
                                  "two_adapters_ragged", "parts_1024", "whole_1025",
                                  "chunked40_parts", "chunked100_parts"])
@pytest.mark.parametrize("P", [2, 4, 8])
def test_build_and_delta_with_exchange(sg, name, P):
    """Every piece splits its shrink over K with its partners; the single launch advances
    each piece's arrival counter by 64, as the two-call path does."""
    w = _workload(name, seed=P)
    pool, x, y0, ids = upload(w, sg)
    PL = large_splits(sg, pool, w.M, P)
    opts = sg.LaunchOpts(n_split_small=P, n_split_large=PL, exchange=1)
    sep, ya, one, yb = _both(sg, w, pool, x, y0, ids, opts)
    _same_segments(sep, one)
    assert torch.equal(ya, yb)
    _check_control(sg, sep, 1, pool)
    _check_control_any_slot(sg, one, 1, pool)
    # partials of late partners recomputed locally: the same bits
    local = sg.LaunchOpts(n_split_small=P, n_split_large=PL, exchange=1, exchange_wait=-1)
    yc = _delta(sg, w, x, y0, lambda y, o: sg.sgmv_lora_delta_ids(ids, x, pool, one, y, opts=o),
                local)
    assert torch.equal(ya, yc)
    # the single launch leaves the counters running; two launches rebuild, which clears them
    single = pool.desc.R_pad == 16 and 1 <= w.M <= 512 and w.dtype == torch.bfloat16
    _check_control_any_slot(sg, one, 2 if single else 1, pool)
    compare(np32(yb), oracle_y(w, np32(w.y0)), w.dtype, what=f"{name} P={P}")


# The single launch's adapter-major pieces when every adapter has rank 16 (A loaded before the
# tokens are known) with the K-split exchange at several split counts. Ragged K (steps not a
# multiple of the eight K slices: some slices empty), ragged N (column splits with empty
# column groups), adapters whose tokens make no small piece or a small piece next to large
# ones.
ROLE_CASES = {
    "decode_like": dict(M=256, K=4096, N=4096, L=64, R=16),
    "few_tokens": dict(M=40, K=1024, N=1024, L=8, R=16, no_lora_frac=0.1),
    "many_per_adapter": dict(M=300, K=2048, N=2048, L=5, R=16),
    "ragged": dict(M=100, K=1152, N=640, L=10, R=16),
}


@pytest.mark.parametrize("name", sorted(ROLE_CASES))
@pytest.mark.parametrize("P", [2, 4, 8])
def test_single_launch_rank16_exchange(sg, name, P):
    """Bit-exact against two launches, also with every partner's partial computed locally."""
    w = workloads.custom(name=name, seed=20 + P, **ROLE_CASES[name])
    pool, x, y0, ids = upload(w, sg)
    PL = large_splits(sg, pool, w.M, P)
    opts = sg.LaunchOpts(n_split_small=P, n_split_large=PL, exchange=1)
    sep, ya, one, yb = _both(sg, w, pool, x, y0, ids, opts)
    _same_segments(sep, one)
    assert torch.equal(ya, yb)
    local = sg.LaunchOpts(n_split_small=P, n_split_large=PL, exchange=1, exchange_wait=-1)
    yc = _delta(sg, w, x, y0, lambda y, o: sg.sgmv_lora_delta_ids(ids, x, pool, one, y, opts=o),
                local)
    assert torch.equal(ya, yc)
    _check_control_any_slot(sg, one, 2, pool)
    compare(np32(yb), oracle_y(w, np32(w.y0)), w.dtype, what=f"{name} P={P}")
    check_no_adapter_rows(w, yb, w.y0)


def test_build_and_delta_decode_full_size(sg):
    """The decode workload (one token per sequence, ids uniform over the pool)."""
    w = workloads.get("decode")
    pool, x, y0, ids = upload(w, sg)
    sep, ya, one, yb = _both(sg, w, pool, x, y0, ids, None)
    _same_segments(sep, one)
    assert torch.equal(ya, yb)
    compare(np32(yb), oracle_y(w, np32(w.y0)), w.dtype, what="decode")
    check_no_adapter_rows(w, yb, w.y0)
    # the delta alone (zero base) through the single launch
    z = torch.zeros_like(y0)
    yz = _delta(sg, w, x, z, lambda v, o: sg.sgmv_lora_delta_ids(ids, x, pool, one, v), None)
    compare(np32(yz), oracle_y(w, np.zeros((w.M, w.N))), w.dtype, what="decode zero base")


def test_build_and_delta_reuse_per_step(sg):
    """Successive steps with new ids reuse one segments object, as a serving loop does."""
    w = _workload("mixed_rank")
    pool, x, y0, _ = upload(w, sg)
    seg = sg.sgmv_segments_alloc(w.M, w.L, 0, DEV)
    for step in range(3):
        ids = torch.from_numpy(np.random.default_rng(100 + step).integers(-1, w.L, w.M)
                               .astype(np.int32)).to(DEV)
        y = _delta(sg, w, x, y0, lambda v, o: sg.sgmv_lora_delta_ids(ids, x, pool, seg, v), None)
        ref_seg = sg.sgmv_build_segments(ids, w.L, 0, on_device=True)
        ref = _delta(sg, w, x, y0, lambda v, o: sg.sgmv_lora_delta(x, pool, ref_seg, v), None)
        _same_segments(ref_seg, seg)
        assert torch.equal(y, ref), step


def test_build_and_delta_bad_ids(sg):
    """Ids outside {-1} U [0, L) count as -1 and are flagged in info[3]."""
    w = _workload("mixed_rank")
    ids_np = w.ids.numpy().copy()
    bad = np.array([3, 50, 51, 170])
    ids_np[bad] = [w.L, -2, 1 << 20, -(1 << 30)]
    pool, x, y0, _ = upload(w, sg)
    ids = torch.from_numpy(ids_np).to(DEV)
    sep, ya, one, yb = _both(sg, w, pool, x, y0, ids, None)
    h = _same_segments(sep, one)
    assert h["status"] == sg.SGMV_EBADID
    assert torch.equal(ya, yb)
    assert torch.equal(yb[torch.from_numpy(bad)].cpu(), w.y0[torch.from_numpy(bad)])
    clean = ids_np.copy()
    clean[bad] = -1
    w.ids = torch.from_numpy(clean)
    compare(np32(yb), oracle_y(w, np32(w.y0)), w.dtype, what="bad ids")
