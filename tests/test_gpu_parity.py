"""GPU parity: the HIP path through the C-ABI against the fp64 oracle on the same seeded
inputs.

Bars: segment and index arrays bit-exact (device builder vs host builder vs oracle); y for
bf16 within relative L2 5e-3 and max-abs 1e-2 * max|ref|, for fp32 within relative L2 1e-4
(plus the Fused-LoRA page's own max-abs < 1e-3 on its test recipe); every check repeated on
a zero-base twin (y0 = 0) so the delta itself is held to the bar; rows of tokens without an
adapter bit-identical to y0; h of the unfused shrink within relative L2 1e-4.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

BF16_REL_L2 = 5e-3
BF16_MAX_FRAC = 1e-2
F32_REL_L2 = 1e-4


@pytest.fixture(scope="module")
def sg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import segmented_gather_gemv_amd as m
    return m


DEV = "cuda"


def np32(t):
    return t.detach().float().cpu().numpy()


def upload(w, sg, y0_zero=False):
    pool = sg.sgmv_pool_pack(w.a.to(DEV), w.b.to(DEV), w.rank.tolist(), w.alpha.tolist())
    x = w.x.to(DEV)
    y = torch.zeros_like(w.y0).to(DEV) if y0_zero else w.y0.to(DEV)
    ids = w.ids.to(DEV)
    return pool, x, y, ids


def slice_views(w, y):
    """Output slices as separate tensors holding the matching columns of y."""
    return [(y[:, n0:n0 + n].contiguous(), n0) for n0, n in w.slices]


def compare(got, ref, dtype, rows=None, what=""):
    if rows is not None:
        got, ref = got[rows], ref[rows]
    diff = got.astype(np.float64) - ref
    nref = np.linalg.norm(ref)
    rel = np.linalg.norm(diff) / max(nref, 1e-30)
    mx = np.max(np.abs(diff)) if diff.size else 0.0
    if dtype == torch.bfloat16:
        assert rel <= BF16_REL_L2, f"{what} rel-L2 {rel:.3e}"
        assert mx <= BF16_MAX_FRAC * np.max(np.abs(ref)), f"{what} max-abs {mx:.3e}"
    else:
        assert rel <= F32_REL_L2, f"{what} rel-L2 {rel:.3e}"
    return rel, mx


def oracle_y(w, y0, rows=None):
    return oracle.lora_delta(np32(w.x), y0, w.ids.numpy(), np32(w.a), np32(w.b),
                             w.rank.numpy(), w.alpha.numpy(), rows=rows)


def run_fused(w, sg, y0_zero=False, chunk=None, on_device=True):
    pool, x, y, ids = upload(w, sg, y0_zero)
    C = w.chunk_size if chunk is None else chunk
    if on_device:
        seg = sg.sgmv_build_segments(ids, w.L, C, on_device=True)
    else:
        seg = sg.sgmv_build_segments(w.ids, w.L, C, on_device=False).to(DEV)
    outs = slice_views(w, y)
    sg.sgmv_lora_delta(x, pool, seg, outs if len(outs) > 1 else outs[0][0])
    torch.cuda.synchronize()
    yy = y.clone()
    for t, n0 in outs:
        n = t.shape[1]
        yy[:, n0:n0 + n] = t
    return yy, seg


def check_no_adapter_rows(w, y_gpu, y0):
    neg = (w.ids == -1).numpy()
    if neg.any():
        assert torch.equal(y_gpu[torch.from_numpy(neg)].cpu(), y0[torch.from_numpy(neg)].cpu())


def sample_rows(w, n, seed=0):
    """Tokens to check one by one: random ones plus the first and last token of every
    segment, so the edges of pieces and segments are covered."""
    seg = oracle.segments(w.ids.numpy(), w.L, w.chunk_size)
    st, ip = seg["sorted_token_ids"], seg["seg_indptr"]
    edge = set()
    for s in range(seg["num_segments"]):
        edge.add(int(st[ip[s]]))
        edge.add(int(st[ip[s + 1] - 1]))
    rng = np.random.default_rng(seed)
    rnd = set(rng.choice(w.M, size=min(n, w.M), replace=False).tolist())
    return sorted(edge | rnd)


# ---------------------------------------------------------------------------------------
# segment builder: device == host == oracle, bit for bit
# ---------------------------------------------------------------------------------------
def builder_cases():
    rng = np.random.default_rng(0)
    cases = [
        ("example", np.array([2, 2, 2, 5, 5, 1, 1]), 6, 0),
        ("empty", np.zeros(0, dtype=np.int64), 4, 0),
        ("all_neg", np.full(3000, -1), 7, 64),
        ("one", np.array([0]), 1, 0),
        ("uniform_dec", rng.integers(0, 64, 256), 64, 0),
        ("distinct_each_lane", np.arange(2048) % 1024, 1024, 0),
        ("runs", np.repeat(rng.integers(0, 50, 40), rng.integers(1, 300, 40)), 50, 0),
        ("runs_chunk", np.repeat(rng.integers(0, 50, 40), rng.integers(1, 300, 40)), 50, 7),
        ("neg_mix_c1", rng.integers(-1, 5, 1500), 5, 1),
        ("ragged", rng.integers(-1, 300, 5001), 300, 64),
        ("big_L", rng.integers(-1, 1024, 9000), 1024, 0),
        # one-round fast path (M <= 1024)
        ("fast_full_one_key", np.full(1024, 3), 4, 0),
        ("fast_full_c1", rng.integers(-1, 7, 1024), 7, 1),
        ("fast_1000_c16", rng.integers(-1, 40, 1000), 40, 16),
        ("fast_1025", rng.integers(-1, 40, 1025), 40, 0),
        ("fast_all_distinct", rng.permutation(1024), 1024, 0),
        ("fast_runs_c64", np.repeat(rng.integers(0, 9, 12), rng.integers(1, 90, 12)), 9, 64),
        ("fast_pool_1024", rng.integers(-1, 1024, 700), 1024, 5),
        # fewest waves covering M: 4 waves up to 256 tokens, 8 up to 512
        ("fast_256_distinct", rng.permutation(256), 256, 0),
        ("fast_257", rng.integers(-1, 30, 257), 30, 0),
        ("fast_300_c3", rng.integers(-1, 90, 300), 90, 3),
        ("fast_512_one_key", np.full(512, 7), 8, 16),
        ("fast_513", rng.integers(-1, 600, 513), 600, 0),
        # mid-size kernel (ids staged in LDS, per-wave ranges), its bounds, and beyond them
        ("mid_1025_c3", rng.integers(-1, 7, 1025), 7, 3),
        ("mid_L600", rng.integers(-1, 600, 2000), 600, 0),
        ("beyond_mid_lds", rng.integers(-1, 900, 2000), 900, 0),
        ("mid_runs_c64", np.repeat(rng.integers(-1, 40, 90), rng.integers(1, 400, 90)), 40, 64),
        ("mid_16k", rng.integers(-1, 50, 16384), 50, 0),
        ("mid_29k_c7", rng.integers(-1, 10, 29000), 10, 7),
        ("mid_over", rng.integers(-1, 50, 32769), 50, 16),
    ]
    for name in ("decode", "prefill", "mixed", "qkv"):
        w = workloads.get(name)
        cases.append((name, w.ids.numpy(), w.L, w.chunk_size))
    return cases


@pytest.mark.parametrize("case", builder_cases(), ids=lambda c: c[0])
def test_device_builder_bit_exact(sg, case):
    name, ids, L, C = case
    ids_t = torch.as_tensor(np.asarray(ids, dtype=np.int32))
    dev = sg.sgmv_build_segments(ids_t.to(DEV), L, C, on_device=True).host()
    host = sg.sgmv_build_segments(ids_t, L, C, on_device=False).host()
    ref = oracle.segments(ids_t.numpy(), L, C)
    M = ids_t.numel()
    assert dev["status"] == sg.SGMV_OK
    assert np.array_equal(dev["sorted_token_ids"].numpy()[:M], ref["sorted_token_ids"])
    for k in ("sorted_token_ids", "seg_indptr", "seg_lora_ids", "large_tiles", "small_tiles"):
        assert torch.equal(dev[k][:M] if k == "sorted_token_ids" else dev[k],
                           host[k][:M] if k == "sorted_token_ids" else host[k]), k
    assert dev["num_segments"] == host["num_segments"] == ref["num_segments"]
    from test_abi_host import check_records
    check_records(dev, ref)


@pytest.mark.parametrize("M", [6, 700, 5000, 40000])  # each builder kernel
def test_device_builder_bad_ids_flagged(sg, M):
    rng = np.random.default_rng(M)
    ids = rng.integers(-1, 3, M).astype(np.int32)
    bad = rng.choice(M, size=max(1, M // 100), replace=False)
    ids[bad] = rng.choice([5, -3, 3, 1 << 20], size=bad.size)
    dev = sg.sgmv_build_segments(torch.from_numpy(ids).to(DEV), 3, 0, on_device=True).host()
    assert dev["status"] == sg.SGMV_EBADID
    clean = ids.copy()
    clean[bad] = -1
    ref = oracle.segments(clean, 3, 0)
    assert np.array_equal(dev["sorted_token_ids"].numpy(), ref["sorted_token_ids"])
    assert np.array_equal(dev["seg_indptr"].numpy(), ref["seg_indptr"])
    # the same ids without the bad ones are clean
    ok = sg.sgmv_build_segments(torch.from_numpy(clean).to(DEV), 3, 0, on_device=True).host()
    assert ok["status"] == sg.SGMV_OK


def test_device_builder_reuse_of_buffers(sg):
    """Building twice into the same arrays (the per-step pattern) gives the same result."""
    w = workloads.get("decode")
    ids = w.ids.to(DEV)
    seg = sg.sgmv_build_segments(ids, w.L, 0, on_device=True)
    first = seg.host()
    sg.sgmv_build_segments(ids, w.L, 0, on_device=True, out=seg)
    again = seg.host()
    for k in ("sorted_token_ids", "seg_indptr", "seg_lora_ids", "large_tiles", "small_tiles"):
        assert torch.equal(first[k], again[k])


# ---------------------------------------------------------------------------------------
# the Fused-LoRA page's test recipe (fp32)
# ---------------------------------------------------------------------------------------
def test_tiny_recipe_fp32(sg):
    rec = json.load(open(os.path.join(GOLDEN, "fused_lora_test_recipe.json")))
    w = workloads.tiny()
    assert w.ids.tolist() == rec["lora_indices"] and w.M == rec["batch_size"]
    assert (w.K, w.N, w.L, w.R) == (rec["in_dim"], rec["out_dim"], rec["num_loras"], rec["r"])
    y_gpu, _ = run_fused(w, sg, y0_zero=True)
    ref = oracle_y(w, np.zeros((w.M, w.N)))
    got = np32(y_gpu)
    assert np.max(np.abs(got - ref)) < rec["max_abs_tol"]
    compare(got, ref, torch.float32, what="tiny")


# ---------------------------------------------------------------------------------------
# parity on small shapes spanning several pieces and ragged tails
# ---------------------------------------------------------------------------------------
SMALL_CASES = {
    # name: custom() kwargs
    "bf16_ragged": dict(M=300, K=512, N=640, L=8, R=16, no_lora_frac=0.1),
    "bf16_mixed_rank": dict(M=333, K=384, N=320, L=12, R=64, ranks=[3, 8, 16, 24, 33, 64],
                            no_lora_frac=0.15),
    "bf16_prefill_like": dict(M=700, K=256, N=512, L=6, R=32,
                              seq_lens=[200, 17, 1, 64, 130, 288]),
    "bf16_odd_shape": dict(M=77, K=100, N=37, L=5, R=3),
    "bf16_odd_shape_rank": dict(M=150, K=136, N=200, L=4, R=40, ranks=[1, 9, 17, 40]),
    "bf16_chunked": dict(M=500, K=256, N=256, L=3, R=16, chunk=13, no_lora_frac=0.05),
    "f32_ragged": dict(M=130, K=200, N=96, L=5, R=16, dtype=torch.float32, w_std=0.1,
                       no_lora_frac=0.1),
    "f32_odd": dict(M=40, K=100, N=37, L=3, R=3, dtype=torch.float32, w_std=0.1),
    "f32_mixed_rank": dict(M=90, K=64, N=70, L=6, R=64, ranks=[1, 5, 16, 64],
                           dtype=torch.float32, w_std=0.1, seq_lens=[70, 20]),
    # fp32 pieces at the expand's row-count branches: 16, 17, 32, 33, 64 rows, a 64 + 16
    # segment, one row
    "f32_piece_edges": dict(M=243, K=160, N=200, L=7, R=16, dtype=torch.float32, w_std=0.1,
                            seq_lens=[16, 17, 32, 33, 64, 80, 1],
                            seq_adapters=[3, 0, 6, 1, 5, 2, 4]),
    "f32_piece_edges_c16": dict(M=243, K=160, N=200, L=7, R=16, dtype=torch.float32,
                                w_std=0.1, seq_lens=[16, 17, 32, 33, 64, 80, 1],
                                seq_adapters=[3, 0, 6, 1, 5, 2, 4], chunk=16),
}


def small_workload(name, y0_zero=False):
    kw = dict(SMALL_CASES[name])
    return workloads.custom(name=name, y0_zero=y0_zero, seed=7, **kw)


@pytest.mark.parametrize("name", sorted(SMALL_CASES))
@pytest.mark.parametrize("zero_base", [False, True])
def test_fused_small(sg, name, zero_base):
    w = small_workload(name, y0_zero=zero_base)
    y_gpu, _ = run_fused(w, sg)
    ref = oracle_y(w, np32(w.y0))
    compare(np32(y_gpu), ref, w.dtype, what=name)
    check_no_adapter_rows(w, y_gpu, w.y0)


@pytest.mark.parametrize("name", sorted(SMALL_CASES))
def test_unfused_small(sg, name):
    w = small_workload(name)
    pool, x, y, ids = upload(w, sg)
    seg = sg.sgmv_build_segments(ids, w.L, w.chunk_size, on_device=True)
    h = sg.sgmv_shrink(x, pool, seg)
    torch.cuda.synchronize()
    h_ref = oracle.shrink(np32(w.x), w.ids.numpy(), np32(w.a), w.rank.numpy())
    lora = w.ids.numpy() >= 0
    hg = h.cpu().numpy()[lora]
    hr = h_ref[lora]
    assert np.linalg.norm(hg - hr) / max(np.linalg.norm(hr), 1e-30) <= 1e-4
    # expand from the GPU h
    sg.sgmv_expand(h, pool, seg, y)
    torch.cuda.synchronize()
    ref = oracle.expand(h_ref, np32(w.y0), w.ids.numpy(), np32(w.b), w.rank.numpy(),
                        w.alpha.numpy())
    compare(np32(y), ref, w.dtype, what=name + " unfused")
    check_no_adapter_rows(w, y, w.y0)


def test_rank_padding_never_read(sg):
    """Poison every pool entry at ranks >= r_l with NaN: y must not change at all."""
    w = small_workload("bf16_mixed_rank")
    pool, x, y, ids = upload(w, sg)
    seg = sg.sgmv_build_segments(ids, w.L, 0, on_device=True)
    y_clean = y.clone()
    sg.sgmv_lora_delta(x, pool, seg, y_clean)
    torch.cuda.synchronize()
    nan = float("nan")
    for l, r in enumerate(w.rank.tolist()):
        pool.a[l, r:, :] = nan
        # rank octets: ranks j >= r live at b[l, j // 8, :, j % 8]
        for j in range(r, pool.b.shape[1] * 8):
            pool.b[l, j // 8, :, j % 8] = nan
    y_nan = y.clone()
    sg.sgmv_lora_delta(x, pool, seg, y_nan)
    torch.cuda.synchronize()
    assert torch.equal(y_clean, y_nan)


def test_guard_bands_and_strides(sg):
    """x and y as strided views inside larger buffers: nothing outside the views changes."""
    w = small_workload("bf16_ragged")
    pool = sg.sgmv_pool_pack(w.a.to(DEV), w.b.to(DEV), w.rank.tolist(), w.alpha.tolist())
    xb = torch.randn(w.M + 6, w.K + 40, generator=torch.Generator().manual_seed(3)).to(
        torch.bfloat16).to(DEV)
    xb[3:3 + w.M, 8:8 + w.K] = w.x.to(DEV)
    x = xb[3:3 + w.M, 8:8 + w.K]
    yb = torch.full((w.M + 4, w.N + 24), 7.0, dtype=torch.bfloat16, device=DEV)
    yb[2:2 + w.M, 8:8 + w.N] = w.y0.to(DEV)
    y = yb[2:2 + w.M, 8:8 + w.N]
    before = yb.clone()
    seg = sg.sgmv_build_segments(w.ids.to(DEV), w.L, 0, on_device=True)
    sg.sgmv_lora_delta(x, pool, seg, y)
    torch.cuda.synchronize()
    mask = torch.ones_like(yb, dtype=torch.bool)
    mask[2:2 + w.M, 8:8 + w.N] = False
    assert torch.equal(yb[mask], before[mask])
    compare(np32(y), oracle_y(w, np32(w.y0)), w.dtype, what="strided")


def test_chunk_size_and_host_segments_agree(sg):
    w = small_workload("bf16_ragged")
    ref = oracle_y(w, np32(w.y0))
    for C in (0, 1, 5, 64):
        for on_dev in (True, False):
            y_gpu, _ = run_fused(w, sg, chunk=C, on_device=on_dev)
            compare(np32(y_gpu), ref, w.dtype, what=f"chunk {C} dev {on_dev}")


def test_token_permutation(sg):
    w = small_workload("bf16_ragged", y0_zero=True)
    y_a, _ = run_fused(w, sg)
    perm = torch.from_numpy(np.random.default_rng(4).permutation(w.M))
    wp = workloads.Workload(w.name, w.dtype, w.ids[perm], w.x[perm], w.a, w.b, w.y0[perm],
                            w.rank, w.alpha)
    y_b, _ = run_fused(wp, sg)
    compare(np32(y_b), np32(y_a)[perm.numpy()].astype(np.float64), w.dtype, what="perm")


def test_all_no_adapter_and_empty(sg):
    w = small_workload("bf16_ragged")
    w.ids[:] = -1
    y_gpu, _ = run_fused(w, sg)
    assert torch.equal(y_gpu.cpu(), w.y0)
    e = workloads.custom(M=0, K=64, N=64, L=2, R=16)
    y_gpu, _ = run_fused(e, sg)
    assert y_gpu.numel() == 0


def test_bad_ids_on_device_are_skipped(sg):
    w = small_workload("bf16_ragged")
    bad = w.ids.clone()
    bad[5] = 99
    bad[17] = -4
    pool, x, y, _ = upload(w, sg)
    seg = sg.sgmv_build_segments(bad.to(DEV), w.L, 0, on_device=True)
    sg.sgmv_lora_delta(x, pool, seg, y)
    torch.cuda.synchronize()
    assert int(seg.info[3].item()) == sg.SGMV_EBADID
    clean = bad.clone()
    clean[5] = -1
    clean[17] = -1
    ref = oracle.lora_delta(np32(w.x), np32(w.y0), clean.numpy(), np32(w.a), np32(w.b),
                            w.rank.numpy(), w.alpha.numpy())
    compare(np32(y), ref, w.dtype, what="bad ids")
    assert torch.equal(y[5].cpu(), w.y0[5]) and torch.equal(y[17].cpu(), w.y0[17])


def test_slices_in_any_order(sg):
    """Three output slices listed out of pool order, each its own tensor."""
    w = workloads.custom(M=120, K=256, N=320, L=5, R=32, seed=3, no_lora_frac=0.1,
                         slices=[(0, 192), (192, 64), (256, 64)])
    pool, x, y, ids = upload(w, sg)
    seg = sg.sgmv_build_segments(ids, w.L, 0, on_device=True)
    q = y[:, 0:192].contiguous()
    k = y[:, 192:256].contiguous()
    v = y[:, 256:320].contiguous()
    sg.sgmv_lora_delta(x, pool, seg, [(v, 256), (q, 0), (k, 192)])
    torch.cuda.synchronize()
    got = torch.cat([q, k, v], dim=1)
    compare(np32(got), oracle_y(w, np32(w.y0)), w.dtype, what="slices")


# ---------------------------------------------------------------------------------------
# full-size workloads, every row against the oracle
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "mixed", "qkv"])
@pytest.mark.parametrize("zero_base", [False, True])
def test_fused_full_size(sg, name, zero_base):
    w = workloads.get(name)
    if zero_base:
        w.y0 = torch.zeros_like(w.y0)
    print(f"fused full size {name} zero_base={zero_base}", flush=True)
    y_gpu, seg = run_fused(w, sg)
    assert int(seg.info[3].item()) == sg.SGMV_OK
    ref = oracle_y(w, np32(w.y0))
    compare(np32(y_gpu), ref, w.dtype, what=name)
    check_no_adapter_rows(w, y_gpu, w.y0)


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "mixed", "qkv"])
@pytest.mark.parametrize("zero_base", [False, True])
def test_unfused_full_size(sg, name, zero_base):
    w = workloads.get(name)
    if zero_base:
        w.y0 = torch.zeros_like(w.y0)
    print(f"unfused full size {name} zero_base={zero_base}", flush=True)
    pool, x, y, ids = upload(w, sg)
    seg = sg.sgmv_build_segments(ids, w.L, w.chunk_size, on_device=True)
    h = sg.sgmv_shrink(x, pool, seg)
    outs = slice_views(w, y)
    sg.sgmv_expand(h, pool, seg, outs if len(outs) > 1 else outs[0][0])
    torch.cuda.synchronize()
    for t, n0 in outs:
        y[:, n0:n0 + t.shape[1]] = t
    h_ref = oracle.shrink(np32(w.x), w.ids.numpy(), np32(w.a), w.rank.numpy())
    lora = w.ids.numpy() >= 0
    hg = h.cpu().numpy()[lora]
    hr = h_ref[lora]
    assert np.linalg.norm(hg - hr) / np.linalg.norm(hr) <= 1e-4
    ref = oracle_y(w, np32(w.y0))
    compare(np32(y), ref, w.dtype, what=name + " unfused")
    check_no_adapter_rows(w, y, w.y0)


# ---------------------------------------------------------------------------------------
# K-split exchange of small pieces (fused calls): column-split workgroups of one piece share
# the shrink over K through the segments' workspace
# ---------------------------------------------------------------------------------------
XCH_CASES = {
    "xch_decode": dict(M=200, K=2048, N=1024, L=40, R=16, no_lora_frac=0.05),
    "xch_mixed_rank": dict(M=180, K=1536, N=768, L=30, R=64, ranks=[5, 16, 31, 64]),
    "xch_odd": dict(M=90, K=1000, N=300, L=20, R=24),          # unaligned kernel, ragged K
    "xch_narrow": dict(M=64, K=1024, N=64, L=8, R=16),          # splits without columns
    "xch_chunked": dict(M=240, K=1024, N=512, L=4, R=32, chunk=5, no_lora_frac=0.1),
    # large pieces (17..64 rows) and ragged tails, several rank tiles
    "xch_prefill": dict(M=400, K=2048, N=768, L=6, R=64, ranks=[16, 40, 64],
                        seq_lens=[200, 17, 64, 119]),
    "xch_prefill_r16": dict(M=300, K=1024, N=512, L=3, R=16, seq_lens=[100, 150, 50]),
    "xch_prefill_odd": dict(M=150, K=700, N=200, L=4, R=48, seq_lens=[33, 90, 27]),
    # the LDS-staged shrink of whole large pieces at its edges: a last K chunk of 8 columns
    # (K % 64 = 8, aligned), pieces of 17..64 rows (2, 3 and 4 row tiles), ranks that end
    # inside a 16-rank tile
    "xch_prefill_kedge": dict(M=400, K=2120, N=384, L=6, R=64, ranks=[17, 33, 47, 64],
                              seq_lens=[113, 17, 48, 97, 125]),
    # past the part-split batch size: large pieces run whole
    "xch_prefill_whole": dict(M=1100, K=1024, N=384, L=5, R=32, ranks=[8, 32],
                              seq_lens=[500, 17, 300, 83, 200]),
}


def _xch_control(sg, seg):
    """Control words [large_cap + small_cap][16], indexed like the records: word 0 of each
    piece is its arrival counter."""
    n = (seg.desc.large_cap + seg.desc.small_cap) * 16
    return seg.exchange[:n * 4].view(torch.int32).view(-1, 16).cpu()


def runs_parts(sg, pool, M):
    """Fused bf16 calls run large pieces as 16-row parts on batches up to PART_SPLIT_MAX_M
    tokens at pool ranks up to 32."""
    return M <= sg.PART_SPLIT_MAX_M and pool.desc.R_pad <= 32


def large_counters(sg, seg, calls, parts):
    """Expected control words of the large records after `calls` exchange calls: word 0 of
    each large piece, or, when large pieces run as 16-row parts, word j of part j (parts
    0 .. ceil(rows / 16) - 1); every other word zero."""
    lc = seg.desc.large_cap
    want = torch.zeros(lc, 16, dtype=torch.int32)
    nl = int(seg.info[1].item())
    rows = seg.tiles.view(-1, sg.TILE_INTS)[:nl, 2].cpu()
    for i in range(nl):
        want[i, :-(-int(rows[i]) // sg.SMALL_ROWS) if parts else 1] = 64 * calls
    return want


def large_splits(sg, pool, M, P):
    """The most column splits up to P that large pieces take with the exchange: 16-row parts
    hold 8 at ranks up to 32; whole pieces, and parts at larger ranks, 4."""
    return min(P, 8 if runs_parts(sg, pool, M) else 4)


def _check_control(sg, seg, calls, pool):
    """Every exchange call advances the counter of every piece (or part) by exactly 64."""
    ctl = _xch_control(sg, seg)
    ns = int(seg.info[2].item())
    lc = seg.desc.large_cap
    want = large_counters(sg, seg, calls, runs_parts(sg, pool, seg.desc.M))
    assert torch.equal(ctl[:lc], want), ctl[:lc, :4]
    assert torch.all(ctl[lc:lc + ns, 0] == 64 * calls), ctl[lc:lc + ns, 0]
    assert torch.all(ctl[lc + ns:, 0] == 0) and torch.all(ctl[lc:, 1:] == 0)


def _fused_opts(sg, w, seg, pool, x, y0, **kw):
    y = y0.clone()
    sg.sgmv_lora_delta(x, pool, seg, y, opts=sg.LaunchOpts(**kw))
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("name", sorted(XCH_CASES))
@pytest.mark.parametrize("P", [2, 3, 4, 8])
def test_exchange_parity_and_determinism(sg, name, P):
    w = workloads.custom(name=name, seed=11, **XCH_CASES[name])
    pool, x, y0, ids = upload(w, sg)
    seg = sg.sgmv_build_segments(ids, w.L, w.chunk_size, on_device=True)
    assert seg.exchange is not None
    torch.cuda.synchronize()
    _check_control(sg, seg, 0, pool)
    ref = oracle_y(w, np32(w.y0))
    PL = large_splits(sg, pool, w.M, P)
    off = _fused_opts(sg, w, seg, pool, x, y0, n_split_small=P, n_split_large=PL, exchange=-1)
    _check_control(sg, seg, 0, pool)
    on = _fused_opts(sg, w, seg, pool, x, y0, n_split_small=P, n_split_large=PL, exchange=1)
    compare(np32(off), ref, w.dtype, what=f"{name} P={P} no exchange")
    compare(np32(on), ref, w.dtype, what=f"{name} P={P} exchange")
    check_no_adapter_rows(w, on, w.y0)
    _check_control(sg, seg, 1, pool)
    # the sum is taken in split order: the same bits on every call, and when the partials
    # of late partners are recomputed locally (no wait at all)
    again = _fused_opts(sg, w, seg, pool, x, y0, n_split_small=P, n_split_large=PL, exchange=1)
    local = _fused_opts(sg, w, seg, pool, x, y0, n_split_small=P, n_split_large=PL, exchange=1,
                        exchange_wait=-1)
    assert torch.equal(on, again)
    assert torch.equal(on, local)
    _check_control(sg, seg, 3, pool)
    # a rebuild clears the control words
    sg.sgmv_build_segments(ids, w.L, w.chunk_size, on_device=True, out=seg)
    torch.cuda.synchronize()
    _check_control(sg, seg, 0, pool)


def test_exchange_workspace_optional(sg):
    """Segments without a workspace take the path without exchange; results agree."""
    w = workloads.custom(name="xch_opt", seed=12, **XCH_CASES["xch_decode"])
    pool, x, y0, ids = upload(w, sg)
    seg = sg.sgmv_build_segments(ids, w.L, 0, on_device=True)
    bare = sg.sgmv_segments_alloc(w.M, w.L, 0, DEV, exchange=False)
    sg.sgmv_build_segments(ids, w.L, 0, on_device=True, out=bare)
    assert bare.exchange is None
    a = _fused_opts(sg, w, seg, pool, x, y0)
    b = _fused_opts(sg, w, bare, pool, x, y0)
    ref = oracle_y(w, np32(w.y0))
    compare(np32(a), ref, w.dtype, what="with workspace")
    compare(np32(b), ref, w.dtype, what="without workspace")


def test_exchange_full_decode_forced_local(sg):
    """The decode workload with every missing partial computed locally, bit-identical to the
    default call, every row against the oracle."""
    w = workloads.get("decode")
    pool, x, y0, ids = upload(w, sg)
    seg = sg.sgmv_build_segments(ids, w.L, 0, on_device=True)
    a = _fused_opts(sg, w, seg, pool, x, y0)
    b = _fused_opts(sg, w, seg, pool, x, y0, exchange_wait=-1)
    assert torch.equal(a, b)
    compare(np32(a), oracle_y(w, np32(w.y0)), w.dtype, what="decode")


@pytest.mark.parametrize("name", ["prefill", "mixed", "qkv"])
@pytest.mark.parametrize("zero_base", [False, True])
def test_exchange_full_size_forced_local(sg, name, zero_base):
    """Full-size workloads with large pieces: the default call (large and small pieces split
    their shrink over K) is bit-identical to the call that computes every partner's partial
    locally, and every row matches the oracle."""
    w = workloads.get(name)
    if zero_base:
        w.y0 = torch.zeros_like(w.y0)
    print(f"exchange forced local {name} zero_base={zero_base}", flush=True)
    pool, x, y0, ids = upload(w, sg)
    seg = sg.sgmv_build_segments(ids, w.L, w.chunk_size, on_device=True)
    def call(**kw):
        y = y0.clone()
        views = [(y[:, n0:n0 + n].contiguous(), n0) for n0, n in w.slices]
        sg.sgmv_lora_delta(x, pool, seg, views if len(views) > 1 else views[0][0],
                           opts=sg.LaunchOpts(**kw))
        torch.cuda.synchronize()
        for t, n0 in views:
            y[:, n0:n0 + t.shape[1]] = t
        return y

    a = call()
    b = call(exchange_wait=-1)
    assert torch.equal(a, b)
    compare(np32(a), oracle_y(w, np32(w.y0)), w.dtype, what=name)
    check_no_adapter_rows(w, a, w.y0)
