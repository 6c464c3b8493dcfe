"""GPU parity of the scale folded into B at pack time (sgmv_pool_pack_ex with
SGMV_PACK_FOLD_SCALE; Ascend article 2.1 and 3.2: the alpha/r factor on either side of the
expand, or folded into B when the weights are loaded).

Bar:
  * the packed B of a folded pool equals the oracle's fold (fp32 product, one rounding to
    the pool dtype) bit for bit, ranks past r_l and all padding zero, stored scales 1;
  * with power-of-two scales the folded pool gives y bit-identical to the unfolded pool on
    every path (fused, fused with the K-split exchange, single launch, shrink + expand);
  * with other scales y meets the usual bar against the oracle's delta over the folded B.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from test_gpu_parity import DEV, check_no_adapter_rows, compare, np32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import segmented_gather_gemv_amd as m
    return m


def _pack(sg, w, fold):
    return sg.sgmv_pool_pack(w.a.to(DEV), w.b.to(DEV), w.rank.tolist(), w.alpha.tolist(),
                             fold_scale=fold)


def _unpack_b(pool, L, N, R):
    """The pool's B in the user layout (L, N, R_pad) from its rank octets."""
    d = pool.desc
    b = pool.b.view(L, d.R_pad // 8, d.N_pad, 8).permute(0, 2, 1, 3).reshape(L, d.N_pad, d.R_pad)
    return b[:, :N, :], b[:, N:, :]


def _non_pow2(w, seed):
    """Replace the alphas by values whose alpha/r is not a power of two."""
    rng = np.random.default_rng(seed)
    w.alpha = torch.from_numpy(rng.uniform(0.3, 40.0, w.L).astype(np.float32))
    return w


CASES = {
    "mixed_rank_bf16": dict(M=150, K=520, N=300, L=12, R=40, ranks=[3, 16, 29, 40],
                            no_lora_frac=0.1),
    "decode_like_bf16": dict(M=64, K=1024, N=1024, L=16, R=16),
    "unaligned_f32": dict(M=40, K=100, N=37, L=5, R=8, ranks=[1, 5, 8], dtype=torch.float32,
                          w_std=0.1),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_folded_pool_matches_oracle_fold(sg, name):
    w = _non_pow2(workloads.custom(name=name, seed=31, **CASES[name]), 1)
    pool = _pack(sg, w, True)
    torch.cuda.synchronize()
    assert pool.desc.scale_folded == 1
    assert torch.equal(pool.scale.cpu(), torch.ones(w.L))
    bf16 = w.dtype == torch.bfloat16
    ref, _ = oracle.fold_scale(np32(w.b), w.rank.numpy(), w.alpha.numpy(), bf16)
    got, pad_n = _unpack_b(pool, w.L, w.N, w.R)
    got = np32(got)
    for l in range(w.L):
        r = int(w.rank[l])
        assert np.array_equal(got[l, :, :r].view(np.uint32), ref[l, :, :r].view(np.uint32)), l
        assert not np.any(got[l, :, r:])
    assert not torch.any(pad_n != 0)
    plain = _pack(sg, w, False)
    torch.cuda.synchronize()
    assert plain.desc.scale_folded == 0


@pytest.mark.parametrize("name", sorted(CASES))
def test_folded_delta_against_oracle(sg, name):
    w = _non_pow2(workloads.custom(name=name, seed=32, **CASES[name]), 2)
    pool = _pack(sg, w, True)
    x, y0, ids = w.x.to(DEV), w.y0.to(DEV), w.ids.to(DEV)
    bf, alpha1 = oracle.fold_scale(np32(w.b), w.rank.numpy(), w.alpha.numpy(),
                                   w.dtype == torch.bfloat16)
    ref = oracle.lora_delta(np32(w.x), np32(w.y0), w.ids.numpy(), np32(w.a), bf,
                            w.rank.numpy(), alpha1)
    seg = sg.sgmv_build_segments(ids, w.L, 0)
    y = y0.clone()
    sg.sgmv_lora_delta(x, pool, seg, y)
    h = sg.sgmv_shrink(x, pool, seg)
    y2 = y0.clone()
    sg.sgmv_expand(h, pool, seg, y2)
    torch.cuda.synchronize()
    compare(np32(y), ref, w.dtype, what=f"{name} fused")
    compare(np32(y2), ref, w.dtype, what=f"{name} unfused")
    check_no_adapter_rows(w, y, w.y0)
    if w.dtype == torch.bfloat16:
        one = sg.sgmv_segments_alloc(w.M, w.L, 0, DEV)
        y3 = y0.clone()
        sg.sgmv_lora_delta_ids(ids, x, pool, one, y3)
        torch.cuda.synchronize()
        assert torch.equal(y3, y)


def _all_paths(sg, w, pool, x, y0, ids):
    out = {}
    seg = sg.sgmv_build_segments(ids, w.L, w.chunk_size)
    y = y0.clone()
    sg.sgmv_lora_delta(x, pool, seg, y)
    out["fused"] = y
    y = y0.clone()
    sg.sgmv_lora_delta(x, pool, seg, y, opts=sg.LaunchOpts(n_split_small=4, n_split_large=2,
                                                           exchange=1))
    out["exchange"] = y
    h = sg.sgmv_shrink(x, pool, seg)
    y = y0.clone()
    sg.sgmv_expand(h, pool, seg, y)
    out["unfused"] = y
    if w.dtype == torch.bfloat16 and w.M <= 512:
        one = sg.sgmv_segments_alloc(w.M, w.L, w.chunk_size, DEV)
        y = y0.clone()
        sg.sgmv_lora_delta_ids(ids, x, pool, one, y)
        out["single launch"] = y
    torch.cuda.synchronize()
    return out


def _pow2(w, seed):
    """alpha_l = r_l times a power of two (1/4 .. 8), so every scale is a power of two."""
    rng = np.random.default_rng(seed)
    w.alpha = w.rank.float() * torch.from_numpy(rng.choice([0.25, 0.5, 1.0, 2.0, 8.0], w.L)
                                                .astype(np.float32))
    return w


POW2 = {
    "decode": lambda: workloads.get("decode"),
    "mixed_rank_pow2": lambda: _pow2(workloads.custom(M=200, K=1024, N=640, L=10, R=64,
                                                      ranks=[8, 16, 32, 64], name="pow2",
                                                      seed=33), 3),
    "prefill_like": lambda: _pow2(workloads.custom(M=400, K=2048, N=768, L=6, R=64,
                                                   ranks=[16, 32, 64], seq_lens=[200, 17, 64, 119],
                                                   name="pow2p", seed=34), 4),
}


@pytest.mark.parametrize("name", sorted(POW2))
def test_power_of_two_fold_is_bit_identical(sg, name):
    w = POW2[name]()
    s = w.alpha.numpy() / w.rank.numpy().astype(np.float32)
    assert np.all(np.frexp(s)[0] == 0.5), "the workload's scales are powers of two"
    x, y0, ids = w.x.to(DEV), w.y0.to(DEV), w.ids.to(DEV)
    a = _all_paths(sg, w, _pack(sg, w, False), x, y0, ids)
    b = _all_paths(sg, w, _pack(sg, w, True), x, y0, ids)
    for k in a:
        assert torch.equal(a[k], b[k]), k
    ref = oracle.lora_delta(np32(w.x), np32(w.y0), w.ids.numpy(), np32(w.a), np32(w.b),
                            w.rank.numpy(), w.alpha.numpy())
    compare(np32(b["fused"]), ref, w.dtype, what=name)
