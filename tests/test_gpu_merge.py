"""GPU parity of the merged weight (sgmv_merge_adapter; Ascend article 1.1 and 4.4, Punica page
SGMV section): W' = W + scale_l B_l A_l.

Bar, element by element against the fp64 oracle's merge_weight: bf16 |W' - ref| <= 2^-8 |ref|
(one rounding to bf16) + 2^-16 (|W| + |scale| sum_j |B A|) for the fp32 accumulation; fp32
2^-20 (|W| + |scale| sum_j |B A|). Also: ranks past r_l poisoned with NaN change nothing, in
place equals out of place bit for bit, untouched columns past K keep their bytes, and the
merged GEMM x W'^T agrees with the base GEMM plus the library's own delta (the merged vs
unmerged consistency check of Ascend article 5.2).
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from test_gpu_parity import DEV, compare, np32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import segmented_gather_gemv_amd as m
    return m


def _check(got, w, a, b, rank, alpha, l, bf16, what):
    ref = oracle.merge_weight(w, a, b, rank, alpha, l)
    r = int(rank[l])
    mag = np.abs(np.asarray(w, np.float64)) + abs(float(alpha[l]) / r) * (
        np.abs(np.asarray(b[l, :, :r], np.float64)) @ np.abs(np.asarray(a[l, :r, :], np.float64)))
    diff = np.abs(got.astype(np.float64) - ref)
    bound = (2.0 ** -8 * np.abs(ref) + 2.0 ** -16 * mag) if bf16 else 2.0 ** -20 * mag
    bad = diff > bound
    assert not bad.any(), f"{what}: {int(bad.sum())} elements, worst {float((diff - bound).max()):.3e}"


CASES = {
    # name: (custom workload arguments, base weight std)
    "decode_r16": (dict(M=4, K=4096, N=4096, L=2, R=16), 0.02),
    "mixed_rank_r64": (dict(M=4, K=1024, N=640, L=6, R=64, ranks=[1, 8, 33, 64]), 0.02),
    "ragged_rows_cols": (dict(M=4, K=520, N=100, L=4, R=24, ranks=[5, 24]), 0.5),
    "unaligned_k": (dict(M=4, K=999, N=77, L=2, R=16, ranks=[3, 16]), 0.5),
    "f32": (dict(M=4, K=300, N=130, L=3, R=8, ranks=[1, 8], dtype=torch.float32, w_std=0.1),
            0.5),
    "tiny": (dict(M=2, K=7, N=5, L=2, R=2, ranks=[1, 2]), 0.5),
    "tiny_f32": (dict(M=2, K=3, N=9, L=1, R=3, dtype=torch.float32, w_std=0.1), 0.5),
}


def _base(w, std, seed):
    g = torch.Generator().manual_seed(seed)
    return (torch.randn(w.N, w.K, generator=g) * std).to(w.dtype)


@pytest.mark.parametrize("name", sorted(CASES))
def test_merge_against_oracle(sg, name):
    kw, std = CASES[name]
    w = workloads.custom(name=name, seed=41, **kw)
    W = _base(w, std, 5)
    pool = sg.sgmv_pool_pack(w.a.to(DEV), w.b.to(DEV), w.rank.tolist(), w.alpha.tolist())
    Wd = W.to(DEV)
    bf16 = w.dtype == torch.bfloat16
    for l in range(w.L):
        out = sg.sgmv_merge_adapter(Wd, pool, l)
        torch.cuda.synchronize()
        _check(np32(out), np32(W), np32(w.a), np32(w.b), w.rank.numpy(), w.alpha.numpy(), l,
               bf16, f"{name} adapter {l}")
    assert torch.equal(Wd.cpu(), W)  # out of place leaves w alone


def test_merge_in_place_and_strided(sg):
    """In place equals out of place bit for bit; a strided w (ld > K) and out leave the
    columns past K untouched."""
    w = workloads.custom(name="ip", seed=42, M=4, K=512, N=200, L=2, R=16)
    W = _base(w, 0.05, 6)
    pool = sg.sgmv_pool_pack(w.a.to(DEV), w.b.to(DEV), w.rank.tolist(), w.alpha.tolist())
    ref = sg.sgmv_merge_adapter(W.to(DEV), pool, 1)
    Wi = W.to(DEV)
    sg.sgmv_merge_adapter(Wi, pool, 1, out=Wi)
    wide = torch.full((w.N, w.K + 24), 7.0, dtype=w.dtype, device=DEV)
    wide[:, :w.K] = W.to(DEV)
    owide = torch.full_like(wide, -3.0)
    sg.sgmv_merge_adapter(wide[:, :w.K], pool, 1, out=owide[:, :w.K])
    torch.cuda.synchronize()
    assert torch.equal(Wi, ref)
    assert torch.equal(owide[:, :w.K], ref)
    assert bool((owide[:, w.K:] == -3.0).all()) and bool((wide[:, w.K:] == 7.0).all())


def test_merge_never_reads_rank_padding(sg):
    w = workloads.custom(name="nanpad", seed=43, M=4, K=768, N=256, L=3, R=40, ranks=[7, 40, 17])
    W = _base(w, 0.05, 7).to(DEV)
    pool = sg.sgmv_pool_pack(w.a.to(DEV), w.b.to(DEV), w.rank.tolist(), w.alpha.tolist())
    clean = [sg.sgmv_merge_adapter(W, pool, l) for l in range(w.L)]
    nan = float("nan")
    for l in range(w.L):
        r = int(w.rank[l])
        pool.a[l, r:, :] = nan
        for j in range(r, pool.desc.R_pad):
            pool.b[l, j // 8, :, j % 8] = nan
    for l in range(w.L):
        assert torch.equal(sg.sgmv_merge_adapter(W, pool, l), clean[l]), l


def test_merged_gemm_matches_base_plus_delta(sg):
    """One adapter for the whole batch (Ascend article 4.4): x W'^T against x W^T plus the
    fused delta, both GEMMs in fp32 on the host from the GPU's bf16 operands."""
    w = workloads.custom(name="mg", seed=44, M=96, K=1024, N=768, L=4, R=16)
    w.ids = torch.full((w.M,), 2, dtype=torch.int32)
    W = _base(w, 0.02, 8)
    pool = sg.sgmv_pool_pack(w.a.to(DEV), w.b.to(DEV), w.rank.tolist(), w.alpha.tolist())
    Wm = sg.sgmv_merge_adapter(W.to(DEV), pool, 2)
    x = w.x.to(DEV)
    base = (w.x.float() @ W.float().T).to(w.dtype)          # bf16 base output
    y = base.to(DEV)
    seg = sg.sgmv_build_segments(w.ids.to(DEV), w.L, 0)
    sg.sgmv_lora_delta(x, pool, seg, y)
    torch.cuda.synchronize()
    merged = w.x.float() @ Wm.cpu().float().T
    compare(np32(y), merged.double().numpy(), w.dtype, what="merged vs unmerged")
