"""sgmv_lora_delta_ids_noalloc: the build + fused delta with the exchange workspace in the
library's static device array, for callers that cannot allocate.

Bar: through the C-ABI, each call leaves y and the segment arrays bit-identical to
sgmv_lora_delta_ids on segments with their own workspace (the same kernels, so the same bits),
and y meets the oracle's bf16 bar with rows of tokens without adapter untouched. Calls follow
one another on one stream with the array keeping the previous call's contents: the decode
batch, a larger two-launch batch with large pieces, then smaller batches (a different pool and
fewer tokens). A batch whose exchange does not fit the array is refused before anything runs.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import workloads

pytestmark = pytest.mark.gpu

DEV = "cuda"


@pytest.fixture(scope="module")
def sg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import segmented_gather_gemv_amd as m
    return m


def _np32(t):
    return t.detach().float().cpu().numpy()


def _run(sg, w, fn_name):
    """One call of the named C-ABI entry point on fresh copies of the inputs; returns y and
    the segments."""
    pool = sg.sgmv_pool_pack(w.a.to(DEV), w.b.to(DEV), w.rank.tolist(), w.alpha.tolist())
    x = w.x.to(DEV)
    y = w.y0.to(DEV)
    ids = w.ids.to(DEV)
    seg = sg.sgmv_segments_alloc(w.M, w.L, w.chunk_size, DEV,
                                 exchange=(fn_name == "sgmv_lora_delta_ids"))
    for t in (seg.sorted_token_ids, seg.seg_indptr, seg.seg_lora_ids, seg.tiles, seg.info):
        t.fill_(-5)  # every entry the call must write is poisoned first
    arr, n = sg._slices(y, pool, w.M)
    lib = sg.library()
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    rc = getattr(lib, fn_name)(ctypes.c_void_p(ids.data_ptr()), ctypes.c_void_p(x.data_ptr()),
                               x.stride(0), w.M, ctypes.byref(pool.desc),
                               ctypes.byref(seg.desc), arr, n, stream)
    torch.cuda.synchronize()
    assert rc == sg.SGMV_OK, f"{fn_name}: status {rc}"
    return y, seg


def _check_against_existing(sg, w, label):
    print(f"no-alloc call: {label} M={w.M} L={w.L}", flush=True)
    y_ref, seg_ref = _run(sg, w, "sgmv_lora_delta_ids")
    y_na, seg_na = _run(sg, w, "sgmv_lora_delta_ids_noalloc")
    assert torch.equal(y_na, y_ref), label
    h_ref, h_na = seg_ref.host(), seg_na.host()
    for k in ("sorted_token_ids", "seg_indptr", "seg_lora_ids", "large_tiles", "small_tiles"):
        assert torch.equal(h_na[k], h_ref[k]), f"{label}: {k}"
    assert h_na["num_segments"] == h_ref["num_segments"] and h_na["status"] == sg.SGMV_OK
    ref = oracle.lora_delta(_np32(w.x), _np32(w.y0), w.ids.numpy(), _np32(w.a), _np32(w.b),
                            w.rank.numpy(), w.alpha.numpy())
    got = _np32(y_na)
    diff = got - ref
    rel = np.linalg.norm(diff) / np.linalg.norm(ref)
    assert rel <= 5e-3, f"{label}: rel-L2 {rel:.3e}"
    assert np.max(np.abs(diff)) <= 1e-2 * np.max(np.abs(ref)), label
    neg = w.ids.numpy() < 0
    assert np.array_equal(got[neg], _np32(w.y0)[neg]), label


def test_noalloc_matches_existing_entry_point_on_successive_calls(sg):
    # the decode batch (one launch), a larger batch with large pieces (two launches), then
    # smaller batches on another pool: each call finds the array as the last one left it
    calls = [
        ("decode", workloads.get("decode")),
        ("two launches", workloads.custom(M=600, K=1024, N=768, L=12, R=16, seed=21,
                                          seq_lens=[150, 9, 300, 141], name="na_two")),
        ("smaller", workloads.custom(M=96, K=2048, N=1024, L=24, R=16, seed=22,
                                     no_lora_frac=0.1, name="na_small")),
        ("smallest", workloads.custom(M=17, K=512, N=256, L=5, R=16, seed=23, name="na_17")),
    ]
    for label, w in calls:
        _check_against_existing(sg, w, label)


def test_noalloc_refuses_batches_beyond_the_array(sg):
    w = workloads.custom(M=512, K=256, N=256, L=512, R=16, seed=24, name="na_big")
    pool = sg.sgmv_pool_pack(w.a.to(DEV), w.b.to(DEV), w.rank.tolist(), w.alpha.tolist())
    seg = sg.sgmv_segments_alloc(w.M, w.L, 0, DEV, exchange=False)
    assert seg.desc.exchange_bytes > sg.NOALLOC_SCRATCH_BYTES
    y = w.y0.to(DEV)
    before = y.clone()
    with pytest.raises(sg.SgmvError) as e:
        sg.sgmv_lora_delta_ids_noalloc(w.ids.to(DEV), w.x.to(DEV), pool, seg, y)
    assert e.value.status == sg.SGMV_EUNSUPPORTED
    torch.cuda.synchronize()
    assert torch.equal(y, before)
