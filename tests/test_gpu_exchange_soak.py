"""Bounded soak of the K-split exchange (GPU).

The column-split workgroups of a piece exchange fp32 partial sums of its shrink through device
memory: relaxed agent-scope atomic stores, a wait for their completion, an agent-scope counter,
then agent-scope atomic loads. Results must never depend on timing: a workgroup that sees its
partners' partials uses them, one that does not computes them itself by the same steps, and
both give the same bits. This test repeats the default call many times and requires every y to
be bit-identical to the call that computes every partner's partial locally (no wait at all),
which itself meets the oracle's bar. It stops at the first mismatch and reports the launch.

  decode  (one launch, sgmv_lora_delta_ids): 2,000 launches
  prefill (built segments, sgmv_lora_delta): 200 launches
"""
import pytest
import torch

import oracle
import workloads
from test_gpu_parity import compare, np32, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sg():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import segmented_gather_gemv_amd as m
    return m


def _soak(call, y0, ref, n, batch=16, what=""):
    """n calls of call(y) on fresh copies of y0, `batch` outputs in flight between checks;
    returns the number of launches checked."""
    ys = [torch.empty_like(y0) for _ in range(batch)]
    done = 0
    while done < n:
        k = min(batch, n - done)
        for j in range(k):
            ys[j].copy_(y0)
            call(ys[j])
        torch.cuda.synchronize()
        for j in range(k):
            assert torch.equal(ys[j], ref), f"{what}: launch {done + j} differs from local"
        done += k
    return done


def test_exchange_soak_decode_single_launch(sg):
    w = workloads.get("decode")
    pool, x, y0, ids = upload(w, sg)
    seg = sg.sgmv_segments_alloc(w.M, w.L, 0, "cuda")
    ref = y0.clone()
    sg.sgmv_lora_delta_ids(ids, x, pool, seg, ref, opts=sg.LaunchOpts(exchange_wait=-1))
    torch.cuda.synchronize()
    compare(np32(ref), oracle.lora_delta(np32(w.x), np32(w.y0), w.ids.numpy(), np32(w.a),
                                         np32(w.b), w.rank.numpy(), w.alpha.numpy()),
            w.dtype, what="decode local")
    print("exchange soak: decode, 2000 launches", flush=True)
    n = _soak(lambda y: sg.sgmv_lora_delta_ids(ids, x, pool, seg, y), y0, ref, 2000,
              what="decode")
    assert n == 2000


def test_exchange_soak_prefill(sg):
    w = workloads.get("prefill")
    pool, x, y0, ids = upload(w, sg)
    seg = sg.sgmv_build_segments(ids, w.L, w.chunk_size, on_device=True)
    ref = y0.clone()
    sg.sgmv_lora_delta(x, pool, seg, ref, opts=sg.LaunchOpts(exchange_wait=-1))
    torch.cuda.synchronize()
    compare(np32(ref), oracle.lora_delta(np32(w.x), np32(w.y0), w.ids.numpy(), np32(w.a),
                                         np32(w.b), w.rank.numpy(), w.alpha.numpy()),
            w.dtype, what="prefill local")
    print("exchange soak: prefill, 200 launches", flush=True)
    n = _soak(lambda y: sg.sgmv_lora_delta(x, pool, seg, y), y0, ref, 200, batch=8,
              what="prefill")
    assert n == 200


def test_exchange_placement(sg):
    """The exchange's partners (equal launch index modulo 8) run on one XCD: every workgroup
    b of a 2048-workgroup grid reads XCD id equal to that of workgroup b mod 8."""
    ok, n_xcd = sg.sgmv_exchange_placement("cuda")
    assert ok, f"workgroups b and b mod 8 ran on different XCDs ({n_xcd} XCDs seen)"
    assert n_xcd in (1, 2, 4, 8)
    seg = sg.sgmv_segments_alloc(256, 64, 0, "cuda")
    assert seg.exchange is not None
