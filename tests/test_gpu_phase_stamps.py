"""The profiling copy of the library (libsgmv_stamps.so, phase stamps compiled into the
single-launch kernel): the same results, bit for bit, as libsgmv.so, and stamps that follow the
phase order in every workgroup that ran a small piece."""
import ctypes
import os

import numpy as np
import pytest
import torch

import segmented_gather_gemv_amd as sg
import workloads

pytestmark = pytest.mark.gpu

STAMPS = os.path.join(os.path.dirname(sg.LIB_PATH), "libsgmv_stamps.so")


def _stamps_lib():
    lib = ctypes.CDLL(STAMPS)
    f = lib.sgmv_lora_delta_ids_ex
    f.argtypes, f.restype = sg.library().sgmv_lora_delta_ids_ex.argtypes, ctypes.c_int
    lib.sgmv_phase_stamps.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    lib.sgmv_phase_stamps.restype = ctypes.c_int
    return lib


@pytest.mark.parametrize("M,L", [(256, 64), (37, 9)])
def test_stamps_library_matches_the_library(M, L):
    print(f"phase stamps: M={M} L={L}", flush=True)
    dev = torch.device("cuda:0")
    w = workloads.custom(M=M, K=4096, N=4096, L=L, R=16, seed=M + L, name="stamps")
    pool = sg.sgmv_pool_pack(w.a.to(dev), w.b.to(dev), w.rank.tolist(), w.alpha.tolist())
    x, ids = w.x.to(dev), w.ids.to(dev)
    y_ref = w.y0.to(dev)
    seg_ref = sg.sgmv_segments_alloc(M, L, 0, dev)
    sg.sgmv_lora_delta_ids(ids, x, pool, seg_ref, y_ref)

    lib = _stamps_lib()
    y = w.y0.to(dev)
    seg = sg.sgmv_segments_alloc(M, L, 0, dev)
    sl, n_sl = sg._slices([(y, 0)], pool, M)
    stream = ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)
    rc = lib.sgmv_lora_delta_ids_ex(ctypes.c_void_p(ids.data_ptr()),
                                    ctypes.c_void_p(x.data_ptr()), x.stride(0), M,
                                    ctypes.byref(pool.desc), ctypes.byref(seg.desc), sl, n_sl,
                                    None, stream)
    assert rc == 0
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref)
    assert torch.equal(seg.sorted_token_ids, seg_ref.sorted_token_ids)

    buf = np.zeros(8192 * 16, dtype=np.uint64)
    assert lib.sgmv_phase_stamps(buf.ctypes.data_as(ctypes.c_void_p), buf.nbytes) == 0
    s = buf.reshape(8192, 16).astype(np.int64)
    full = (s[:, 0] > 0) & (s[:, 8] > s[:, 0])
    # one row per adapter split that found tokens: at least one per adapter in the batch
    n_ad = len(set(w.ids[w.ids >= 0].tolist()))
    assert full.sum() >= n_ad
    assert (np.diff(s[full, :9], axis=1) >= 0).all()
