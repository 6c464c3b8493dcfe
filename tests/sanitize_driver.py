"""Host-side workload for the sanitizer build of libsgmv (run by test_host_sanitize.py in a
child process with the AddressSanitizer runtime preloaded; no GPU is touched).

Drives, through the C-ABI of the instrumented library given as argv[1]: the host segment
builder on every id string of length 0-5 over {-1, 0, 1, 2} with chunk sizes 0-3 and on
random batches up to 40,000 tokens (each compared with the oracle's segments), the grouping
cache's host path, bad ids, and every argument-error path of the entry points that returns
before a launch. numpy and ctypes only (no torch), so the instrumented library is the only
native code of interest in the process. Prints "sanitize driver ok" at the end.
"""
import ctypes
import itertools
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import oracle  # noqa: E402

OK, EINVAL, EBADID, EUNSUP, ECAP, EHIP = range(6)
TILE_INTS, TILE_ROWS, SMALL_ROWS = 32, 64, 16
i32, i64, vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p


class Pool(ctypes.Structure):
    _fields_ = [("a", vp), ("b", vp), ("rank", vp), ("scale", vp), ("L", i32), ("R_max", i32),
                ("R_pad", i32), ("K", i32), ("N", i32), ("K_pad", i32), ("N_pad", i32),
                ("dtype", i32), ("rank_min", i32), ("scale_folded", i32)]


class Segs(ctypes.Structure):
    _fields_ = [("sorted_token_ids", vp), ("seg_indptr", vp), ("seg_lora_ids", vp),
                ("tiles", vp), ("info", vp), ("M", i32), ("L", i32), ("chunk_size", i32),
                ("seg_cap", i32), ("large_cap", i32), ("small_cap", i32), ("exchange", vp),
                ("exchange_bytes", i64)]


class Slice(ctypes.Structure):
    _fields_ = [("y", vp), ("ldy", i64), ("n_begin", i32), ("n_len", i32)]


class Opts(ctypes.Structure):
    _fields_ = [("start_event", vp), ("stop_event", vp), ("n_split_small", i32),
                ("n_split_large", i32), ("exchange", i32), ("exchange_wait", i32)]


lib = ctypes.CDLL(sys.argv[1])
for f in ("sgmv_pool_init", "sgmv_pool_pack", "sgmv_pool_pack_ex", "sgmv_segments_init",
          "sgmv_build_segments", "sgmv_build_segments_cached", "sgmv_shrink", "sgmv_expand",
          "sgmv_lora_delta", "sgmv_lora_delta_ex", "sgmv_lora_delta_ids",
          "sgmv_lora_delta_ids_noalloc", "sgmv_merge_adapter", "sgmv_chunk_size_for_batch",
          "sgmv_version"):
    getattr(lib, f).restype = ctypes.c_int
lib.sgmv_status_string.restype = ctypes.c_char_p
P = ctypes.byref


def ptr(a):
    return a.ctypes.data_as(vp)


class HostSegs:
    """Host arrays for M tokens of L adapters, sized exactly as sgmv_segments_init says (so
    any write past them is an out-of-bounds access the sanitizer reports)."""

    def __init__(self, M, L, C):
        self.d = Segs()
        assert lib.sgmv_segments_init(M, L, C, P(self.d)) == OK
        d = self.d
        self.sorted = np.full(max(M, 1), -9, np.int32)
        self.indptr = np.full(d.seg_cap + 1, -9, np.int32)
        self.lora = np.full(max(d.seg_cap, 1), -9, np.int32)
        # 16-byte aligned records, exactly the stated count
        n = (d.large_cap + d.small_cap) * TILE_INTS
        raw = np.full(n + 4, -9, np.int32)
        off = (-raw.ctypes.data % 16) // 4
        self.tiles = raw[off:off + n]
        self.info = np.full(4, -9, np.int32)
        d.sorted_token_ids, d.seg_indptr, d.seg_lora_ids = (ptr(self.sorted), ptr(self.indptr),
                                                            ptr(self.lora))
        d.tiles, d.info, d.exchange = ptr(self.tiles), ptr(self.info), None


def host_build_check(ids, L, C):
    ids = np.ascontiguousarray(ids, dtype=np.int32)
    M = ids.shape[0]
    s = HostSegs(M, L, C)
    rc = lib.sgmv_build_segments(ptr(ids) if M else None, M, L, C, 0, P(s.d), None)
    assert rc == OK, rc
    ref = oracle.segments(ids, L, C)
    S = int(s.info[0])
    assert S == ref["num_segments"]
    assert np.array_equal(s.sorted[:M], ref["sorted_token_ids"])
    assert np.array_equal(s.indptr[:S + 1], ref["seg_indptr"])
    assert np.array_equal(s.lora[:S], ref["seg_lora_ids"])
    return s


def main():
    # exhaustive short strings and random batches through the host builder
    n = 0
    for M in range(0, 6):
        for ids in itertools.product((-1, 0, 1, 2), repeat=M):
            for C in (0, 1, 2, 3):
                host_build_check(list(ids), 3, C)
                n += 1
    rng = np.random.default_rng(0)
    for _ in range(40):
        M = int(rng.integers(1, 40000))
        L = int(rng.integers(1, 1000))
        C = int(rng.choice([0, 1, 7, 64, 300]))
        ids = rng.integers(-1, L, size=M)
        ids[: M // 3] = rng.integers(0, L)
        host_build_check(ids, L, C)
        n += 1
    # bad ids: EBADID from the host builder
    for bad in ([0, 3, 1], [-2], [1 << 30, 0]):
        a = np.asarray(bad, np.int32)
        s = HostSegs(len(bad), 3, 0)
        assert lib.sgmv_build_segments(ptr(a), len(bad), 3, 0, 0, P(s.d), None) == EBADID

    # grouping cache, host path: build, hit, miss, forced rebuild, bad id never cached
    M, L = 300, 20
    ids = rng.integers(-1, L, size=M).astype(np.int32)
    s = HostSegs(M, L, 0)
    cache = np.zeros(4 + M, np.int32)
    for _ in range(2):
        assert lib.sgmv_build_segments_cached(ptr(ids), M, L, 0, 0, P(s.d), ptr(cache),
                                              None) == OK
    ids[7] = (ids[7] + 1) % L
    assert lib.sgmv_build_segments_cached(ptr(ids), M, L, 0, 0, P(s.d), ptr(cache), None) == OK
    cache[0] = 0
    assert lib.sgmv_build_segments_cached(ptr(ids), M, L, 0, 0, P(s.d), ptr(cache), None) == OK
    ids[3] = L
    assert lib.sgmv_build_segments_cached(ptr(ids), M, L, 0, 0, P(s.d), ptr(cache),
                                          None) == EBADID
    assert cache[0] == 0
    assert lib.sgmv_build_segments_cached(ptr(ids), M, L, 0, 0, P(s.d), None, None) == EINVAL

    # segments descriptor errors
    d = Segs()
    assert lib.sgmv_segments_init(-1, 4, 0, P(d)) == EINVAL
    assert lib.sgmv_segments_init(4, 0, 0, P(d)) == EINVAL
    assert lib.sgmv_segments_init(4, 4, -1, P(d)) == EINVAL
    assert lib.sgmv_segments_init(4, 4, 0, None) == EINVAL
    a = np.zeros(8, np.int32)
    s = HostSegs(8, 4, 0)
    assert lib.sgmv_build_segments(ptr(a), 7, 4, 0, 0, P(s.d), None) == EINVAL   # wrong M
    assert lib.sgmv_build_segments(ptr(a), 8, 4, 3, 0, P(s.d), None) == EINVAL   # wrong C
    assert lib.sgmv_build_segments(None, 8, 4, 0, 0, P(s.d), None) == EINVAL
    s.d.tiles = ctypes.c_void_p(s.d.tiles + 4)                                     # misaligned
    assert lib.sgmv_build_segments(ptr(a), 8, 4, 0, 0, P(s.d), None) == EINVAL
    s = HostSegs(8, 4, 0)
    s.d.large_cap += 1
    assert lib.sgmv_build_segments(ptr(a), 8, 4, 0, 0, P(s.d), None) == EINVAL
    assert lib.sgmv_build_segments(ptr(a), 8, 2000, 0, 1, P(HostSegs(8, 2000, 0).d),
                                   None) == EUNSUP

    # pool errors
    p = Pool()
    ab, bb = ctypes.c_size_t(), ctypes.c_size_t()
    assert lib.sgmv_pool_init(4, 16, 128, 256, 1, P(p), P(ab), P(bb)) == OK
    for args in [(0, 16, 128, 256, 1), (4, 0, 128, 256, 1), (4, 16, 0, 256, 1),
                 (4, 16, 128, 0, 1), (4, 16, 128, 256, 7), (70000, 16, 8, 8, 1)]:
        assert lib.sgmv_pool_init(*args, P(p), P(ab), P(bb)) == EINVAL
    assert lib.sgmv_pool_init(4, 65, 128, 256, 1, P(p), P(ab), P(bb)) == EUNSUP
    assert lib.sgmv_pool_init(4, 16, 128, 256, 1, None, P(ab), P(bb)) == EINVAL
    # a pool with (never dereferenced) host addresses for the validation paths
    assert lib.sgmv_pool_init(4, 16, 128, 256, 1, P(p), P(ab), P(bb)) == OK
    fake = np.zeros(64, np.int64)
    p.a = p.b = p.rank = p.scale = ptr(fake)
    rank = np.array([16, 8, 0, 4], np.int32)
    alpha = np.ones(4, np.float32)
    assert lib.sgmv_pool_pack(ptr(fake), ptr(fake), ptr(rank), ptr(alpha), P(p), None) == EINVAL
    rank[2] = 17
    assert lib.sgmv_pool_pack(ptr(fake), ptr(fake), ptr(rank), ptr(alpha), P(p), None) == EINVAL
    rank[2] = 16
    alpha[1] = np.inf
    assert lib.sgmv_pool_pack(ptr(fake), ptr(fake), ptr(rank), ptr(alpha), P(p), None) == EINVAL
    assert lib.sgmv_pool_pack_ex(ptr(fake), ptr(fake), ptr(rank), ptr(alpha), 4, P(p),
                                 None) == EINVAL

    # delta entry points: errors returned before any launch, and M = 0 no-ops
    M = 8
    s = HostSegs(M, 4, 0)
    y = np.zeros((M, 256), np.uint16)
    sl = (Slice * 2)()
    sl[0].y, sl[0].ldy, sl[0].n_begin, sl[0].n_len = ptr(y), 256, 0, 256
    x = np.zeros((M, 128), np.uint16)
    h = np.zeros((M, 16), np.float32)
    assert lib.sgmv_lora_delta(ptr(x), 128, -1, P(p), P(s.d), sl, 1, None) == EINVAL
    assert lib.sgmv_lora_delta(ptr(x), 128, M, None, P(s.d), sl, 1, None) == EINVAL
    assert lib.sgmv_lora_delta(ptr(x), 100, M, P(p), P(s.d), sl, 1, None) == EINVAL  # ldx < K
    assert lib.sgmv_lora_delta(None, 128, M, P(p), P(s.d), sl, 1, None) == EINVAL
    assert lib.sgmv_lora_delta(ptr(x), 128, M, P(p), P(s.d), sl, 0, None) == EINVAL
    assert lib.sgmv_lora_delta(ptr(x), 128, M, P(p), P(s.d), sl, 5, None) == EINVAL
    assert lib.sgmv_lora_delta(ptr(x), 128, M, P(p), P(s.d), None, 1, None) == EINVAL
    sl[1].y, sl[1].ldy, sl[1].n_begin, sl[1].n_len = ptr(y), 256, 100, 50          # overlap
    assert lib.sgmv_lora_delta(ptr(x), 128, M, P(p), P(s.d), sl, 2, None) == EINVAL
    sl[1].n_begin, sl[1].n_len = 250, 20                                           # past N
    assert lib.sgmv_lora_delta(ptr(x), 128, M, P(p), P(s.d), sl, 2, None) == EINVAL
    sl[0].ldy = 100                                                                # ldy < len
    assert lib.sgmv_lora_delta(ptr(x), 128, M, P(p), P(s.d), sl, 1, None) == EINVAL
    sl[0].ldy = 256
    s0 = HostSegs(0, 4, 0)
    assert lib.sgmv_lora_delta(None, 128, 0, P(p), P(s0.d), sl, 1, None) == OK      # no-op
    assert lib.sgmv_shrink(ptr(x), 128, M, P(p), P(s.d), ptr(h), 8, None) == EINVAL  # ldh
    assert lib.sgmv_shrink(ptr(x), 128, M, P(p), P(s.d), None, 16, None) == EINVAL
    assert lib.sgmv_expand(None, 16, M, P(p), P(s.d), sl, 1, None) == EINVAL
    for o in (Opts(None, None, 65, 0, 0, 0), Opts(None, None, 0, -1, 0, 0),
              Opts(None, None, 0, 0, 2, 0), Opts(None, None, 0, 0, 0, -2)):
        assert lib.sgmv_lora_delta_ex(ptr(x), 128, M, P(p), P(s.d), sl, 1, P(o), None) == EINVAL
    ids = np.zeros(M, np.int32)
    assert lib.sgmv_lora_delta_ids(None, ptr(x), 128, M, P(p), P(s.d), sl, 1, None) == EINVAL
    assert lib.sgmv_lora_delta_ids(ptr(ids), ptr(x), 128, M, P(p), P(HostSegs(M, 5, 0).d), sl,
                                   1, None) == EINVAL                              # L differs
    assert lib.sgmv_lora_delta_ids_noalloc(ptr(ids), ptr(x), 128, M, P(p), None, sl, 1,
                                           None) == EINVAL
    big = HostSegs(512, 512, 0)                     # exchange beyond the static array
    p2 = Pool()
    assert lib.sgmv_pool_init(512, 16, 128, 256, 1, P(p2), P(ab), P(bb)) == OK
    p2.a = p2.b = p2.rank = p2.scale = ptr(fake)
    xb = np.zeros((512, 128), np.uint16)
    idb = np.zeros(512, np.int32)
    assert lib.sgmv_lora_delta_ids_noalloc(ptr(idb), ptr(xb), 128, 512, P(p2), P(big.d), sl, 1,
                                           None) == EUNSUP
    assert lib.sgmv_merge_adapter(ptr(fake), 128, ptr(fake), 128, P(p), 4, None) == EINVAL
    assert lib.sgmv_merge_adapter(ptr(fake), 100, ptr(fake), 128, P(p), 0, None) == EINVAL
    assert lib.sgmv_merge_adapter(None, 128, ptr(fake), 128, P(p), 0, None) == EINVAL

    # plain host functions
    assert lib.sgmv_version() >= 100
    for st in range(7):
        assert lib.sgmv_status_string(st)
    for Mq in (-5, 0, 1, 256, 512, 513, 1024, 1025, 1 << 20):
        for na in (0, 1, 64, 1 << 20):
            c = lib.sgmv_chunk_size_for_batch(Mq, na)
            assert c in (0, 16)
    print(f"sanitize driver ok ({n} host builds)", flush=True)


def plant_overflow():
    """A call that breaks the contract on purpose: sorted_token_ids one entry short of M. The
    host builder writes M entries, so an instrumented build must report the overflow."""
    M, L = 64, 4
    s = HostSegs(M, L, 0)
    short = np.full(M - 1, -9, np.int32)
    s.d.sorted_token_ids = ptr(short)
    ids = np.zeros(M, np.int32)
    lib.sgmv_build_segments(ptr(ids), M, L, 0, 0, P(s.d), None)
    print("planted overflow was not reported", flush=True)


if __name__ == "__main__":
    if len(sys.argv) > 2 and sys.argv[2] == "--plant-overflow":
        plant_overflow()
    else:
        main()
