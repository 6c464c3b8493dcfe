"""CPU tests of the C-ABI: the library loads, exports every function include/sgmv.h
declares, the host segment builder matches the oracle bit for bit, and argument errors come
back as the documented status codes. No GPU work is launched here."""
import ctypes
import itertools
import os
import re
import subprocess

import numpy as np
import pytest
import torch

import oracle
import segmented_gather_gemv_amd as sg
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sgmv.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sgmv_[a-z_]+)\s*\(", text)))


def test_header_declares_the_boundary_calls():
    names = declared_functions()
    for n in ["sgmv_build_segments", "sgmv_shrink", "sgmv_expand", "sgmv_lora_delta",
              "sgmv_pool_pack"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = sg.library()
    names = declared_functions()
    assert names
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", sg.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if l.strip())
    assert set(names) <= exported
    assert set(sg.EXPORTED) <= exported
    assert "sgmv_phase_stamps" not in exported  # profiling builds only


def test_stamps_library_exports_the_same_calls_and_the_stamp_reader():
    """libsgmv_stamps.so (the profiling copy behind bench.py --phase-stamps) is the library
    with phase stamps compiled into the single-launch kernel: the same C-ABI plus the reader."""
    path = os.path.join(os.path.dirname(sg.LIB_PATH), "libsgmv_stamps.so")
    assert os.path.exists(path), "build.py builds libsgmv_stamps.so beside libsgmv.so"
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True, text=True,
                         check=True).stdout
    exported = set(l.split()[-1] for l in out.splitlines() if l.strip())
    assert set(declared_functions()) <= exported
    assert "sgmv_phase_stamps" in exported


def test_binding_constants_match_the_header():
    text = open(HEADER).read()
    defs = dict(re.findall(r"#define SGMV_([A-Z_0-9]+) (\d+)", text))
    for name in ["TILE_ROWS", "SMALL_ROWS", "TILE_INTS", "MAX_RANK", "MAX_SLICES",
                 "DEVICE_BUILDER_MAX_L", "FUSED_BUILD_MAX_M", "PART_SPLIT_MAX_M"]:
        assert int(defs[name]) == getattr(sg, name), name
    assert int(defs["TILE_ROWS"]) % int(defs["SMALL_ROWS"]) == 0


def test_version_and_status_strings():
    lib = sg.library()
    assert lib.sgmv_version() >= 100
    for s in range(6):
        assert lib.sgmv_status_string(s).startswith(b"SGMV_")


def host_build(ids, L, C):
    seg = sg.sgmv_build_segments(torch.as_tensor(np.asarray(ids, dtype=np.int32)), L, C,
                                 on_device=False)
    return seg.host()


def assert_same_as_oracle(ids, L, C):
    got = host_build(ids, L, C)
    ref = oracle.segments(ids, L, C)
    assert np.array_equal(got["sorted_token_ids"].numpy()[:len(ids)], ref["sorted_token_ids"])
    assert np.array_equal(got["seg_indptr"].numpy(), ref["seg_indptr"])
    assert np.array_equal(got["seg_lora_ids"].numpy(), ref["seg_lora_ids"])
    assert got["num_segments"] == ref["num_segments"]
    check_records(got, ref)
    assert got["status"] == sg.SGMV_OK


def check_records(got, ref):
    """Descriptor records against the oracle's segments, by the invariants include/sgmv.h
    states for them (the piece split is the library's, with the library's constants): every
    segment is cut, from its first sorted row, into pieces of SGMV_TILE_ROWS rows, the last
    one shorter; each record names its segment's adapter, its first row and its rows, in
    segment order within its class; a piece is small exactly when it has at most
    SGMV_SMALL_ROWS rows; together the pieces cover every sorted row of a segment once;
    [4..16) are zero; the token slots of a small piece hold its sorted token ids then -1,
    those of a large piece all -1."""
    st = np.asarray(ref["sorted_token_ids"])
    ip = np.asarray(ref["seg_indptr"])
    sl = np.asarray(ref["seg_lora_ids"])
    S = int(ref["num_segments"])
    n_rows = int(ip[S]) if S else 0
    covered = np.zeros(n_rows, dtype=np.int64)
    pieces = {}
    for recs, small in ((got["large_tiles"], False), (got["small_tiles"], True)):
        recs = recs.numpy().reshape(-1, sg.TILE_INTS)
        if len(recs):
            assert np.all(np.diff(recs[:, 1]) > 0), "records follow segment order"
        for rec in recs:
            lora, start, rows, s = (int(v) for v in rec[:4])
            assert 0 <= s < S
            assert lora == int(sl[s])
            assert 1 <= rows <= sg.TILE_ROWS
            assert (rows <= sg.SMALL_ROWS) == small
            assert int(ip[s]) <= start and start + rows <= int(ip[s + 1])
            assert (start - int(ip[s])) % sg.TILE_ROWS == 0, "pieces start every TILE_ROWS"
            covered[start:start + rows] += 1
            pieces.setdefault(s, []).append((start, rows))
            assert np.all(rec[4:16] == 0)
            toks = np.full(16, -1)
            if small:
                toks[:rows] = st[start:start + rows]
            assert np.array_equal(rec[16:], toks)
    assert np.all(covered == 1), "every sorted row of a segment in exactly one piece"
    for s in range(S):  # all pieces of a segment but its last are full
        ps = sorted(pieces[s])
        assert all(r == sg.TILE_ROWS for _, r in ps[:-1])


def test_record_checker_catches_corrupted_records():
    """check_records itself: each plausible corruption of a correct build is rejected."""
    ids = np.concatenate([np.full(150, 3), np.arange(40) % 5, np.full(20, 1), [-1, -1]])
    ref = oracle.segments(ids, 6, 0)
    good = host_build(ids, 6, 0)
    check_records(good, ref)

    def corrupt(cls, row, col, delta):
        bad = {k: (v.clone() if torch.is_tensor(v) else v) for k, v in good.items()}
        recs = bad[cls].view(-1, sg.TILE_INTS)
        recs[row, col] += delta
        return bad

    n_small = good["small_tiles"].numel() // sg.TILE_INTS
    assert n_small >= 2 and good["large_tiles"].numel() // sg.TILE_INTS >= 2
    for cls, row, col, delta in [("large_tiles", 0, 0, 1),    # wrong adapter
                                 ("large_tiles", 1, 1, -1),   # overlapping pieces
                                 ("large_tiles", 0, 2, -1),   # a row left out
                                 ("small_tiles", 0, 3, 1),    # wrong segment
                                 ("small_tiles", 1, 16, 1),   # wrong token in a slot
                                 ("small_tiles", 0, 5, 7)]:   # reserved word not zero
        with pytest.raises(AssertionError):
            check_records(corrupt(cls, row, col, delta), ref)


def test_host_builder_worked_example():
    got = host_build([2, 2, 2, 5, 5, 1, 1], 6, 0)
    assert got["seg_indptr"].tolist() == [0, 3, 5, 7]
    assert got["seg_lora_ids"].tolist() == [2, 5, 1]
    assert got["sorted_token_ids"].tolist() == list(range(7))


def test_host_builder_exhaustive_small():
    for M in range(0, 6):
        for ids in itertools.product((-1, 0, 1, 2), repeat=M):
            for C in (0, 1, 2, 3):
                assert_same_as_oracle(list(ids), 3, C)


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill", "mixed", "qkv"])
def test_host_builder_workloads(name):
    w = workloads.get(name)
    assert_same_as_oracle(w.ids.numpy(), w.L, w.chunk_size)


@pytest.mark.parametrize("seed", range(6))
def test_host_builder_random(seed):
    rng = np.random.default_rng(seed)
    M = int(rng.integers(1, 5000))
    L = int(rng.integers(1, 300))
    C = int(rng.choice([0, 1, 7, 64, 200]))
    ids = rng.integers(-1, L, size=M)
    # long runs to produce many large tiles
    ids[: M // 3] = rng.integers(0, L)
    assert_same_as_oracle(ids, L, C)


def test_host_builder_bad_id():
    with pytest.raises(sg.SgmvError) as e:
        host_build([0, 3, 1], 3, 0)
    assert e.value.status == sg.SGMV_EBADID
    with pytest.raises(sg.SgmvError) as e:
        host_build([0, -2], 3, 0)
    assert e.value.status == sg.SGMV_EBADID


def test_host_builder_empty_and_all_negative():
    got = host_build([], 4, 0)
    assert got["num_segments"] == 0 and got["seg_indptr"].tolist() == [0]
    got = host_build([-1] * 9, 4, 3)
    assert got["num_segments"] == 0
    assert got["sorted_token_ids"].tolist() == list(range(9))


def test_capacities_bound_the_outputs():
    """The capacities sgmv_segments_init reports bound what the oracle's segments need: one
    entry per segment, and per piece of SGMV_TILE_ROWS rows in its class."""
    rng = np.random.default_rng(1)
    for _ in range(50):
        M = int(rng.integers(0, 3000))
        L = int(rng.integers(1, 100))
        C = int(rng.choice([0, 1, 3, 64]))
        seg = sg.sgmv_segments_alloc(M, L, C, "cpu")
        d = seg.desc
        ids = rng.integers(-1, L, size=M)
        if M:
            ids[: M // 3] = rng.integers(0, L)  # long buckets: many large pieces
        ref = oracle.segments(ids, L, C)
        lens = np.diff(ref["seg_indptr"])
        n_large = int(sum(c // sg.TILE_ROWS + (c % sg.TILE_ROWS > sg.SMALL_ROWS) for c in lens))
        n_small = int(sum(0 < c % sg.TILE_ROWS <= sg.SMALL_ROWS for c in lens))
        assert ref["num_segments"] <= d.seg_cap
        assert n_large <= d.large_cap and n_small <= d.small_cap


# ---------------------------------------------------------------------------------------
# argument errors (returned before any launch)
# ---------------------------------------------------------------------------------------
def test_pool_init_errors():
    lib = sg.library()
    p = sg._Pool()
    a, b = ctypes.c_size_t(), ctypes.c_size_t()
    ok = lib.sgmv_pool_init(4, 16, 128, 256, sg.SGMV_BF16, ctypes.byref(p), ctypes.byref(a),
                            ctypes.byref(b))
    assert ok == sg.SGMV_OK
    assert (p.R_pad, p.K_pad, p.N_pad) == (16, 128, 256)
    assert a.value == 4 * 16 * 128 * 2 and b.value == 4 * 16 * 256 * 2
    assert lib.sgmv_pool_init(4, 65, 128, 256, 1, ctypes.byref(p), ctypes.byref(a),
                              ctypes.byref(b)) == sg.SGMV_EUNSUPPORTED
    for args in [(0, 16, 128, 256, 1), (4, 0, 128, 256, 1), (4, 16, 0, 256, 1),
                 (4, 16, 128, 0, 1), (4, 16, 128, 256, 7)]:
        assert lib.sgmv_pool_init(*args, ctypes.byref(p), ctypes.byref(a),
                                  ctypes.byref(b)) == sg.SGMV_EINVAL
    assert lib.sgmv_pool_init(4, 3, 100, 37, 0, ctypes.byref(p), ctypes.byref(a),
                              ctypes.byref(b)) == sg.SGMV_OK
    assert (p.R_pad, p.K_pad, p.N_pad) == (16, 128, 64)


def test_segments_init_errors():
    lib = sg.library()
    s = sg._Segments()
    assert lib.sgmv_segments_init(-1, 4, 0, ctypes.byref(s)) == sg.SGMV_EINVAL
    assert lib.sgmv_segments_init(4, 0, 0, ctypes.byref(s)) == sg.SGMV_EINVAL
    assert lib.sgmv_segments_init(4, 4, -1, ctypes.byref(s)) == sg.SGMV_EINVAL
    assert lib.sgmv_segments_init(256, 64, 0, ctypes.byref(s)) == sg.SGMV_OK
    assert (s.seg_cap, s.large_cap, s.small_cap) == (64, 256 // 17, 64)
    assert lib.sgmv_segments_init(2048, 128, 64, ctypes.byref(s)) == sg.SGMV_OK
    assert s.seg_cap == min(2048, 128 + 2048 // 64)
    # exchange workspace
    # (control words [large_cap + small_cap][16] padded to 256 B, small tiles [8][16][64],
    # large tiles [4][64][64], fp32)
    assert lib.sgmv_segments_init(256, 64, 0, ctypes.byref(s)) == sg.SGMV_OK
    assert (s.large_cap, s.small_cap) == (15, 64)
    assert s.exchange_bytes == 5120 + 64 * 8 * 16 * 64 * 4 + 15 * 4 * 64 * 64 * 4
    assert lib.sgmv_segments_init(7, 3, 0, ctypes.byref(s)) == sg.SGMV_OK
    assert s.exchange_bytes == 256 + 3 * 8 * 16 * 64 * 4
    assert lib.sgmv_segments_init(0, 4, 0, ctypes.byref(s)) == sg.SGMV_OK
    assert s.exchange_bytes == 0


def test_build_segments_errors():
    lib = sg.library()
    seg = sg.sgmv_segments_alloc(8, 4, 0, "cpu")
    ids = torch.zeros(8, dtype=torch.int32)
    # descriptor initialised for another M / chunk size
    assert lib.sgmv_build_segments(ctypes.c_void_p(ids.data_ptr()), 7, 4, 0, 0,
                                   ctypes.byref(seg.desc), None) == sg.SGMV_EINVAL
    assert lib.sgmv_build_segments(ctypes.c_void_p(ids.data_ptr()), 8, 4, 2, 0,
                                   ctypes.byref(seg.desc), None) == sg.SGMV_EINVAL
    assert lib.sgmv_build_segments(None, 8, 4, 0, 0, ctypes.byref(seg.desc),
                                   None) == sg.SGMV_EINVAL
    # descriptor records must be 16-byte aligned
    d = sg._Segments()
    ctypes.memmove(ctypes.byref(d), ctypes.byref(seg.desc), ctypes.sizeof(d))
    d.tiles = seg.desc.tiles + 4
    assert lib.sgmv_build_segments(ctypes.c_void_p(ids.data_ptr()), 8, 4, 0, 0, ctypes.byref(d),
                                   None) == sg.SGMV_EINVAL
    # device builder limit on the pool size is checked before any launch
    big = sg.sgmv_segments_alloc(8, 5000, 0, "cpu")
    assert lib.sgmv_build_segments(ctypes.c_void_p(ids.data_ptr()), 8, 5000, 0, 1,
                                   ctypes.byref(big.desc), None) == sg.SGMV_EUNSUPPORTED


def _fake_pool(L=4, R=16, K=128, N=256, dtype=sg.SGMV_BF16):
    p = sg._Pool()
    a, b = ctypes.c_size_t(), ctypes.c_size_t()
    assert sg.library().sgmv_pool_init(L, R, K, N, dtype, ctypes.byref(p), ctypes.byref(a),
                                       ctypes.byref(b)) == 0
    # non-null placeholders: validation never dereferences them
    p.a = p.b = p.rank = p.scale = 0x1000
    return p


def test_delta_argument_errors():
    lib = sg.library()
    pool = _fake_pool()
    seg = sg.sgmv_segments_alloc(8, 4, 0, "cpu")
    y = sg._Slice(0x2000, 256, 0, 256)
    x = ctypes.c_void_p(0x3000)
    call = lambda *a: lib.sgmv_lora_delta(*a)
    # ldx < K
    assert call(x, 64, 8, ctypes.byref(pool), ctypes.byref(seg.desc), ctypes.byref(y), 1,
                None) == sg.SGMV_EINVAL
    # M does not match the segments
    assert call(x, 128, 9, ctypes.byref(pool), ctypes.byref(seg.desc), ctypes.byref(y), 1,
                None) == sg.SGMV_EINVAL
    # slice past N, zero slices, too many slices, overlapping slices
    bad = sg._Slice(0x2000, 256, 200, 100)
    assert call(x, 128, 8, ctypes.byref(pool), ctypes.byref(seg.desc), ctypes.byref(bad), 1,
                None) == sg.SGMV_EINVAL
    assert call(x, 128, 8, ctypes.byref(pool), ctypes.byref(seg.desc), ctypes.byref(y), 0,
                None) == sg.SGMV_EINVAL
    arr = (sg._Slice * 5)(*[sg._Slice(0x2000, 256, 0, 8)] * 5)
    assert call(x, 128, 8, ctypes.byref(pool), ctypes.byref(seg.desc), arr, 5,
                None) == sg.SGMV_EINVAL
    ov = (sg._Slice * 2)(sg._Slice(0x2000, 256, 0, 100), sg._Slice(0x4000, 256, 50, 100))
    assert call(x, 128, 8, ctypes.byref(pool), ctypes.byref(seg.desc), ov, 2,
                None) == sg.SGMV_EINVAL
    # null x, null pool pointer fields
    assert call(None, 128, 8, ctypes.byref(pool), ctypes.byref(seg.desc), ctypes.byref(y), 1,
                None) == sg.SGMV_EINVAL
    p2 = _fake_pool()
    p2.a = 0
    assert call(x, 128, 8, ctypes.byref(p2), ctypes.byref(seg.desc), ctypes.byref(y), 1,
                None) == sg.SGMV_EINVAL
    # shrink: ldh < R_max
    assert lib.sgmv_shrink(x, 128, 8, ctypes.byref(pool), ctypes.byref(seg.desc),
                           ctypes.c_void_p(0x5000), 8, None) == sg.SGMV_EINVAL
    # expand: null h
    assert lib.sgmv_expand(None, 16, 8, ctypes.byref(pool), ctypes.byref(seg.desc),
                           ctypes.byref(y), 1, None) == sg.SGMV_EINVAL


def test_exchange_and_option_errors():
    """Workspace and option checks happen before any launch."""
    lib = sg.library()
    pool = _fake_pool()
    seg = sg.sgmv_segments_alloc(8, 4, 0, "cpu")
    y = sg._Slice(0x2000, 256, 0, 256)
    x = ctypes.c_void_p(0x3000)
    call = lambda d, o: lib.sgmv_lora_delta_ex(x, 128, 8, ctypes.byref(pool), ctypes.byref(d),
                                              ctypes.byref(y), 1, o, None)
    d = sg._Segments()
    ctypes.memmove(ctypes.byref(d), ctypes.byref(seg.desc), ctypes.sizeof(d))
    d.exchange = 0x10080  # not 256-byte aligned
    assert call(d, None) == sg.SGMV_EINVAL
    d.exchange = 0x10000
    d.exchange_bytes = seg.desc.exchange_bytes - 1  # too small
    assert call(d, None) == sg.SGMV_EINVAL
    for kw in [dict(exchange=2), dict(exchange=-2), dict(exchange_wait=-2),
               dict(n_split_small=65), dict(n_split_large=-1)]:
        assert call(seg.desc, sg.LaunchOpts(**kw).ref()) == sg.SGMV_EINVAL, kw


def test_empty_batch_is_a_noop():
    lib = sg.library()
    pool = _fake_pool()
    seg = sg.sgmv_segments_alloc(0, 4, 0, "cpu")
    y = sg._Slice(0x2000, 256, 0, 256)
    assert lib.sgmv_lora_delta(ctypes.c_void_p(0x3000), 128, 0, ctypes.byref(pool),
                               ctypes.byref(seg.desc), ctypes.byref(y), 1, None) == sg.SGMV_OK


def test_pool_pack_rejects_bad_rank_before_launch():
    lib = sg.library()
    pool = _fake_pool(L=2, R=8)
    rank = torch.tensor([8, 9], dtype=torch.int32)
    alpha = torch.tensor([1.0, 1.0])
    assert lib.sgmv_pool_pack(ctypes.c_void_p(0x10), ctypes.c_void_p(0x10),
                              ctypes.c_void_p(rank.data_ptr()), ctypes.c_void_p(alpha.data_ptr()),
                              ctypes.byref(pool), None) == sg.SGMV_EINVAL
    rank = torch.tensor([0, 3], dtype=torch.int32)
    assert lib.sgmv_pool_pack(ctypes.c_void_p(0x10), ctypes.c_void_p(0x10),
                              ctypes.c_void_p(rank.data_ptr()), ctypes.c_void_p(alpha.data_ptr()),
                              ctypes.byref(pool), None) == sg.SGMV_EINVAL


def test_delta_ids_argument_errors():
    """The build-and-delta call checks its arguments before any launch, on both of its
    paths (one launch for small bf16 batches, build + delta otherwise)."""
    lib = sg.library()
    y = sg._Slice(0x2000, 256, 0, 256)
    x = ctypes.c_void_p(0x3000)
    ids = ctypes.c_void_p(0x4000)
    for M, dtype in [(8, sg.SGMV_BF16), (600, sg.SGMV_BF16), (8, sg.SGMV_F32)]:
        pool = _fake_pool(dtype=dtype)
        seg = sg.sgmv_segments_alloc(M, 4, 0, "cpu")
        call = lambda i, xx, d, n=1, o=None: lib.sgmv_lora_delta_ids_ex(
            i, xx, 128, M, ctypes.byref(pool), ctypes.byref(d), ctypes.byref(y), n, o, None)
        assert call(None, x, seg.desc) == sg.SGMV_EINVAL           # no ids
        assert call(ids, None, seg.desc) == sg.SGMV_EINVAL         # no x
        assert call(ids, x, seg.desc, n=0) == sg.SGMV_EINVAL       # no slice
        other = sg.sgmv_segments_alloc(M + 1, 4, 0, "cpu")
        assert call(ids, x, other.desc) == sg.SGMV_EINVAL          # segments for another M
        assert call(ids, x, seg.desc, o=sg.LaunchOpts(exchange=3).ref()) == sg.SGMV_EINVAL


def test_chunk_size_rule():
    """sgmv_chunk_size_for_batch: no chunks for small batches whose adapters are many enough
    that buckets are already small pieces, 16-row chunks up to 1024 tokens, none above."""
    f = sg.sgmv_chunk_size_for_batch
    assert f(0, 0) == 0 and f(-3, 5) == 0
    assert f(256, 64) == 0 and f(512, 64) == 0 and f(512, 100) == 0
    assert f(256, 16) == 16 and f(256, 1) == 16 and f(256, 0) == 16   # unknown: chunks
    assert f(513, 1000) == 16 and f(1024, 1) == 16
    assert f(1025, 0) == 0 and f(8192, 12) == 0 and f(1 << 20, 3) == 0
    # the answer is a valid chunk size for the segment calls
    for M, n in [(1, 1), (300, 2), (5000, 40)]:
        C = f(M, n)
        assert C >= 0
        seg = sg.sgmv_segments_alloc(M, 64, C, "cpu")
        assert seg.desc.chunk_size == C


def test_merge_and_pack_argument_errors():
    """sgmv_merge_adapter and sgmv_pool_pack_ex reject bad arguments before any launch."""
    lib = sg.library()
    pool = _fake_pool(L=4, R=16, K=128, N=256)
    w, wo = ctypes.c_void_p(0x6000), ctypes.c_void_p(0x7000)
    merge = lambda *a: lib.sgmv_merge_adapter(*a)
    assert merge(None, 128, wo, 128, ctypes.byref(pool), 0, None) == sg.SGMV_EINVAL
    assert merge(w, 128, None, 128, ctypes.byref(pool), 0, None) == sg.SGMV_EINVAL
    assert merge(w, 127, wo, 128, ctypes.byref(pool), 0, None) == sg.SGMV_EINVAL  # ldw < K
    assert merge(w, 128, wo, 100, ctypes.byref(pool), 0, None) == sg.SGMV_EINVAL  # ldo < K
    assert merge(w, 128, wo, 128, ctypes.byref(pool), -1, None) == sg.SGMV_EINVAL
    assert merge(w, 128, wo, 128, ctypes.byref(pool), 4, None) == sg.SGMV_EINVAL   # L = 4
    bad = _fake_pool()
    bad.b = 0
    assert merge(w, 128, wo, 128, ctypes.byref(bad), 0, None) == sg.SGMV_EINVAL
    bad_opts = sg.LaunchOpts(n_split_small=-3)
    assert lib.sgmv_merge_adapter_ex(w, 128, wo, 128, ctypes.byref(pool), 0, bad_opts.ref(),
                                     None) == sg.SGMV_EINVAL
    # unknown pack flags (checked with the pool before any copy)
    rank = torch.full((4,), 16, dtype=torch.int32)
    alpha = torch.full((4,), 32.0)
    assert lib.sgmv_pool_pack_ex(w, wo, ctypes.c_void_p(rank.data_ptr()),
                                 ctypes.c_void_p(alpha.data_ptr()), 2, ctypes.byref(pool),
                                 None) == sg.SGMV_EINVAL
    # the Python binding checks shapes and dtypes of w
    p = sg.Pool.__new__(sg.Pool)
    p.desc = pool
    p.a = torch.zeros(1, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        sg.sgmv_merge_adapter(torch.zeros(3, 3, dtype=torch.bfloat16), p, 0)
