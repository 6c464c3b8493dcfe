"""Pins for the fp64 oracle: each check ties it to something other than itself.

  * the worked segment example printed on the Punica page (golden fixture);
  * exhaustive comparison of the segment builder with a second, differently written
    definition (a stable sort by first-appearance key) over every short id string;
  * structural invariants of segments;
  * merged vs unmerged equivalence x(W + s A^T B^T) = xW + s (x A^T) B^T through a dense
    K x N matrix (Punica page, SGMV section; Ascend article 1.1 and 5.2);
  * the single-adapter special case as two plain matmuls over the whole batch;
  * pure-Python triple loops on tiny inputs;
  * closed forms: all tokens without adapter leave y bit-identical, power-of-two scales act
    exactly, an adapter of rank r stored in a wider pool equals the same adapter in a pool
    of rank r, permuting tokens permutes rows;
  * bf16 rounding of the scale fold: hand-worked bit patterns, agreement with torch's
    float32 -> bfloat16 conversion, exactness for power-of-two scales, the half-unit error
    bound on the folded B and on the folded delta;
  * planted mistakes: plausible bugs injected into copies of the oracle are each caught by
    at least one of the checks above.
"""
import itertools
import json
import os

import numpy as np
import pytest

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------------------------------
# helpers: an independent segment definition and independent delta loops
# ---------------------------------------------------------------------------------------
def alt_segments(ids, C):
    """Second definition of the segments: a stable sort of token indices by the position
    where their adapter first appears (no-adapter tokens last), then runs of equal ids cut
    every C rows."""
    ids = [int(v) for v in ids]
    first = {}
    for t, v in enumerate(ids):
        if v >= 0 and v not in first:
            first[v] = t
    inf = len(ids) + 1
    perm = sorted(range(len(ids)), key=lambda t: (first[ids[t]] if ids[t] >= 0 else inf, t))
    n_lora = sum(1 for v in ids if v >= 0)
    indptr, lora = [0], []
    run_id, run_len = None, 0
    for pos in range(n_lora):
        v = ids[perm[pos]]
        if v != run_id or (C and run_len == C):
            if pos > 0:
                indptr.append(pos)
            lora.append(v)
            run_id, run_len = v, 0
        run_len += 1
    if n_lora:
        indptr.append(n_lora)
    return perm, indptr, lora


def brute_delta(x, y0, ids, A, B, rank, alpha):
    """Pure-Python loops, no numpy: y[t][n] = y0[t][n] + alpha/r * sum_j B[n][j] sum_k
    A[j][k] x[t][k]."""
    M, N = len(y0), len(y0[0])
    K = len(x[0])
    out = [list(map(float, row)) for row in y0]
    for t in range(M):
        l = int(ids[t])
        if l < 0:
            continue
        r = int(rank[l])
        s = float(alpha[l]) / r
        hs = []
        for j in range(r):
            acc = 0.0
            for k in range(K):
                acc += float(A[l][j][k]) * float(x[t][k])
            hs.append(acc)
        for n in range(N):
            acc = 0.0
            for j in range(r):
                acc += float(B[l][n][j]) * hs[j]
            out[t][n] += s * acc
    return np.asarray(out)


def rand_problem(rng, M, K, N, L, R, ranks=None, neg_frac=0.0):
    ids = rng.integers(0, L, size=M).astype(np.int32)
    if neg_frac:
        ids[rng.random(M) < neg_frac] = -1
    x = rng.standard_normal((M, K))
    A = rng.standard_normal((L, R, K))
    B = rng.standard_normal((L, N, R))
    y0 = rng.standard_normal((M, N))
    rank = np.asarray(ranks if ranks is not None else [R] * L, dtype=np.int32)
    alpha = rng.choice([1.0, 2.0, 8.0, 16.0, 3.0], size=L)
    return x, y0, ids, A, B, rank, alpha


def rel_err(a, b):
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


# ---------------------------------------------------------------------------------------
# segment pins
# ---------------------------------------------------------------------------------------
def check_worked_example(seg_fn):
    g = json.load(open(os.path.join(GOLDEN, "punica_segment_example.json")))
    out = seg_fn(g["lora_ids"], max(g["lora_ids"]) + 1, 0)
    return (list(out["seg_indptr"]) == g["s"]
            and list(out["sorted_token_ids"]) == list(range(len(g["lora_ids"]))))


def test_worked_example_from_page():
    assert check_worked_example(oracle.segments)
    out = oracle.segments([2, 2, 2, 5, 5, 1, 1], 6, 0)
    assert list(out["seg_lora_ids"]) == [2, 5, 1]
    assert out["num_segments"] == 3


def check_exhaustive(seg_fn, max_len=6):
    for M in range(0, max_len + 1):
        for ids in itertools.product((-1, 0, 1, 2), repeat=M):
            for C in (0, 1, 2, 3):
                out = seg_fn(list(ids), 3, C)
                perm, indptr, lora = alt_segments(ids, C)
                if (list(out["sorted_token_ids"]) != perm or list(out["seg_indptr"]) != indptr
                        or list(out["seg_lora_ids"]) != lora or out["num_segments"] != len(lora)):
                    return False
    return True


def test_segments_exhaustive_against_second_definition():
    assert check_exhaustive(oracle.segments)


def check_invariants(out, ids, C):
    ids = np.asarray(ids)
    M = ids.shape[0]
    st = np.asarray(out["sorted_token_ids"])
    ip = np.asarray(out["seg_indptr"])
    sl = np.asarray(out["seg_lora_ids"])
    S = out["num_segments"]
    assert sorted(st.tolist()) == list(range(M))             # a permutation
    assert ip[0] == 0 and len(ip) == S + 1 and len(sl) == S
    assert np.all(np.diff(ip) > 0)                            # no empty segment
    n_lora = int((ids >= 0).sum())
    assert ip[-1] == n_lora
    for s in range(S):
        toks = st[ip[s]:ip[s + 1]]
        assert np.all(ids[toks] == sl[s])                     # one adapter per segment
        assert np.all(np.diff(toks) > 0)                      # ascending inside a segment
        if C:
            assert len(toks) <= C
    if C == 0:
        assert len(set(sl.tolist())) == S                     # one segment per adapter
    tail = st[n_lora:]
    assert np.all(ids[tail] == -1) and np.all(np.diff(tail) > 0)


@pytest.mark.parametrize("C", [0, 1, 5, 64])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_segment_invariants_random(C, seed):
    rng = np.random.default_rng(seed)
    ids = rng.integers(-1, 37, size=1000)
    check_invariants(oracle.segments(ids, 37, C), ids, C)


def test_segments_degenerate():
    out = oracle.segments([], 4, 0)
    assert out["num_segments"] == 0 and list(out["seg_indptr"]) == [0]
    out = oracle.segments([-1, -1, -1], 4, 2)
    assert out["num_segments"] == 0 and list(out["sorted_token_ids"]) == [0, 1, 2]
    out = oracle.segments([3] * 10, 4, 4)
    assert list(out["seg_indptr"]) == [0, 4, 8, 10] and list(out["seg_lora_ids"]) == [3, 3, 3]


@pytest.mark.parametrize("bad", [[-2], [0, 4], [0, 1, 7, -1]])
def test_bad_ids_raise(bad):
    with pytest.raises(oracle.BadAdapterId):
        oracle.segments(bad, 4, 0)
    with pytest.raises(oracle.BadAdapterId):
        oracle.lora_delta(np.zeros((len(bad), 2)), np.zeros((len(bad), 2)), np.asarray(bad),
                          np.zeros((4, 1, 2)), np.zeros((4, 2, 1)), np.ones(4, np.int32),
                          np.ones(4))


# ---------------------------------------------------------------------------------------
# delta pins
# ---------------------------------------------------------------------------------------
def check_merged(delta_fn, seed=0):
    rng = np.random.default_rng(seed)
    M, K, N, L, R = 9, 24, 20, 3, 6
    x, _, ids, A, B, rank, alpha = rand_problem(rng, M, K, N, L, R, ranks=[6, 3, 5],
                                                neg_frac=0.2)
    W = rng.standard_normal((K, N))
    y0 = x @ W
    y = delta_fn(x, y0, ids, A, B, rank, alpha)
    for t in range(M):
        l = int(ids[t])
        if l < 0:
            Wp = W
        else:
            r = int(rank[l])
            Wp = W + (alpha[l] / r) * (A[l, :r, :].T @ B[l, :, :r].T)   # dense merged weight
        ym = x[t] @ Wp
        if rel_err(y[t], ym) > 1e-12:
            return False
    return True


def test_merged_equals_unmerged():
    for seed in range(4):
        assert check_merged(oracle.lora_delta, seed)


def check_single_adapter(delta_fn):
    rng = np.random.default_rng(11)
    M, K, N, L, R = 17, 40, 33, 4, 5
    x, y0, _, A, B, rank, alpha = rand_problem(rng, M, K, N, L, R)
    ids = np.full(M, 2, dtype=np.int32)
    y = delta_fn(x, y0, ids, A, B, rank, alpha)
    ref = y0 + (alpha[2] / R) * np.matmul(np.matmul(x, A[2].T), B[2].T)
    return rel_err(y, ref) <= 1e-12


def test_single_adapter_is_two_matmuls():
    assert check_single_adapter(oracle.lora_delta)


def check_brute(delta_fn, seed=0):
    rng = np.random.default_rng(100 + seed)
    M, K, N, L, R = 6, 12, 11, 3, 4
    x, y0, ids, A, B, rank, alpha = rand_problem(rng, M, K, N, L, R, ranks=[4, 1, 3],
                                                neg_frac=0.25)
    y = delta_fn(x, y0, ids, A, B, rank, alpha)
    ref = brute_delta(x.tolist(), y0.tolist(), ids.tolist(), A.tolist(), B.tolist(),
                      rank.tolist(), alpha.tolist())
    return np.max(np.abs(y - ref)) <= 1e-12 * max(1.0, np.max(np.abs(ref)))


def test_bruteforce_tiny():
    for seed in range(6):
        assert check_brute(oracle.lora_delta, seed)


def test_all_no_adapter_is_identity():
    rng = np.random.default_rng(7)
    x, y0, _, A, B, rank, alpha = rand_problem(rng, 8, 10, 12, 3, 4)
    ids = np.full(8, -1, dtype=np.int32)
    y = oracle.lora_delta(x, y0, ids, A, B, rank, alpha)
    assert np.array_equal(y, y0)


def test_power_of_two_scale_is_exact():
    rng = np.random.default_rng(8)
    x, y0, ids, A, B, rank, _ = rand_problem(rng, 10, 16, 14, 3, 4, ranks=[4, 2, 3])
    zero = np.zeros_like(y0)
    d1 = oracle.lora_delta(x, zero, ids, A, B, rank, rank.astype(np.float64))      # scale 1
    d4 = oracle.lora_delta(x, zero, ids, A, B, rank, 4.0 * rank.astype(np.float64))  # scale 4
    assert np.array_equal(d4, 4.0 * d1)


def check_rank_pool(delta_fn):
    rng = np.random.default_rng(9)
    M, K, N, L = 12, 20, 18, 3
    ranks = [2, 5, 3]
    x, y0, ids, A, B, rank, alpha = rand_problem(rng, M, K, N, L, 8, ranks=ranks)
    y_wide = delta_fn(x, y0, ids, A, B, rank, alpha)
    ok = True
    for l in range(L):
        r = ranks[l]
        sel = np.asarray(ids) == l
        A1 = A[l:l + 1, :r, :].copy()
        B1 = B[l:l + 1, :, :r].copy()
        ids1 = np.where(sel, 0, -1).astype(np.int32)
        y1 = delta_fn(x, y0, ids1, A1, B1, np.asarray([r], np.int32), alpha[l:l + 1])
        ok &= bool(np.array_equal(y1[sel], y_wide[sel]))
    return ok


def test_rank_r_in_wide_pool_equals_rank_r_pool():
    assert check_rank_pool(oracle.lora_delta)


def test_token_permutation_permutes_rows():
    rng = np.random.default_rng(10)
    x, y0, ids, A, B, rank, alpha = rand_problem(rng, 15, 9, 7, 4, 3, neg_frac=0.2)
    perm = rng.permutation(15)
    y = oracle.lora_delta(x, y0, ids, A, B, rank, alpha)
    yp = oracle.lora_delta(x[perm], y0[perm], ids[perm], A, B, rank, alpha)
    assert np.array_equal(yp, y[perm])


def test_shrink_then_expand_matches_delta():
    rng = np.random.default_rng(12)
    x, y0, ids, A, B, rank, alpha = rand_problem(rng, 20, 30, 25, 5, 8,
                                                ranks=[8, 1, 4, 7, 2], neg_frac=0.2)
    h = oracle.shrink(x, ids, A, rank)
    y = oracle.expand(h, y0, ids, B, rank, alpha)
    assert rel_err(y, oracle.lora_delta(x, y0, ids, A, B, rank, alpha)) <= 1e-13
    # h of one adapter is a plain matmul of the batch against A^T, zero past the rank
    sel = ids == 3
    assert np.allclose(h[sel, :7], x[sel] @ A[3, :7].T, rtol=1e-13, atol=0)
    assert np.all(h[sel, 7:] == 0) and np.all(h[ids == -1] == 0)


def test_rows_subset_matches_full():
    rng = np.random.default_rng(13)
    x, y0, ids, A, B, rank, alpha = rand_problem(rng, 30, 12, 10, 4, 3, neg_frac=0.1)
    full = oracle.lora_delta(x, y0, ids, A, B, rank, alpha)
    rows = [0, 7, 29, 13]
    part = oracle.lora_delta(x, y0, ids, A, B, rank, alpha, rows=rows)
    assert np.array_equal(part[rows], full[rows])


def test_algorithmic_counts():
    import workloads
    ids = np.asarray([0, 0, 1, -1])
    rank = np.asarray([4, 2])
    # x: 3 rows * K, y: 3 rows * N read+write, weights (4+2)*(K+N), 12 B index per token
    K, N = 10, 6
    assert workloads.algorithmic_bytes(ids, rank, K, N, 2) == (3 * K + 2 * 3 * N + 6 * (K + N)) * 2 + 48
    assert workloads.algorithmic_flops(ids, rank, K, N) == 2 * (K + N) * (4 + 4 + 2)


# ---------------------------------------------------------------------------------------
# planted mistakes: each plausible bug must trip at least one pin
# ---------------------------------------------------------------------------------------
def _seg_ascending_id(ids, L, C=0):
    ids = np.asarray(ids)
    order = sorted(set(int(v) for v in ids if v >= 0))
    st, ip, sl = [], [0], []
    for l in order:
        b = np.nonzero(ids == l)[0]
        st.extend(b.tolist())
        ip.append(ip[-1] + len(b))
        sl.append(l)
    st.extend(np.nonzero(ids == -1)[0].tolist())
    return {"sorted_token_ids": np.asarray(st), "seg_indptr": np.asarray(ip),
            "seg_lora_ids": np.asarray(sl), "num_segments": len(sl)}


def _seg_run_length(ids, L, C=0):
    ids = [int(v) for v in ids]
    st, ip, sl = [], [0], []
    prev = None
    for t, v in enumerate(ids):
        if v < 0:
            continue
        if v != prev:
            if st:
                ip.append(len(st))
            sl.append(v)
            prev = v
        st.append(t)
    if st:
        ip.append(len(st))
    st.extend(t for t, v in enumerate(ids) if v < 0)
    return {"sorted_token_ids": np.asarray(st), "seg_indptr": np.asarray(ip),
            "seg_lora_ids": np.asarray(sl), "num_segments": len(sl)}


def _seg_neg_first(ids, L, C=0):
    out = oracle.segments(ids, L, C)
    ids = np.asarray(ids)
    st = out["sorted_token_ids"]
    n_neg = int((ids == -1).sum())
    out = dict(out)
    out["sorted_token_ids"] = np.concatenate([st[len(st) - n_neg:], st[:len(st) - n_neg]])
    return out


def _seg_chunk_from_stream(ids, L, C=0):
    """Chunks cut over the whole reordered stream instead of per bucket."""
    out = oracle.segments(ids, L, 0)
    if not C:
        return out
    ids = np.asarray(ids)
    st = out["sorted_token_ids"]
    n = int(out["seg_indptr"][-1])
    ip = list(range(0, n, C)) + [n] if n else [0]
    sl = [int(ids[st[p]]) for p in ip[:-1]]
    return {"sorted_token_ids": st, "seg_indptr": np.asarray(ip),
            "seg_lora_ids": np.asarray(sl), "num_segments": len(sl)}


def _delta_variant(kind):
    def fn(x, y0, ids, A, B, rank, alpha):
        y = np.array(y0, dtype=np.float64, copy=True)
        R = A.shape[1]
        for t in range(x.shape[0]):
            l = int(ids[t])
            if l < 0:
                if kind == "touches_negative":
                    y[t] = y[t] + 1e-3
                continue
            r = int(rank[l])
            if kind == "rank_off_by_one":
                r = max(1, r - 1)
            scale = alpha[l] / (R if kind == "scale_by_max_rank" else int(rank[l]))
            if kind == "dropped_scale":
                scale = 1.0
            h = A[l, :r, :] @ x[t]
            if kind == "b_reversed_rank":
                d = B[l, :, :r][:, ::-1] @ h
            else:
                d = B[l, :, :r] @ h
            if kind == "wrong_sign":
                d = -d
            if kind == "wrong_adapter_b":
                d = B[(l + 1) % B.shape[0], :, :r] @ h
            y[t] = y[t] + scale * d
        return y
    return fn


SEG_MUTANTS = [_seg_ascending_id, _seg_run_length, _seg_neg_first, _seg_chunk_from_stream]
DELTA_MUTANTS = ["rank_off_by_one", "scale_by_max_rank", "dropped_scale", "b_reversed_rank",
                 "wrong_sign", "wrong_adapter_b", "touches_negative"]


@pytest.mark.parametrize("mut", SEG_MUTANTS, ids=lambda f: f.__name__)
def test_planted_segment_mistakes_are_caught(mut):
    caught = not check_worked_example(mut) or not check_exhaustive(mut, max_len=5)
    assert caught


@pytest.mark.parametrize("kind", DELTA_MUTANTS)
def test_planted_delta_mistakes_are_caught(kind):
    fn = _delta_variant(kind)
    caught = (not check_merged(fn) or not check_single_adapter(fn) or not check_brute(fn)
              or not check_rank_pool(fn))
    assert caught
    # and the unmutated variant passes them all
    ok = _delta_variant("none")
    assert check_merged(ok) and check_single_adapter(ok) and check_brute(ok) and check_rank_pool(ok)


# ---------------------------------------------------------------------------------------
# scale folded into B (reading R8): bf16 rounding and the fold
# ---------------------------------------------------------------------------------------
# (fp32 bit pattern, bf16 result as an fp32 pattern), worked out by hand from the definition
# of round-to-nearest-even on the low 16 bits
ROUND_CASES = [
    (0x3F800000, 0x3F800000),  # 1.0
    (0x3F808000, 0x3F800000),  # 1 + 2^-8: halfway, kept part even -> down
    (0x3F818000, 0x3F820000),  # 1 + 2^-7 + 2^-8: halfway, kept part odd -> up
    (0x3F808001, 0x3F810000),  # just above halfway -> up
    (0x3F807FFF, 0x3F800000),  # just below halfway -> down
    (0xBF808000, 0xBF800000),  # negative halfway, even -> toward zero here
    (0xBF818000, 0xBF820000),  # negative halfway, odd -> away from zero
    (0x3FFFFFFF, 0x40000000),  # carry into the exponent
    (0x7F7FFFFF, 0x7F800000),  # largest finite fp32 rounds to infinity
    (0x7F800000, 0x7F800000),  # infinity
    (0x00008000, 0x00000000),  # subnormal halfway, even
    (0x00018000, 0x00020000),  # subnormal halfway, odd
    (0x80000000, 0x80000000),  # -0
]


def _bits(v):
    return np.asarray(v, dtype=np.float32).view(np.uint32)


def check_round_cases(round_fn):
    src = np.asarray([c[0] for c in ROUND_CASES], dtype=np.uint32).view(np.float32)
    want = np.asarray([c[1] for c in ROUND_CASES], dtype=np.uint32)
    got = _bits(round_fn(src))
    nan = round_fn(np.asarray([0x7FC00001, 0xFF800001], dtype=np.uint32).view(np.float32))
    return bool(np.array_equal(got, want)) and bool(np.isnan(nan).all())


def test_round_bf16_hand_values():
    assert check_round_cases(oracle.round_bf16)


def test_round_bf16_matches_torch_cast():
    """torch's CPU float32 -> bfloat16 conversion (a library routine) on 2^20 random fp32 bit
    patterns, NaNs aside (their payloads may differ)."""
    import torch
    pat = np.random.default_rng(5).integers(0, 2 ** 32, size=1 << 20, dtype=np.uint64)
    v = pat.astype(np.uint32).view(np.float32)
    keep = ~np.isnan(v)
    ref = torch.from_numpy(v.copy()).to(torch.bfloat16).float().numpy()
    assert np.array_equal(_bits(oracle.round_bf16(v))[keep], _bits(ref)[keep])


def _bf16_problem(rng, M, K, N, L, R, ranks):
    x, y0, ids, A, B, rank, _ = rand_problem(rng, M, K, N, L, R, ranks=ranks)
    # bf16-representable operands, as a bf16 pool holds them
    A = oracle.round_bf16(A.astype(np.float32)).astype(np.float64)
    B = oracle.round_bf16(B.astype(np.float32)).astype(np.float64)
    x = oracle.round_bf16(x.astype(np.float32)).astype(np.float64)
    return x, y0, ids, A, B, rank


def check_fold_power_of_two(fold_fn):
    """Power-of-two scales: the folded B is scale * B exactly, and the folded delta equals
    the unfolded one bit for bit."""
    rng = np.random.default_rng(21)
    ranks = [4, 2, 3, 1]
    x, y0, ids, A, B, rank = _bf16_problem(rng, 12, 16, 20, 4, 4, ranks)
    alpha = np.asarray([8.0, 1.0, 0.75, 0.25]) * np.asarray(ranks)   # scales 8, 1, 0.75, 0.25
    alpha[2] = 0.5 * ranks[2]                                          # keep powers of two
    for bf16 in (True, False):
        Bf, alpha1 = fold_fn(B, rank, alpha, bf16)
        for l, r in enumerate(ranks):
            if not np.array_equal(Bf[l, :, :r], B[l, :, :r] * (alpha[l] / r)):
                return False
        if not np.array_equal(oracle.lora_delta(x, y0, ids, A, Bf, rank, alpha1),
                              oracle.lora_delta(x, y0, ids, A, B, rank, alpha)):
            return False
    return True


def test_fold_power_of_two_is_exact():
    assert check_fold_power_of_two(oracle.fold_scale)


def check_fold_error_bound(fold_fn):
    """Other scales: every folded entry is a bf16 value within half a bf16 unit (2^-8
    relative) of the fp32 product, and each folded delta element is within that bound (plus
    the fp32 product and quotient roundings, 2^-23) of the exact one, term by term."""
    rng = np.random.default_rng(22)
    ranks = [5, 3, 7]
    x, y0, ids, A, B, rank = _bf16_problem(rng, 30, 24, 40, 3, 8, ranks)
    alpha = np.asarray([3.0, 10.0, 0.3])
    Bf, alpha1 = fold_fn(B, rank, alpha, True)
    for l, r in enumerate(ranks):
        prod = B[l, :, :r].astype(np.float32) * (np.float32(alpha[l]) / np.float32(r))
        f = Bf[l, :, :r].astype(np.float32)
        if np.any(_bits(f) & 0xFFFF):
            return False
        if np.any(np.abs(f.astype(np.float64) - prod) > 2.0 ** -8 * np.abs(prod.astype(np.float64))):
            return False
    zero = np.zeros_like(y0)
    yf = oracle.lora_delta(x, zero, ids, A, Bf, rank, alpha1)
    yu = oracle.lora_delta(x, zero, ids, A, B, rank, alpha)
    for t in range(x.shape[0]):
        l = int(ids[t])
        if l < 0:
            if np.any(yf[t] != 0):
                return False
            continue
        r = ranks[l]
        h = A[l, :r, :] @ x[t]
        bound = (2.0 ** -8 + 2.0 ** -23) * (np.abs(B[l, :, :r] * (alpha[l] / r)) @ np.abs(h))
        if np.any(np.abs(yf[t] - yu[t]) > bound + 1e-12 * np.max(np.abs(yu[t]))):
            return False
    # a scale that is not a power of two does change some entries
    return not np.array_equal(Bf[0, :, :5], B[0, :, :5] * (alpha[0] / 5))


def test_fold_error_bound():
    assert check_fold_error_bound(oracle.fold_scale)


def _round_variant(kind):
    def fn(v):
        bits = np.asarray(v, dtype=np.float32).view(np.uint32).astype(np.uint64)
        if kind == "truncate":
            out = (bits >> 16) << 16
        elif kind == "ties_away":
            out = ((bits + 0x8000) >> 16) << 16
        else:  # "ties_up_only_even_bit_ignored": always adds half minus one
            out = ((bits + 0x7FFF) >> 16) << 16
        return out.astype(np.uint32).view(np.float32)
    return fn


def _fold_variant(kind):
    def fn(b, rank, alpha, bf16):
        b32 = np.asarray(b, dtype=np.float32)
        out = np.zeros_like(b32)
        R = b32.shape[2]
        for l in range(b32.shape[0]):
            r = int(rank[l])
            s = np.float32(alpha[l]) / np.float32(R if kind == "scale_by_max_rank" else r)
            if kind == "no_scale":
                s = np.float32(1.0)
            prod = b32[l, :, :r] * s
            if bf16:
                prod = _round_variant("truncate")(prod) if kind == "truncate" else \
                    oracle.round_bf16(prod)
            out[l, :, :r] = prod
        return out, np.asarray(rank, dtype=np.float64).copy()
    return fn


@pytest.mark.parametrize("kind", ["truncate", "ties_away", "ties_up_only_even_bit_ignored"])
def test_planted_rounding_mistakes_are_caught(kind):
    assert not check_round_cases(_round_variant(kind))


@pytest.mark.parametrize("kind", ["no_scale", "scale_by_max_rank", "truncate"])
def test_planted_fold_mistakes_are_caught(kind):
    fn = _fold_variant(kind)
    assert not (check_fold_power_of_two(fn) and check_fold_error_bound(fn))
    ok = _fold_variant("none")
    assert check_fold_power_of_two(ok) and check_fold_error_bound(ok)


# ---------------------------------------------------------------------------------------
# merged weight (Ascend article 1.1 and 4.4; Punica page, SGMV section)
# ---------------------------------------------------------------------------------------
def check_merge_equivalence(merge_fn):
    """x W'^T equals the base product plus the unmerged delta of the (independently pinned)
    per-token oracle, for every token of the merged adapter."""
    rng = np.random.default_rng(31)
    M, K, N, L, R = 9, 14, 11, 3, 6
    x, _, _, A, B, rank, alpha = rand_problem(rng, M, K, N, L, R, ranks=[6, 2, 5])
    W = rng.standard_normal((N, K))
    for l in range(L):
        ids = np.full(M, l, dtype=np.int32)
        base = x @ W.T
        ref = oracle.lora_delta(x, base, ids, A, B, rank, alpha)
        got = x @ merge_fn(W, A, B, rank, alpha, l).T
        if rel_err(got, ref) > 1e-12:
            return False
    return True


def check_merge_brute(merge_fn):
    """Pure-Python loops on a tiny case, with entries past each rank set to NaN (never read)."""
    rng = np.random.default_rng(32)
    N, K, L, R = 5, 7, 2, 4
    A = rng.standard_normal((L, R, K))
    B = rng.standard_normal((L, N, R))
    rank = np.asarray([3, 1], dtype=np.int32)
    alpha = np.asarray([1.5, 4.0])
    A[0, 3:, :] = np.nan
    B[0, :, 3:] = np.nan
    A[1, 1:, :] = np.nan
    B[1, :, 1:] = np.nan
    W = rng.standard_normal((N, K))
    for l in range(L):
        got = merge_fn(W, A, B, rank, alpha, l)
        r = int(rank[l])
        for n in range(N):
            for k in range(K):
                v = float(W[n, k]) + (float(alpha[l]) / r) * sum(
                    float(B[l, n, j]) * float(A[l, j, k]) for j in range(r))
                if not abs(got[n, k] - v) <= 1e-12 * max(1.0, abs(v)):
                    return False
    return True


def test_merge_equals_unmerged_delta():
    assert check_merge_equivalence(oracle.merge_weight)


def test_merge_bruteforce_tiny():
    assert check_merge_brute(oracle.merge_weight)


def _merge_variant(kind):
    def fn(w, a, b, rank, alpha, l):
        R = a.shape[1]
        r = int(rank[l])
        s = float(alpha[l]) / (R if kind == "scale_by_max_rank" else r)
        if kind == "no_scale":
            s = 1.0
        if kind == "all_ranks":
            r = R
        d = np.asarray(b[l, :, :r], np.float64) @ np.asarray(a[l, :r, :], np.float64)
        if kind == "wrong_sign":
            d = -d
        return np.asarray(w, np.float64) + s * d
    return fn


@pytest.mark.parametrize("kind", ["scale_by_max_rank", "no_scale", "all_ranks", "wrong_sign"])
def test_planted_merge_mistakes_are_caught(kind):
    fn = _merge_variant(kind)
    assert not (check_merge_equivalence(fn) and check_merge_brute(fn))
    ok = _merge_variant("none")
    assert check_merge_equivalence(ok) and check_merge_brute(ok)
