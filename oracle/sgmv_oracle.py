"""fp64 CPU oracle for the multi-LoRA segmented gather GEMV (SGMV) delta.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import or call this module. The library under
``segmented_gather_gemv_amd/`` never does, and this module imports nothing from it: the
two share no code. Inputs come in as numpy arrays (any float dtype; bf16 values are handed
over as their exact fp32 copies) and every floating step below runs in fp64.

Sources, cited by page title and section:
  * Fused-LoRA page: "09. Triton Fused LoRA" (llm-algo-leetcode), Steps 1-3 (pool layout
    A (L, r, in), B (L, out, r); per-token routing by ``lora_indices``) and its test
    (per-token loop ``x[i] @ A.T @ B.T``).
  * Punica page: "III. Punica: Multi-Tenant LoRA Serving", section SGMV (Y = XW + (x_i A_i
    B_i)_i), section on the batching effect (worked example: ids 2,2,2,5,5,1,1 give the
    boundary array s = [0,3,5,7]) and the code section (tokens reordered by adapter, then
    cut into fixed-size chunks, each chunk one segment with one adapter; weight index per
    segment; rows resolved through sorted token ids).
  * Ascend article: vLLM-Ascend LoRA operator article, sections 1.1 (delta
    (alpha/r)(x A^T) B^T added to the base output), 2.1 (per-adapter rank r and alpha; a
    maximum rank), 3.3 (decode SGMV: group rows by adapter), 3.2 (the scale on either side
    of the expand, or folded into B at load time), 4.4 (a merged weight for batches with
    one or two adapters),
    5.2 (merged vs unmerged consistency) and 5.3 (rows without adapter are skipped).

Readings where the pages are silent or disagree (each one is listed with its reason in the
project's design notes):
  R1 shapes: A is (L, R, K) and B is (L, N, R); the delta is (x A^T) B^T (Fused-LoRA page).
  R2 segment order: buckets in order of first appearance of the adapter among the tokens,
     tokens ascending inside a bucket (the only order that reproduces the worked example
     and still groups scattered tokens).
  R3 id -1 means "no adapter": such tokens are in no segment, go to the tail of
     ``sorted_token_ids`` in ascending order, and their y rows are left unchanged.
  R4 any other id outside [0, L) is an error.
  R5 with chunk size C > 0 each bucket is cut into ceil(c/C) chunks, all of C rows but the
     last; chunks never cross buckets and follow bucket order.
  R6 scale_l = alpha_l / rank_l with the adapter's own rank.
  R7 the rank-r adapter uses only A[l, :r, :] and B[l, :, :r]; entries past r are ignored.
  R8 folding the scale into B at load time (Ascend article 2.1 and 3.2 allow the factor on
     either side of the expand, or folded into B) forms scale_l * B in fp32, with scale_l
     the fp32 quotient alpha_l / r_l, and rounds it once to the pool's element type
     (bf16: nearest, ties to even). The pages fix no precision for this step.
"""
from __future__ import annotations

from typing import Dict, Optional, Sequence, Tuple

import numpy as np


class BadAdapterId(ValueError):
    """An id outside {-1} U [0, L) (reading R4)."""


# ----------------------------------------------------------------------------------------
# O1: validation
# ----------------------------------------------------------------------------------------
def validate_ids(ids: np.ndarray, L: int) -> None:
    """Every token id is -1 (no adapter, Ascend article 5.3) or an index into the pool of
    L adapters (Fused-LoRA page, Step 1). Anything else raises BadAdapterId."""
    ids = np.asarray(ids)
    bad = (ids < -1) | (ids >= L)
    if bad.any():
        t = int(np.nonzero(bad)[0][0])
        raise BadAdapterId(f"token {t} has adapter id {int(ids[t])}, pool holds {L}")


# ----------------------------------------------------------------------------------------
# O2: segments (definitional, O(M * distinct adapters))
# ----------------------------------------------------------------------------------------
def segments(ids: Sequence[int], L: int, chunk_size: int = 0) -> Dict[str, np.ndarray]:
    """Group tokens by adapter (Punica page, code section: reorder tokens by adapter, then
    optionally cut the reordered stream into fixed-size chunks, each chunk being one
    segment with one adapter; batching-effect section: boundary array s).

    Returns int32 arrays ``sorted_token_ids`` [M], ``seg_indptr`` [S+1], ``seg_lora_ids``
    [S] and the int ``num_segments`` S.
    """
    ids = np.asarray(ids, dtype=np.int64)
    validate_ids(ids, L)
    if chunk_size < 0:
        raise ValueError("chunk_size must be >= 0")
    M = ids.shape[0]
    # adapters in order of their first appearance among tokens that carry one (R2)
    order = []
    seen = set()
    for t in range(M):
        l = int(ids[t])
        if l >= 0 and l not in seen:
            seen.add(l)
            order.append(l)
    sorted_ids = []
    indptr = [0]
    seg_lora = []
    for l in order:
        bucket = np.nonzero(ids == l)[0]          # ascending token index inside the bucket
        sorted_ids.extend(int(t) for t in bucket)
        c = bucket.shape[0]
        if chunk_size == 0:
            pieces = [c]
        else:                                     # R5
            n = -(-c // chunk_size)
            pieces = [chunk_size] * (n - 1) + [c - chunk_size * (n - 1)]
        for p in pieces:
            indptr.append(indptr[-1] + p)
            seg_lora.append(l)
    sorted_ids.extend(int(t) for t in np.nonzero(ids == -1)[0])   # R3: tail
    return {
        "sorted_token_ids": np.asarray(sorted_ids, dtype=np.int32),
        "seg_indptr": np.asarray(indptr, dtype=np.int32),
        "seg_lora_ids": np.asarray(seg_lora, dtype=np.int32),
        "num_segments": len(seg_lora),
    }


# ----------------------------------------------------------------------------------------
# O3 / O4: the delta, per token, in fp64
# ----------------------------------------------------------------------------------------
def _rows(M: int, rows: Optional[Sequence[int]]):
    return range(M) if rows is None else [int(t) for t in rows]


def shrink(x: np.ndarray, ids: np.ndarray, a: np.ndarray, rank: np.ndarray,
           rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """First stage of the two-stage projection (Ascend article 3.2): for a token t with
    adapter l of rank r, h[t, :r] = A[l, :r, :] @ x[t] (unscaled). Columns j >= r and rows
    of tokens without adapter are 0. Returns fp64 [M, R]."""
    ids = np.asarray(ids)
    L, R, K = a.shape
    validate_ids(ids, L)
    M = x.shape[0]
    h = np.zeros((M, R), dtype=np.float64)
    for t in _rows(M, rows):
        l = int(ids[t])
        if l < 0:
            continue
        r = int(rank[l])
        h[t, :r] = a[l, :r, :].astype(np.float64) @ x[t].astype(np.float64)
    return h


def expand(h: np.ndarray, y0: np.ndarray, ids: np.ndarray, b: np.ndarray, rank: np.ndarray,
           alpha: np.ndarray, rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Second stage (Ascend article 3.2, 3.3): y[t] = y0[t] + (alpha_l / r) * B[l, :, :r]
    @ h[t, :r]; rows of tokens without adapter keep y0. Returns fp64 [M, N]."""
    ids = np.asarray(ids)
    L, N, R = b.shape
    validate_ids(ids, L)
    y = np.array(y0, dtype=np.float64, copy=True)
    for t in _rows(y.shape[0], rows):
        l = int(ids[t])
        if l < 0:
            continue
        r = int(rank[l])
        scale = float(alpha[l]) / r                                     # R6
        y[t] = y[t] + scale * (b[l, :, :r].astype(np.float64) @ np.asarray(h[t, :r], np.float64))
    return y


def lora_delta(x: np.ndarray, y0: np.ndarray, ids: np.ndarray, a: np.ndarray, b: np.ndarray,
               rank: np.ndarray, alpha: np.ndarray,
               rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """The multi-LoRA delta added to a base output (Ascend article 1.1 and 2.3; Punica page,
    SGMV section; Fused-LoRA page test loop), token by token in fp64:

        y[t] = y0[t] + (alpha_l / r_l) * B[l, :, :r_l] @ (A[l, :r_l, :] @ x[t])   if l >= 0
        y[t] = y0[t]                                                            if l == -1

    with l = ids[t]. It does not depend on how tokens are grouped into segments.
    ``rows`` restricts the work to those tokens (others keep y0). Returns fp64 [M, N]."""
    ids = np.asarray(ids)
    L, R, K = a.shape
    validate_ids(ids, L)
    y = np.array(y0, dtype=np.float64, copy=True)
    for t in _rows(y.shape[0], rows):
        l = int(ids[t])
        if l < 0:
            continue
        r = int(rank[l])
        h = a[l, :r, :].astype(np.float64) @ x[t].astype(np.float64)
        y[t] = y[t] + (float(alpha[l]) / r) * (b[l, :, :r].astype(np.float64) @ h)
    return y


def round_bf16(v) -> np.ndarray:
    """Round fp32 values to bfloat16 (the upper 16 bits of an fp32 pattern), to nearest with
    ties to even, returned as fp32. Written from the definition on the bit pattern: add half
    of the dropped range, minus one unless the kept part is odd, then drop the low 16 bits;
    a carry moves into the exponent (up to infinity). NaN stays a quiet NaN."""
    bits = np.ascontiguousarray(np.asarray(v, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    keep_odd = (bits >> np.uint64(16)) & np.uint64(1)
    rounded = ((bits + np.uint64(0x7FFF) + keep_odd) >> np.uint64(16)) << np.uint64(16)
    is_nan = ((bits & np.uint64(0x7F800000)) == np.uint64(0x7F800000)) & \
        ((bits & np.uint64(0x007FFFFF)) != np.uint64(0))
    quiet = ((bits >> np.uint64(16)) << np.uint64(16)) | np.uint64(0x00400000)
    out = np.where(is_nan, quiet, rounded).astype(np.uint32)
    return out.view(np.float32)


def fold_scale(b: np.ndarray, rank: np.ndarray, alpha: np.ndarray,
               bf16: bool) -> Tuple[np.ndarray, np.ndarray]:
    """B with each adapter's scale folded in (reading R8): for j < r_l,
    B'[l, n, j] = round(fp32(scale_l) * fp32(B[l, n, j])) with scale_l = fp32(alpha_l) /
    fp32(r_l) in fp32 arithmetic; round is round_bf16 for a bf16 pool and the identity for
    an fp32 pool (the fp32 product is already rounded). Entries j >= r_l are set to 0.
    Returns (B' as fp32 (L, N, R), alpha' = r so that every remaining scale alpha'/r is 1)."""
    b32 = np.asarray(b, dtype=np.float32)
    L, N, R = b32.shape
    out = np.zeros_like(b32)
    for l in range(L):
        r = int(rank[l])
        s32 = np.float32(alpha[l]) / np.float32(r)        # fp32 division (IEEE, nearest)
        prod = b32[l, :, :r] * s32                         # fp32 products (IEEE, nearest)
        out[l, :, :r] = round_bf16(prod) if bf16 else prod
    return out, np.asarray(rank, dtype=np.float64).copy()


def merge_weight(w: np.ndarray, a: np.ndarray, b: np.ndarray, rank: np.ndarray,
                 alpha: np.ndarray, l: int) -> np.ndarray:
    """Adapter l merged into a base weight (Ascend article 1.1 and 4.4; Punica page, SGMV
    section): W' = W + (alpha_l / r_l) * B[l, :, :r_l] @ A[l, :r_l, :] in fp64, where W (N, K)
    is the base weight of y = x W^T, so that x W'^T = x W^T + the adapter's delta."""
    r = int(rank[l])
    w64 = np.asarray(w, dtype=np.float64)
    return w64 + (float(alpha[l]) / r) * (np.asarray(b[l, :, :r], np.float64)
                                          @ np.asarray(a[l, :r, :], np.float64))


__all__ = [
    "BadAdapterId", "validate_ids", "segments", "shrink", "expand", "lora_delta",
    "round_bf16", "fold_scale", "merge_weight",
]
