"""Seeded synthetic inputs for the multi-LoRA delta workloads.

This module only draws inputs: token adapter ids, activations, user-layout adapter
pools, base outputs, per-adapter ranks and alphas. It holds no step of the method
itself (no segment building, no contraction, no scaling), so both the fp64 oracle
and the GPU library can be fed from it without sharing any arithmetic.

Conventions for every workload:
  * a CPU ``torch.Generator`` seeded with 42 (or the seed given);
  * draw order: sequence lengths and ids, then x, then A, then B, then y0, then ranks
    and alphas;
  * floating values are drawn in fp32 and cast once to the workload dtype with
    round-to-nearest-even, so the fp32 copy handed to the oracle holds exactly the
    values the GPU receives;
  * ids, ranks and lengths are int32; id -1 means "no adapter".

User layouts (as in the Fused-LoRA page, Step 1): ``a`` is (L, R, K) and ``b`` is
(L, N, R). Entries at ranks >= rank[l] are filled with random values on purpose:
nothing may read them.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence, Tuple

import numpy as _np
import torch

SEED = 42


@dataclass
class Workload:
    name: str
    dtype: torch.dtype
    ids: torch.Tensor            # int32 [M]
    x: torch.Tensor              # [M, K]
    a: torch.Tensor              # [L, R, K]
    b: torch.Tensor              # [L, N, R]
    y0: torch.Tensor             # [M, N]
    rank: torch.Tensor           # int32 [L]
    alpha: torch.Tensor          # float32 [L]
    chunk_size: int = 0
    # output slices as (first pool column, number of columns); one slice covers all N
    slices: List[Tuple[int, int]] = field(default_factory=list)
    note: str = ""

    @property
    def M(self) -> int:
        return int(self.ids.shape[0])

    @property
    def K(self) -> int:
        return int(self.x.shape[1])

    @property
    def N(self) -> int:
        return int(self.b.shape[1])

    @property
    def L(self) -> int:
        return int(self.a.shape[0])

    @property
    def R(self) -> int:
        return int(self.a.shape[1])

    def __post_init__(self):
        if not self.slices:
            self.slices = [(0, int(self.b.shape[1]))]


def _normal(g: torch.Generator, shape, std: float, dtype: torch.dtype) -> torch.Tensor:
    t = torch.randn(*shape, generator=g, dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def rescale_lengths(raw: Sequence[int], total: int) -> List[int]:
    """Scale integer lengths to sum to ``total``: floor of the exact rational share,
    then hand the remainder to the largest fractional parts (ties to the lower index)."""
    s = int(sum(raw))
    num = [int(r) * total for r in raw]
    base = [n // s for n in num]
    rem = [n % s for n in num]
    short = total - sum(base)
    order = sorted(range(len(raw)), key=lambda i: (-rem[i], i))
    for i in order[:short]:
        base[i] += 1
    return base


def _sequence_lengths(g: torch.Generator, n_seq: int, lo: int, hi: int, total: int) -> List[int]:
    raw = torch.randint(lo, hi + 1, (n_seq,), generator=g, dtype=torch.int64).tolist()
    return rescale_lengths(raw, total)


def tiny(seed: int = SEED) -> Workload:
    """Fused-LoRA page test: M=4, 128 -> 256, 3 adapters of rank 16, fp32, ids [2,0,1,2],
    scale 1, y starting at zero."""
    g = torch.Generator().manual_seed(seed)
    M, K, N, L, R = 4, 128, 256, 3, 16
    ids = torch.tensor([2, 0, 1, 2], dtype=torch.int32)
    x = _normal(g, (M, K), 1.0, torch.float32)
    a = _normal(g, (L, R, K), 1.0, torch.float32)
    b = _normal(g, (L, N, R), 1.0, torch.float32)
    y0 = torch.zeros(M, N, dtype=torch.float32)
    rank = torch.full((L,), R, dtype=torch.int32)
    alpha = torch.full((L,), float(R), dtype=torch.float32)  # alpha/r = 1
    return Workload("tiny", torch.float32, ids, x, a, b, y0, rank, alpha,
                    note="M=4 K=128 N=256 L=3 r=16 fp32 ids=[2,0,1,2] scale=1 y0=0")


def decode(seed: int = SEED, M: int = 256, K: int = 4096, N: int = 4096, L: int = 64,
           r: int = 16, alpha: float = 32.0) -> Workload:
    """Decode SGMV: one row per sequence, ids uniform over the pool, bf16,
    x ~ N(0,1), A,B ~ N(0, 0.02^2), y0 ~ N(0,1)."""
    g = torch.Generator().manual_seed(seed)
    ids = torch.randint(0, L, (M,), generator=g, dtype=torch.int32)
    x = _normal(g, (M, K), 1.0, torch.bfloat16)
    a = _normal(g, (L, r, K), 0.02, torch.bfloat16)
    b = _normal(g, (L, N, r), 0.02, torch.bfloat16)
    y0 = _normal(g, (M, N), 1.0, torch.bfloat16)
    rank = torch.full((L,), r, dtype=torch.int32)
    al = torch.full((L,), float(alpha), dtype=torch.float32)
    return Workload("decode", torch.bfloat16, ids, x, a, b, y0, rank, al,
                    note=f"decode bs={M} d_in={K} d_out={N} r={r} L={L} bf16")


def prefill(seed: int = SEED, M: int = 8192, n_seq: int = 16, K: int = 4096, N: int = 4096,
            L: int = 32, r: int = 64, alpha: float = 32.0) -> Workload:
    """Prefill segmented grouped GEMM: n_seq sequences with lengths uniform in [64, 1024]
    rescaled to sum to M, laid out in sequence order (unsorted by adapter), one uniform id
    per sequence."""
    g = torch.Generator().manual_seed(seed)
    lens = _sequence_lengths(g, n_seq, 64, 1024, M)
    seq_ids = torch.randint(0, L, (n_seq,), generator=g, dtype=torch.int32)
    ids = torch.repeat_interleave(seq_ids, torch.tensor(lens, dtype=torch.int64))
    x = _normal(g, (M, K), 1.0, torch.bfloat16)
    a = _normal(g, (L, r, K), 0.02, torch.bfloat16)
    b = _normal(g, (L, N, r), 0.02, torch.bfloat16)
    y0 = _normal(g, (M, N), 1.0, torch.bfloat16)
    rank = torch.full((L,), r, dtype=torch.int32)
    al = torch.full((L,), float(alpha), dtype=torch.float32)
    return Workload("prefill", torch.bfloat16, ids.to(torch.int32), x, a, b, y0, rank, al,
                    note=f"prefill {M} tokens in {n_seq} sequences d={K}->{N} r={r} L={L} bf16")


def zipf_ids(g: torch.Generator, M: int, L: int, s: float) -> torch.Tensor:
    """i.i.d. ids from a Zipf law truncated to the pool: p_k ~ k^-s for k=1..L, id = k-1."""
    k = torch.arange(1, L + 1, dtype=torch.float64)
    p = k.pow(-s)
    p = p / p.sum()
    return torch.multinomial(p, M, replacement=True, generator=g).to(torch.int32)


def mixed(seed: int = SEED, M: int = 2048, K: int = 4096, N: int = 11008, L: int = 128,
          R: int = 64, ranks: Sequence[int] = (8, 16, 32, 64), zipf_s: float = 1.1,
          no_lora_frac: float = 0.1, chunk: int = 64, alpha: float = 32.0) -> Workload:
    """Mixed-rank chunked: Zipf ids, a tenth of the tokens without adapter, per-adapter
    ranks from {8,16,32,64} padded to R, segments re-chunked to 64 rows."""
    g = torch.Generator().manual_seed(seed)
    ids = zipf_ids(g, M, L, zipf_s)
    n_neg = int(round(no_lora_frac * M))
    neg = torch.randperm(M, generator=g)[:n_neg]
    ids[neg] = -1
    x = _normal(g, (M, K), 1.0, torch.bfloat16)
    a = _normal(g, (L, R, K), 0.02, torch.bfloat16)
    b = _normal(g, (L, N, R), 0.02, torch.bfloat16)
    y0 = _normal(g, (M, N), 1.0, torch.bfloat16)
    choice = torch.tensor(list(ranks), dtype=torch.int32)
    rank = choice[torch.randint(0, len(ranks), (L,), generator=g)]
    al = torch.full((L,), float(alpha), dtype=torch.float32)
    return Workload("mixed", torch.bfloat16, ids, x, a, b, y0, rank, al, chunk_size=chunk,
                    note=f"mixed-rank M={M} d={K}->{N} L={L} ranks={tuple(ranks)} "
                         f"zipf s={zipf_s} {n_neg} tokens without adapter chunk={chunk} bf16")


def qkv(seed: int = SEED, K: int = 8192, slices: Sequence[int] = (8192, 1024, 1024),
        r: int = 32, L: int = 512, n_prefill_seq: int = 8, prefill_tokens: int = 3840,
        decode_tokens: int = 256, alphas: Sequence[float] = (16.0, 32.0, 64.0)) -> Workload:
    """Fused QKV slices on a mixed batch: one shared A per adapter, B concatenated over the
    three output slices; prefill sequences first, then one-token decode sequences."""
    g = torch.Generator().manual_seed(seed)
    N = int(sum(slices))
    lens = _sequence_lengths(g, n_prefill_seq, 64, 1024, prefill_tokens)
    seq_ids = torch.randint(0, L, (n_prefill_seq,), generator=g, dtype=torch.int32)
    dec_ids = torch.randint(0, L, (decode_tokens,), generator=g, dtype=torch.int32)
    ids = torch.cat([torch.repeat_interleave(seq_ids, torch.tensor(lens, dtype=torch.int64)),
                     dec_ids]).to(torch.int32)
    M = int(ids.shape[0])
    x = _normal(g, (M, K), 1.0, torch.bfloat16)
    a = _normal(g, (L, r, K), 0.02, torch.bfloat16)
    b = _normal(g, (L, N, r), 0.02, torch.bfloat16)
    y0 = _normal(g, (M, N), 1.0, torch.bfloat16)
    rank = torch.full((L,), r, dtype=torch.int32)
    choice = torch.tensor(list(alphas), dtype=torch.float32)
    al = choice[torch.randint(0, len(alphas), (L,), generator=g)]
    sl, off = [], 0
    for n in slices:
        sl.append((off, int(n)))
        off += int(n)
    return Workload("qkv", torch.bfloat16, ids, x, a, b, y0, rank, al, slices=sl,
                    note=f"fused QKV d={K}->{tuple(slices)} r={r} L={L} "
                         f"{prefill_tokens} prefill + {decode_tokens} decode tokens bf16")


def custom(M: int, K: int, N: int, L: int, R: int, dtype: torch.dtype = torch.bfloat16,
           seed: int = SEED, ranks: Optional[Sequence[int]] = None, no_lora_frac: float = 0.0,
           seq_lens: Optional[Sequence[int]] = None, w_std: float = 0.02, chunk: int = 0,
           alphas: Optional[Sequence[float]] = None, y0_zero: bool = False,
           slices: Optional[Sequence[Tuple[int, int]]] = None, name: str = "custom",
           seq_adapters: Optional[Sequence[int]] = None) -> Workload:
    """General generator for parity cases: odd shapes, ragged tails, mixed ranks, id -1.

    ``ranks``: per-adapter rank choices (uniform over the list); default all R.
    ``seq_lens``: if given, ids are constant per sequence (prefill-like), else i.i.d.
    ``seq_adapters``: with seq_lens, the adapter of each sequence (else drawn uniformly).
    """
    g = torch.Generator().manual_seed(seed)
    if seq_lens is not None:
        seq_lens = [int(v) for v in seq_lens]
        assert sum(seq_lens) == M
        seq_ids = torch.randint(0, L, (len(seq_lens),), generator=g, dtype=torch.int32)
        if seq_adapters is not None:
            assert len(seq_adapters) == len(seq_lens)
            seq_ids = torch.tensor(list(seq_adapters), dtype=torch.int32)
        ids = torch.repeat_interleave(seq_ids, torch.tensor(seq_lens, dtype=torch.int64))
        ids = ids.to(torch.int32)
    else:
        ids = torch.randint(0, L, (M,), generator=g, dtype=torch.int32)
    n_neg = int(round(no_lora_frac * M))
    if n_neg:
        ids[torch.randperm(M, generator=g)[:n_neg]] = -1
    x = _normal(g, (M, K), 1.0, dtype)
    a = _normal(g, (L, R, K), w_std, dtype)
    b = _normal(g, (L, N, R), w_std, dtype)
    y0 = torch.zeros(M, N, dtype=dtype) if y0_zero else _normal(g, (M, N), 1.0, dtype)
    if ranks is None:
        rank = torch.full((L,), R, dtype=torch.int32)
    else:
        choice = torch.tensor(list(ranks), dtype=torch.int32)
        rank = choice[torch.randint(0, len(ranks), (L,), generator=g)]
    if alphas is None:
        al = rank.to(torch.float32) * 2.0
    else:
        choice = torch.tensor(list(alphas), dtype=torch.float32)
        al = choice[torch.randint(0, len(alphas), (L,), generator=g)]
    return Workload(name, dtype, ids, x, a, b, y0, rank, al, chunk_size=chunk,
                    slices=list(slices) if slices else [],
                    note=f"custom M={M} K={K} N={N} L={L} R={R} {dtype}")


# ---------------------------------------------------------------------------------------
# accounting (counts only; used for roofline figures)
# ---------------------------------------------------------------------------------------
def algorithmic_bytes(ids, rank, K: int, N: int, elem_bytes: int) -> int:
    """Bytes the method itself must move for one delta over a batch: x rows of tokens with
    an adapter (read once), their y rows (read and written), each used adapter's true-rank
    A[l, :r, :] and B[l, :, :r] (read once), and the int32 index arrays (ids, sorted ids,
    segment arrays: about 12 B per token). Padding, re-reads and the intermediate h are
    excluded."""
    ids = _np.asarray(ids)
    lora = ids[ids >= 0]
    m = int(lora.shape[0])
    used = _np.unique(lora)
    w = sum(int(rank[l]) * (K + N) for l in used)
    return (m * K + 2 * m * N + w) * elem_bytes + 12 * int(ids.shape[0])


def algorithmic_flops(ids, rank, K: int, N: int) -> int:
    """2 * r * (K + N) per token with an adapter (Ascend article 3.2: about 2 d r M per
    stage)."""
    ids = _np.asarray(ids)
    return int(sum(2 * int(rank[l]) * (K + N) for l in ids[ids >= 0]))



def decode_trace(steps: int, M: int = 256, L: int = 64, mean_len: int = 256,
                 admit_every: int = 8, seed: int = SEED) -> torch.Tensor:
    """Per-step token adapter ids [steps, M] of a decode batch with M slots, one token per
    sequence per step. A sequence keeps its adapter (uniform on [0, L)) for its whole life,
    whose length in steps is uniform on [1, 2 * mean_len - 1]; when it ends its slot holds -1
    until the next admission, which fills every free slot with a new sequence every
    `admit_every` steps. Step 0 starts with every slot occupied, each sequence with a
    remaining life drawn like a new one's."""
    g = torch.Generator().manual_seed(seed)
    ids = torch.randint(0, L, (M,), generator=g, dtype=torch.int32)
    left = torch.randint(1, 2 * mean_len, (M,), generator=g, dtype=torch.int32)
    out = torch.empty(steps, M, dtype=torch.int32)
    for s in range(steps):
        if s > 0 and s % admit_every == 0:
            free = ids < 0
            n = int(free.sum())
            if n:
                ids[free] = torch.randint(0, L, (n,), generator=g, dtype=torch.int32)
                left[free] = torch.randint(1, 2 * mean_len, (n,), generator=g, dtype=torch.int32)
        out[s] = ids
        left -= (ids >= 0).to(torch.int32)
        ids[(ids >= 0) & (left <= 0)] = -1
    return out


BY_NAME = {"tiny": tiny, "decode": decode, "prefill": prefill, "mixed": mixed, "qkv": qkv}


def get(name: str, **kw) -> Workload:
    return BY_NAME[name](**kw)


def segment_example_ids() -> torch.Tensor:
    """Token ids of the Punica page's worked segment example (batching-effect section)."""
    return torch.tensor([2, 2, 2, 5, 5, 1, 1], dtype=torch.int32)
