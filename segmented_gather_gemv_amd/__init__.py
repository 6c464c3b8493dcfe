"""Python binding of libsgmv, the multi-LoRA SGMV delta for MI355X (gfx950).

Argument marshalling only: torch tensors provide device memory and the current HIP stream,
every step of the computation runs in the library's HIP kernels. The function names are
those of the C-ABI in ``include/sgmv.h``:

    sgmv_pool_pack(a, b, rank, alpha)                 -> Pool
    sgmv_build_segments(ids, L, chunk_size, on_device) -> Segments
    sgmv_shrink(x, pool, seg, h=None)                 -> h   (fp32 [M, R_max])
    sgmv_expand(h, pool, seg, y | [slices])           -> None (y updated in place)
    sgmv_lora_delta(x, pool, seg, y | [slices])       -> None (y updated in place)

The shared library is loaded from this package directory; importing raises if it is
missing (build it with ``python -m segmented_gather_gemv_amd.build``).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import List, Optional, Sequence, Tuple, Union

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsgmv.so")

SGMV_OK, SGMV_EINVAL, SGMV_EBADID, SGMV_EUNSUPPORTED, SGMV_ECAPACITY, SGMV_EHIP = range(6)
SGMV_F32, SGMV_BF16 = 0, 1
TILE_ROWS = 64
SMALL_ROWS = 16
TILE_INTS = 32
MAX_RANK = 64
MAX_SLICES = 4
DEVICE_BUILDER_MAX_L = 1024
FUSED_BUILD_MAX_M = 512
PART_SPLIT_MAX_M = 1024
CACHE_HEADER = 4
FOLD_SCALE = 1
NOALLOC_SCRATCH_BYTES = 16 << 20

EXPORTED = [
    "sgmv_pool_init", "sgmv_pool_pack", "sgmv_segments_init", "sgmv_build_segments",
    "sgmv_shrink", "sgmv_expand", "sgmv_lora_delta", "sgmv_build_segments_ex",
    "sgmv_shrink_ex", "sgmv_expand_ex", "sgmv_lora_delta_ex", "sgmv_lora_delta_ids",
    "sgmv_lora_delta_ids_ex", "sgmv_build_segments_cached", "sgmv_build_segments_cached_ex",
    "sgmv_pool_pack_ex", "sgmv_merge_adapter", "sgmv_merge_adapter_ex", "sgmv_status_string",
    "sgmv_version", "sgmv_chunk_size_for_batch", "sgmv_lora_delta_ids_noalloc",
    "sgmv_exchange_placement",
]


class SgmvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {_status_string(status)} (status {status})")


class _Pool(ctypes.Structure):
    _fields_ = [("a", ctypes.c_void_p), ("b", ctypes.c_void_p), ("rank", ctypes.c_void_p),
                ("scale", ctypes.c_void_p), ("L", ctypes.c_int32), ("R_max", ctypes.c_int32),
                ("R_pad", ctypes.c_int32), ("K", ctypes.c_int32), ("N", ctypes.c_int32),
                ("K_pad", ctypes.c_int32), ("N_pad", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("rank_min", ctypes.c_int32), ("scale_folded", ctypes.c_int32)]


class _Segments(ctypes.Structure):
    _fields_ = [("sorted_token_ids", ctypes.c_void_p), ("seg_indptr", ctypes.c_void_p),
                ("seg_lora_ids", ctypes.c_void_p), ("tiles", ctypes.c_void_p),
                ("info", ctypes.c_void_p), ("M", ctypes.c_int32), ("L", ctypes.c_int32),
                ("chunk_size", ctypes.c_int32), ("seg_cap", ctypes.c_int32),
                ("large_cap", ctypes.c_int32), ("small_cap", ctypes.c_int32),
                ("exchange", ctypes.c_void_p), ("exchange_bytes", ctypes.c_int64)]


class _LaunchOpts(ctypes.Structure):
    _fields_ = [("start_event", ctypes.c_void_p), ("stop_event", ctypes.c_void_p),
                ("n_split_small", ctypes.c_int32), ("n_split_large", ctypes.c_int32),
                ("exchange", ctypes.c_int32), ("exchange_wait", ctypes.c_int32)]


class LaunchOpts:
    """Optional launch settings: HIP events (raw hipEvent_t handles) that the kernel's own
    dispatch records at its start and end, column-split overrides (0 = library's choice),
    the K-split exchange of small pieces (0 = library's choice, 1 = on where possible,
    -1 = off) and its wait bound (10 ns units; 0 = default, -1 = no wait)."""

    def __init__(self, start_event=None, stop_event=None, n_split_small=0, n_split_large=0,
                 exchange=0, exchange_wait=0):
        self.c = _LaunchOpts(start_event, stop_event, int(n_split_small), int(n_split_large),
                             int(exchange), int(exchange_wait))

    def ref(self):
        return ctypes.byref(self.c)


def _opts(opts):
    return None if opts is None else opts.ref()


class _Slice(ctypes.Structure):
    _fields_ = [("y", ctypes.c_void_p), ("ldy", ctypes.c_int64), ("n_begin", ctypes.c_int32),
                ("n_len", ctypes.c_int32)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with "
                          f"'python -m segmented_gather_gemv_amd.build'")
    lib = ctypes.CDLL(LIB_PATH)
    i32, i64, vp, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_size_t
    P = ctypes.POINTER
    lib.sgmv_pool_init.argtypes = [i32, i32, i32, i32, i32, P(_Pool), P(sz), P(sz)]
    lib.sgmv_pool_pack.argtypes = [vp, vp, vp, vp, P(_Pool), vp]
    lib.sgmv_pool_pack_ex.argtypes = [vp, vp, vp, vp, i32, P(_Pool), vp]
    lib.sgmv_merge_adapter.argtypes = [vp, i64, vp, i64, P(_Pool), i32, vp]
    lib.sgmv_segments_init.argtypes = [i32, i32, i32, P(_Segments)]
    lib.sgmv_build_segments.argtypes = [vp, i32, i32, i32, i32, P(_Segments), vp]
    lib.sgmv_shrink.argtypes = [vp, i64, i32, P(_Pool), P(_Segments), vp, i64, vp]
    lib.sgmv_expand.argtypes = [vp, i64, i32, P(_Pool), P(_Segments), P(_Slice), i32, vp]
    lib.sgmv_lora_delta.argtypes = [vp, i64, i32, P(_Pool), P(_Segments), P(_Slice), i32, vp]
    O = P(_LaunchOpts)
    lib.sgmv_build_segments_ex.argtypes = [vp, i32, i32, i32, i32, P(_Segments), O, vp]
    lib.sgmv_build_segments_cached.argtypes = [vp, i32, i32, i32, i32, P(_Segments), vp, vp]
    lib.sgmv_build_segments_cached_ex.argtypes = [vp, i32, i32, i32, i32, P(_Segments), vp, O,
                                                  vp]
    lib.sgmv_shrink_ex.argtypes = [vp, i64, i32, P(_Pool), P(_Segments), vp, i64, O, vp]
    lib.sgmv_expand_ex.argtypes = [vp, i64, i32, P(_Pool), P(_Segments), P(_Slice), i32, O, vp]
    lib.sgmv_lora_delta_ex.argtypes = [vp, i64, i32, P(_Pool), P(_Segments), P(_Slice), i32, O,
                                       vp]
    lib.sgmv_lora_delta_ids.argtypes = [vp, vp, i64, i32, P(_Pool), P(_Segments), P(_Slice),
                                        i32, vp]
    lib.sgmv_lora_delta_ids_ex.argtypes = [vp, vp, i64, i32, P(_Pool), P(_Segments), P(_Slice),
                                           i32, O, vp]
    lib.sgmv_merge_adapter_ex.argtypes = [vp, i64, vp, i64, P(_Pool), i32, O, vp]
    lib.sgmv_lora_delta_ids_noalloc.argtypes = [vp, vp, i64, i32, P(_Pool), P(_Segments),
                                                P(_Slice), i32, vp]
    for f in ["sgmv_pool_init", "sgmv_pool_pack", "sgmv_segments_init", "sgmv_build_segments",
              "sgmv_shrink", "sgmv_expand", "sgmv_lora_delta", "sgmv_build_segments_ex",
              "sgmv_shrink_ex", "sgmv_expand_ex", "sgmv_lora_delta_ex", "sgmv_lora_delta_ids",
              "sgmv_lora_delta_ids_ex", "sgmv_build_segments_cached",
              "sgmv_build_segments_cached_ex", "sgmv_pool_pack_ex", "sgmv_merge_adapter",
              "sgmv_merge_adapter_ex", "sgmv_lora_delta_ids_noalloc"]:
        getattr(lib, f).restype = ctypes.c_int
    lib.sgmv_status_string.argtypes = [ctypes.c_int]
    lib.sgmv_status_string.restype = ctypes.c_char_p
    lib.sgmv_version.restype = ctypes.c_int32
    lib.sgmv_chunk_size_for_batch.argtypes = [i32, i32]
    lib.sgmv_chunk_size_for_batch.restype = ctypes.c_int32
    lib.sgmv_exchange_placement.argtypes = [P(i32), vp]
    lib.sgmv_exchange_placement.restype = ctypes.c_int
    return lib


_lib = _load()


def _status_string(s: int) -> str:
    return _lib.sgmv_status_string(int(s)).decode()


def _check(status: int, where: str):
    if status != SGMV_OK:
        raise SgmvError(status, where)


def library():
    """The loaded ctypes library (for tests of the raw C-ABI)."""
    return _lib


def _stream(device: torch.device):
    if device.type != "cuda":
        return None
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _dtype_code(dt: torch.dtype) -> int:
    if dt == torch.bfloat16:
        return SGMV_BF16
    if dt == torch.float32:
        return SGMV_F32
    raise TypeError(f"libsgmv takes bfloat16 or float32, got {dt}")


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


# ---------------------------------------------------------------------------------------
# pool
# ---------------------------------------------------------------------------------------
@dataclass
class Pool:
    a: torch.Tensor        # [L, R_pad, K_pad]
    b: torch.Tensor        # [L, R_pad/8, N_pad, 8]
    rank: torch.Tensor     # int32 [L]
    scale: torch.Tensor    # fp32 [L]
    desc: _Pool

    @property
    def L(self): return self.desc.L

    @property
    def R_max(self): return self.desc.R_max

    @property
    def K(self): return self.desc.K

    @property
    def N(self): return self.desc.N

    @property
    def dtype(self): return self.a.dtype


def sgmv_pool_init(L: int, R_max: int, K: int, N: int, dtype: torch.dtype,
                   device: Union[str, torch.device] = "cuda") -> Pool:
    """Allocate an empty pool (zero-filled) in the library layout."""
    desc = _Pool()
    ab, bb = ctypes.c_size_t(), ctypes.c_size_t()
    _check(_lib.sgmv_pool_init(L, R_max, K, N, _dtype_code(dtype), ctypes.byref(desc),
                               ctypes.byref(ab), ctypes.byref(bb)), "sgmv_pool_init")
    dev = torch.device(device)
    a = torch.zeros(L, desc.R_pad, desc.K_pad, dtype=dtype, device=dev)
    b = torch.zeros(L, desc.R_pad // 8, desc.N_pad, 8, dtype=dtype, device=dev)
    assert a.numel() * a.element_size() == ab.value and b.numel() * b.element_size() == bb.value
    rank = torch.zeros(L, dtype=torch.int32, device=dev)
    scale = torch.zeros(L, dtype=torch.float32, device=dev)
    desc.a, desc.b = a.data_ptr(), b.data_ptr()
    desc.rank, desc.scale = rank.data_ptr(), scale.data_ptr()
    return Pool(a, b, rank, scale, desc)


def sgmv_pool_pack(a: torch.Tensor, b: torch.Tensor, rank: Sequence[int],
                   alpha: Sequence[float], fold_scale: bool = False) -> Pool:
    """Pack user-layout adapters A (L, R, K) and B (L, N, R) (device tensors of the pool
    dtype) with per-adapter rank and alpha into a new pool. ``fold_scale`` stores
    alpha/r * B (formed in fp32, rounded once to the pool dtype) and unit scales."""
    if a.dim() != 3 or b.dim() != 3:
        raise ValueError("a must be (L, R, K) and b (L, N, R)")
    L, R, K = a.shape
    if b.shape[0] != L or b.shape[2] != R:
        raise ValueError(f"b shape {tuple(b.shape)} does not match a shape {tuple(a.shape)}")
    if a.dtype != b.dtype:
        raise TypeError("a and b must share a dtype")
    N = b.shape[1]
    pool = sgmv_pool_init(L, R, K, N, a.dtype, a.device)
    a = a.contiguous()
    b = b.contiguous()
    rank_h = torch.as_tensor(rank, dtype=torch.int32).cpu().contiguous()
    alpha_h = torch.as_tensor(alpha, dtype=torch.float32).cpu().contiguous()
    if rank_h.numel() != L or alpha_h.numel() != L:
        raise ValueError("rank and alpha need one entry per adapter")
    _check(_lib.sgmv_pool_pack_ex(_ptr(a), _ptr(b), _ptr(rank_h), _ptr(alpha_h),
                                  FOLD_SCALE if fold_scale else 0, ctypes.byref(pool.desc),
                                  _stream(a.device)), "sgmv_pool_pack")
    return pool


# ---------------------------------------------------------------------------------------
# segments
# ---------------------------------------------------------------------------------------
@dataclass
class Segments:
    sorted_token_ids: torch.Tensor
    seg_indptr: torch.Tensor
    seg_lora_ids: torch.Tensor
    tiles: torch.Tensor          # [(large_cap + small_cap), TILE_INTS] descriptor records
    info: torch.Tensor           # [4]: num_segments, n_large, n_small, status
    desc: _Segments
    exchange: Optional[torch.Tensor] = None  # fused-call workspace (device, zero-filled)

    @property
    def M(self): return self.desc.M

    def to(self, device) -> "Segments":
        """Copy (e.g. host-built) segments to another device; a GPU copy gets a fresh
        exchange workspace."""
        d = _Segments()
        ctypes.memmove(ctypes.byref(d), ctypes.byref(self.desc), ctypes.sizeof(_Segments))
        dev = torch.device(device)
        out = Segments(*(t.to(dev) for t in (self.sorted_token_ids, self.seg_indptr,
                                             self.seg_lora_ids, self.tiles, self.info)), d,
                       _exchange_buffer(d, dev))
        out._bind()
        return out

    def _bind(self):
        self.desc.sorted_token_ids = self.sorted_token_ids.data_ptr()
        self.desc.seg_indptr = self.seg_indptr.data_ptr()
        self.desc.seg_lora_ids = self.seg_lora_ids.data_ptr()
        self.desc.tiles = self.tiles.data_ptr()
        self.desc.info = self.info.data_ptr()
        self.desc.exchange = None if self.exchange is None else self.exchange.data_ptr()

    def host(self) -> dict:
        """Synchronous host view: the trimmed arrays and the counters."""
        info = self.info.cpu().tolist()
        S, nl, ns, st = info
        tiles = self.tiles.cpu()
        return {
            "sorted_token_ids": self.sorted_token_ids.cpu(),
            "seg_indptr": self.seg_indptr.cpu()[:S + 1],
            "seg_lora_ids": self.seg_lora_ids.cpu()[:S],
            "num_segments": S,
            "large_tiles": tiles[:nl],
            "small_tiles": tiles[self.desc.large_cap:self.desc.large_cap + ns],
            "status": st,
        }


_PLACEMENT = {}


def sgmv_exchange_placement(device: Union[str, torch.device] = "cuda") -> Tuple[bool, int]:
    """Whether the fused call's K-split exchange may be used on `device` (the workgroups of
    a piece run on one XCD), and the number of XCDs seen; checked once per device."""
    dev = torch.device(device)
    key = dev.index if dev.index is not None else torch.cuda.current_device()
    if key not in _PLACEMENT:
        n = ctypes.c_int32(0)
        with torch.cuda.device(key):
            st = _lib.sgmv_exchange_placement(ctypes.byref(n),
                                              ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        if st not in (SGMV_OK, SGMV_EUNSUPPORTED):
            _check(st, "sgmv_exchange_placement")
        _PLACEMENT[key] = (st == SGMV_OK, int(n.value))
    return _PLACEMENT[key]


def _exchange_buffer(desc: _Segments, dev: torch.device) -> Optional[torch.Tensor]:
    if dev.type != "cuda" or desc.exchange_bytes <= 0:
        return None
    if not sgmv_exchange_placement(dev)[0]:
        return None  # partners of a piece would not share an L2: fused calls run without it
    buf = torch.zeros(int(desc.exchange_bytes) + 256, dtype=torch.uint8, device=dev)
    off = (-buf.data_ptr()) % 256  # the library wants 256-byte alignment
    return buf[off:off + int(desc.exchange_bytes)]


def sgmv_segments_alloc(M: int, L: int, chunk_size: int = 0,
                        device: Union[str, torch.device] = "cuda",
                        exchange: bool = True) -> Segments:
    """Allocate segment arrays for M tokens and L adapters; on a GPU, also the zero-filled
    exchange workspace of the fused call unless ``exchange`` is False."""
    desc = _Segments()
    _check(_lib.sgmv_segments_init(M, L, chunk_size, ctypes.byref(desc)), "sgmv_segments_init")
    dev = torch.device(device)
    z = lambda n: torch.zeros(max(int(n), 1), dtype=torch.int32, device=dev)
    seg = Segments(z(M), z(desc.seg_cap + 1), z(desc.seg_cap),
                   torch.zeros(max(desc.large_cap + desc.small_cap, 1), TILE_INTS,
                               dtype=torch.int32, device=dev), z(4), desc,
                   _exchange_buffer(desc, dev) if exchange else None)
    seg._bind()
    return seg


def sgmv_build_segments(ids: torch.Tensor, L: int, chunk_size: int = 0, on_device: bool = True,
                        out: Optional[Segments] = None,
                        opts: Optional[LaunchOpts] = None) -> Segments:
    """Group tokens by adapter (id -1: no adapter). ``on_device`` runs the GPU builder on the
    current stream without a host sync (ids must be a device tensor); otherwise the host
    builder runs on CPU tensors and raises on a bad id."""
    ids = ids.to(torch.int32).contiguous()
    M = int(ids.numel())
    dev = ids.device
    if on_device and dev.type != "cuda":
        raise ValueError("on_device=True needs ids on the GPU")
    if not on_device and dev.type != "cpu":
        raise ValueError("on_device=False needs ids on the CPU")
    seg = out if out is not None else sgmv_segments_alloc(M, L, chunk_size, dev)
    _check(_lib.sgmv_build_segments_ex(_ptr(ids), M, L, chunk_size, 1 if on_device else 0,
                                       ctypes.byref(seg.desc), _opts(opts), _stream(dev)),
           "sgmv_build_segments")
    return seg


def sgmv_chunk_size_for_batch(M: int, n_adapters: int = 0) -> int:
    """The library's chunk size for a batch of M tokens over n_adapters distinct adapters
    (0 = unknown), measured: see include/sgmv.h."""
    return int(_lib.sgmv_chunk_size_for_batch(int(M), int(n_adapters)))


def sgmv_segments_cache_alloc(M: int, device: Union[str, torch.device] = "cuda") -> torch.Tensor:
    """An empty grouping cache for batches of M tokens: SGMV_CACHE_HEADER + M zeroed int32."""
    return torch.zeros(CACHE_HEADER + max(int(M), 0), dtype=torch.int32, device=device)


def sgmv_build_segments_cached(ids: torch.Tensor, seg: Segments, cache: torch.Tensor,
                               on_device: bool = True,
                               opts: Optional[LaunchOpts] = None) -> Segments:
    """Build ``seg`` from ``ids`` unless the cache shows that seg already holds the build of
    these very ids (then nothing is written). ``cache`` comes from sgmv_segments_cache_alloc
    and is used with this seg only; on the device nothing syncs with the host."""
    ids = ids.to(torch.int32).contiguous()
    M = int(ids.numel())
    dev = ids.device
    if (dev.type == "cuda") != bool(on_device) or cache.device != dev:
        raise ValueError("ids and cache must both be on the GPU (on_device) or on the CPU")
    if cache.dtype != torch.int32 or not cache.is_contiguous() or cache.numel() < CACHE_HEADER + M:
        raise ValueError("cache must be a contiguous int32 tensor of SGMV_CACHE_HEADER + M")
    _check(_lib.sgmv_build_segments_cached_ex(_ptr(ids), M, seg.desc.L, seg.desc.chunk_size,
                                              1 if on_device else 0, ctypes.byref(seg.desc),
                                              _ptr(cache), _opts(opts), _stream(dev)),
           "sgmv_build_segments_cached")
    return seg


# ---------------------------------------------------------------------------------------
# shrink / expand / fused delta
# ---------------------------------------------------------------------------------------
SliceSpec = Tuple[torch.Tensor, int]   # (y tensor [M, n_len], first pool column)


def _slices(y_or_slices, pool: Pool, M: int):
    if isinstance(y_or_slices, torch.Tensor):
        specs = [(y_or_slices, 0)]
    else:
        specs = list(y_or_slices)
    arr = (_Slice * len(specs))()
    for i, (y, n0) in enumerate(specs):
        if y.dim() != 2 or y.shape[0] != M or y.stride(1) != 1:
            raise ValueError("each output slice must be a row-major [M, n] tensor")
        if y.dtype != pool.dtype or y.device != pool.a.device:
            raise TypeError("output slice dtype/device must match the pool")
        arr[i].y = y.data_ptr()
        arr[i].ldy = y.stride(0)
        arr[i].n_begin = int(n0)
        arr[i].n_len = int(y.shape[1])
    return arr, len(specs)


def _check_x(x: torch.Tensor, pool: Pool):
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a row-major [M, K] tensor")
    if x.dtype != pool.dtype or x.device != pool.a.device:
        raise TypeError("x dtype/device must match the pool")
    if x.shape[1] != pool.K:
        raise ValueError(f"x has {x.shape[1]} columns, pool K is {pool.K}")


def sgmv_shrink(x: torch.Tensor, pool: Pool, seg: Segments,
                h: Optional[torch.Tensor] = None,
                opts: Optional[LaunchOpts] = None) -> torch.Tensor:
    """h[t, :r] = A[l, :r, :] @ x[t] for tokens with an adapter (fp32, unscaled)."""
    _check_x(x, pool)
    M = x.shape[0]
    if h is None:
        h = torch.zeros(M, pool.R_max, dtype=torch.float32, device=x.device)
    if h.dtype != torch.float32 or h.stride(1) != 1:
        raise TypeError("h must be a row-major fp32 tensor")
    _check(_lib.sgmv_shrink_ex(_ptr(x), x.stride(0), M, ctypes.byref(pool.desc),
                               ctypes.byref(seg.desc), _ptr(h), h.stride(0), _opts(opts),
                               _stream(x.device)), "sgmv_shrink")
    return h


def sgmv_expand(h: torch.Tensor, pool: Pool, seg: Segments,
                y: Union[torch.Tensor, Sequence[SliceSpec]],
                opts: Optional[LaunchOpts] = None) -> None:
    """y[t] += scale_l * B[l, :, :r] @ h[t, :r] (in place; list of (y, first column) for
    several output slices)."""
    if h.dtype != torch.float32 or h.stride(1) != 1:
        raise TypeError("h must be a row-major fp32 tensor")
    M = h.shape[0]
    arr, n = _slices(y, pool, M)
    _check(_lib.sgmv_expand_ex(_ptr(h), h.stride(0), M, ctypes.byref(pool.desc),
                               ctypes.byref(seg.desc), arr, n, _opts(opts), _stream(h.device)),
           "sgmv_expand")


def sgmv_lora_delta(x: torch.Tensor, pool: Pool, seg: Segments,
                    y: Union[torch.Tensor, Sequence[SliceSpec]],
                    opts: Optional[LaunchOpts] = None) -> None:
    """Fused y[t] += scale_l * B[l, :, :r] @ (A[l, :r, :] @ x[t]) (in place)."""
    _check_x(x, pool)
    M = x.shape[0]
    arr, n = _slices(y, pool, M)
    _check(_lib.sgmv_lora_delta_ex(_ptr(x), x.stride(0), M, ctypes.byref(pool.desc),
                                   ctypes.byref(seg.desc), arr, n, _opts(opts),
                                   _stream(x.device)), "sgmv_lora_delta")


def sgmv_lora_delta_ids(ids: torch.Tensor, x: torch.Tensor, pool: Pool, seg: Segments,
                        y: Union[torch.Tensor, Sequence[SliceSpec]],
                        opts: Optional[LaunchOpts] = None) -> None:
    """Build ``seg`` from the device ids and apply the fused delta, as sgmv_build_segments
    (on device) followed by sgmv_lora_delta; a single launch for small bf16 batches."""
    _check_x(x, pool)
    M = x.shape[0]
    if ids.dtype != torch.int32 or ids.device != x.device or ids.numel() != M:
        raise TypeError("ids must be an int32 tensor of M entries on x's device")
    ids = ids.contiguous()
    arr, n = _slices(y, pool, M)
    _check(_lib.sgmv_lora_delta_ids_ex(_ptr(ids), _ptr(x), x.stride(0), M,
                                       ctypes.byref(pool.desc), ctypes.byref(seg.desc), arr, n,
                                       _opts(opts), _stream(x.device)), "sgmv_lora_delta_ids")


def sgmv_lora_delta_ids_noalloc(ids: torch.Tensor, x: torch.Tensor, pool: Pool,
                                seg: Segments,
                                y: Union[torch.Tensor, Sequence[SliceSpec]]) -> None:
    """sgmv_lora_delta_ids with the exchange workspace in the library's static device array
    (seg.exchange is not used): for callers that cannot allocate device memory. Calls that
    overlap on one GPU share that array; order them on one stream."""
    _check_x(x, pool)
    M = x.shape[0]
    if ids.dtype != torch.int32 or ids.device != x.device or ids.numel() != M:
        raise TypeError("ids must be an int32 tensor of M entries on x's device")
    ids = ids.contiguous()
    arr, n = _slices(y, pool, M)
    _check(_lib.sgmv_lora_delta_ids_noalloc(_ptr(ids), _ptr(x), x.stride(0), M,
                                            ctypes.byref(pool.desc), ctypes.byref(seg.desc),
                                            arr, n, _stream(x.device)),
           "sgmv_lora_delta_ids_noalloc")


def sgmv_merge_adapter(w: torch.Tensor, pool: Pool, adapter: int,
                       out: Optional[torch.Tensor] = None,
                       opts: Optional[LaunchOpts] = None) -> torch.Tensor:
    """W' = W + scale_l B_l A_l for the base weight w (N, K) of y = x W^T, into ``out`` (a new
    tensor by default; ``out=w`` merges in place)."""
    if w.dim() != 2 or tuple(w.shape) != (pool.N, pool.K):
        raise ValueError(f"w must be (N, K) = ({pool.N}, {pool.K})")
    if w.dtype != pool.dtype or w.device != pool.a.device or w.stride(1) != 1:
        raise ValueError("w must be a row-contiguous tensor of the pool's dtype and device")
    if out is None:
        out = torch.empty_like(w, memory_format=torch.contiguous_format)
    if tuple(out.shape) != tuple(w.shape) or out.dtype != w.dtype or out.stride(1) != 1:
        raise ValueError("out must match w")
    _check(_lib.sgmv_merge_adapter_ex(_ptr(w), w.stride(0), _ptr(out), out.stride(0),
                                      ctypes.byref(pool.desc), int(adapter), _opts(opts),
                                      _stream(w.device)), "sgmv_merge_adapter")
    return out


__all__ = [
    "LIB_PATH", "EXPORTED", "SgmvError", "Pool", "Segments", "LaunchOpts", "library",
    "sgmv_pool_init", "sgmv_pool_pack", "sgmv_segments_alloc", "sgmv_build_segments",
    "sgmv_shrink", "sgmv_expand", "sgmv_lora_delta", "sgmv_lora_delta_ids",
    "sgmv_lora_delta_ids_noalloc", "sgmv_segments_cache_alloc", "sgmv_build_segments_cached", "sgmv_merge_adapter",
    "sgmv_chunk_size_for_batch", "sgmv_exchange_placement",
]
