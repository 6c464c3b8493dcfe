// On-device segment builder: the same stable counting sort as the host builder, in one
// workgroup, with no host synchronisation (Ascend article 4.2: a per-step sort that syncs
// host and device sits on the critical path).
//
// Shared definitions: keys are adapter ids, with key L standing for "no adapter" (-1, or a
// bad id, which also raises the status flag). Buckets follow the order in which adapters
// first appear; tokens ascend inside a bucket (Punica page, code section; worked example in
// the batching-effect section). A token lands at bucket start + (equal keys before it).
//
// Two kernels:
//  * small batches (M <= 1024, one token per thread, 4, 8 or 16 waves): each wave ranks its
//    64 keys in registers (one ballot per lane), a per-(key, wave) byte table in LDS adds the
//    counts of lower waves, and one workgroup scan over the tokens of (first-appearance flag,
//    bucket size, segments, large and small descriptors) places every bucket;
//  * larger batches: the same in rounds of 1024 tokens with a running count per key, lanes
//    of equal keys grouped by ballots.
// Every global write index is checked against its array bound. Both kernels also clear the
// control words of the fused call's exchange workspace, when the segments carry one.
#include <climits>

#include "common.h"

namespace sgmv {

constexpr int BUILD_THREADS = 1024;
constexpr int BUILD_WAVES = BUILD_THREADS / WAVE;

__host__ __device__ inline size_t align16(size_t v) { return (v + 15) & ~size_t(15); }

// Inclusive scan across the 64 lanes of a wave with DPP row shifts and row broadcasts.
__device__ __forceinline__ int wave_incl_scan(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// Exclusive scan of NV ints per thread across a workgroup of NW waves. s_w holds NV * NW
// ints. Contains barriers: call from all threads.
template <int NV, int NW = BUILD_WAVES>
__device__ void block_scan(const int (&v)[NV], int (&ex)[NV], int (&tot)[NV], int* s_w) {
  const int lane = threadIdx.x & (WAVE - 1), w = threadIdx.x / WAVE;
  int x[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    x[i] = wave_incl_scan(v[i]);
    if (lane == WAVE - 1) s_w[i * NW + w] = x[i];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int4* q = reinterpret_cast<const int4*>(s_w + i * NW);
    int before = 0, all = 0;
#pragma unroll
    for (int j = 0; j < NW / 4; ++j) {
      const int4 s = q[j];
      const int vals[4] = {s.x, s.y, s.z, s.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        all += vals[e];
        before += (4 * j + e < w) ? vals[e] : 0;
      }
    }
    ex[i] = before + x[i] - v[i];
    tot[i] = all;
  }
  __syncthreads();
}

// Counts of equal keys in lower waves (pre), in this wave (cw) and in higher waves (post),
// from the per-(key, wave) byte table of a workgroup of NW waves.
template <int NW = BUILD_WAVES>
__device__ __forceinline__ void wave_counts(const uint8_t* rc, int key, int& pre, int& cw,
                                            int& post) {
  const int w = threadIdx.x / WAVE;
  const uint32_t* q = reinterpret_cast<const uint32_t*>(rc + key * NW);
  pre = cw = post = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int v = (q[i >> 2] >> (8 * (i & 3))) & 0xff;
    if (i < w) pre += v;
    else if (i == w) cw = v;
    else post += v;
  }
}

// Descriptor counts of one segment of `len` rows.
__device__ __forceinline__ void piece_tiles(int len, int& nl, int& ns) {
  const int rem = len % SGMV_TILE_ROWS;
  nl = len / SGMV_TILE_ROWS + (rem > SGMV_SMALL_ROWS ? 1 : 0);
  ns = (rem > 0 && rem <= SGMV_SMALL_ROWS) ? 1 : 0;
}

// Writes the descriptors of one bucket (adapter `lora`, `cnt` rows from sorted row `start`,
// chunk size C) and its segments. Token slots of small descriptors are left to the tokens'
// own threads (token_slot); every other token slot gets -1.
__device__ void write_bucket(int lora, int cnt, int C, int start, int seg0, int lt, int st,
                             int32_t* indptr, int32_t* seg_lora, int32_t* tiles, int seg_cap,
                             int large_cap, int small_cap) {
  const int np = C > 0 ? (cnt + C - 1) / C : 1;
  for (int i = 0; i < np; ++i) {
    const int seg = seg0 + i;
    const int s0 = start + (C > 0 ? i * C : 0);
    const int len = C > 0 ? min(C, cnt - i * C) : cnt;
    if (seg < seg_cap) {
      indptr[seg] = s0;
      seg_lora[seg] = lora;
    }
    for (int r0 = 0; r0 < len; r0 += SGMV_TILE_ROWS) {
      const int rows = min(SGMV_TILE_ROWS, len - r0);
      const bool small = rows <= SGMV_SMALL_ROWS;
      const int idx = small ? st++ : lt++;
      if (small ? idx >= small_cap : idx >= large_cap) continue;
      int4* d = reinterpret_cast<int4*>(tiles + (size_t)(small ? large_cap + idx : idx) *
                                                    SGMV_TILE_INTS);
      d[0] = make_int4(lora, s0 + r0, rows, seg);
      d[1] = d[2] = d[3] = make_int4(0, 0, 0, 0);
      // token slots past the piece's rows; the others belong to the tokens' own threads
      const int first_free = small ? rows : 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (4 * q >= first_free) {
          d[4 + q] = make_int4(-1, -1, -1, -1);
        } else if (4 * q + 4 > first_free) {
          int32_t* e = reinterpret_cast<int32_t*>(d + 4 + q);
          for (int i = first_free - 4 * q; i < 4; ++i) e[i] = -1;
        }
      }
    }
  }
}

// The token with in-bucket rank `rank` of a bucket of `cnt` rows whose first small
// descriptor is `sbase`: if it lands in a small descriptor, store its id in that record.
__device__ __forceinline__ void token_slot(int t, int rank, int cnt, int C, int sbase,
                                           int32_t* tiles, int large_cap, int small_cap) {
  const int i = C > 0 ? rank / C : 0;                  // segment (chunk) inside the bucket
  const int in_seg = C > 0 ? rank - i * C : rank;
  const int len = C > 0 ? min(C, cnt - i * C) : cnt;
  const int piece = in_seg / SGMV_TILE_ROWS;
  const int rows = min(SGMV_TILE_ROWS, len - piece * SGMV_TILE_ROWS);
  if (rows > SGMV_SMALL_ROWS) return;
  int nl_full, ns_full;
  piece_tiles(C > 0 ? C : cnt, nl_full, ns_full);
  const int sidx = sbase + (C > 0 ? i * ns_full : 0);  // one small piece at most per segment
  const int slot = in_seg - piece * SGMV_TILE_ROWS;
  if (sidx < small_cap && slot < SGMV_SMALL_ROWS)
    tiles[(size_t)(large_cap + sidx) * SGMV_TILE_INTS + 16 + slot] = t;
}

// ---------------------------------------------------------------------------------------
// small batches: M <= 1024
// ---------------------------------------------------------------------------------------
size_t build_small_lds_bytes(int L, int nw) {
  const size_t nk = (size_t)L + 1;
  return align16(nk * nw) + 2 * align16(nk * sizeof(int));
}

// One token per thread, NW waves (the fewest that cover M).
template <int NW>
__global__ __launch_bounds__(NW * WAVE) void build_segments_small_kernel(
    const int32_t* __restrict__ ids, int M, int L, int C, int32_t* __restrict__ sorted,
    int32_t* __restrict__ indptr, int32_t* __restrict__ seg_lora, int32_t* __restrict__ tiles,
    int32_t* __restrict__ info, int seg_cap, int large_cap, int small_cap,
    int32_t* __restrict__ xctl, int n_xctl) {
  constexpr int NT = NW * WAVE;
  extern __shared__ __align__(16) unsigned char smem[];
  const int NK = L + 1;
  uint8_t* rc = smem;                                                     // [NK][NW]
  int* s_base = reinterpret_cast<int*>(smem + align16((size_t)NK * NW));  // [NK]
  int* s_sbase = s_base + align16((size_t)NK * sizeof(int)) / sizeof(int);  // [NK]
  __shared__ __align__(16) int s_w[5 * NW];
  __shared__ int s_bad;

  const int t = threadIdx.x, lane = t & (WAVE - 1), w = t / WAVE;
  const bool valid = t < M;
  for (int i = t; i < n_xctl; i += NT) xctl[i] = 0;
  for (int i = t; i < NK * (NW / 4); i += NT) reinterpret_cast<uint32_t*>(rc)[i] = 0;
  if (t == 0) s_bad = 0;
  int key = -2;  // never equal to a real key (0..L)
  if (valid) {
    int id = ids[t];
    if (id < -1 || id >= L) {
      s_bad = 1;
      id = -1;
    }
    key = id < 0 ? L : id;
  }
  // rank among equal keys of lower lanes, and the count in this wave: lane j keeps the
  // ballot of the lanes holding its key (lanes past M hold a key no token has)
  uint64_t same = 0;
  if (w * WAVE < M) {  // uniform; waves without tokens skip it
#pragma unroll
    for (int j = 0; j < WAVE; ++j) {
      const uint64_t m = __ballot(key == __builtin_amdgcn_readlane(key, j));
      same = lane == j ? m : same;
    }
  }
  const int rk = __popcll(same & lanemask_lt(lane));
  const int cw = __popcll(same);
  __syncthreads();
  if (valid && rk == 0) rc[key * NW + w] = (uint8_t)cw;
  __syncthreads();
  int pre = 0, cwt = 0, post = 0;
  if (valid) wave_counts<NW>(rc, key, pre, cwt, post);
  const int rank = pre + rk;
  const int cnt = pre + cwt + post;
  const bool first = valid && key < L && rank == 0;
  int v[5] = {0, 0, 0, 0, 0};
  if (first) {
    const int np = C > 0 ? (cnt + C - 1) / C : 1;
    const int last = C > 0 ? cnt - C * (np - 1) : cnt;
    int nl, ns, nl1, ns1;
    piece_tiles(C > 0 ? C : cnt, nl, ns);
    piece_tiles(last, nl1, ns1);
    v[0] = 1;
    v[1] = cnt;
    v[2] = np;
    v[3] = (np - 1) * nl + nl1;
    v[4] = (np - 1) * ns + ns1;
  }
  int ex[5], tot[5];
  block_scan<5, NW>(v, ex, tot, s_w);
  const int n_lora = tot[1], n_seg = tot[2], n_large = tot[3], n_small = tot[4];
  const bool overflow = n_seg > seg_cap || n_large > large_cap || n_small > small_cap;
  if (first) {
    s_base[key] = ex[1];
    s_sbase[key] = ex[4];
    if (!overflow)
      write_bucket(key, cnt, C, ex[1], ex[2], ex[3], ex[4], indptr, seg_lora, tiles, seg_cap,
                   large_cap, small_cap);
  }
  if (t == 0) {
    if (!overflow) indptr[n_seg] = n_lora;
    info[0] = overflow ? 0 : n_seg;
    info[1] = overflow ? 0 : n_large;
    info[2] = overflow ? 0 : n_small;
    info[3] = overflow ? SGMV_ECAPACITY : (s_bad ? SGMV_EBADID : SGMV_OK);
    s_base[L] = n_lora;
  }
  __syncthreads();
  if (valid) {
    const int pos = s_base[key] + rank;
    if (pos < M) sorted[pos] = t;
    if (key < L && !overflow)
      token_slot(t, rank, cnt, C, s_sbase[key], tiles, large_cap, small_cap);
  }
}

// ---------------------------------------------------------------------------------------
// larger batches: rounds of 1024 tokens
// ---------------------------------------------------------------------------------------
size_t build_lds_bytes(int L) {
  const size_t nk = (size_t)L + 1;
  return align16(nk * BUILD_WAVES) + 7 * align16((nk + 1) * sizeof(int));
}

// Group lanes of this wave holding equal keys. Returns the lane's rank among lanes with the
// same key and a lower lane index. The lowest lane of each group writes the group size to
// rc[key * 16 + wave] and, when `first` is given and key < L, folds its token into first[].
__device__ int match_rank(bool valid, int key, int t, uint8_t* rc, int* first, int L) {
  const int lane = threadIdx.x & (WAVE - 1), w = threadIdx.x / WAVE;
  uint64_t active = __ballot(valid);
  int myrank = 0;
  while (active) {
    const int leader = __ffsll((unsigned long long)active) - 1;
    const int lkey = __builtin_amdgcn_readlane(key, leader);
    const uint64_t m = __ballot(valid && key == lkey);
    if (valid && key == lkey) myrank = __popcll(m & lanemask_lt(lane));
    if (lane == leader) {
      rc[lkey * BUILD_WAVES + w] = (uint8_t)__popcll(m);
      if (first != nullptr && lkey < L) atomicMin(&first[lkey], t);
    }
    active &= ~m;
  }
  return myrank;
}

__global__ __launch_bounds__(BUILD_THREADS) void build_segments_kernel(
    const int32_t* __restrict__ ids, int M, int L, int C, int32_t* __restrict__ sorted,
    int32_t* __restrict__ indptr, int32_t* __restrict__ seg_lora, int32_t* __restrict__ tiles,
    int32_t* __restrict__ info, int seg_cap, int large_cap, int small_cap,
    int32_t* __restrict__ xctl, int n_xctl) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int NK = L + 1;  // key L = "no adapter"
  uint8_t* rc = smem;
  int* run = reinterpret_cast<int*>(smem + align16((size_t)NK * BUILD_WAVES));
  const size_t stride = align16((size_t)(NK + 1) * sizeof(int)) / sizeof(int);
  int* first = run + stride;      // first token of each adapter, then its first large piece
  int* bidx = first + stride;     // bucket of each adapter
  int* ord = bidx + stride;       // adapter of each bucket
  int* bstart = ord + stride;     // first sorted row of each bucket
  int* pstart = bstart + stride;  // first segment of each bucket
  int* sbase = pstart + stride;   // first small descriptor of each bucket
  __shared__ __align__(16) int s_w[4 * BUILD_WAVES];
  __shared__ int s_bad;

  const int tid = threadIdx.x;
  for (int i = tid; i < n_xctl; i += BUILD_THREADS) xctl[i] = 0;
  for (int i = tid; i < NK * (BUILD_WAVES / 4); i += BUILD_THREADS)
    reinterpret_cast<uint32_t*>(rc)[i] = 0;
  for (int i = tid; i < NK; i += BUILD_THREADS) {
    run[i] = 0;
    first[i] = INT_MAX;
  }
  if (tid == 0) s_bad = 0;
  __syncthreads();

  const int rounds = (M + BUILD_THREADS - 1) / BUILD_THREADS;

  // ---- pass 1: per-key totals and first appearance ----
  for (int rd = 0; rd < rounds; ++rd) {
    const int t = rd * BUILD_THREADS + tid;
    const bool valid = t < M;
    int key = 0;
    if (valid) {
      int id = ids[t];
      if (id < -1 || id >= L) {
        s_bad = 1;
        id = -1;
      }
      key = id < 0 ? L : id;
    }
    const int myrank = match_rank(valid, key, t, rc, first, L);
    __syncthreads();
    int pre = 0, cw = 0, post = 0;
    if (valid) wave_counts(rc, key, pre, cw, post);
    __syncthreads();
    if (valid) {
      if (post == 0 && myrank == cw - 1) run[key] += pre + cw;
      rc[key * BUILD_WAVES + tid / WAVE] = 0;
    }
  }
  __syncthreads();

  // ---- bucket order: the first appearances, in token order ----
  int n_buckets = 0;
  for (int rd = 0; rd < rounds; ++rd) {
    const int t = rd * BUILD_THREADS + tid;
    int key = L;
    if (t < M) {
      const int id = ids[t];
      key = (id < 0 || id >= L) ? L : id;
    }
    const int v[1] = {(t < M && key < L && first[key] == t) ? 1 : 0};
    int ex[1], tot[1];
    block_scan<1>(v, ex, tot, s_w);
    if (v[0]) {
      bidx[key] = n_buckets + ex[0];
      ord[n_buckets + ex[0]] = key;
    }
    n_buckets += tot[0];
  }
  __syncthreads();

  // ---- bucket starts, first segment and first descriptors of each bucket ----
  int n_lora = 0, n_seg = 0, n_large = 0, n_small = 0;
  for (int b0 = 0; b0 < n_buckets; b0 += BUILD_THREADS) {
    const int b = b0 + tid;
    int v[4] = {0, 0, 0, 0};
    if (b < n_buckets) {
      const int cnt = run[ord[b]];
      const int np = C > 0 ? (cnt + C - 1) / C : 1;
      const int last = C > 0 ? cnt - C * (np - 1) : cnt;
      int nl, ns, nl1, ns1;
      piece_tiles(C > 0 ? C : cnt, nl, ns);
      piece_tiles(last, nl1, ns1);
      v[0] = cnt;
      v[1] = np;
      v[2] = (np - 1) * nl + nl1;
      v[3] = (np - 1) * ns + ns1;
    }
    int ex[4], tot[4];
    block_scan<4>(v, ex, tot, s_w);
    if (b < n_buckets) {
      bstart[b] = n_lora + ex[0];
      pstart[b] = n_seg + ex[1];
      first[ord[b]] = n_large + ex[2];  // first[] is free after the bucket order
      sbase[b] = n_small + ex[3];
    }
    n_lora += tot[0];
    n_seg += tot[1];
    n_large += tot[2];
    n_small += tot[3];
  }
  if (tid == 0) {
    bstart[n_buckets] = n_lora;
    pstart[n_buckets] = n_seg;
  }
  const bool overflow = n_seg > seg_cap || n_large > large_cap || n_small > small_cap;
  __syncthreads();
  if (!overflow) {
    for (int b = tid; b < n_buckets; b += BUILD_THREADS) {
      const int lora = ord[b];
      write_bucket(lora, bstart[b + 1] - bstart[b], C, bstart[b], pstart[b], first[lora],
                   sbase[b], indptr, seg_lora, tiles, seg_cap, large_cap, small_cap);
    }
  }
  if (tid == 0) {
    if (!overflow) indptr[n_seg] = n_lora;
    info[0] = overflow ? 0 : n_seg;
    info[1] = overflow ? 0 : n_large;
    info[2] = overflow ? 0 : n_small;
    info[3] = overflow ? SGMV_ECAPACITY : (s_bad ? SGMV_EBADID : SGMV_OK);
  }

  // ---- pass 2: stable scatter ----
  __syncthreads();
  for (int b = tid; b < n_buckets; b += BUILD_THREADS) run[ord[b]] = bstart[b];
  if (tid == 0) run[L] = n_lora;
  __syncthreads();
  for (int rd = 0; rd < rounds; ++rd) {
    const int t = rd * BUILD_THREADS + tid;
    const bool valid = t < M;
    int key = 0;
    if (valid) {
      const int id = ids[t];
      key = (id < 0 || id >= L) ? L : id;
    }
    const int myrank = match_rank(valid, key, t, rc, nullptr, L);
    __syncthreads();
    int pre = 0, cw = 0, post = 0;
    if (valid) {
      wave_counts(rc, key, pre, cw, post);
      const int pos = run[key] + pre + myrank;
      if (pos < M) sorted[pos] = t;
      if (key < L && !overflow) {
        const int b = bidx[key];
        token_slot(t, pos - bstart[b], bstart[b + 1] - bstart[b], C, sbase[b], tiles, large_cap,
                   small_cap);
      }
    }
    __syncthreads();
    if (valid) {
      if (post == 0 && myrank == cw - 1) run[key] += pre + cw;
      rc[key * BUILD_WAVES + tid / WAVE] = 0;
    }
  }
}

hipError_t launch_build_segments(const int32_t* ids, int M, int L, int C, int32_t* sorted,
                                 int32_t* indptr, int32_t* seg_lora, int32_t* tiles,
                                 int32_t* info, int seg_cap, int large_cap, int small_cap,
                                 int32_t* xctl, int n_xctl, LaunchEvents ev,
                                 hipStream_t stream) {
  if (M <= BUILD_THREADS) {
#define SGMV_SMALL_BUILD(NW_)                                                                 \
  hipExtLaunchKernelGGL(build_segments_small_kernel<NW_>, dim3(1), dim3(NW_ * WAVE),         \
                        build_small_lds_bytes(L, NW_), stream, ev.start, ev.stop, 0, ids, M, \
                        L, C, sorted, indptr, seg_lora, tiles, info, seg_cap, large_cap,     \
                        small_cap, xctl, n_xctl)
    if (M <= 4 * WAVE) SGMV_SMALL_BUILD(4);
    else if (M <= 8 * WAVE) SGMV_SMALL_BUILD(8);
    else SGMV_SMALL_BUILD(16);
#undef SGMV_SMALL_BUILD
  } else {
    hipExtLaunchKernelGGL(build_segments_kernel, dim3(1), dim3(BUILD_THREADS),
                          build_lds_bytes(L), stream, ev.start, ev.stop, 0, ids, M, L, C, sorted,
                          indptr, seg_lora, tiles, info, seg_cap, large_cap, small_cap, xctl,
                          n_xctl);
  }
  return hipGetLastError();
}

}  // namespace sgmv
