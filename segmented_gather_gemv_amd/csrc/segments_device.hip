// On-device segment builder: the same stable counting sort as the host builder, in one
// workgroup, with no host synchronisation (Ascend article 4.2: a per-step sort that syncs
// host and device sits on the critical path).
//
// One workgroup of 16 waves walks the tokens in rounds of 1024 (one 64-token chunk per
// wave). Inside a chunk, lanes holding the same key are grouped with ballots: the lowest
// lane leads, its group's size goes into a per-(key, wave) byte table in LDS, and each lane
// learns its rank among the equal keys of lower lanes. Across the waves of a round, the
// table gives each lane the count of equal keys in lower waves. A per-key running counter
// carries the count over rounds. Pass 1 counts keys and records where each adapter first
// appears; the bucket order (by first appearance), bucket starts, segment arrays and work
// descriptors follow from scans; pass 2 repeats the rounds and scatters every token to
// base[key] + (equal keys before it), which keeps tokens ascending inside a bucket.
#include <climits>

#include "common.h"

namespace sgmv {

constexpr int BUILD_THREADS = 1024;
constexpr int BUILD_WAVES = BUILD_THREADS / WAVE;

__host__ __device__ inline size_t align16(size_t v) { return (v + 15) & ~size_t(15); }

// Dynamic LDS bytes for a pool of L adapters.
size_t build_lds_bytes(int L) {
  const size_t nk = (size_t)L + 1;
  return align16(nk * BUILD_WAVES) + 6 * align16((nk + 1) * sizeof(int));
}

// Exclusive scan of one int per thread across the workgroup. s_w holds BUILD_WAVES + 1
// ints; on return *total is the sum. Contains barriers: call from all threads.
__device__ int block_exclusive_scan(int v, int* s_w, int* total) {
  const int lane = threadIdx.x & (WAVE - 1), w = threadIdx.x / WAVE;
  int x = v;
#pragma unroll
  for (int off = 1; off < WAVE; off <<= 1) {
    const int y = __shfl_up(x, off, WAVE);
    if (lane >= off) x += y;
  }
  if (lane == WAVE - 1) s_w[w] = x;
  __syncthreads();
  if (threadIdx.x == 0) {
    int acc = 0;
    for (int i = 0; i < BUILD_WAVES; ++i) {
      const int t = s_w[i];
      s_w[i] = acc;
      acc += t;
    }
    s_w[BUILD_WAVES] = acc;
  }
  __syncthreads();
  const int res = s_w[w] + x - v;
  *total = s_w[BUILD_WAVES];
  __syncthreads();
  return res;
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

// Counts of equal keys in lower waves (pre), in this wave (cw) and in higher waves (post).
__device__ inline void wave_counts(const uint8_t* rc, int key, int& pre, int& cw, int& post) {
  const int w = threadIdx.x / WAVE;
  const u32x4_t q = *reinterpret_cast<const u32x4_t*>(rc + key * BUILD_WAVES);
  pre = cw = post = 0;
#pragma unroll
  for (int i = 0; i < BUILD_WAVES; ++i) {
    const int v = (q[i >> 2] >> (8 * (i & 3))) & 0xff;
    if (i < w) pre += v;
    else if (i == w) cw = v;
    else post += v;
  }
}

__global__ __launch_bounds__(BUILD_THREADS) void build_segments_kernel(
    const int32_t* __restrict__ ids, int M, int L, int C, int32_t* __restrict__ sorted,
    int32_t* __restrict__ indptr, int32_t* __restrict__ seg_lora, int32_t* __restrict__ tiles,
    int32_t* __restrict__ info, int seg_cap, int large_cap, int small_cap) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int NK = L + 1;  // key L = "no adapter"
  uint8_t* rc = smem;
  int* run = reinterpret_cast<int*>(smem + align16((size_t)NK * BUILD_WAVES));
  const size_t stride = align16((size_t)(NK + 1) * sizeof(int)) / sizeof(int);
  int* first = run + stride;
  int* bidx = first + stride;
  int* ord = bidx + stride;
  int* bstart = ord + stride;
  int* pstart = bstart + stride;
  __shared__ int s_w[BUILD_WAVES + 1];
  __shared__ int s_bad;

  const int tid = threadIdx.x;
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
    const int flag = (t < M && key < L && first[key] == t) ? 1 : 0;
    int tot;
    const int ex = block_exclusive_scan(flag, s_w, &tot);
    if (flag) {
      bidx[key] = n_buckets + ex;
      ord[n_buckets + ex] = key;
    }
    n_buckets += tot;
  }
  __syncthreads();

  // ---- bucket starts and chunk counts ----
  int n_lora = 0, n_seg = 0;
  for (int b0 = 0; b0 < n_buckets; b0 += BUILD_THREADS) {
    const int b = b0 + tid;
    const int sz = b < n_buckets ? run[ord[b]] : 0;
    const int np = b < n_buckets ? (C > 0 ? (sz + C - 1) / C : 1) : 0;
    int tot1, tot2;
    const int e1 = block_exclusive_scan(sz, s_w, &tot1);
    const int e2 = block_exclusive_scan(np, s_w, &tot2);
    if (b < n_buckets) {
      bstart[b] = n_lora + e1;
      pstart[b] = n_seg + e2;
    }
    n_lora += tot1;
    n_seg += tot2;
  }
  if (tid == 0) {
    bstart[n_buckets] = n_lora;
    pstart[n_buckets] = n_seg;
  }
  const bool seg_overflow = n_seg > seg_cap;  // cannot happen with the stated capacities
  if (seg_overflow) n_seg = 0;
  __syncthreads();

  // ---- segment arrays ----
  for (int p = tid; p < n_seg; p += BUILD_THREADS) {
    int lo = 0, hi = n_buckets - 1;  // last bucket b with pstart[b] <= p
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (pstart[mid] <= p) lo = mid;
      else hi = mid - 1;
    }
    const int i = p - pstart[lo];
    indptr[p] = bstart[lo] + (C > 0 ? i * C : 0);
    seg_lora[p] = ord[lo];
  }
  if (tid == 0) indptr[n_seg] = seg_overflow ? 0 : n_lora;

  // ---- work descriptors ----
  int n_large = 0, n_small = 0;
  bool tile_overflow = false;
  for (int p0 = 0; p0 < n_seg; p0 += BUILD_THREADS) {
    const int p = p0 + tid;
    int nl = 0, ns = 0, start = 0, len = 0, lora = 0;
    if (p < n_seg) {
      int lo = 0, hi = n_buckets - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (pstart[mid] <= p) lo = mid;
        else hi = mid - 1;
      }
      const int i = p - pstart[lo];
      const int size = bstart[lo + 1] - bstart[lo];
      start = bstart[lo] + (C > 0 ? i * C : 0);
      len = C > 0 ? min(C, size - i * C) : size;
      lora = ord[lo];
      const int rem = len % SGMV_TILE_ROWS;
      nl = len / SGMV_TILE_ROWS + (rem > SGMV_SMALL_ROWS ? 1 : 0);
      ns = (rem > 0 && rem <= SGMV_SMALL_ROWS) ? 1 : 0;
    }
    int totl, tots;
    const int el = block_exclusive_scan(nl, s_w, &totl);
    const int es = block_exclusive_scan(ns, s_w, &tots);
    if (n_large + totl > large_cap || n_small + tots > small_cap) {
      tile_overflow = true;  // cannot happen with the stated capacities
      break;
    }
    for (int i = 0; i < nl; ++i) {
      int32_t* d = tiles + (size_t)(n_large + el + i) * 4;
      d[0] = lora;
      d[1] = start + i * SGMV_TILE_ROWS;
      d[2] = min(SGMV_TILE_ROWS, len - i * SGMV_TILE_ROWS);
      d[3] = p;
    }
    if (ns) {
      int32_t* d = tiles + (size_t)(large_cap + n_small + es) * 4;
      const int q = len / SGMV_TILE_ROWS;
      d[0] = lora;
      d[1] = start + q * SGMV_TILE_ROWS;
      d[2] = len - q * SGMV_TILE_ROWS;
      d[3] = p;
    }
    n_large += totl;
    n_small += tots;
  }
  if (tid == 0) {
    info[0] = n_seg;
    info[1] = tile_overflow ? 0 : n_large;
    info[2] = tile_overflow ? 0 : n_small;
    info[3] = (seg_overflow || tile_overflow) ? SGMV_ECAPACITY : (s_bad ? SGMV_EBADID : SGMV_OK);
  }

  // ---- pass 2: stable scatter ----
  for (int u = tid; u < L; u += BUILD_THREADS)
    if (first[u] != INT_MAX) run[u] = bstart[bidx[u]];
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
      sorted[run[key] + pre + myrank] = t;
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
                                 hipStream_t stream) {
  const size_t lds = build_lds_bytes(L);
  hipLaunchKernelGGL(build_segments_kernel, dim3(1), dim3(BUILD_THREADS), lds, stream, ids, M, L,
                     C, sorted, indptr, seg_lora, tiles, info, seg_cap, large_cap, small_cap);
  return hipGetLastError();
}

}  // namespace sgmv
