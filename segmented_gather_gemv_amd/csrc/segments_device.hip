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
//    bucket size, segments, large and small descriptors) places every bucket; each token's
//    thread writes its sorted position and, if it starts a chunk or a piece, that entry;
//  * mid-size batches (up to 32768 tokens, tables within 64 KB of LDS): ids loaded once into
//    LDS, each wave walks its own contiguous range with a private row of per-key counts;
//  * larger batches: the same counting in rounds of 1024 tokens with a running count per
//    key, lanes of equal keys grouped by ballots.
// Every global write index is checked against its array bound. The kernels also clear the
// control words of the fused call's exchange workspace, when the segments carry one. Given a
// grouping cache, a kernel first compares the batch's ids (and M, L, C) with the cached ones
// and, if nothing changed, exits before writing anything: the segments already hold this
// build.
#include <climits>

#include "cache.h"
#include "segments_common.h"

namespace sgmv {

// ---------------------------------------------------------------------------------------
// grouping cache (Ascend article 4.2, 5.3): a build is skipped when the ids, M, L and C equal
// those of the last build made with the same cache
// ---------------------------------------------------------------------------------------
// True on every thread if the cache holds exactly this call's (M, L, C) and, for each token
// i < M handled by this thread, `differ` says whether ids[i] differs from the cached id.
__device__ __forceinline__ bool cache_unchanged(const int32_t* cache, int M, int L, int C,
                                                bool differ) {
  if (threadIdx.x == 0)
    differ = differ || cache[0] != CACHE_TAG || cache[1] != M || cache[2] != L || cache[3] != C;
  return !__syncthreads_or(differ);
}

__device__ __forceinline__ void cache_header(int32_t* cache, int M, int L, int C) {
  if (threadIdx.x == 0) {
    cache[0] = CACHE_TAG;
    cache[1] = M;
    cache[2] = L;
    cache[3] = C;
  }
}

// Strided compare of the whole batch (kernels that do not hold one token per thread).
template <int NT>
__device__ bool cache_hit(const int32_t* ids, int M, int L, int C, const int32_t* cache) {
  bool differ = false;
  for (int i = threadIdx.x; i < M; i += NT) differ |= ids[i] != cache[SGMV_CACHE_HEADER + i];
  return cache_unchanged(cache, M, L, C, differ);
}

// Stores the ids and header of this call's segment build; called once it is known to run.
template <int NT>
__device__ void cache_store(const int32_t* ids, int M, int L, int C, int32_t* cache) {
  for (int i = threadIdx.x; i < M; i += NT) cache[SGMV_CACHE_HEADER + i] = ids[i];
  cache_header(cache, M, L, C);
}

// ---------------------------------------------------------------------------------------
// small batches: M <= 1024
// ---------------------------------------------------------------------------------------
size_t build_small_lds_bytes(int L, int nw) {
  const size_t nk = (size_t)L + 1;
  return align16(nk * nw) + 4 * align16(nk * sizeof(int));
}

// One token per thread, NW waves (the fewest that cover M).
template <int NW>
__global__ __launch_bounds__(NW * WAVE) void build_segments_small_kernel(
    const int32_t* __restrict__ ids, int M, int L, int C, int32_t* __restrict__ sorted,
    int32_t* __restrict__ indptr, int32_t* __restrict__ seg_lora, int32_t* __restrict__ tiles,
    int32_t* __restrict__ info, int seg_cap, int large_cap, int small_cap,
    int32_t* __restrict__ xctl, int n_xctl, int32_t* __restrict__ cache) {
  constexpr int NT = NW * WAVE;
  extern __shared__ __align__(16) unsigned char smem[];
  const int NK = L + 1;
  uint8_t* rc = smem;                                                     // [NK][NW]
  int* s_base = reinterpret_cast<int*>(smem + align16((size_t)NK * NW));  // [NK]
  const size_t kstride = align16((size_t)NK * sizeof(int)) / sizeof(int);
  int* s_sbase = s_base + kstride;  // [NK] first small descriptor of each bucket
  int* s_seg0 = s_sbase + kstride;  // [NK] first segment
  int* s_lbase = s_seg0 + kstride;  // [NK] first large descriptor
  __shared__ __align__(16) int s_w[6 * NW];

  const int t = threadIdx.x, lane = t & (WAVE - 1), w = t / WAVE;
  const bool valid = t < M;
  const int raw = valid ? ids[t] : 0;
  if (cache != nullptr) {
    if (cache_unchanged(cache, M, L, C, valid && cache[SGMV_CACHE_HEADER + t] != raw)) return;
    if (valid) cache[SGMV_CACHE_HEADER + t] = raw;
    cache_header(cache, M, L, C);
  }
  for (int i = t; i < n_xctl; i += NT) xctl[i] = 0;
  for (int i = t; i < NK * (NW / 4); i += NT) reinterpret_cast<uint32_t*>(rc)[i] = 0;
  int key = -2;  // never equal to a real key (0..L)
  bool bad = false;
  if (valid) {
    int id = raw;
    if (id < -1 || id >= L) {
      bad = true;  // counted by the workgroup scan below
      id = -1;
    }
    key = id < 0 ? L : id;
  }
  // rank among equal keys of lower lanes, and the count in this wave
  uint64_t same = 0;
  if (w * WAVE < M) same = match_key(key, valid, L);  // uniform; waves without tokens skip it
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
  int v[6] = {0, 0, 0, 0, 0, bad ? 1 : 0};
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
  int ex[6], tot[6];
  block_scan<6, NW>(v, ex, tot, s_w);
  const int n_lora = tot[1], n_seg = tot[2], n_large = tot[3], n_small = tot[4];
  const bool overflow = n_seg > seg_cap || n_large > large_cap || n_small > small_cap;
  if (first) {
    s_base[key] = ex[1];
    s_sbase[key] = ex[4];
    s_seg0[key] = ex[2];
    s_lbase[key] = ex[3];
  }
  if (t == 0) {
    if (!overflow) indptr[n_seg] = n_lora;
    info[0] = overflow ? 0 : n_seg;
    info[1] = overflow ? 0 : n_large;
    info[2] = overflow ? 0 : n_small;
    info[3] = overflow ? SGMV_ECAPACITY : (tot[5] > 0 ? SGMV_EBADID : SGMV_OK);
    s_base[L] = n_lora;
  }
  __syncthreads();
  if (valid) {
    const int pos = s_base[key] + rank;
    if (pos < M) sorted[pos] = t;
    if (key < L && !overflow) {
      token_slot(t, rank, cnt, C, s_sbase[key], tiles, large_cap, small_cap);
      bucket_entries(key, rank, cnt, C, s_base[key], s_seg0[key], s_lbase[key], s_sbase[key],
                     indptr, seg_lora, tiles, seg_cap, large_cap, small_cap);
    }
  }
}

// Segment entries and piece records of every bucket, written by the whole workgroup: one
// thread per 16-byte quad of a record (a wave writes eight whole records) and one per segment,
// each finding its bucket by a binary search over the buckets' first record or segment.
// Per bucket b (in bucket order): bstart first sorted row (bstart[n_buckets] = the total),
// pstart first segment, lstart / sbase first large / small record, ord its adapter.
__device__ void write_entries_coop(int n_large, int n_small, int n_seg, int n_buckets,
                                   const int* bstart, const int* pstart, const int* lstart,
                                   const int* sbase, const int* ord, int C, int32_t* indptr,
                                   int32_t* seg_lora, int32_t* tiles, int large_cap) {
  const int tid = threadIdx.x;
  for (int idx = tid; idx < (n_large + n_small) * 8; idx += BUILD_THREADS) {
    const int rec = idx >> 3, q = idx & 7;
    const bool small = rec >= n_large;
    const int r = small ? rec - n_large : rec;
    const int b = last_at_most(small ? sbase : lstart, n_buckets, r);
    const int cnt_b = bstart[b + 1] - bstart[b];
    const PieceDesc pd = small ? small_piece_desc(r - sbase[b], C, cnt_b, bstart[b], pstart[b])
                               : large_piece_desc(r - lstart[b], C, cnt_b, bstart[b], pstart[b]);
    int4* d = reinterpret_cast<int4*>(tiles + (size_t)(small ? large_cap + r : r) *
                                                  SGMV_TILE_INTS) + q;
    if (q == 0) {
      *d = make_int4(ord[b], pd.start, pd.rows, pd.seg);
    } else if (q < 4) {
      *d = make_int4(0, 0, 0, 0);
    } else {  // token slots past the piece's rows; the others belong to the tokens' threads
      const int first_free = small ? pd.rows : 0, s0 = 4 * (q - 4);
      if (s0 >= first_free) {
        *d = make_int4(-1, -1, -1, -1);
      } else if (s0 + 4 > first_free) {
        int32_t* e = reinterpret_cast<int32_t*>(d);
        for (int i = first_free - s0; i < 4; ++i) e[i] = -1;
      }
    }
  }
  for (int sg = tid; sg < n_seg; sg += BUILD_THREADS) {
    const int b = last_at_most(pstart, n_buckets, sg);
    indptr[sg] = bstart[b] + (C > 0 ? (sg - pstart[b]) * C : 0);
    seg_lora[sg] = ord[b];
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
    int32_t* __restrict__ xctl, int n_xctl, int32_t* __restrict__ cache) {
  extern __shared__ __align__(16) unsigned char smem[];
  const int NK = L + 1;  // key L = "no adapter"
  uint8_t* rc = smem;
  int* run = reinterpret_cast<int*>(smem + align16((size_t)NK * BUILD_WAVES));
  const size_t stride = align16((size_t)(NK + 1) * sizeof(int)) / sizeof(int);
  int* first = run + stride;      // first token per adapter, then first large piece per bucket
  int* bidx = first + stride;     // bucket of each adapter
  int* ord = bidx + stride;       // adapter of each bucket
  int* bstart = ord + stride;     // first sorted row of each bucket
  int* pstart = bstart + stride;  // first segment of each bucket
  int* sbase = pstart + stride;   // first small descriptor of each bucket
  __shared__ __align__(16) int s_w[4 * BUILD_WAVES];
  __shared__ int s_bad;

  const int tid = threadIdx.x;
  if (cache != nullptr) {
    if (cache_hit<BUILD_THREADS>(ids, M, L, C, cache)) return;
    cache_store<BUILD_THREADS>(ids, M, L, C, cache);
  }
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
      first[b] = n_large + ex[2];  // first[] is free after the bucket order: large starts
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
  if (!overflow)
    write_entries_coop(n_large, n_small, n_seg, n_buckets, bstart, pstart, first, sbase, ord, C,
                       indptr, seg_lora, tiles, large_cap);
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

// ---------------------------------------------------------------------------------------
// mid-size batches: 1024 < M <= MID_MAX_M with every table in 64 KB of LDS
// ---------------------------------------------------------------------------------------
// All ids are loaded once into LDS. Each wave owns a contiguous range of tokens and a private
// row of per-key counts: pass 1 counts with LDS atomics (counts and first appearances do not
// depend on order), an exclusive scan over the waves turns the rows into per-wave starting
// ranks, and pass 2 walks each wave's range in rounds of 64, in order, placing the tokens. Buckets are ordered by first appearance through a
// bitmap of the tokens that appear first for their adapter and a prefix popcount over it.
constexpr int MID_MAX_M = 32768;

struct MidLds {
  size_t keys, hist, first, cnt, bidx, ord, bstart, pstart, sbase, lstart, bitmap, wpre, lanes,
      bytes;
};

__host__ __device__ inline MidLds mid_lds(int M, int L) {
  const size_t nk = (size_t)L + 1, nw = ((size_t)M + 31) / 32;
  MidLds m;
  size_t o = 0;
  m.keys = o;   o += align16((size_t)M * sizeof(uint16_t));
  m.hist = o;   o += align16(BUILD_WAVES * nk * sizeof(int));
  m.first = o;  o += align16(nk * sizeof(int));
  m.cnt = o;    o += align16(nk * sizeof(int));
  m.bidx = o;   o += align16(nk * sizeof(int));
  m.ord = o;    o += align16(nk * sizeof(int));
  m.bstart = o; o += align16((nk + 1) * sizeof(int));
  m.pstart = o; o += align16((nk + 1) * sizeof(int));
  m.sbase = o;  o += align16((nk + 1) * sizeof(int));
  m.lstart = o; o += align16((nk + 1) * sizeof(int));
  m.bitmap = o; o += align16(nw * sizeof(uint32_t));
  m.wpre = o;   o += align16(nw * sizeof(int));
  m.lanes = o;  o += BUILD_WAVES * WAVE * sizeof(int);
  m.bytes = o;
  return m;
}

// Lanes of a wave holding equal keys (valid lanes only): the lane's rank among lower lanes
// with its key, the size of its group, and whether it is the group's lowest lane. A wave
// whose lanes share one key (runs of one adapter) takes one ballot; otherwise every lane
// compares its key with the wave's 64 keys, staged in a per-wave row of LDS (s_k).
__device__ __forceinline__ void group_lanes(bool valid, int key, int* s_k, int& rank,
                                            int& size, bool& leader) {
  const int lane = threadIdx.x & (WAVE - 1);
  const uint64_t active = __ballot(valid);
  rank = size = 0;
  leader = false;
  if (!active) return;
  const int ld = __ffsll((unsigned long long)active) - 1;
  const int lkey = __builtin_amdgcn_readlane(key, ld);
  const uint64_t m0 = __ballot(valid && key == lkey);
  if (m0 == active) {  // uniform
    if (valid) {
      rank = __popcll(m0 & lanemask_lt(lane));
      size = __popcll(m0);
      leader = lane == ld;
    }
    return;
  }
  const int k = valid ? key : -1;  // no valid key is negative
  s_k[lane] = k;                   // read back by this wave only: LDS keeps the wave's order
  uint32_t lo = 0, hi = 0;  // bit j: lane j holds this lane's key
#pragma unroll
  for (int j4 = 0; j4 < WAVE; j4 += 4) {
    const int4 q = *reinterpret_cast<const int4*>(s_k + j4);
    const int kj[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int j = j4 + e;
      if (j < 32) lo |= kj[e] == k ? (1u << j) : 0u;
      else hi |= kj[e] == k ? (1u << (j - 32)) : 0u;
    }
  }
  const uint64_t same = ((uint64_t)hi << 32) | lo;
  if (valid) {
    rank = __popcll(same & lanemask_lt(lane));
    size = __popcll(same);
    leader = rank == 0;
  }
}

__global__ __launch_bounds__(BUILD_THREADS) void build_segments_mid_kernel(
    const int32_t* __restrict__ ids, int M, int L, int C, int32_t* __restrict__ sorted,
    int32_t* __restrict__ indptr, int32_t* __restrict__ seg_lora, int32_t* __restrict__ tiles,
    int32_t* __restrict__ info, int seg_cap, int large_cap, int small_cap,
    int32_t* __restrict__ xctl, int n_xctl, int32_t* __restrict__ cache) {
  extern __shared__ __align__(16) unsigned char smem[];
  const MidLds lay = mid_lds(M, L);
  const int NK = L + 1, nwords = (M + 31) / 32;
  uint16_t* keys = reinterpret_cast<uint16_t*>(smem + lay.keys);    // [M]
  int* hist = reinterpret_cast<int*>(smem + lay.hist);  // [16][NK] counts, then first ranks
  int* first = reinterpret_cast<int*>(smem + lay.first);            // [NK]
  int* cnt = reinterpret_cast<int*>(smem + lay.cnt);                // [NK]
  int* bidx = reinterpret_cast<int*>(smem + lay.bidx);              // [NK]
  int* ord = reinterpret_cast<int*>(smem + lay.ord);                // [NK]
  int* bstart = reinterpret_cast<int*>(smem + lay.bstart);          // [NK + 1]
  int* pstart = reinterpret_cast<int*>(smem + lay.pstart);          // [NK + 1]
  int* sbase = reinterpret_cast<int*>(smem + lay.sbase);            // [NK + 1]
  int* lstart = reinterpret_cast<int*>(smem + lay.lstart);          // [NK + 1]
  uint32_t* bitmap = reinterpret_cast<uint32_t*>(smem + lay.bitmap);  // [nwords]
  int* wpre = reinterpret_cast<int*>(smem + lay.wpre);              // [nwords]
  int* s_k = reinterpret_cast<int*>(smem + lay.lanes) + (threadIdx.x / WAVE) * WAVE;  // [64]
  __shared__ __align__(16) int s_w[4 * BUILD_WAVES];
  __shared__ int s_bad;

  const int tid = threadIdx.x, lane = tid & (WAVE - 1), w = tid / WAVE;
  if (cache != nullptr) {
    if (cache_hit<BUILD_THREADS>(ids, M, L, C, cache)) return;
    cache_store<BUILD_THREADS>(ids, M, L, C, cache);
  }
  for (int i = tid; i < n_xctl; i += BUILD_THREADS) xctl[i] = 0;
  for (int i = tid; i < BUILD_WAVES * NK; i += BUILD_THREADS) hist[i] = 0;
  for (int i = tid; i < NK; i += BUILD_THREADS) first[i] = INT_MAX;
  for (int i = tid; i < nwords; i += BUILD_THREADS) bitmap[i] = 0u;
  if (tid == 0) s_bad = 0;
  __syncthreads();
  // the ids into LDS: each thread's loads of a round are issued together (a row of loads past
  // M is skipped as a whole; the index clamped into [0, M)), so a round costs one memory round
  // trip
  constexpr int IPT = 16;
  for (int base = 0; base < M; base += IPT * BUILD_THREADS) {
    int v[IPT];
#pragma unroll
    for (int i = 0; i < IPT; ++i)
      v[i] = base + i * BUILD_THREADS < M ? ids[min(base + i * BUILD_THREADS + tid, M - 1)] : 0;
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
      const int t = base + i * BUILD_THREADS + tid;
      int id = v[i];
      if (t < M) {
        if (id < -1 || id >= L) {
          s_bad = 1;
          id = -1;
        }
        keys[t] = (uint16_t)(id < 0 ? L : id);
      }
    }
  }
  __syncthreads();

  // ---- pass 1: per-wave counts and first appearances (order-free: LDS atomics) ----
  const int chunk = (((M + BUILD_WAVES - 1) / BUILD_WAVES) + WAVE - 1) & ~(WAVE - 1);
  const int t0 = w * chunk, t1 = min(M, t0 + chunk);
  int* hw = hist + w * NK;
  for (int base = t0; base < t1; base += WAVE) {
    const int t = base + lane;
    const bool valid = t < t1;
    const int key = valid ? keys[t] : -1;
    const int k0 = __builtin_amdgcn_readfirstlane(key);  // lane 0 is always valid
    if (__ballot(valid && key == k0) == __ballot(valid)) {  // one key: one update
      if (lane == 0) {
        hw[k0] += min(WAVE, t1 - base);
        if (k0 < L) atomicMin(&first[k0], base);
      }
    } else if (valid) {
      atomicAdd(&hw[key], 1);
      if (key < L) atomicMin(&first[key], t);
    }
  }
  __syncthreads();

  // ---- per key: exclusive scan over the waves, total, first-appearance bit ----
  for (int k = tid; k < NK; k += BUILD_THREADS) {
    int run = 0;
    for (int v = 0; v < BUILD_WAVES; ++v) {
      const int c = hist[v * NK + k];
      hist[v * NK + k] = run;
      run += c;
    }
    cnt[k] = run;
    if (k < L && run > 0) atomicOr(&bitmap[first[k] >> 5], 1u << (first[k] & 31));
  }
  __syncthreads();

  // ---- bucket order: rank of each first appearance among all first appearances ----
  int n_buckets;
  {
    const int v[1] = {tid < nwords ? (int)__popc(bitmap[tid]) : 0};
    int ex[1], tot[1];
    block_scan<1>(v, ex, tot, s_w);  // nwords <= BUILD_THREADS
    if (tid < nwords) wpre[tid] = ex[0];
    n_buckets = tot[0];
  }
  __syncthreads();
  for (int k = tid; k < L; k += BUILD_THREADS) {
    if (cnt[k] > 0) {
      const int f = first[k];
      const int b = wpre[f >> 5] + __popc(bitmap[f >> 5] & ((1u << (f & 31)) - 1u));
      bidx[k] = b;
      ord[b] = k;
    }
  }
  __syncthreads();

  // ---- bucket starts, first segment and first descriptors of each bucket ----
  int n_lora = 0, n_seg = 0, n_large = 0, n_small = 0;
  for (int b0 = 0; b0 < n_buckets; b0 += BUILD_THREADS) {
    const int b = b0 + tid;
    int v[4] = {0, 0, 0, 0};
    if (b < n_buckets) {
      const int c = cnt[ord[b]];
      const int np = C > 0 ? (c + C - 1) / C : 1;
      const int last = C > 0 ? c - C * (np - 1) : c;
      int nl, ns, nl1, ns1;
      piece_tiles(C > 0 ? C : c, nl, ns);
      piece_tiles(last, nl1, ns1);
      v[0] = c;
      v[1] = np;
      v[2] = (np - 1) * nl + nl1;
      v[3] = (np - 1) * ns + ns1;
    }
    int ex[4], tot[4];
    block_scan<4>(v, ex, tot, s_w);
    if (b < n_buckets) {
      bstart[b] = n_lora + ex[0];
      pstart[b] = n_seg + ex[1];
      lstart[b] = n_large + ex[2];
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
    lstart[n_buckets] = n_large;
    sbase[n_buckets] = n_small;
  }
  const bool overflow = n_seg > seg_cap || n_large > large_cap || n_small > small_cap;
  __syncthreads();
  if (!overflow)
    write_entries_coop(n_large, n_small, n_seg, n_buckets, bstart, pstart, lstart, sbase, ord, C,
                       indptr, seg_lora, tiles, large_cap);
  if (tid == 0) {
    if (!overflow) indptr[n_seg] = n_lora;
    info[0] = overflow ? 0 : n_seg;
    info[1] = overflow ? 0 : n_large;
    info[2] = overflow ? 0 : n_small;
    info[3] = overflow ? SGMV_ECAPACITY : (s_bad ? SGMV_EBADID : SGMV_OK);
  }

  // ---- pass 2: every wave places its tokens, in token order ----
  for (int base = t0; base < t1; base += WAVE) {
    const int t = base + lane;
    const bool valid = t < t1;
    const int key = valid ? keys[t] : -1;
    int rank, size;
    bool leader;
    group_lanes(valid, key, s_k, rank, size, leader);
    if (valid) {
      const int b = key < L ? bidx[key] : 0;
      const int start = key < L ? bstart[b] : n_lora;
      const int pos = start + hw[key] + rank;
      if (pos < M) sorted[pos] = t;
      if (key < L && !overflow && sbase[b + 1] > sbase[b])  // the bucket has small pieces
        token_slot(t, pos - start, bstart[b + 1] - start, C, sbase[b], tiles, large_cap,
                   small_cap);
    }
    if (leader) hw[key] += size;  // after every lane has read it
  }
}

hipError_t launch_build_segments(const int32_t* ids, int M, int L, int C, int32_t* sorted,
                                 int32_t* indptr, int32_t* seg_lora, int32_t* tiles,
                                 int32_t* info, int seg_cap, int large_cap, int small_cap,
                                 int32_t* xctl, int n_xctl, int32_t* cache, LaunchEvents ev,
                                 hipStream_t stream) {
  if (M <= BUILD_THREADS) {
#define SGMV_SMALL_BUILD(NW_)                                                                 \
  hipExtLaunchKernelGGL(build_segments_small_kernel<NW_>, dim3(1), dim3(NW_ * WAVE),         \
                        build_small_lds_bytes(L, NW_), stream, ev.start, ev.stop, 0, ids, M, \
                        L, C, sorted, indptr, seg_lora, tiles, info, seg_cap, large_cap,     \
                        small_cap, xctl, n_xctl, cache)
    if (M <= 4 * WAVE) SGMV_SMALL_BUILD(4);
    else if (M <= 8 * WAVE) SGMV_SMALL_BUILD(8);
    else SGMV_SMALL_BUILD(16);
#undef SGMV_SMALL_BUILD
  } else if (M <= MID_MAX_M && mid_lds(M, L).bytes <= 65536) {
    hipExtLaunchKernelGGL(build_segments_mid_kernel, dim3(1), dim3(BUILD_THREADS),
                          mid_lds(M, L).bytes, stream, ev.start, ev.stop, 0, ids, M, L, C,
                          sorted, indptr, seg_lora, tiles, info, seg_cap, large_cap, small_cap,
                          xctl, n_xctl, cache);
  } else {
    hipExtLaunchKernelGGL(build_segments_kernel, dim3(1), dim3(BUILD_THREADS),
                          build_lds_bytes(L), stream, ev.start, ev.stop, 0, ids, M, L, C, sorted,
                          indptr, seg_lora, tiles, info, seg_cap, large_cap, small_cap, xctl,
                          n_xctl, cache);
  }
  return hipGetLastError();
}

}  // namespace sgmv
