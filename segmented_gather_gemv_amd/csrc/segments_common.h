// Device helpers shared by the segment builders and the fused build + delta launch: the
// workgroup scan, per-wave key counts, descriptor counts of a segment, descriptor records and
// token slots, and the position of a piece inside its bucket. The counting sort itself is
// described in segments_device.hip.
#pragma once

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
// ints. Contains barriers: call from all threads. Without REUSE the final barrier, which
// lets a later call write s_w again, is left out.
template <int NV, int NW = BUILD_WAVES, bool REUSE = true>
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
  if (REUSE) __syncthreads();
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

constexpr int PARTS_PER_PIECE = SGMV_TILE_ROWS / SGMV_SMALL_ROWS;

// Parts of SGMV_SMALL_ROWS rows in the large pieces of a segment (chunk) of len rows: four per
// full piece, and ceil(rem / 16) for a ragged large piece.
__device__ __forceinline__ int large_parts(int len) {
  const int rem = len % SGMV_TILE_ROWS;
  return PARTS_PER_PIECE * (len / SGMV_TILE_ROWS) +
         (rem > SGMV_SMALL_ROWS ? (rem + SGMV_SMALL_ROWS - 1) / SGMV_SMALL_ROWS : 0);
}

// Large piece li (within the bucket) and part `sub` of the bucket's lp-th part. A chunk's large
// pieces come in row order, all but a ragged last one with four parts.
__device__ __forceinline__ void part_of(int lp, int C, int cnt, int& li, int& sub) {
  int chunk = 0, r = lp, nlf = 0;
  if (C > 0) {
    int nsf;
    piece_tiles(C, nlf, nsf);
    const int np = (cnt + C - 1) / C;
    const int pf = large_parts(C);
    chunk = (pf > 0 && lp < (np - 1) * pf) ? lp / pf : np - 1;
    r = lp - chunk * pf;
  }
  li = chunk * nlf + r / PARTS_PER_PIECE;
  sub = r % PARTS_PER_PIECE;
}

// The segment entries and piece records of one bucket (adapter `lora`, `cnt` rows from sorted
// row `start`, chunk size C), written by the bucket's own token threads (one token per
// thread): the first token of each chunk writes that segment's start and adapter, the first
// token of each piece writes the piece's record, with -1 in the token slots that the piece's
// tokens do not fill (those write their own ids, token_slot). A long bucket's hundreds of
// stores are spread over many waves instead of queueing behind one lane's store limit. `rank`
// is the token's rank in its bucket; seg0, lt and st are the bucket's first segment, large
// and small descriptor.
__device__ __forceinline__ void bucket_entries(int lora, int rank, int cnt, int C, int start,
                                               int seg0, int lt, int st, int32_t* indptr,
                                               int32_t* seg_lora, int32_t* tiles, int seg_cap,
                                               int large_cap, int small_cap) {
  const int i = C > 0 ? rank / C : 0;  // chunk (segment) inside the bucket
  const int in_seg = C > 0 ? rank - i * C : rank;
  if (in_seg % SGMV_TILE_ROWS != 0) return;
  const int len = C > 0 ? min(C, cnt - i * C) : cnt;
  const int s0 = start + (C > 0 ? i * C : 0);
  const int seg = seg0 + i;
  if (in_seg == 0 && seg < seg_cap) {
    indptr[seg] = s0;
    seg_lora[seg] = lora;
  }
  const int rows = min(SGMV_TILE_ROWS, len - in_seg);
  const bool small = rows <= SGMV_SMALL_ROWS;
  // every chunk before this one is full: nl_full large pieces and ns_full (0 or 1) small
  // ones each; inside a chunk only the last piece can be small
  int nl_full = 0, ns_full = 0;
  if (C > 0) piece_tiles(C, nl_full, ns_full);
  const int idx = small ? st + i * ns_full : lt + i * nl_full + in_seg / SGMV_TILE_ROWS;
  if (small ? idx >= small_cap : idx >= large_cap) return;
  int4* d = reinterpret_cast<int4*>(tiles + (size_t)(small ? large_cap + idx : idx) *
                                                SGMV_TILE_INTS);
  d[0] = make_int4(lora, s0 + in_seg, rows, seg);
  d[1] = d[2] = d[3] = make_int4(0, 0, 0, 0);
  const int first_free = small ? rows : 0;  // token slots past the piece's rows
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    if (4 * q >= first_free) {
      d[4 + q] = make_int4(-1, -1, -1, -1);
    } else if (4 * q + 4 > first_free) {
      int32_t* e = reinterpret_cast<int32_t*>(d + 4 + q);
      for (int k = first_free - 4 * q; k < 4; ++k) e[k] = -1;
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

// Largest b in [0, n) with a[b] <= x, for a non-decreasing a with a[0] <= x.
__device__ __forceinline__ int last_at_most(const int* a, int n, int x) {
  int lo = 0, hi = n - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a[mid] <= x) lo = mid;
    else hi = mid - 1;
  }
  return lo;
}

// First sorted row, rows and segment of one piece of a bucket of cnt rows that starts at
// sorted row `start` and segment `seg0` (chunk size C, 0 = no chunks). Pieces are numbered
// chunk by chunk, then by row within a chunk; every chunk holds at most one small piece.
struct PieceDesc {
  int start, rows, seg;
};

// li-th large piece (17..64 rows) of the bucket.
__device__ __forceinline__ PieceDesc large_piece_desc(int li, int C, int cnt, int start,
                                                      int seg0) {
  int chunk = 0, p = li;
  if (C > 0) {
    const int np = (cnt + C - 1) / C;
    int nlf, nsf;
    piece_tiles(C, nlf, nsf);  // large pieces of every chunk but the last
    if (nlf > 0 && li < (np - 1) * nlf) {
      chunk = li / nlf;
      p = li - chunk * nlf;
    } else {
      chunk = np - 1;
      p = li - (np - 1) * nlf;
    }
  }
  const int len = C > 0 ? min(C, cnt - chunk * C) : cnt;
  const int r0 = SGMV_TILE_ROWS * p;
  return PieceDesc{start + (C > 0 ? chunk * C : 0) + r0, min(SGMV_TILE_ROWS, len - r0),
                   seg0 + chunk};
}

// si-th small piece (1..16 rows) of the bucket: the tail of a chunk.
__device__ __forceinline__ PieceDesc small_piece_desc(int si, int C, int cnt, int start,
                                                      int seg0) {
  int chunk = 0;
  if (C > 0) {
    int nlf, nsf;
    piece_tiles(C, nlf, nsf);  // nsf: whether every full chunk ends in a small piece
    chunk = nsf ? si : (cnt + C - 1) / C - 1;
  }
  const int len = C > 0 ? min(C, cnt - chunk * C) : cnt;
  const int r0 = SGMV_TILE_ROWS * (len / SGMV_TILE_ROWS);
  return PieceDesc{start + (C > 0 ? chunk * C : 0) + r0, len - r0, seg0 + chunk};
}

// Lanes of this wave that hold the same key as this lane (keys 0..L; lanes with `valid`
// false are in no mask): one ballot per bit of the largest key, each lane keeping the lanes
// that agree with it on that bit.
__device__ __forceinline__ uint64_t match_key(int key, bool valid, int L) {
  uint64_t same = __ballot(valid);
  const int nb = 32 - __builtin_clz((unsigned)(L | 1));
  for (int b = 0; b < nb; ++b) {
    const bool bit = (key >> b) & 1;
    const uint64_t m = __ballot(bit);
    same &= bit ? m : ~m;
  }
  return same;
}

// Lanes of this wave's block of 64 tokens whose id is l. A full block is read with scalar
// loads (through the constant address space; the ids are read-only for the launch), whose
// latency does not queue behind the wave's vector loads; a partial block with one vector
// load per lane.
__device__ __forceinline__ uint64_t wave_adapter_mask(const int32_t* ids, int M, int l) {
  typedef const int32_t __attribute__((address_space(4))) cint;
  const int base = __builtin_amdgcn_readfirstlane((int)(threadIdx.x / WAVE)) * WAVE;
  const int n = M - base;
  uint64_t m = 0;
  if (n >= WAVE) {
    const cint* cp = (const cint*)(ids + base);
#pragma unroll
    for (int j = 0; j < WAVE; ++j) m |= (uint64_t)(cp[j] == l) << j;
  } else if (n > 0) {
    const int lane = threadIdx.x & (WAVE - 1);
    const int id = ids[base + (lane < n ? lane : 0)];
    m = __ballot(lane < n && id == l);
  }
  return m;
}

// The small piece of an adapter's bucket when there is no chunking: its last c % 64 tokens
// when that is 1..16 (c: the adapter's tokens), in token order, as the device builder makes
// it. Call from all threads of a workgroup of NW waves, each wave passing the mask of its
// block of 64 tokens whose id is the adapter's (ids past M never set); s_wc holds NW ints.
// Returns the piece's rows (0: no small piece; uniform) and writes its tokens to s_tok,
// visible after the caller's next barrier.
template <int NW>
__device__ __forceinline__ int adapter_small_piece(uint64_t m, int* s_wc, int* s_tok) {
  const int t = threadIdx.x, lane = t & (WAVE - 1), w = t / WAVE;
  const bool mine = (m >> lane) & 1u;
  if (lane == 0) s_wc[w] = __popcll(m);
  __syncthreads();
  int before = 0, c = 0;
#pragma unroll
  for (int i = 0; i < NW; ++i) {
    const int v = s_wc[i];
    c += v;
    before += i < w ? v : 0;
  }
  const int rem = c % SGMV_TILE_ROWS;
  const int rows = rem <= SGMV_SMALL_ROWS ? rem : 0;
  if (mine) {
    const int r = before + __popcll(m & lanemask_lt(lane)) - (c - rows);
    if (r >= 0) s_tok[r] = t;
  }
  return rows;
}

// ---------------------------------------------------------------------------------------
// In-workgroup segment build for the fused build + delta launch
// ---------------------------------------------------------------------------------------
// A workgroup of 8 waves, one token per thread (M <= 512), ranks the adapter ids exactly as
// the device builder does (buckets in order of first appearance, tokens ascending inside a
// bucket, ids -1 and bad ids last): every workgroup of the launch does it, then takes its own
// descriptor from the result without any global round trip. The `writer` workgroup also
// writes the segment arrays, records and info exactly as the builder does, so that later
// calls can use them.
constexpr int FUSED_BUILD_WAVES = 8;
constexpr int FUSED_BUILD_MAX_M = FUSED_BUILD_WAVES * WAVE;
static_assert(FUSED_BUILD_MAX_M == SGMV_FUSED_BUILD_MAX_M, "one token per thread");

struct WgBuildLds {
  uint8_t* rc;  // [L + 1][8] per-(key, wave) counts
  int* base;    // [L + 1] first sorted row of each bucket (L: the tail)
  int* sbase;   // [L + 1] first small descriptor of each bucket
  int* seg0;    // [L + 1] first segment of each bucket
  int* lbase;   // [L + 1] first large descriptor of each bucket
  int* w;       // [6 * 8] workgroup scan scratch
  int* rec;     // [6] this workgroup's piece or part: adapter, first row, rows, segment,
                // descriptor, part
};

inline size_t wg_build_lds_bytes(int L) {
  const size_t nk = (size_t)L + 1;
  return align16(nk * FUSED_BUILD_WAVES) + 4 * align16(nk * sizeof(int)) +
         align16(6 * FUSED_BUILD_WAVES * sizeof(int)) + align16(6 * sizeof(int));
}

__device__ __forceinline__ WgBuildLds wg_build_lds(unsigned char* p, int L) {
  const size_t nk = (size_t)L + 1;
  WgBuildLds s;
  s.rc = p;
  p += align16(nk * FUSED_BUILD_WAVES);
  s.base = reinterpret_cast<int*>(p);
  p += align16(nk * sizeof(int));
  s.sbase = reinterpret_cast<int*>(p);
  p += align16(nk * sizeof(int));
  s.seg0 = reinterpret_cast<int*>(p);
  p += align16(nk * sizeof(int));
  s.lbase = reinterpret_cast<int*>(p);
  p += align16(nk * sizeof(int));
  s.w = reinterpret_cast<int*>(p);
  p += align16(6 * FUSED_BUILD_WAVES * sizeof(int));
  s.rec = reinterpret_cast<int*>(p);
  return s;
}

struct WgBuildOut {
  int n_large, n_small;  // 0 when an array would overflow
  int tile;               // this workgroup's descriptor, -1 if none
  int sub;                // its 16-row part when large pieces run in parts (else 0)
  int lora, start, rows;  // of the descriptor, or of the part
};

struct WgBuildDst {  // the builder's outputs, written by the writer workgroup only
  int32_t *sorted, *indptr, *seg_lora, *tiles, *info;
  int seg_cap, large_cap, small_cap;
};

// Call from all 512 threads; thread t passes the id of token t (any value for t >= M). For
// descriptor `tile` of class `small` (a large piece's `tile` is its cyclic slot, dealt in
// blocks by blocked_tile once the count is known), returns the descriptor, its adapter, first
// sorted row and rows, and writes its token ids to s_tok. With `parts`, a large slot stands
// for one 16-row part of a large piece instead: the parts of the batch are numbered densely
// (bucket by bucket, piece by piece) and dealt in blocks like pieces, and the part's
// descriptor, part index, first row, rows and tokens are returned. Ends without a barrier:
// the caller's next barrier makes s_tok visible, and S may be written again only after it.
__device__ __forceinline__ WgBuildOut wg_build(int id, int M, int L, int C, bool small, int tile,
                                               bool parts, bool writer, const WgBuildDst& D,
                                               const WgBuildLds& S, int* s_tok) {
  constexpr int NW = FUSED_BUILD_WAVES;
  const int t = threadIdx.x, lane = t & (WAVE - 1), w = t / WAVE;
  const int NK = L + 1;
  const bool valid = t < M;
  for (int i = t; i < NK * (NW / 4); i += NW * WAVE) reinterpret_cast<uint32_t*>(S.rc)[i] = 0;
  int key = -2;  // never equal to a real key (0..L)
  bool bad = false;
  if (valid) {
    if (id < -1 || id >= L) {
      bad = true;
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
  if (valid && rk == 0) S.rc[key * NW + w] = (uint8_t)cw;
  __syncthreads();
  int pre = 0, cwt = 0, post = 0;
  if (valid) wave_counts<NW>(S.rc, key, pre, cwt, post);
  const int rank = pre + rk;
  const int cnt = pre + cwt + post;
  const bool first = valid && key < L && rank == 0;
  // per bucket, at its first token: tokens, segments, large and small descriptors; and the
  // bad-id count
  // and the large pieces' 16-row parts
  int v[6] = {0, 0, 0, 0, bad ? 1 : 0, 0};
  if (first) {
    const int np = C > 0 ? (cnt + C - 1) / C : 1;
    const int last = C > 0 ? cnt - C * (np - 1) : cnt;
    int nl, ns, nl1, ns1;
    piece_tiles(C > 0 ? C : cnt, nl, ns);
    piece_tiles(last, nl1, ns1);
    v[0] = cnt;
    v[1] = np;
    v[2] = (np - 1) * nl + nl1;
    v[3] = (np - 1) * ns + ns1;
    v[5] = C > 0 ? (np - 1) * large_parts(C) + large_parts(last) : large_parts(cnt);
  }
  int ex[6], tot[6];
  block_scan<6, NW, false>(v, ex, tot, S.w);
  const int n_lora = tot[0], n_seg = tot[1], n_large = tot[2], n_small = tot[3];
  const bool overflow = n_seg > D.seg_cap || n_large > D.large_cap || n_small > D.small_cap;
  const bool by_part = parts && !small;
  const int n_slots = overflow ? 0 : (small ? n_small : (by_part ? tot[5] : n_large));
  if (!small) tile = blocked_tile(tile, n_slots);
  if (first) {
    S.base[key] = ex[0];
    S.sbase[key] = ex[3];
    S.seg0[key] = ex[1];
    S.lbase[key] = ex[2];
    if (!overflow) {
      // this workgroup's descriptor (or part), if it belongs to this bucket
      const int first_d = small ? ex[3] : (by_part ? ex[5] : ex[2]);
      const int nd = small ? v[3] : (by_part ? v[5] : v[2]);
      if (tile >= first_d && tile < first_d + nd) {
        int li = tile - first_d, sub = 0;
        if (by_part) part_of(li, C, cnt, li, sub);
        const PieceDesc pd = small ? small_piece_desc(li, C, cnt, ex[0], ex[1])
                                   : large_piece_desc(li, C, cnt, ex[0], ex[1]);
        S.rec[0] = key;
        S.rec[1] = pd.start + SGMV_SMALL_ROWS * sub;
        S.rec[2] = by_part ? min(SGMV_SMALL_ROWS, pd.rows - SGMV_SMALL_ROWS * sub) : pd.rows;
        S.rec[3] = pd.seg;
        S.rec[4] = (small ? ex[3] : ex[2]) + li;
        S.rec[5] = sub;
      }
    }
  }
  if (t == 0) {
    S.base[L] = n_lora;
    if (writer) {
      if (!overflow) D.indptr[n_seg] = n_lora;
      D.info[0] = overflow ? 0 : n_seg;
      D.info[1] = overflow ? 0 : n_large;
      D.info[2] = overflow ? 0 : n_small;
      D.info[3] = overflow ? SGMV_ECAPACITY : (tot[4] > 0 ? SGMV_EBADID : SGMV_OK);
    }
  }
  __syncthreads();
  WgBuildOut out;
  out.n_large = overflow ? 0 : n_large;
  out.n_small = overflow ? 0 : n_small;
  const bool mine = tile >= 0 && tile < n_slots;
  out.tile = mine ? S.rec[4] : -1;
  out.sub = mine ? S.rec[5] : 0;
  out.lora = mine ? S.rec[0] : 0;
  out.start = mine ? S.rec[1] : 0;
  out.rows = mine ? S.rec[2] : 0;
  if (valid) {
    const int pos = S.base[key] + rank;
    if (key < L && pos >= out.start && pos < out.start + out.rows) s_tok[pos - out.start] = t;
    if (writer) {
      if (pos < M) D.sorted[pos] = t;
      if (key < L && !overflow) {
        token_slot(t, rank, cnt, C, S.sbase[key], D.tiles, D.large_cap, D.small_cap);
        bucket_entries(key, rank, cnt, C, S.base[key], S.seg0[key], S.lbase[key],
                       S.sbase[key], D.indptr, D.seg_lora, D.tiles, D.seg_cap, D.large_cap,
                       D.small_cap);
      }
    }
  }
  return out;
}

}  // namespace sgmv
