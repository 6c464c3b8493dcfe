// libsgmv C-ABI: argument validation, launch geometry and dispatch. Stateless; every call
// runs on the caller's stream. Declarations and contracts are in include/sgmv.h.
#include <cmath>
#include <cstring>

#include "cache.h"
#include "common.h"
#include "segments_host.h"

namespace sgmv {
size_t build_lds_bytes(int L);
hipError_t launch_build_segments(const int32_t* ids, int M, int L, int C, int32_t* sorted,
                                 int32_t* indptr, int32_t* seg_lora, int32_t* tiles,
                                 int32_t* info, int seg_cap, int large_cap, int small_cap,
                                 int32_t* xctl, int n_xctl, int32_t* cache, LaunchEvents ev,
                                 hipStream_t stream);
hipError_t launch_pool_pack(const void* a_user, const void* b_user, const sgmv_pool& p,
                            bool fold_scale, hipStream_t stream);
hipError_t launch_delta_bf16(int mode, bool aligned, DeltaArgs A, LaunchEvents ev,
                             hipStream_t stream);
hipError_t launch_delta_f32(int mode, DeltaArgs A, LaunchEvents ev, hipStream_t stream);
hipError_t launch_delta_bf16_build(bool aligned, DeltaArgs A, LaunchEvents ev,
                                   hipStream_t stream);
hipError_t launch_merge(const void* w, int64_t ldw, void* w_out, int64_t ldo, const sgmv_pool& p,
                        int l, LaunchEvents ev, hipStream_t stream);

namespace {

inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }

bool pool_ok(const sgmv_pool* p) {
  if (!p || !p->a || !p->b || !p->rank || !p->scale) return false;
  if (p->L < 1 || p->R_max < 1 || p->K < 1 || p->N < 1) return false;
  if (p->dtype != SGMV_F32 && p->dtype != SGMV_BF16) return false;
  if (p->R_pad != round_up(p->R_max, 16) || p->K_pad != round_up(p->K, 32) ||
      p->N_pad != round_up(p->N, 32))
    return false;
  return true;
}

bool seg_ok(const sgmv_segments* s, int32_t M, int32_t L) {
  if (!s || !s->sorted_token_ids || !s->seg_indptr || !s->seg_lora_ids || !s->tiles || !s->info)
    return false;
  if (s->M != M || s->L != L || s->chunk_size < 0) return false;
  if ((reinterpret_cast<uintptr_t>(s->tiles) % 16) != 0) return false;
  int32_t sc, lc, smc;
  segment_capacities(M, L, s->chunk_size, &sc, &lc, &smc);
  if (s->seg_cap != sc || s->large_cap != lc || s->small_cap != smc) return false;
  return !s->exchange || (s->exchange_bytes >= exchange_layout(lc, smc).bytes &&
                          (reinterpret_cast<uintptr_t>(s->exchange) % 256) == 0);
}

inline bool aligned_to(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Validates the output slices and fills the slice part of the kernel arguments.
sgmv_status fill_slices(const sgmv_pool* p, int32_t M, const sgmv_slice* out, int32_t n_slices,
                        DeltaArgs& A, bool& aligned) {
  if (!out || n_slices < 1 || n_slices > SGMV_MAX_SLICES) return SGMV_EINVAL;
  int v = 0;
  for (int i = 0; i < n_slices; ++i) {
    const sgmv_slice& s = out[i];
    if (!s.y || s.n_len < 1 || s.n_begin < 0 || (int64_t)s.n_begin + s.n_len > p->N ||
        s.ldy < s.n_len)
      return SGMV_EINVAL;
    for (int j = 0; j < i; ++j) {  // pool column ranges must be disjoint
      const sgmv_slice& t = out[j];
      if (s.n_begin < t.n_begin + t.n_len && t.n_begin < s.n_begin + s.n_len) return SGMV_EINVAL;
    }
    A.slices[i].y = s.y;
    A.slices[i].ldy = s.ldy;
    A.slices[i].n_begin = s.n_begin;
    A.slices[i].v_begin = v;
    A.slices[i].n_len = s.n_len;
    if (s.n_len % 4 != 0 || s.ldy % 4 != 0 || !aligned_to(s.y, 8)) aligned = false;
    v += s.n_len;
  }
  for (int i = n_slices; i < SGMV_MAX_SLICES; ++i) {
    A.slices[i] = A.slices[0];
    A.slices[i].v_begin = 0x7fffffff;
  }
  A.n_slices = n_slices;
  A.v_total = v;
  (void)M;
  return SGMV_OK;
}

void fill_common(const sgmv_pool* p, const sgmv_segments* seg, DeltaArgs& A) {
  A.a = p->a;
  A.b = p->b;
  A.rank = p->rank;
  A.scale = p->scale;
  A.R_max = p->R_max;
  A.R_pad = p->R_pad;
  A.K = p->K;
  A.K_pad = p->K_pad;
  A.N_pad = p->N_pad;
  A.L = p->L;
  A.sorted = seg->sorted_token_ids;
  A.tiles = seg->tiles;
  A.info = seg->info;
  A.large_cap = seg->large_cap;
  A.small_cap = seg->small_cap;
}

// Column splits per work descriptor: enough workgroups to cover the chip for decode-like
// pieces, few enough that x rows and A are not re-read too often for prefill-like ones
// (every split of a piece recomputes its shrink unless the K-split exchange is on, in which
// case the splits share it and more of them pay). Caller overrides win.
void choose_splits(int v_total, int M, int L, bool exchange, const sgmv_launch_opts* opts,
                   DeltaArgs& A) {
  auto clamp = [](int v, int lo, int hi) { return v < lo ? lo : (v > hi ? hi : v); };
  const int ps = clamp(v_total / 1024, 1, exchange ? SGMV_EXCHANGE_MAX_SPLITS : 16);
  int pl = clamp(v_total / 2048, 1, 16);
  if (exchange) {
    // large pieces are long-running: keep their workgroups within what is resident at once
    // (two per CU); about M/64 pieces plus one ragged piece per segment
    const int pieces = M / SGMV_TILE_ROWS + (L < 64 ? L : 64);
    const int fit = (2 * 256) / (pieces > 0 ? pieces : 1);
    pl = clamp(v_total / 1024, 1, clamp(fit, 2, SGMV_EXCHANGE_MAX_SPLITS_LARGE));
  }
  A.n_split_small = (opts && opts->n_split_small > 0) ? opts->n_split_small : ps;
  A.n_split_large = (opts && opts->n_split_large > 0) ? opts->n_split_large : pl;
}

bool opts_ok(const sgmv_launch_opts* o) {
  return !o || (o->n_split_small >= 0 && o->n_split_small <= 64 && o->n_split_large >= 0 &&
                o->n_split_large <= 64 && o->exchange >= -1 && o->exchange <= 1 &&
                o->exchange_wait >= -1);
}

// Most column splits of a 16-row part that a large piece's partial slots hold: 8 when every
// partial row is 32 floats (ranks up to 32), else 4.
int part_splits_max(int R_pad) {
  return R_pad <= 32 ? SGMV_EXCHANGE_MAX_SPLITS : SGMV_EXCHANGE_MAX_SPLITS_LARGE;
}

// K-split exchange of a fused call, per piece class: needs the workspace and a split count
// in range (small pieces 2..8, large 2..4); by default also at least two 128-wide K steps per
// split, so that every workgroup has work of its own.
void choose_exchange(const sgmv_segments* seg, const sgmv_launch_opts* o, DeltaArgs& A) {
  const int want = o ? o->exchange : 0;
  auto on = [&](int P, int pmax) {
    bool v = want >= 0 && seg->exchange && P >= 2 && P <= pmax;
    if (v && want == 0) v = A.K >= 256 * P;
    return v;
  };
  A.xch_small = on(A.n_split_small, SGMV_EXCHANGE_MAX_SPLITS) ? 1 : 0;
  A.xch_large =
      on(A.n_split_large, A.rsplit > 1 ? part_splits_max(A.R_pad) : SGMV_EXCHANGE_MAX_SPLITS_LARGE)
          ? 1
          : 0;
  if (!A.xch_small && !A.xch_large) return;
  const ExchangeLayout x = exchange_layout(seg->large_cap, seg->small_cap);
  char* base = static_cast<char*>(seg->exchange);
  A.xctl = reinterpret_cast<int32_t*>(base);
  A.xpart_small = reinterpret_cast<float*>(base + x.small_off);
  A.xpart_large = reinterpret_cast<float*>(base + x.large_off);
  const int wait = o ? o->exchange_wait : 0;
  A.xwait = wait == 0 ? 2000 : (wait < 0 ? -1 : wait);
  A.xwait_large = A.xwait < 0 ? -1 : 10 * A.xwait;
}

LaunchEvents events_of(const sgmv_launch_opts* o) {
  LaunchEvents e;
  if (o) {
    e.start = static_cast<hipEvent_t>(o->start_event);
    e.stop = static_cast<hipEvent_t>(o->stop_event);
  }
  return e;
}

sgmv_status hip_status(hipError_t e) { return e == hipSuccess ? SGMV_OK : SGMV_EHIP; }

// `ids` (fused mode, bf16, 1 <= M <= SGMV_FUSED_BUILD_MAX_M only): the launch also builds
// the segments of seg from these device ids.
sgmv_status run_delta(int mode, const void* x, int64_t ldx, const float* h_in, float* h_out,
                      int64_t ldh, int32_t M, const sgmv_pool* pool, const sgmv_segments* seg,
                      const sgmv_slice* out, int32_t n_slices, const sgmv_launch_opts* opts,
                      void* stream, const int32_t* ids = nullptr) {
  if (M < 0 || !pool_ok(pool) || !opts_ok(opts)) return SGMV_EINVAL;
  if (pool->R_max > SGMV_MAX_RANK) return SGMV_EUNSUPPORTED;
  if (!seg_ok(seg, M, pool->L)) return SGMV_EINVAL;
  if (M == 0) {  // no-op; empty buffers may have null addresses
    if (mode != MODE_SHRINK && (!out || n_slices < 1 || n_slices > SGMV_MAX_SLICES))
      return SGMV_EINVAL;
    return SGMV_OK;
  }
  DeltaArgs A;
  std::memset(&A, 0, sizeof(A));
  bool aligned = true;
  if (mode != MODE_EXPAND) {
    if (!x || ldx < pool->K) return SGMV_EINVAL;
    A.x = x;
    A.ldx = ldx;
    if (pool->K % 8 != 0 || ldx % 8 != 0 || !aligned_to(x, 16)) aligned = false;
  }
  if (mode == MODE_SHRINK) {
    if (!h_out || ldh < pool->R_max) return SGMV_EINVAL;
    A.h = h_out;
    A.ldh = ldh;
  }
  if (mode == MODE_EXPAND) {
    if (!h_in || ldh < pool->R_max) return SGMV_EINVAL;
    A.h = const_cast<float*>(h_in);
    A.ldh = ldh;
  }
  if (mode != MODE_SHRINK) {
    const sgmv_status st = fill_slices(pool, M, out, n_slices, A, aligned);
    if (st != SGMV_OK) return st;
  } else {
    A.n_slices = 0;
    A.v_total = 0;
  }
  fill_common(pool, seg, A);
  A.rsplit = 1;
  if (mode == MODE_SHRINK) {
    A.n_split_large = A.n_split_small = 1;
  } else {
    const bool xch = mode == MODE_FUSED && pool->dtype == SGMV_BF16 && seg->exchange &&
                     !(opts && opts->exchange < 0);
    choose_splits(A.v_total, M, pool->L, xch, opts, A);
    // small batches: large pieces run as 16-row parts with the small pieces' column split
    // (few-adapter batches then spread over as many workgroups as 16-row chunks would give);
    // with the exchange, at most the splits a large piece's partial slots hold for parts
    if (mode == MODE_FUSED && pool->dtype == SGMV_BF16 && M <= SGMV_PART_SPLIT_MAX_M &&
        pool->R_pad <= 32) {
      A.rsplit = SGMV_TILE_ROWS / SGMV_SMALL_ROWS;
      // the small pieces' split; with the exchange (where more splits cost no extra reads of
      // x and A) up to about 128 part workgroups for a batch of one adapter (M / 16 parts)
      int pp = A.n_split_small;
      if (xch) {
        if (2048 / M > pp) pp = 2048 / M;
        if (pp > part_splits_max(pool->R_pad)) pp = part_splits_max(pool->R_pad);
      }
      if (!(opts && opts->n_split_large > 0)) A.n_split_large = pp;
    }
  }
  if (mode == MODE_FUSED && pool->dtype == SGMV_BF16) choose_exchange(seg, opts, A);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const LaunchEvents ev = events_of(opts);
  if (ids) {
    A.ids = ids;
    A.M = M;
    A.chunk = seg->chunk_size;
    A.seg_cap = seg->seg_cap;
    A.w_sorted = seg->sorted_token_ids;
    A.w_indptr = seg->seg_indptr;
    A.w_seg_lora = seg->seg_lora_ids;
    A.w_tiles = seg->tiles;
    A.w_info = seg->info;
    A.amajor = (seg->chunk_size == 0 && pool->L <= seg->small_cap) ? 1 : 0;
    // every adapter at the full rank of one tile: a small piece's A and B loads need
    // neither its rank nor its tokens and are issued first
    A.spec = (A.amajor && pool->R_pad == 16 && pool->rank_min == pool->R_pad) ? 1 : 0;
    // the in-launch build's kernels run large pieces only as 16-row parts
    if (A.rsplit != SGMV_TILE_ROWS / SGMV_SMALL_ROWS) return SGMV_EUNSUPPORTED;
    return hip_status(launch_delta_bf16_build(aligned, A, ev, s));
  }
  if (pool->dtype == SGMV_BF16) return hip_status(launch_delta_bf16(mode, aligned, A, ev, s));
  return hip_status(launch_delta_f32(mode, A, ev, s));
}

// Both builders; `cache` (may be null) as in sgmv_build_segments_cached.
sgmv_status build_segments(const int32_t* lora_indices, int32_t M, int32_t L, int32_t chunk_size,
                           int32_t on_device, const sgmv_segments* seg, int32_t* cache,
                           const sgmv_launch_opts* opts, void* stream) {
  if (M < 0 || L < 1 || chunk_size < 0 || (M > 0 && !lora_indices)) return SGMV_EINVAL;
  if (!seg || seg->chunk_size != chunk_size || !seg_ok(seg, M, L)) return SGMV_EINVAL;
  if (!opts_ok(opts)) return SGMV_EINVAL;
  if (on_device == 0) {
    if (cache) {
      if (cache[0] == CACHE_TAG && cache[1] == M && cache[2] == L && cache[3] == chunk_size &&
          (M == 0 ||
           std::memcmp(cache + SGMV_CACHE_HEADER, lora_indices, sizeof(int32_t) * M) == 0))
        return SGMV_OK;  // seg already holds these segments (only successful builds are cached)
      cache[0] = 0;  // a failed build leaves the cache empty
    }
    const int st = host_build_segments(lora_indices, M, L, chunk_size, seg->sorted_token_ids,
                                       seg->seg_indptr, seg->seg_lora_ids, seg->tiles, seg->info,
                                       seg->seg_cap, seg->large_cap, seg->small_cap);
    if (cache && st == SGMV_OK) {
      if (M > 0) std::memcpy(cache + SGMV_CACHE_HEADER, lora_indices, sizeof(int32_t) * M);
      cache[1] = M;
      cache[2] = L;
      cache[3] = chunk_size;
      cache[0] = CACHE_TAG;
    }
    return (sgmv_status)st;
  }
  if (L > SGMV_DEVICE_BUILDER_MAX_L) return SGMV_EUNSUPPORTED;
  int32_t* xctl = static_cast<int32_t*>(seg->exchange);
  const int n_xctl = xctl ? (seg->large_cap + seg->small_cap) * XCH_CTL_INTS : 0;
  return hip_status(launch_build_segments(lora_indices, M, L, chunk_size, seg->sorted_token_ids,
                                          seg->seg_indptr, seg->seg_lora_ids, seg->tiles,
                                          seg->info, seg->seg_cap, seg->large_cap, seg->small_cap,
                                          xctl, n_xctl, cache, events_of(opts),
                                          static_cast<hipStream_t>(stream)));
}

// The XCD (hardware register XCC_ID) of every workgroup of the grid, from its first lane.
__global__ void xcd_probe_kernel(int32_t* out) {
  const int xcc = __builtin_amdgcn_s_getreg((3 << 11) | 20);  // HW_REG_XCC_ID, bits 0..3
  if (threadIdx.x == 0) out[blockIdx.x] = xcc;
}

}  // namespace
}  // namespace sgmv

using namespace sgmv;

extern "C" {

const char* sgmv_status_string(sgmv_status s) {
  switch (s) {
    case SGMV_OK: return "SGMV_OK";
    case SGMV_EINVAL: return "SGMV_EINVAL: invalid argument";
    case SGMV_EBADID: return "SGMV_EBADID: adapter id outside {-1} U [0, L)";
    case SGMV_EUNSUPPORTED: return "SGMV_EUNSUPPORTED: outside the kernels' limits";
    case SGMV_ECAPACITY: return "SGMV_ECAPACITY: output array smaller than its bound";
    case SGMV_EHIP: return "SGMV_EHIP: HIP runtime error";
  }
  return "unknown sgmv_status";
}

int32_t sgmv_version(void) { return 100; }

sgmv_status sgmv_exchange_placement(int32_t* n_xcd, void* stream) {
  constexpr int G = 2048;
  int32_t* d = nullptr;
  if (hipMalloc(&d, G * sizeof(int32_t)) != hipSuccess) return SGMV_EHIP;
  hipStream_t s = static_cast<hipStream_t>(stream);
  xcd_probe_kernel<<<G, WAVE, 0, s>>>(d);
  int32_t h[G];
  hipError_t e = hipGetLastError();
  if (e == hipSuccess) e = hipMemcpyAsync(h, d, sizeof(h), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (hipFree(d) != hipSuccess && e == hipSuccess) e = hipErrorUnknown;
  if (e != hipSuccess) return SGMV_EHIP;
  int32_t most = 0;
  bool ok = true;
  for (int b = 0; b < G; ++b) {
    most = h[b] > most ? h[b] : most;
    ok = ok && h[b] == h[b % 8];
  }
  if (n_xcd) *n_xcd = most + 1;
  return ok ? SGMV_OK : SGMV_EUNSUPPORTED;
}

int32_t sgmv_chunk_size_for_batch(int32_t M, int32_t n_adapters) {
  if (M <= 0) return 0;
  if (M <= SGMV_FUSED_BUILD_MAX_M && n_adapters > 0 && M <= 8 * n_adapters) return 0;
  return M <= 1024 ? 16 : 0;
}

sgmv_status sgmv_pool_init(int32_t L, int32_t R_max, int32_t K, int32_t N, int32_t dtype,
                           sgmv_pool* pool, size_t* a_bytes, size_t* b_bytes) {
  if (!pool || !a_bytes || !b_bytes) return SGMV_EINVAL;
  if (L < 1 || R_max < 1 || K < 1 || N < 1 || L > 65535) return SGMV_EINVAL;
  if (dtype != SGMV_F32 && dtype != SGMV_BF16) return SGMV_EINVAL;
  if (R_max > SGMV_MAX_RANK) return SGMV_EUNSUPPORTED;
  std::memset(pool, 0, sizeof(*pool));
  pool->L = L;
  pool->R_max = R_max;
  pool->R_pad = (int32_t)round_up(R_max, 16);
  pool->K = K;
  pool->N = N;
  pool->K_pad = (int32_t)round_up(K, 32);
  pool->N_pad = (int32_t)round_up(N, 32);
  pool->dtype = dtype;
  const size_t e = dtype == SGMV_BF16 ? 2 : 4;
  *a_bytes = (size_t)L * pool->R_pad * pool->K_pad * e;
  *b_bytes = (size_t)L * pool->R_pad * pool->N_pad * e;
  return SGMV_OK;
}

sgmv_status sgmv_pool_pack_ex(const void* a_user, const void* b_user, const int32_t* rank,
                              const float* alpha, int32_t flags, sgmv_pool* pool, void* stream) {
  if (!a_user || !b_user || !rank || !alpha || !pool_ok(pool)) return SGMV_EINVAL;
  if ((flags & ~SGMV_PACK_FOLD_SCALE) != 0) return SGMV_EINVAL;
  const bool fold = (flags & SGMV_PACK_FOLD_SCALE) != 0;
  const int L = pool->L;
  float* scale = static_cast<float*>(std::malloc(sizeof(float) * (size_t)L));
  if (!scale) return SGMV_EINVAL;
  for (int l = 0; l < L; ++l) {
    if (rank[l] < 1 || rank[l] > pool->R_max || !std::isfinite(alpha[l])) {
      std::free(scale);
      return SGMV_EINVAL;
    }
    scale[l] = alpha[l] / (float)rank[l];
  }
  int32_t rmin = pool->R_max;
  for (int l = 0; l < L; ++l) rmin = rank[l] < rmin ? rank[l] : rmin;
  pool->rank_min = rmin;
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = hipMemcpyAsync(pool->rank, rank, sizeof(int32_t) * L, hipMemcpyHostToDevice, s);
  if (e == hipSuccess)
    e = hipMemcpyAsync(pool->scale, scale, sizeof(float) * L, hipMemcpyHostToDevice, s);
  // folding: B is packed with the true scales, then the stored scales become 1
  if (e == hipSuccess) e = launch_pool_pack(a_user, b_user, *pool, fold, s);
  if (e == hipSuccess && fold) {
    for (int l = 0; l < L; ++l) scale[l] = 1.f;
    e = hipMemcpyAsync(pool->scale, scale, sizeof(float) * L, hipMemcpyHostToDevice, s);
  }
  if (e == hipSuccess) e = hipStreamSynchronize(s);  // host staging buffers end here
  std::free(scale);
  if (e != hipSuccess) return SGMV_EHIP;
  pool->scale_folded = fold ? 1 : 0;
  return SGMV_OK;
}

sgmv_status sgmv_pool_pack(const void* a_user, const void* b_user, const int32_t* rank,
                           const float* alpha, sgmv_pool* pool, void* stream) {
  return sgmv_pool_pack_ex(a_user, b_user, rank, alpha, 0, pool, stream);
}

sgmv_status sgmv_segments_init(int32_t M, int32_t L, int32_t chunk_size, sgmv_segments* seg) {
  if (!seg || M < 0 || L < 1 || chunk_size < 0) return SGMV_EINVAL;
  seg->M = M;
  seg->L = L;
  seg->chunk_size = chunk_size;
  segment_capacities(M, L, chunk_size, &seg->seg_cap, &seg->large_cap, &seg->small_cap);
  seg->exchange_bytes = exchange_layout(seg->large_cap, seg->small_cap).bytes;
  return SGMV_OK;
}

sgmv_status sgmv_build_segments_ex(const int32_t* lora_indices, int32_t M, int32_t L,
                                   int32_t chunk_size, int32_t on_device,
                                   const sgmv_segments* seg, const sgmv_launch_opts* opts,
                                   void* stream) {
  return build_segments(lora_indices, M, L, chunk_size, on_device, seg, nullptr, opts, stream);
}

sgmv_status sgmv_build_segments_cached_ex(const int32_t* lora_indices, int32_t M, int32_t L,
                                          int32_t chunk_size, int32_t on_device,
                                          const sgmv_segments* seg, int32_t* cache,
                                          const sgmv_launch_opts* opts, void* stream) {
  if (!cache && M > 0) return SGMV_EINVAL;
  return build_segments(lora_indices, M, L, chunk_size, on_device, seg, cache, opts, stream);
}

sgmv_status sgmv_build_segments_cached(const int32_t* lora_indices, int32_t M, int32_t L,
                                       int32_t chunk_size, int32_t on_device,
                                       const sgmv_segments* seg, int32_t* cache, void* stream) {
  return sgmv_build_segments_cached_ex(lora_indices, M, L, chunk_size, on_device, seg, cache,
                                       nullptr, stream);
}

sgmv_status sgmv_build_segments(const int32_t* lora_indices, int32_t M, int32_t L,
                                int32_t chunk_size, int32_t on_device, const sgmv_segments* seg,
                                void* stream) {
  return sgmv_build_segments_ex(lora_indices, M, L, chunk_size, on_device, seg, nullptr, stream);
}

sgmv_status sgmv_shrink_ex(const void* x, int64_t ldx, int32_t M, const sgmv_pool* pool,
                           const sgmv_segments* seg, float* h, int64_t ldh,
                           const sgmv_launch_opts* opts, void* stream) {
  return run_delta(MODE_SHRINK, x, ldx, nullptr, h, ldh, M, pool, seg, nullptr, 0, opts, stream);
}

sgmv_status sgmv_shrink(const void* x, int64_t ldx, int32_t M, const sgmv_pool* pool,
                        const sgmv_segments* seg, float* h, int64_t ldh, void* stream) {
  return sgmv_shrink_ex(x, ldx, M, pool, seg, h, ldh, nullptr, stream);
}

sgmv_status sgmv_expand_ex(const float* h, int64_t ldh, int32_t M, const sgmv_pool* pool,
                           const sgmv_segments* seg, const sgmv_slice* out, int32_t n_slices,
                           const sgmv_launch_opts* opts, void* stream) {
  return run_delta(MODE_EXPAND, nullptr, 0, h, nullptr, ldh, M, pool, seg, out, n_slices, opts,
                   stream);
}

sgmv_status sgmv_expand(const float* h, int64_t ldh, int32_t M, const sgmv_pool* pool,
                        const sgmv_segments* seg, const sgmv_slice* out, int32_t n_slices,
                        void* stream) {
  return sgmv_expand_ex(h, ldh, M, pool, seg, out, n_slices, nullptr, stream);
}

sgmv_status sgmv_lora_delta_ex(const void* x, int64_t ldx, int32_t M, const sgmv_pool* pool,
                               const sgmv_segments* seg, const sgmv_slice* out,
                               int32_t n_slices, const sgmv_launch_opts* opts, void* stream) {
  return run_delta(MODE_FUSED, x, ldx, nullptr, nullptr, 0, M, pool, seg, out, n_slices, opts,
                   stream);
}

sgmv_status sgmv_lora_delta(const void* x, int64_t ldx, int32_t M, const sgmv_pool* pool,
                            const sgmv_segments* seg, const sgmv_slice* out, int32_t n_slices,
                            void* stream) {
  return sgmv_lora_delta_ex(x, ldx, M, pool, seg, out, n_slices, nullptr, stream);
}

sgmv_status sgmv_lora_delta_ids_ex(const int32_t* lora_indices, const void* x, int64_t ldx,
                                   int32_t M, const sgmv_pool* pool, const sgmv_segments* seg,
                                   const sgmv_slice* out, int32_t n_slices,
                                   const sgmv_launch_opts* opts, void* stream) {
  if (M < 0 || (M > 0 && !lora_indices) || !pool_ok(pool) || !opts_ok(opts)) return SGMV_EINVAL;
  if (!seg_ok(seg, M, pool->L)) return SGMV_EINVAL;
  // one launch where it measured faster than two: small bf16 batches whose ranks fit one
  // 16-rank tile (with wider ranks every workgroup's in-kernel grouping cost more than the
  // builder launch it saves)
  if (pool->dtype == SGMV_BF16 && M >= 1 && M <= SGMV_FUSED_BUILD_MAX_M &&
      pool->L <= SGMV_DEVICE_BUILDER_MAX_L && pool->R_pad == 16)
    return run_delta(MODE_FUSED, x, ldx, nullptr, nullptr, 0, M, pool, seg, out, n_slices, opts,
                     stream, lora_indices);
  // two launches: validate the delta's arguments first so that a bad call changes nothing
  if (M > 0 && (!x || ldx < pool->K)) return SGMV_EINVAL;
  if (!out || n_slices < 1 || n_slices > SGMV_MAX_SLICES) return SGMV_EINVAL;
  sgmv_launch_opts ob, od;
  std::memset(&ob, 0, sizeof(ob));
  std::memset(&od, 0, sizeof(od));
  if (opts) {
    od = *opts;
    ob.start_event = opts->start_event;
    od.start_event = nullptr;
  }
  const sgmv_status st = sgmv_build_segments_ex(lora_indices, M, pool->L, seg->chunk_size, 1,
                                                seg, &ob, stream);
  if (st != SGMV_OK) return st;
  return sgmv_lora_delta_ex(x, ldx, M, pool, seg, out, n_slices, &od, stream);
}

sgmv_status sgmv_merge_adapter_ex(const void* w, int64_t ldw, void* w_out, int64_t ldo,
                                  const sgmv_pool* pool, int32_t adapter,
                                  const sgmv_launch_opts* opts, void* stream) {
  if (!w || !w_out || !pool_ok(pool) || !opts_ok(opts)) return SGMV_EINVAL;
  if (adapter < 0 || adapter >= pool->L || ldw < pool->K || ldo < pool->K) return SGMV_EINVAL;
  return hip_status(launch_merge(w, ldw, w_out, ldo, *pool, adapter, events_of(opts),
                                 static_cast<hipStream_t>(stream)));
}

sgmv_status sgmv_merge_adapter(const void* w, int64_t ldw, void* w_out, int64_t ldo,
                               const sgmv_pool* pool, int32_t adapter, void* stream) {
  return sgmv_merge_adapter_ex(w, ldw, w_out, ldo, pool, adapter, nullptr, stream);
}

sgmv_status sgmv_lora_delta_ids(const int32_t* lora_indices, const void* x, int64_t ldx,
                                int32_t M, const sgmv_pool* pool, const sgmv_segments* seg,
                                const sgmv_slice* out, int32_t n_slices, void* stream) {
  return sgmv_lora_delta_ids_ex(lora_indices, x, ldx, M, pool, seg, out, n_slices, nullptr,
                                stream);
}

}  // extern "C"
