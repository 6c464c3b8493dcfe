// bf16 multi-LoRA delta on gfx950 matrix cores (device code; instantiated by
// delta_bf16_fused.hip and delta_bf16_unfused.hip).
//
// One workgroup (8 waves) takes one work descriptor -- a piece of at most 64 rows of one
// segment, i.e. of one adapter (Ascend article 3.3: start row, row count, adapter) -- and
// one range of output columns:
//
//   shrink  h[rows, r] = x[rows, :] @ A[l, :r, :]^T            (Ascend article 3.2)
//   expand  y[rows, cols] += scale_l * h @ B[l, cols, :r]^T    (second stage, scatter-add)
//
// Rows are gathered through the sorted token ids (Punica page, code section). Both
// contractions run on v_mfma_f32_16x16x32_bf16 with fp32 accumulation. In the fused kernel
// h never leaves the workgroup (Ascend article 4.3): the shrink's partial tiles are reduced
// in LDS, scaled, and split into hi + lo bf16 parts, so the expand keeps about 16
// significant bits of the fp32 h rather than 8.
//
// The path is bound by memory latency and bandwidth, not by the matrix cores, so the work is
// arranged to keep many loads in flight and few dependent memory round trips:
//  * the workgroup -> (piece, column split) map needs no device data: pieces are dealt
//    round-robin to the 8 XCDs (workgroup i runs on XCD i % 8) and all column splits of a
//    piece run on one XCD, sharing x rows and A through its L2;
//  * one round of loads brings the piece record (with the token ids of a small piece), the
//    piece counts and the pool's rank/scale table (into LDS);
//  * small pieces (<= 16 rows, decode) split K eight ways, one slice per wave, and issue all
//    shrink loads together with the expand's B and y loads before the first MFMA;
//  * large pieces (prefill) cover up to four row tiles x two K slices and stream K.
//
// Operand layouts. A K step of 128 is four MFMAs of 32: for MFMA i, lane (c, g) of a wave
// loads the 16 bytes of x row c and of A rank row c at k = 32 i + 8 g, so the four lanes of a
// row read 64 contiguous bytes in one instruction. In the expand, the contraction over rank
// runs in tiles of 32 ranks: lane (c, g) loads rank octet g of the tile (B is stored in rank
// octets, [l][j/8][n][8], so one 16-byte load is one operand fragment), once; the hi and lo
// parts of h go through two MFMAs on that fragment. MFMA q of a 64-column group covers
// column 4 c + q for lane column c, so a lane's four accumulators are four adjacent columns
// of one output row and y moves 8 bytes per lane access.
#pragma once

#include "common.h"
#include "segments_common.h"

namespace sgmv {

// Phase stamps, for profiling builds only (libsgmv_stamps.so). With SGMV_PHASE_STAMPS defined,
// thread 0 of each of the first STAMP_WGS workgroups records the 100 MHz real-time counter at
// the phase points of a small piece into slot k of its row; sgmv_phase_stamps reads the array
// back. Without it (the library itself) the macros are empty and no stamp code is compiled.
#ifdef SGMV_PHASE_STAMPS
constexpr int STAMP_WGS = 8192, STAMP_SLOTS = 16;
static __device__ uint64_t g_phase_stamps[STAMP_WGS * STAMP_SLOTS];
#define SGMV_STAMP(k)                                                                   \
  do {                                                                                  \
    if (threadIdx.x == 0 && blockIdx.x < STAMP_WGS)                                     \
      g_phase_stamps[blockIdx.x * STAMP_SLOTS + (k)] = __builtin_amdgcn_s_memrealtime(); \
  } while (0)
// stamp k once the wave-uniform value v is in its scalar registers
#define SGMV_STAMP_AFTER(k, v)                                      \
  do {                                                              \
    if (threadIdx.x == 0) asm volatile("" ::"s"(v));                \
    SGMV_STAMP(k);                                                  \
  } while (0)
// stamp k after every store of the workgroup has completed
#define SGMV_STAMP_DRAINED(k)        \
  do {                               \
    __builtin_amdgcn_s_waitcnt(0);   \
    __syncthreads();                 \
    SGMV_STAMP(k);                   \
  } while (0)
#else
#define SGMV_STAMP(k) \
  do {                \
  } while (0)
#define SGMV_STAMP_AFTER(k, v) \
  do {                         \
  } while (0)
#define SGMV_STAMP_DRAINED(k) \
  do {                        \
  } while (0)
#endif

constexpr int DT_THREADS = 512;
constexpr int DT_WAVES = DT_THREADS / WAVE;
constexpr int KSTEP = 128;
constexpr int HS = 68;                // LDS row stride of the h tile (64 ranks + 4 pad floats)
constexpr int RANK_TABLE_MAX = 1024;  // pools up to this size get rank/scale staged in LDS
// LDS-staged large shrink: K chunks of 64, each a 64-row x tile and a 64-rank A tile (8 KB
// each) brought in by direct global-to-LDS loads into a ring of STAGES buffers at the start
// of the dynamic LDS, STAGES - 1 chunks in flight
constexpr int STAGE_BYTES = 16384;
constexpr int STAGES = 4;
// The h tile (64 rows of HS floats) lives in the dynamic LDS too, over the ring's last buffer
// (a staged shrink writes it only once its last chunk is consumed): the dynamic part holds
// the ring and the tile in 65 KB, and with the static part two workgroups still fit a CU.
constexpr int SH_OFFSET = (STAGES - 1) * STAGE_BYTES;
constexpr int SH_BYTES = SGMV_TILE_ROWS * HS * 4;
static_assert(SH_BYTES >= STAGE_BYTES, "the h tile covers the ring's last buffer");

struct Piece {
  int lora, start, rows, r;
  float scale;
  int v0, v1;         // column range, in the concatenation of the output slices
  int tile, split, nsplit;  // descriptor index in its class, column split and split count
  int xsub;  // part index when a large piece runs as 16-row parts (its exchange is the
             // large class's), else -1
};

// Where concatenated output column v lives: its slice's y, row stride, y column, pool column.
struct ColMap {
  uint16_t* y;
  int64_t ldy;
  int col, n;
};

__device__ __forceinline__ ColMap map_column(const DeltaArgs& A, int v) {
  ColMap m{static_cast<uint16_t*>(A.slices[0].y), A.slices[0].ldy, v, A.slices[0].n_begin + v};
#pragma unroll
  for (int i = 1; i < SGMV_MAX_SLICES; ++i) {
    if (i < A.n_slices && v >= A.slices[i].v_begin) {
      m.y = static_cast<uint16_t*>(A.slices[i].y);
      m.ldy = A.slices[i].ldy;
      m.col = v - A.slices[i].v_begin;
      m.n = A.slices[i].n_begin + m.col;
    }
  }
  return m;
}

template <bool ALIGNED>
__device__ __forceinline__ void map_group(const DeltaArgs& A, int vl, ColMap (&cm)[4]) {
  cm[0] = map_column(A, vl);
#pragma unroll
  for (int q = 1; q < 4; ++q) {
    if (ALIGNED) {  // a 4-column group never straddles slices
      cm[q] = cm[0];
      cm[q].col += q;
      cm[q].n += q;
    } else {
      cm[q] = map_column(A, vl + q);
    }
  }
}

// 8 bf16 of an x row starting at k (zeros past K or for an absent row).
template <bool ALIGNED>
__device__ __forceinline__ u32x4_t load_x8(const uint16_t* xr, int k, int K, bool valid) {
  u32x4_t v = {0u, 0u, 0u, 0u};
  if (!valid) return v;
  if (ALIGNED) {
    if (k < K) v = load_u32x4(xr + k);
  } else {
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const uint32_t lo = (k + e < K) ? xr[k + e] : 0u;
      const uint32_t hi = (k + e + 1 < K) ? xr[k + e + 1] : 0u;
      v[e >> 1] = lo | (hi << 16);
    }
  }
  return v;
}

// B fragments of the four columns of a lane for NE rank tiles of 32: lane group g holds rank
// octet 4 re + g. Zero past the adapter's rank and past the column range.
template <int NE>
__device__ __forceinline__ void load_b_group(const uint16_t* bb, int N_pad, int r, int vl,
                                             int v1, int g, const ColMap (&cm)[4],
                                             u32x4_t (&bq)[NE][4]) {
#pragma unroll
  for (int re = 0; re < NE; ++re) {
    const int o = re * 4 + g;
    const int live = r - 8 * o;  // live ranks in this octet
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      bq[re][q] = (live > 0 && vl + q < v1) ? load_u32x4(bb + ((size_t)o * N_pad + cm[q].n) * 8)
                                             : u32x4_t{0u, 0u, 0u, 0u};
      if (live > 0 && live < 8) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (e >= live) bq[re][q][e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
      }
    }
  }
}

// yacc[q] += h_hi @ B + h_lo @ B over NE rank tiles of 32.
template <int NE>
__device__ __forceinline__ void expand_mfma(const bf16x8_t (&P)[NE][2],
                                            const u32x4_t (&bq)[NE][4], f32x4_t (&yacc)[4]) {
#pragma unroll
  for (int re = 0; re < NE; ++re)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      yacc[q] = mfma_16x16x32_bf16(P[re][0], as_bf16x8(bq[re][q]), yacc[q]);
      yacc[q] = mfma_16x16x32_bf16(P[re][1], as_bf16x8(bq[re][q]), yacc[q]);
    }
}

// Old y of rows 4g..4g+3 of row tile rt at this lane's four columns (aligned path). NT: the
// loads are marked non-temporal (y is read once and rewritten; the caches keep A and B).
template <bool ALIGNED, bool NT = false>
__device__ __forceinline__ void load_y(const int* s_tok, int rows, int rt, int g, int vl, int v1,
                                       const ColMap (&cm)[4], uint2 (&yv)[4]) {
  // the four rows' tokens in one 16-byte LDS read (s_tok is 16-byte aligned)
  const int4 tk = *reinterpret_cast<const int4*>(s_tok + rt * 16 + 4 * g);
  const int toks[4] = {tk.x, tk.y, tk.z, tk.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int row = rt * 16 + 4 * g + e;
    yv[e] = make_uint2(0u, 0u);
    if (ALIGNED && row < rows && vl < v1) {
      const uint2* p =
          reinterpret_cast<const uint2*>(cm[0].y + (size_t)toks[e] * (size_t)cm[0].ldy + cm[0].col);
      if constexpr (NT) {
        const u32x2_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x2_t*>(p));
        yv[e] = make_uint2(t.x, t.y);
      } else {
        yv[e] = *p;
      }
    }
  }
}

// y update of one row tile: yv holds the old values (aligned path), yacc the delta. NT: the
// aligned path's stores are marked non-temporal.
template <bool ALIGNED, bool NT = false>
__device__ __forceinline__ void store_y(const int* s_tok, int rows, int rt, int g, int vl, int v1,
                                        const ColMap (&cm)[4], const uint2 (&yv)[4],
                                        const f32x4_t (&yacc)[4]) {
  const int4 tk = *reinterpret_cast<const int4*>(s_tok + rt * 16 + 4 * g);
  const int toks[4] = {tk.x, tk.y, tk.z, tk.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int row = rt * 16 + 4 * g + e;
    if (row >= rows) continue;
    const size_t tok = (size_t)toks[e];
    if (ALIGNED) {
      if (vl >= v1) continue;
      uint16_t* yp = cm[0].y + tok * (size_t)cm[0].ldy + cm[0].col;
      uint2 v = yv[e];
      const float d0 = bf16_bits_to_f32(v.x & 0xffffu) + yacc[0][e];
      const float d1 = bf16_bits_to_f32(v.x >> 16) + yacc[1][e];
      const float d2 = bf16_bits_to_f32(v.y & 0xffffu) + yacc[2][e];
      const float d3 = bf16_bits_to_f32(v.y >> 16) + yacc[3][e];
      v.x = pack_bf16x2(d0, d1);
      v.y = pack_bf16x2(d2, d3);
      if constexpr (NT) {
        u32x2_t t;
        t.x = v.x;
        t.y = v.y;
        __builtin_nontemporal_store(t, reinterpret_cast<u32x2_t*>(yp));
      } else {
        *reinterpret_cast<uint2*>(yp) = v;
      }
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (vl + q >= v1) continue;
        uint16_t* yp = cm[q].y + tok * (size_t)cm[q].ldy + cm[q].col;
        *yp = (uint16_t)pack_bf16x2(bf16_bits_to_f32(*yp) + yacc[q][e], 0.f);
      }
    }
  }
}

// Sums the partial h tiles of the K slices (s_part, [wave][rank tile][16][16]) into s_h,
// multiplied by `mult`; columns >= r are 0. nrt row tiles, ntp row tiles per K slice.
template <int NRK>
__device__ void reduce_partials(int nrt, int ntp, int ks, int r, float mult, const float* s_part,
                                float* s_h) {
  const int ncol = (NRK + 1) / 2 * 32, nrow = nrt * 16;  // whole 32-rank expand tiles
  for (int idx = threadIdx.x; idx < nrow * ncol; idx += DT_THREADS) {
    const int row = idx / ncol, j = idx - row * ncol;
    const int rtt = row >> 4, rr = row & 15, rk = j >> 4, cc = j & 15;
    float s = 0.f;
    if (j < r)
      for (int q = 0; q < ks; ++q) s += s_part[(((q * ntp + rtt) * NRK + rk) * 16 + rr) * 16 + cc];
    s_h[row * HS + j] = s * mult;
  }
}

// hi and lo bf16 parts of 8 consecutive h values (16-byte aligned in LDS): hi = rne(h),
// lo = rne(h - hi), so hi + lo keeps about 16 significant bits of h.
__device__ __forceinline__ void split_hi_lo(const float* hp, u32x4_t& hi, u32x4_t& lo) {
  const float4 a = *reinterpret_cast<const float4*>(hp);
  const float4 b = *reinterpret_cast<const float4*>(hp + 4);
  const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    const uint32_t h2 = pack_bf16x2(v[e], v[e + 1]);
    hi[e >> 1] = h2;
    lo[e >> 1] = pack_bf16x2(v[e] - bf16_bits_to_f32(h2 & 0xffffu), v[e + 1] - bf16_bits_to_f32(h2 >> 16));
  }
}

// hi and lo bf16 operand fragments of the h tile into s_pf ([row tile][rank tile of 32][hi,
// lo][lane], 16 B each). Lane (c, g) of fragment (rt, re) holds row rt*16 + c, ranks
// re*32 + 8g + 0..7; the lo part is h - hi, rounded, so hi + lo keeps about 16 bits of h.
template <int NE>
__device__ void build_fragments(int nrt, const float* s_h, u32x4_t* s_pf) {
  const int w = threadIdx.x / WAVE, lane = threadIdx.x & (WAVE - 1);
  const int c = lane & 15, g = lane >> 4;
  for (int f = w; f < nrt * NE; f += DT_WAVES) {
    const int rt = f / NE, re = f - rt * NE;
    u32x4_t hi, lo;
    split_hi_lo(s_h + (rt * 16 + c) * HS + re * 32 + 8 * g, hi, lo);
    s_pf[(2 * f) * WAVE + lane] = hi;
    s_pf[(2 * f + 1) * WAVE + lane] = lo;
  }
}

template <int NE>
__device__ __forceinline__ void read_fragments(const u32x4_t* s_pf, int rt, int lane,
                                               bf16x8_t (&P)[NE][2]) {
#pragma unroll
  for (int re = 0; re < NE; ++re) {
    P[re][0] = as_bf16x8(s_pf[(2 * (rt * NE + re)) * WAVE + lane]);
    P[re][1] = as_bf16x8(s_pf[(2 * (rt * NE + re) + 1) * WAVE + lane]);
  }
}

// The same hi and lo fragments straight from the h tile, for a wave that needs them once.
template <int NE>
__device__ __forceinline__ void h_fragments(const float* s_h, int rt, int lane,
                                            bf16x8_t (&P)[NE][2]) {
  const int c = lane & 15, g = lane >> 4;
#pragma unroll
  for (int re = 0; re < NE; ++re) {
    u32x4_t hi, lo;
    split_hi_lo(s_h + (rt * 16 + c) * HS + re * 32 + 8 * g, hi, lo);
    P[re][0] = as_bf16x8(hi);
    P[re][1] = as_bf16x8(lo);
  }
}

// NSTEP K steps of x and A for one wave (a row tile of 16 rows): loads, then MFMAs.
template <int NRK, int NSTEP, bool ALIGNED>
struct ShrinkSteps {
  u32x4_t xv[NSTEP][4], av[NSTEP][NRK][4];
  __device__ __forceinline__ void load(const uint16_t* xr, bool vx, const uint16_t* ab,
                                       int K_pad, int K, int r, int ch, int c1, int c, int g) {
#pragma unroll
    for (int st = 0; st < NSTEP; ++st) {
      const bool live = ch + st < c1;
      const int kb = (ch + st) * KSTEP + 8 * g;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int k = kb + 32 * i;  // instruction i: 64 contiguous bytes of each row
        xv[st][i] = load_x8<ALIGNED>(xr, k, K, vx && live);
#pragma unroll
        for (int rk = 0; rk < NRK; ++rk) {
          const int j = rk * 16 + c;
          av[st][rk][i] = (live && j < r && k < K) ? load_u32x4(ab + (size_t)j * K_pad + k)
                                                   : u32x4_t{0u, 0u, 0u, 0u};
        }
      }
    }
  }
  // The same loads in two parts: the adapter's A rows (all 16 NRK of them; rows at or past
  // r are zeroed by mask_rank once r is known), then the tokens' x rows. load_a issues its
  // loads unconditionally (an element outside the step reads the row's first 16 bytes and is
  // zeroed), so that later waits can count them exactly.
  __device__ __forceinline__ void load_a(const uint16_t* ab, int K_pad, int K, int ch, int c1,
                                         int c, int g) {
#pragma unroll
    for (int st = 0; st < NSTEP; ++st) {
      const bool live = ch + st < c1;
      const int kb = (ch + st) * KSTEP + 8 * g;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int k = kb + 32 * i;
        const bool in = live && k < K;
#pragma unroll
        for (int rk = 0; rk < NRK; ++rk) {
          const int j = rk * 16 + c;
          const u32x4_t v = load_u32x4(ab + (size_t)j * K_pad + (in ? k : 0));
          av[st][rk][i] = in ? v : u32x4_t{0u, 0u, 0u, 0u};
        }
      }
    }
  }
  __device__ __forceinline__ void mask_rank(int r, int c) {
#pragma unroll
    for (int st = 0; st < NSTEP; ++st)
#pragma unroll
      for (int rk = 0; rk < NRK; ++rk)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (rk * 16 + c >= r) av[st][rk][i] = u32x4_t{0u, 0u, 0u, 0u};
  }
  __device__ __forceinline__ void load_x(const uint16_t* xr, bool vx, int K, int ch, int c1,
                                         int g) {
#pragma unroll
    for (int st = 0; st < NSTEP; ++st) {
      const bool live = ch + st < c1;
      const int kb = (ch + st) * KSTEP + 8 * g;
#pragma unroll
      for (int i = 0; i < 4; ++i) xv[st][i] = load_x8<ALIGNED>(xr, kb + 32 * i, K, vx && live);
    }
  }
  __device__ __forceinline__ void mfma(f32x4_t (&acc)[NRK]) const {
#pragma unroll
    for (int st = 0; st < NSTEP; ++st)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int rk = 0; rk < NRK; ++rk)
          acc[rk] = mfma_16x16x32_bf16(as_bf16x8(xv[st][i]), as_bf16x8(av[st][rk][i]), acc[rk]);
  }
};

// One K step of 128 for one wave, loaded and multiplied in two halves of 64: half the
// registers of ShrinkSteps<NRK, 1> for the loads in flight, the same MFMAs in the same order.
template <int NRK, bool ALIGNED>
__device__ __forceinline__ void shrink_step_halves(const uint16_t* xr, bool vx,
                                                   const uint16_t* ab, int K_pad, int K, int r,
                                                   int ch, int c1, int c, int g,
                                                   f32x4_t (&acc)[NRK]) {
  const bool live = ch < c1;
  const int kb = ch * KSTEP + 8 * g;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    u32x4_t xv[2], av[NRK][2];
#pragma unroll
    for (int i2 = 0; i2 < 2; ++i2) {
      const int k = kb + 32 * (2 * hf + i2);
      xv[i2] = load_x8<ALIGNED>(xr, k, K, vx && live);
#pragma unroll
      for (int rk = 0; rk < NRK; ++rk) {
        const int j = rk * 16 + c;
        av[rk][i2] = (live && j < r && k < K) ? load_u32x4(ab + (size_t)j * K_pad + k)
                                               : u32x4_t{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int i2 = 0; i2 < 2; ++i2)
#pragma unroll
      for (int rk = 0; rk < NRK; ++rk)
        acc[rk] = mfma_16x16x32_bf16(as_bf16x8(xv[i2]), as_bf16x8(av[rk][i2]), acc[rk]);
  }
}

// B fragments and old y of the first PF column groups of a wave (small pieces), loaded
// before the shrink's MFMAs so their latency overlaps the shrink; NT: y loads non-temporal.
template <int NE, int PF, bool ALIGNED, bool NT = false>
struct ExpandPrefetch {
  static constexpr int N = PF > 0 ? PF : 1;  // PF = 0: no prefetch (never loaded)
  ColMap cm[N][4];
  u32x4_t bq[N][NE][4];
  uint2 yv[N][4];
  __device__ __forceinline__ void load(const DeltaArgs& A, const uint16_t* bb, const Piece& pc,
                                       const int* s_tok, int w, int c, int g) {
#pragma unroll
    for (int f = 0; f < PF; ++f) {
      const int vl = pc.v0 + 64 * (w + DT_WAVES * f) + 4 * c;
      map_group<ALIGNED>(A, vl, cm[f]);
      load_b_group<NE>(bb, A.N_pad, pc.r, vl, pc.v1, g, cm[f], bq[f]);
      sgmv::load_y<ALIGNED, NT>(s_tok, pc.rows, 0, g, vl, pc.v1, cm[f], yv[f]);
    }
  }
  // The same loads in three steps: the column groups' maps, the tokens' y rows (load_y,
  // which needs the maps), then B of the adapter at rank r (the pool's full rank, before the
  // adapter's own is known; mask_rank trims it).
  __device__ __forceinline__ void map(const DeltaArgs& A, const Piece& pc, int w, int c) {
#pragma unroll
    for (int f = 0; f < PF; ++f)
      map_group<ALIGNED>(A, pc.v0 + 64 * (w + DT_WAVES * f) + 4 * c, cm[f]);
  }
  __device__ __forceinline__ void load_b(const uint16_t* bb, int N_pad, const Piece& pc, int r,
                                         int w, int c, int g) {
#pragma unroll
    for (int f = 0; f < PF; ++f) {
      const int vl = pc.v0 + 64 * (w + DT_WAVES * f) + 4 * c;
      load_b_group<NE>(bb, N_pad, r, vl, pc.v1, g, cm[f], bq[f]);
    }
  }
  __device__ __forceinline__ void mask_rank(int r, int g) {
#pragma unroll
    for (int f = 0; f < PF; ++f)
#pragma unroll
      for (int re = 0; re < NE; ++re) {
        const int live = r - 8 * (re * 4 + g);  // live ranks in this lane's octet
#pragma unroll
        for (int q = 0; q < 4; ++q)
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (e >= live) bq[f][re][q][e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
      }
  }
  __device__ __forceinline__ void load_y(const Piece& pc, const int* s_tok, int w, int c, int g) {
#pragma unroll
    for (int f = 0; f < PF; ++f) {
      const int vl = pc.v0 + 64 * (w + DT_WAVES * f) + 4 * c;
      sgmv::load_y<ALIGNED, NT>(s_tok, pc.rows, 0, g, vl, pc.v1, cm[f], yv[f]);
    }
  }
};

// ---------------------------------------------------------------------------------------
// K-split exchange between the column-split workgroups of one piece
// ---------------------------------------------------------------------------------------
// Workgroup p of the P that share a piece reduces K steps [p*nch/P, (p+1)*nch/P) of the
// shrink, publishes that fp32 partial tile (rows x ranks) to the workspace and adds its
// share to the piece's arrival counter: 1 for every split but the last, which adds 64 - (P-1),
// so that every call advances the counter by exactly 64 and a workgroup knows that all P
// partials are in once the counter has moved 64 past the multiple of 64 it found (no reset is
// needed between calls; the counter wraps safely). It then adds the P partials in split order,
// so the sum does not depend on which workgroup finished first. If the counter has not moved
// 64 within a bounded wait, the workgroup computes every other split's partial itself, by the
// same steps in the same order as its owner (bit-identical), and uses those instead.
//
// Memory ordering. Partial tiles are written and read only with agent-scope atomic stores and
// loads, which bypass the non-coherent caches (the stores write through to the device's
// coherence point); a workgroup waits for its own stores to complete before it adds to the
// counter, and reads partials only after it has seen the counter complete. This orders data
// and counter without agent-scope fences, whose L2 write-back and invalidate would stall every
// workgroup of the XCD. The partners of a piece run on one XCD and their counter atomics meet
// in its L2; if they are not seen in time, the local fallback keeps the results unchanged.

// Waits until every vector memory operation of this wave has completed (vmcnt = 0).
__device__ __forceinline__ void wait_stores() {
  // s_waitcnt encoding on gfx9: vmcnt [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]
  __builtin_amdgcn_s_waitcnt(0x0f70);
}

// Workgroup barrier for LDS traffic only: this wave's LDS reads and writes are complete
// before it arrives, while its global loads (direct-to-LDS ones included) stay in flight.
// __syncthreads' workgroup fence would also wait for all of those, which takes away the
// overlap of the staged shrink below, which orders its direct-to-LDS loads with explicit
// vmcnt waits instead. The memory clobber keeps the compiler from moving memory accesses
// across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// How the 8 waves of a workgroup share a piece's shrink: wave w takes row tile w % ntp and
// K slice w / ntp (ks slices). Small pieces: one row tile, 8 K slices; large pieces: 2 row
// tiles x 4 slices or 4 row tiles (3 or 4 used) x 2 slices.
struct ShrinkGeom {
  int nrt, ntp, ks;
};

__device__ __forceinline__ ShrinkGeom shrink_geom(bool small, int rows) {
  ShrinkGeom G;
  G.nrt = small ? 1 : (rows + 15) >> 4;
  G.ntp = small ? 1 : (G.nrt == 2 ? 2 : 4);
  G.ks = DT_WAVES / G.ntp;
  return G;
}

// Partial h of (row, rank j) of a piece: the wave partials in s_part
// ([wave][rank tile][16][16]) summed over the K slices in slice order; zero for j >= r.
template <int NRK>
__device__ __forceinline__ float part_sum(const float* s_part, const ShrinkGeom& G, int row,
                                          int j, int r) {
  const int rt = row >> 4, rr = row & 15, rk = j >> 4, cc = j & 15;
  float s = 0.f;
  if (j < r) {
    for (int q = 0; q < G.ks; ++q) s += s_part[(((q * G.ntp + rt) * NRK + rk) * 16 + rr) * 16 + cc];
  }
  return s;
}

template <int NRK>
__device__ __forceinline__ void store_wave_partial(float* s_part, int w, int c, int g,
                                                   const f32x4_t (&acc)[NRK]) {
  // D layout: lane (c, g) holds rows 4g..4g+3 of column c
#pragma unroll
  for (int rk = 0; rk < NRK; ++rk)
#pragma unroll
    for (int e = 0; e < 4; ++e) s_part[((w * NRK + rk) * 16 + 4 * g + e) * 16 + c] = acc[rk][e];
}

// Entries of a partial tile per thread: up to 16 (small) or 64 (large) rows x NCOL ranks
// (whole 32-rank expand tiles); thread t holds entries t, t + DT_THREADS, ...
template <int NRK, bool LARGE>
struct XchShape {
  static constexpr int NCOL = (NRK + 1) / 2 * 32;
  static constexpr int ROWS = LARGE ? 64 : 16;
  static constexpr int PER = (ROWS * NCOL + DT_THREADS - 1) / DT_THREADS;
  static constexpr int MAXS = LARGE ? SGMV_EXCHANGE_MAX_SPLITS_LARGE : SGMV_EXCHANGE_MAX_SPLITS;
  static constexpr int64_t TILE = LARGE ? XCH_LARGE_TILE : XCH_SMALL_TILE;
};

// Wave w's part of the shrink over K steps [k0, k1) of a split, one step at a time, into
// s_part. The MFMAs run in the same order as in the pieces' own loops, which issue several
// steps per load round, so the partial is bit-identical to its owner's.
template <int NRK, bool ALIGNED>
__device__ void shrink_range(const DeltaArgs& A, const Piece& pc, const ShrinkGeom& G,
                             const int* s_tok, int k0, int k1, float* s_part) {
  const int w = threadIdx.x / WAVE, lane = threadIdx.x & (WAVE - 1);
  const int c = lane & 15, g = lane >> 4;
  const int rt = w % G.ntp, kslice = w / G.ntp;
  const int row = rt * 16 + c;
  const bool vx = rt < G.nrt && row < pc.rows;
  const uint16_t* xr =
      static_cast<const uint16_t*>(A.x) + (size_t)(vx ? s_tok[row] : 0) * (size_t)A.ldx;
  const uint16_t* ab = static_cast<const uint16_t*>(A.a) + (size_t)pc.lora * A.R_pad * A.K_pad;
  const int n = k1 - k0;
  const int c0 = k0 + kslice * n / G.ks, c1 = k0 + (kslice + 1) * n / G.ks;
  f32x4_t acc[NRK];
#pragma unroll
  for (int i = 0; i < NRK; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if (rt < G.nrt) {
    for (int ch = c0; ch < c1; ++ch) {
      if constexpr (NRK >= 3) {
        shrink_step_halves<NRK, ALIGNED>(xr, vx, ab, A.K_pad, A.K, pc.r, ch, c1, c, g, acc);
      } else {
        ShrinkSteps<NRK, 1, ALIGNED> S;
        S.load(xr, vx, ab, A.K_pad, A.K, pc.r, ch, c1, c, g);
        S.mfma(acc);
      }
    }
  }
  store_wave_partial<NRK>(s_part, w, c, g, acc);
}

// Shrink of a large piece over K steps [k0, k1) of KSTEP, staged through LDS: the range is
// cut into 64-wide chunks; for each, 16 direct global-to-LDS loads of 1 KB (2 per wave:
// waves 0-3 the 64 x rows, waves 4-7 the 64 A rank rows, 128 bytes of each row) fill one of
// STAGES buffers, STAGES - 1 chunks ahead of the one being multiplied, so loads stay in flight
// without registers. Wave w owns row tiles 2 (w % 2) .. + 1 and rank tiles 2 ((w / 2) % 2)
// .. + 1 over the 32-wide half w / 4 of every chunk (16 accumulator registers), reading its
// MFMA operands from LDS (each wave reads 4 KB of a 16 KB chunk); the two halves' partials
// are added once at the end (half 0 + half 1) and go to s_h (times mult). Within a row of
// 128 bytes the eight 16-byte chunks are stored in the order q ^ ((row / 2) % 8), which makes
// the operand reads of 16 lanes (16 rows) fall in distinct LDS banks. Rows past the piece
// read its first token's row, ranks past the adapter's rank its first rank row, k past K the
// row's first bytes; all of these are zeroed when read. The same steps in the same order serve a piece's own partial and the
// local recomputation of a partner's. Needs STAGES * STAGE_BYTES of s_part.
// This wave's two 1 KB loads of one chunk (k0: the chunk's first K index) into buf. NT: waves
// 0-3's x loads are marked non-temporal (x is read once; A stays cached).
template <bool NT = false>
__device__ __forceinline__ void stage_chunk(const uint16_t* const (&src)[2], const int (&kq)[2],
                                            int k0, int K, unsigned char* buf, int w) {
  typedef __attribute__((address_space(3))) void lds_void;
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int k = k0 + kq[i];
    if (NT && w < 4)
      __builtin_amdgcn_global_load_lds(src[i] + (k < K ? k : 0),
                                       (lds_void*)(buf + (2 * w + i) * 1024), 16, 0, 2 /* nt */);
    else
      __builtin_amdgcn_global_load_lds(src[i] + (k < K ? k : 0),
                                       (lds_void*)(buf + (2 * w + i) * 1024), 16, 0, 0);
  }
}

template <int NRK>
__device__ __forceinline__ void large_shrink_staged(const DeltaArgs& A, const Piece& pc, int nrt,
                                    const int* s_tok, int k0, int k1, float mult,
                                    float* s_part, float* s_h) {
  const int tid = threadIdx.x, w = tid / WAVE, lane = tid & (WAVE - 1);
  const int c = lane & 15, g = lane >> 4;
  unsigned char* stage0 = reinterpret_cast<unsigned char*>(s_part);
  // this lane's two loads per chunk: slot 2w + i covers tile rows 8 (2w + i) .. + 7 (x for
  // slots 0..7, A for 8..15), lane l takes row 8 slot + l / 8 and 16-byte chunk
  // (l % 8) ^ ((row / 2) % 8) of the row's 128 bytes
  const uint16_t* src[2];
  int kq[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int slot = 2 * w + i;
    const int row = 8 * (slot & 7) + (lane >> 3);
    kq[i] = 8 * ((lane & 7) ^ ((row >> 1) & 7));
    if (slot < 8) {
      const int tok = s_tok[row < pc.rows ? row : 0];
      src[i] = static_cast<const uint16_t*>(A.x) + (size_t)tok * (size_t)A.ldx;
    } else {
      const int rk = row < pc.r ? row : 0;  // past the adapter's rank: a row already read
      src[i] = static_cast<const uint16_t*>(A.a) + ((size_t)pc.lora * A.R_pad + rk) * A.K_pad;
    }
  }
  const int nck = 2 * (k1 - k0);  // 64-wide chunks
  const int kbase = k0 * KSTEP, K = A.K;
  // this wave's MFMA work: row tiles 2 tp, 2 tp + 1, rank tiles 2 kp, 2 kp + 1, the 32-wide
  // half ks of every chunk (wave-uniform, from the first lane)
  const int wu = __builtin_amdgcn_readfirstlane(w);
  const int tp = wu & 1, kp = (wu >> 1) & 1, ks = wu >> 2;
  const int q = 4 * ks + g;  // this lane's 16-byte chunk of a 128-byte row
  f32x4_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int t = 0; t < 2; ++t) acc[i][t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  uint32_t mrow[2], mrank[2];  // operand masks: rows past the piece, ranks past the adapter's
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    mrow[i] = (2 * tp + i) * 16 + c < pc.rows ? 0xffffffffu : 0u;
    mrank[i] = (2 * kp + i) * 16 + c < pc.r ? 0xffffffffu : 0u;
  }
#pragma unroll
  for (int ck = 0; ck < STAGES - 1; ++ck)
    if (ck < nck)
      stage_chunk<(NRK >= 2)>(src, kq, kbase + 64 * ck, K, stage0 + (ck % STAGES) * STAGE_BYTES, w);
  for (int ck = 0; ck < nck; ++ck) {
    // this wave's loads of chunk ck are in once at most the later chunk's two are outstanding
    // (only the two loads of each later chunk already issued, up to STAGES - 2 of them, may
    // still be outstanding)
    static_assert(STAGES == 4, "the wait counts below assume two chunks in flight behind");
    if (ck + 2 < nck) __builtin_amdgcn_s_waitcnt(0x0f70 | 4);       // vmcnt(4)
    else if (ck + 1 < nck) __builtin_amdgcn_s_waitcnt(0x0f70 | 2);  // vmcnt(2)
    else __builtin_amdgcn_s_waitcnt(0x0f70);                        // vmcnt(0)
    lds_barrier();  // every wave's loads of chunk ck are in; chunk ck - 1 is consumed
    if (ck + STAGES - 1 < nck) {
      const int cn = ck + STAGES - 1;
      stage_chunk<(NRK >= 2)>(src, kq, kbase + 64 * cn, K, stage0 + (cn % STAGES) * STAGE_BYTES,
                              w);
    }
    // every operand read first, masked by AND (no branches between the reads and the MFMAs)
    const unsigned char* buf = stage0 + (ck % STAGES) * STAGE_BYTES;
    const uint32_t kin = kbase + 64 * ck + 8 * q < K ? 0xffffffffu : 0u;
    u32x4_t xv[2], av[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int row = (2 * tp + i) * 16 + c;
      const int j = (2 * kp + i) * 16 + c;  // rank row
      xv[i] = *reinterpret_cast<const u32x4_t*>(buf + row * 128 + ((q ^ ((row >> 1) & 7)) << 4));
      av[i] = *reinterpret_cast<const u32x4_t*>(buf + 8192 + j * 128 +
                                                ((q ^ ((j >> 1) & 7)) << 4));
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xv[i][e] &= mrow[i] & kin;
        av[i][e] &= mrank[i] & kin;
      }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int t = 0; t < 2; ++t)
        if (2 * tp + i < nrt && (NRK == 4 || 2 * kp + t < NRK))  // tiles with work
          acc[i][t] = mfma_16x16x32_bf16(as_bf16x8(xv[i]), as_bf16x8(av[t]), acc[i][t]);
  }
  __syncthreads();  // the last chunk is consumed: s_part is free again
  // the two halves' partials summed (half 0 + half 1) into s_h, times mult; D layout: lane
  // (c, g) holds rows 4g..4g+3 of rank column c
  constexpr int NCOL = (NRK + 1) / 2 * 32;
  float* red = s_part + (size_t)(wu & 3) * 1024;  // [tile i, t][e][lane] of wave w % 4
  if (ks == 1) {
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) red[((2 * i + t) * 4 + e) * WAVE + lane] = acc[i][t][e];
  }
  __syncthreads();
  if (ks == 0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if (2 * tp + i >= nrt) continue;  // wave-uniform
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int col = (2 * kp + t) * 16 + c;
        if (col < NCOL) {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            s_h[((2 * tp + i) * 16 + 4 * g + e) * HS + col] =
                (acc[i][t][e] + red[((2 * i + t) * 4 + e) * WAVE + lane]) * mult;
        }
      }
    }
  }
  __syncthreads();
}

// Shrink of a large piece over K steps [k0, k1) of KSTEP: the 8 waves split the range into
// 8 slices of 32-wide substeps, and each wave accumulates every row tile x rank tile of the
// piece over its slice, so x and A are each read once per workgroup. The wave partials are
// then summed in wave order, one row tile at a time, into s_h rows (times mult; zero at ranks
// >= r). The same steps in the same order serve a piece's own partial and the local
// recomputation of a partner's, so both are bit-identical.
template <int NRK, bool ALIGNED, bool STAGED = false>
__device__ __forceinline__ void large_shrink(const DeltaArgs& A, const Piece& pc, int nrt, const int* s_tok,
                             int k0, int k1, float mult, float* s_part, float* s_h) {
  if constexpr (ALIGNED && STAGED) {  // every launch gives s_part STAGES * STAGE_BYTES
    large_shrink_staged<NRK>(A, pc, nrt, s_tok, k0, k1, mult, s_part, s_h);
    return;
  }
  constexpr int NCOL = (NRK + 1) / 2 * 32;  // whole 32-rank expand tiles
  const int tid = threadIdx.x, w = tid / WAVE, lane = tid & (WAVE - 1);
  const int c = lane & 15, g = lane >> 4;
  const int n = 4 * (k1 - k0);  // 32-wide substeps of the range
  const int u0 = 4 * k0 + w * n / DT_WAVES, u1 = 4 * k0 + (w + 1) * n / DT_WAVES;
  const uint16_t* ab = static_cast<const uint16_t*>(A.a) + (size_t)pc.lora * A.R_pad * A.K_pad;
  const uint16_t* xr[4];
  bool vx[4];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    const int row = rt * 16 + c;
    vx[rt] = rt < nrt && row < pc.rows;
    xr[rt] = static_cast<const uint16_t*>(A.x) + (size_t)(vx[rt] ? s_tok[row] : 0) * (size_t)A.ldx;
  }
  f32x4_t acc[4][NRK];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int rk = 0; rk < NRK; ++rk) acc[rt][rk] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int u = u0; u < u1; ++u) {
    const int k = 32 * u + 8 * g;
    u32x4_t xv[4], av[NRK];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) xv[rt] = load_x8<ALIGNED>(xr[rt], k, A.K, vx[rt]);
#pragma unroll
    for (int rk = 0; rk < NRK; ++rk) {
      const int j = rk * 16 + c;
      av[rk] = (j < pc.r && k < A.K) ? load_u32x4(ab + (size_t)j * A.K_pad + k)
                                      : u32x4_t{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      if (rt < nrt) {  // uniform
#pragma unroll
        for (int rk = 0; rk < NRK; ++rk)
          acc[rt][rk] = mfma_16x16x32_bf16(as_bf16x8(xv[rt]), as_bf16x8(av[rk]), acc[rt][rk]);
      }
    }
  }
  const ShrinkGeom G1{1, 1, DT_WAVES};  // one row tile, 8 K slices (the waves)
#pragma unroll
  for (int rt = 0; rt < 4; ++rt) {
    if (rt >= nrt) break;  // uniform
    store_wave_partial<NRK>(s_part, w, c, g, acc[rt]);
    __syncthreads();
    for (int idx = tid; idx < 16 * NCOL; idx += DT_THREADS) {
      const int row = idx / NCOL, j = idx - row * NCOL;
      s_h[(rt * 16 + row) * HS + j] = part_sum<NRK>(s_part, G1, row, j, pc.r) * mult;
    }
    __syncthreads();
  }
}

// Writes partial tile `slot` of a piece from this workgroup's partial: large pieces have it
// summed in s_h, small pieces as wave partials in s_part. Call from all threads.
template <int NRK, bool LARGE>
__device__ __forceinline__ void store_partial(const Piece& pc, const ShrinkGeom& G,
                                              const float* s_part, const float* s_h,
                                              float* slot) {
  using S = XchShape<NRK, LARGE>;
  const int entries = G.nrt * 16 * S::NCOL;
#pragma unroll
  for (int e = 0; e < S::PER; ++e) {
    const int idx = threadIdx.x + e * DT_THREADS;
    if (idx < entries) {
      const int row = idx / S::NCOL, j = idx - row * S::NCOL;
      float v;
      if constexpr (LARGE)
        v = s_h[row * HS + j];
      else
        v = part_sum<NRK>(s_part, G, row, j, pc.r);
      __hip_atomic_store(slot + row * S::NCOL + j, v, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Called by all threads once this workgroup's partial for its K range is in s_part (small
// pieces: wave partials) or s_h (large pieces: summed). Leaves the scaled full h tile in s_h
// (nrt * 16 rows x NCOL ranks).
template <int NRK, bool ALIGNED, bool LARGE>
__device__ void exchange_h(const DeltaArgs& A, const Piece& pc, const ShrinkGeom& G,
                           const int* s_tok, int nch, float* s_part, float* s_h, int* s_flag) {
  using S = XchShape<NRK, LARGE>;
  const int tid = threadIdx.x, P = pc.nsplit, p = pc.split;
  const int entries = G.nrt * 16 * S::NCOL;
  // slots: a small piece's, a large piece's, or those of part j of a large piece, which
  // counts arrivals in word j of the piece's control block and keeps its split q partial (16
  // rows of NCOL floats) at q * 64 NCOL + j * 16 NCOL floats into the piece's partial slots
  // (up to 8 splits at NCOL 32, 4 at NCOL 64)
  const bool prt = !LARGE && NRK <= 2 && pc.xsub >= 0;  // parts: ranks up to 32 only
  const size_t rec = (LARGE || prt) ? (size_t)pc.tile : (size_t)A.large_cap + pc.tile;
  uint32_t* counter =
      reinterpret_cast<uint32_t*>(A.xctl) + rec * XCH_CTL_INTS + (prt ? pc.xsub : 0);
  float* part;
  int xs;
  if (LARGE || prt) {
    part = A.xpart_large + (size_t)pc.tile * SGMV_EXCHANGE_MAX_SPLITS_LARGE * XCH_LARGE_TILE;
    xs = (int)XCH_LARGE_TILE;
    if (prt) {
      part += pc.xsub * SGMV_SMALL_ROWS * S::NCOL;
      xs = SGMV_TILE_ROWS * S::NCOL;
    }
  } else {
    part = A.xpart_small + (size_t)pc.tile * SGMV_EXCHANGE_MAX_SPLITS * XCH_SMALL_TILE;
    xs = (int)XCH_SMALL_TILE;
  }
  const int64_t wait = LARGE ? A.xwait_large : A.xwait;

  store_partial<NRK, LARGE>(pc, G, s_part, s_h, part + p * xs);
  wait_stores();
  __syncthreads();
  if (!LARGE) SGMV_STAMP(4);  // the partial is published (and B and y are in)
  if (tid == 0) {
    const uint32_t inc = p == P - 1 ? 64u - (uint32_t)(P - 1) : 1u;
    const uint32_t old =
        __hip_atomic_fetch_add(counter, inc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint32_t base = old & ~63u;
    uint32_t cur = old + inc;
    if (cur - base < 64u && wait >= 0) {
      const uint64_t t0 = wall_clock64();
      do {
        __builtin_amdgcn_s_sleep(2);
        cur = __hip_atomic_load(counter, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      } while (cur - base < 64u && wall_clock64() - t0 < (uint64_t)wait);
    }
    *s_flag = cur - base >= 64u ? 1 : 0;
  }
  __syncthreads();
  if (!LARGE) SGMV_STAMP(5);  // the counter is complete (or the wait is over)

  if (!*s_flag) {  // uniform: a partner is late. Every other partial is computed here, by the
                   // same steps as its owner's, and written to its slot (the owner, if it is
                   // still running, writes the same bits)
    for (int q = 0; q < P; ++q) {
      if (q == p) continue;
      __syncthreads();  // the previous round's readers of s_part / s_h are done
      if constexpr (LARGE)
        large_shrink<NRK, ALIGNED, true>(A, pc, G.nrt, s_tok, q * nch / P, (q + 1) * nch / P, 1.f,
                                   s_part, s_h);
      else
        shrink_range<NRK, ALIGNED>(A, pc, G, s_tok, q * nch / P, (q + 1) * nch / P, s_part);
      __syncthreads();
      store_partial<NRK, LARGE>(pc, G, s_part, s_h, part + q * xs);
    }
    wait_stores();
    __syncthreads();
  }

  // every partial is in its slot: the sum in split order, scaled
  float pv[S::MAXS][S::PER];
#pragma unroll
  for (int q = 0; q < S::MAXS; ++q)
#pragma unroll
    for (int e = 0; e < S::PER; ++e) {
      const int idx = tid + e * DT_THREADS;
      const int row = idx / S::NCOL, j = idx - row * S::NCOL;
      pv[q][e] = (q < P && idx < entries)
                     ? __hip_atomic_load(part + q * xs + row * S::NCOL + j, __ATOMIC_RELAXED,
                                         __HIP_MEMORY_SCOPE_AGENT)
                     : 0.f;
    }
#pragma unroll
  for (int e = 0; e < S::PER; ++e) {
    const int idx = tid + e * DT_THREADS;
    float h = 0.f;
#pragma unroll
    for (int q = 0; q < S::MAXS; ++q)
      if (q < P) h += pv[q][e];
    if (idx < entries) {
      const int row = idx / S::NCOL, j = idx - row * S::NCOL;
      s_h[row * HS + j] = h * pc.scale;
    }
  }
}

// ---------------------------------------------------------------------------------------
// small pieces (<= 16 rows): K split across the 8 waves, expand operands prefetched
// ---------------------------------------------------------------------------------------
// SPEC (fused build + delta, adapter-major, every adapter at full rank 16): pc holds the
// adapter and the columns only; the first K step's A tile is loaded before the adapter's
// tokens are looked up in the batch's ids, the tokens' x and y after, B once x is in; the
// adapter's rank and scale (rank_l, scale_l) mask A and B where they are first used.
template <int MODE, int NRK, bool ALIGNED, bool XCH, bool SPEC = false, bool YNT = false>
__device__ __forceinline__ void small_piece(const DeltaArgs& A, Piece& pc, int* s_tok,
                                            float* s_part, float* s_h, int* s_mask,
                                            int rank_l = 0, float scale_l = 0.f) {
  const int tid = threadIdx.x, w = tid / WAVE, lane = tid & (WAVE - 1);
  const int c = lane & 15, g = lane >> 4;
  constexpr bool xkernel = XCH && MODE == MODE_FUSED;
  const bool xch = xkernel && ((NRK <= 2 && pc.xsub >= 0) ? A.xch_large : A.xch_small);
  // K steps whose loads are issued together, and column groups per wave whose B and y are
  // prefetched, sized so that everything in flight fits in registers. With the exchange a
  // workgroup covers a fraction of K, one step per load round suffices, and the smaller
  // register footprint lets two workgroups share a CU.
  constexpr int NSTEP = xkernel ? 1 : (NRK == 1 ? 4 : (NRK == 2 ? 2 : 1));
  constexpr int PF = NRK == 1 ? 2 : ((xkernel && NRK >= 3) ? 0 : 1);
  constexpr int NE = (NRK + 1) / 2;  // expand rank tiles of 32
  const uint16_t* bb =
      static_cast<const uint16_t*>(A.b) + (size_t)pc.lora * (A.R_pad / 8) * A.N_pad * 8;

  ExpandPrefetch<NE, PF, ALIGNED, YNT> pf;
  bool fetched = false;
  const int nch = (A.K + KSTEP - 1) / KSTEP;

  if (MODE != MODE_EXPAND) {
    f32x4_t acc[NRK];
#pragma unroll
    for (int i = 0; i < NRK; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const uint16_t* ab = static_cast<const uint16_t*>(A.a) + (size_t)pc.lora * A.R_pad * A.K_pad;
    // K steps of this workgroup (all of K, or its split's range), then of this wave
    const int k0 = xch ? pc.split * nch / pc.nsplit : 0;
    const int k1 = xch ? (pc.split + 1) * nch / pc.nsplit : nch;
    const int c0 = k0 + w * (k1 - k0) / DT_WAVES, c1 = k0 + (w + 1) * (k1 - k0) / DT_WAVES;
    int ch = c0;
    if constexpr (SPEC) {
      static_assert(MODE == MODE_FUSED && NRK == 1 && PF > 0, "adapter-major rank-16 pieces");
      ShrinkSteps<NRK, NSTEP, ALIGNED> S;
      S.load_a(ab, A.K_pad, A.K, ch, c1, c, g);
      const uint64_t idmask = wave_adapter_mask(A.ids, A.M, pc.lora);
      SGMV_STAMP_AFTER(1, idmask);  // the ids are in
      pc.rows = adapter_small_piece<DT_WAVES>(idmask, reinterpret_cast<int*>(s_part), s_tok);
      if (pc.rows == 0) {  // uniform: no small piece; let the loads land before leaving
        __builtin_amdgcn_s_waitcnt(0);
        return;
      }
      __syncthreads();  // s_tok; s_part is free again
      SGMV_STAMP(2);  // the piece's tokens are known
      pc.r = rank_l;
      pc.scale = scale_l;
      const bool vx = c < pc.rows;
      S.load_x(static_cast<const uint16_t*>(A.x) + (size_t)(vx ? s_tok[c] : 0) * (size_t)A.ldx,
               vx, A.K, ch, c1, g);
      // y right behind x (loads complete in order, so the MFMAs wait for x alone), B once x is
      // in: y's round trip overlaps the shrink, and x does not queue behind B
      pf.map(A, pc, w, c);
      pf.load_y(pc, s_tok, w, c, g);
      S.mask_rank(pc.r, c);
      S.mfma(acc);
      SGMV_STAMP(3);  // x is in, the first K step multiplied
      pf.load_b(bb, A.N_pad, pc, A.R_pad, w, c, g);
      fetched = true;
      ch += NSTEP;
    }
    const bool vx = c < pc.rows;
    const uint16_t* xr =
        static_cast<const uint16_t*>(A.x) + (size_t)(vx ? s_tok[c] : 0) * (size_t)A.ldx;
    for (; ch < c1; ch += NSTEP) {
      if constexpr (xkernel && NRK >= 3) {
        shrink_step_halves<NRK, ALIGNED>(xr, vx, ab, A.K_pad, A.K, pc.r, ch, c1, c, g, acc);
      } else {
        ShrinkSteps<NRK, NSTEP, ALIGNED> S;
        S.load(xr, vx, ab, A.K_pad, A.K, pc.r, ch, c1, c, g);
        // y rides along the first loads (the MFMAs wait for x and A alone: loads complete in
        // order), B follows once they are in, so x and A do not queue behind it
        const bool first = MODE == MODE_FUSED && PF > 0 && !fetched;
        if (first) {
          pf.map(A, pc, w, c);
          pf.load_y(pc, s_tok, w, c, g);
        }
        S.mfma(acc);
        if (first) {
          pf.load_b(bb, A.N_pad, pc, pc.r, w, c, g);
          fetched = true;
        }
      }
    }
    store_wave_partial<NRK>(s_part, w, c, g, acc);
  }
  if (MODE != MODE_SHRINK && PF > 0 && !fetched) pf.load(A, bb, pc, s_tok, w, c, g);
  __syncthreads();
  if (xch)
    exchange_h<NRK, ALIGNED, false>(A, pc, shrink_geom(true, pc.rows), s_tok, nch, s_part, s_h,
                                    s_mask);
  else if (MODE != MODE_EXPAND)
    reduce_partials<NRK>(1, 1, DT_WAVES, pc.r, MODE == MODE_SHRINK ? 1.f : pc.scale, s_part, s_h);
  __syncthreads();
  if (MODE == MODE_SHRINK) return;

  bf16x8_t P[NE][2];
  h_fragments<NE>(s_h, 0, lane, P);
  if constexpr (SPEC) pf.mask_rank(pc.r, g);
  if constexpr (SPEC) SGMV_STAMP(6);  // h is in LDS

  // prefetched groups
#pragma unroll
  for (int f = 0; f < PF; ++f) {
    const int vg = pc.v0 + 64 * (w + DT_WAVES * f);
    if (vg >= pc.v1) continue;
    f32x4_t yacc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) yacc[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    expand_mfma<NE>(P, pf.bq[f], yacc);
    store_y<ALIGNED, YNT>(s_tok, pc.rows, 0, g, vg + 4 * c, pc.v1, pf.cm[f], pf.yv[f], yacc);
  }
  // remaining groups
  for (int vg = pc.v0 + 64 * (w + DT_WAVES * PF); vg < pc.v1; vg += 64 * DT_WAVES) {
    const int vl = vg + 4 * c;
    ColMap cg[4];
    map_group<ALIGNED>(A, vl, cg);
    u32x4_t b2[NE][4];
    uint2 y2[4];
    load_b_group<NE>(bb, A.N_pad, pc.r, vl, pc.v1, g, cg, b2);
    load_y<ALIGNED, YNT>(s_tok, pc.rows, 0, g, vl, pc.v1, cg, y2);
    f32x4_t yacc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) yacc[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    expand_mfma<NE>(P, b2, yacc);
    store_y<ALIGNED, YNT>(s_tok, pc.rows, 0, g, vl, pc.v1, cg, y2, yacc);
  }
  if constexpr (SPEC) {
    SGMV_STAMP(7);          // the y stores are issued
    SGMV_STAMP_DRAINED(8);  // and complete
  }
}

// ---------------------------------------------------------------------------------------
// large pieces (17..64 rows): waves cover (row tile, K slice) pairs and stream K
// ---------------------------------------------------------------------------------------
template <int MODE, int NRK, bool ALIGNED, bool XCH, bool YNT = false>
__device__ __forceinline__ void large_piece(const DeltaArgs& A, const Piece& pc, const int* s_tok,
                                            float* s_part, float* s_h, int* s_mask) {
  const int tid = threadIdx.x, w = tid / WAVE, lane = tid & (WAVE - 1);
  const int c = lane & 15, g = lane >> 4;
  const ShrinkGeom G = shrink_geom(false, pc.rows);
  const int nrt = G.nrt;  // 2..4 row tiles
  constexpr bool xkernel = XCH && MODE == MODE_FUSED;
  const bool xch = xkernel && A.xch_large;
  if (MODE != MODE_EXPAND) {
    const int nch = (A.K + KSTEP - 1) / KSTEP;
    // K steps of this workgroup: all of K, or its split's range
    const int k0 = xch ? pc.split * nch / pc.nsplit : 0;
    const int k1 = xch ? (pc.split + 1) * nch / pc.nsplit : nch;
    large_shrink<NRK, ALIGNED, MODE == MODE_FUSED>(A, pc, nrt, s_tok, k0, k1,
                               (MODE == MODE_FUSED && !xch) ? pc.scale : 1.f, s_part, s_h);
    if (xch) exchange_h<NRK, ALIGNED, true>(A, pc, G, s_tok, nch, s_part, s_h, s_mask);
  }
  __syncthreads();
  if (MODE == MODE_SHRINK) return;

  constexpr int NE = (NRK + 1) / 2;  // expand rank tiles of 32
  u32x4_t* s_pf = reinterpret_cast<u32x4_t*>(s_part);
  build_fragments<NE>(nrt, s_h, s_pf);
  __syncthreads();
  const uint16_t* bb =
      static_cast<const uint16_t*>(A.b) + (size_t)pc.lora * (A.R_pad / 8) * A.N_pad * 8;
  for (int vg = pc.v0 + 64 * w; vg < pc.v1; vg += 64 * DT_WAVES) {
    const int vl = vg + 4 * c;
    ColMap cm[4];
    map_group<ALIGNED>(A, vl, cm);
    u32x4_t bq[NE][4];  // kept across the row tiles
    load_b_group<NE>(bb, A.N_pad, pc.r, vl, pc.v1, g, cm, bq);
    // old y of every row tile, loaded together with B (one memory round trip per group)
    uint2 yv[4][4];
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      if (rt < nrt) load_y<ALIGNED, YNT>(s_tok, pc.rows, rt, g, vl, pc.v1, cm, yv[rt]);
    }
#pragma unroll
    for (int rt = 0; rt < 4; ++rt) {
      if (rt >= nrt) break;
      bf16x8_t P[NE][2];
      read_fragments<NE>(s_pf, rt, lane, P);
      f32x4_t yacc[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) yacc[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      expand_mfma<NE>(P, bq, yacc);
      store_y<ALIGNED, YNT>(s_tok, pc.rows, rt, g, vl, pc.v1, cm, yv[rt], yacc);
    }
  }
}

// Dispatch on the piece's rank tiles (1..NRKM) and class.
// YNT: y is read and written non-temporally (it streams through once; A and B stay cached).
// The kernels for ranks above 16 take it (prefill-like batches: 10% faster at rank 64); the
// rank-16 kernel, which decode batches run, keeps plain accesses.
template <int MODE, bool ALIGNED, int NRK, bool XCH, bool YNT>
__device__ __forceinline__ void piece_of(const DeltaArgs& A, const Piece& pc, bool small,
                                         const int* s_tok, float* s_part, float* s_h,
                                         int* s_mask) {
  if (small) {
    Piece q = pc;
    small_piece<MODE, NRK, ALIGNED, XCH, false, YNT>(A, q, const_cast<int*>(s_tok), s_part, s_h,
                                                     s_mask);
  } else
    large_piece<MODE, NRK, ALIGNED, XCH, YNT>(A, pc, s_tok, s_part, s_h, s_mask);
}

template <int MODE, bool ALIGNED, int NRKM, bool XCH>
__device__ __forceinline__ void run_piece(const DeltaArgs& A, const Piece& pc, bool small,
                                          int nrk, const int* s_tok, float* s_part, float* s_h,
                                          int* s_mask) {
  constexpr bool YNT = NRKM >= 2;
  if constexpr (NRKM == 1) {
    piece_of<MODE, ALIGNED, 1, XCH, YNT>(A, pc, small, s_tok, s_part, s_h, s_mask);
  } else if constexpr (NRKM == 2) {
    if (nrk <= 1) piece_of<MODE, ALIGNED, 1, XCH, YNT>(A, pc, small, s_tok, s_part, s_h, s_mask);
    else piece_of<MODE, ALIGNED, 2, XCH, YNT>(A, pc, small, s_tok, s_part, s_h, s_mask);
  } else {
    switch (nrk) {
      case 1: piece_of<MODE, ALIGNED, 1, XCH, YNT>(A, pc, small, s_tok, s_part, s_h, s_mask); break;
      case 2: piece_of<MODE, ALIGNED, 2, XCH, YNT>(A, pc, small, s_tok, s_part, s_h, s_mask); break;
      case 3: piece_of<MODE, ALIGNED, 3, XCH, YNT>(A, pc, small, s_tok, s_part, s_h, s_mask); break;
      default: piece_of<MODE, ALIGNED, 4, XCH, YNT>(A, pc, small, s_tok, s_part, s_h, s_mask); break;
    }
  }
}

// Pieces of rank tiles up to NRKM (ranks up to 16 NRKM); XCH: pieces of fused calls split
// their shrink over K with the other column splits of the piece; BUILD: every workgroup
// first builds the segments of the batch itself (fused build + delta, M <= 512).
// Aligned exchange variants are held to 128 registers so that two workgroups share a CU; the
// generic unaligned instance needs more and is left unconstrained.
template <int MODE, bool ALIGNED, int NRKM, bool XCH, bool BUILD>
__global__ __launch_bounds__(DT_THREADS)
__attribute__((amdgpu_waves_per_eu(XCH && ALIGNED ? 4 : 1))) void delta_bf16_kernel(DeltaArgs A) {
  __shared__ __align__(16) int s_tok[SGMV_TILE_ROWS];
  __shared__ int s_rank[RANK_TABLE_MAX];
  __shared__ float s_scale[RANK_TABLE_MAX];
  __shared__ int s_mask;  // K-split exchange: 1 when every partner's partial is in
  // partial shrink tiles, [wave][rank tile][16][16] fp32 (R_pad/16 rank tiles); reused for
  // the expand's h fragments afterwards; the staged shrink's ring; the h tile at SH_OFFSET
  extern __shared__ __align__(16) float s_part[];
  SGMV_STAMP(0);
  float* const s_h = s_part + SH_OFFSET / sizeof(float);

  // ---- which piece and column split (from the workgroup index alone) ----
  const bool split = MODE != MODE_SHRINK;
  if constexpr (BUILD) {
    if (A.amajor && (int)blockIdx.x == A.grid_writer) {  // the segment arrays, no piece
      const int id = threadIdx.x < (unsigned)A.M ? A.ids[threadIdx.x] : 0;
      const WgBuildDst dst{A.w_sorted, A.w_indptr, A.w_seg_lora, A.w_tiles, A.w_info,
                           A.seg_cap, A.large_cap, A.small_cap};
      wg_build(id, A.M, A.L, A.chunk, false, -8 /* a slot with no piece */, false, true, dst,
               wg_build_lds(reinterpret_cast<unsigned char*>(s_part), A.L), s_tok);
      return;
    }
  }
  bool small;
  int tile, p, P, sub = 0;
  if (!locate_piece(A, split, small, tile, p, P, true)) return;
  // large pieces as 16-row parts: fused calls on small batches at ranks up to 32 (the host
  // sets rsplit 1 otherwise; kernels for larger ranks leave the code out)
  const int rsplit = (MODE == MODE_FUSED && NRKM <= 2) ? A.rsplit : 1;

  const int tid = threadIdx.x;
  const bool table = A.L <= RANK_TABLE_MAX;
  Piece pc;
  if (BUILD && A.amajor && small) {
    // ---- adapter-major small piece: slot `tile` is adapter `tile`; no sort needed ----
    if (tile >= A.L) return;
    if constexpr (MODE == MODE_FUSED && NRKM == 1) {
      if (A.spec) {  // A first; the ids, rank and scale come through scalar loads meanwhile
        typedef const int32_t __attribute__((address_space(4))) cint;
        typedef const float __attribute__((address_space(4))) cfloat;
        const int rank_l = ((const cint*)A.rank)[tile];
        const float scale_l = ((const cfloat*)A.scale)[tile];
        pc.lora = tile;
        pc.start = 0;
        pc.rows = 0;
        pc.r = A.R_pad;
        pc.scale = 0.f;
        const int width = (((A.v_total + P - 1) / P) + 63) & ~63;
        pc.v0 = p * width;
        pc.v1 = min(pc.v0 + width, A.v_total);
        pc.tile = tile;
        pc.split = p;
        pc.nsplit = P;
        pc.xsub = -1;
        if (pc.v0 >= pc.v1 && !(XCH && A.xch_small)) return;
        small_piece<MODE, 1, ALIGNED, XCH, true>(A, pc, s_tok, s_part, s_h, &s_mask, rank_l,
                                                 scale_l);
        return;
      }
    }
    const int id = tid < A.M ? A.ids[tid] : -1;
    if (tid == 0) {
      s_rank[tile] = A.rank[tile];
      s_scale[tile] = A.scale[tile];
    }
    pc.rows = adapter_small_piece<DT_WAVES>(__ballot(id == tile),
                                            reinterpret_cast<int*>(s_part), s_tok);
    if (pc.rows == 0) return;  // uniform
    pc.lora = tile;
    pc.start = 0;
    __syncthreads();  // s_tok and the table entry; s_part is free again
  } else if constexpr (BUILD) {
    // ---- the batch's segments, built here; the rank/scale table loads overlap the ids' ----
    static_assert(DT_THREADS == FUSED_BUILD_WAVES * WAVE, "one token per thread");
    const int id = tid < A.M ? A.ids[tid] : 0;  // issued first: one round trip with the table
    if (table) {
      for (int i = tid; i < A.L; i += DT_THREADS) {
        s_rank[i] = A.rank[i];
        s_scale[i] = A.scale[i];
      }
    }
    const WgBuildDst dst{A.w_sorted, A.w_indptr, A.w_seg_lora, A.w_tiles, A.w_info,
                         A.seg_cap, A.large_cap, A.small_cap};
    const WgBuildLds S = wg_build_lds(reinterpret_cast<unsigned char*>(s_part), A.L);
    if (!small && rsplit > 1 && A.amajor) {
      // adapter-indexed launch: the large class has work only if some adapter has more tokens
      // than a small piece holds; a histogram in LDS decides before the full build
      int* s_cnt = reinterpret_cast<int*>(s_part);
      for (int i = tid; i < A.L; i += DT_THREADS) s_cnt[i] = 0;
      __syncthreads();
      if (tid < A.M && id >= 0 && id < A.L) atomicAdd(s_cnt + id, 1);
      __syncthreads();
      bool big = false;
      for (int i = tid; i < A.L; i += DT_THREADS) big = big || s_cnt[i] > SGMV_SMALL_ROWS;
      if (!__syncthreads_or(big)) return;  // uniform: no large piece in this batch
    }
    const WgBuildOut bo = wg_build(id, A.M, A.L, A.chunk, small, tile, rsplit > 1,
                                   !A.amajor && blockIdx.x == 0, dst, S, s_tok);
    if (bo.tile < 0) return;  // uniform across the workgroup
    tile = bo.tile;
    sub = bo.sub;
    pc.lora = bo.lora;
    pc.start = bo.start;
    pc.rows = bo.rows;
    __syncthreads();  // s_tok and the table are in LDS; the build scratch (s_part) is free
  } else {
    // ---- one round of loads: counts, the piece record, its tokens, the rank/scale table
    // (a large piece's record waits for the count, which places it) ----
    const int count = A.info[small ? 2 : 1];
    if (!small) {
      tile = blocked_tile(tile, count * rsplit);
      if (tile < 0) return;  // uniform
      sub = tile % rsplit;
      tile /= rsplit;
    }
    const int32_t* rec = A.tiles + (size_t)(small ? A.large_cap + tile : tile) * SGMV_TILE_INTS;
    pc.lora = rec[0];
    pc.start = rec[1];
    pc.rows = rec[2];
    if (!small && rsplit > 1) {  // part `sub` of the large piece: 16 of its rows
      pc.start += SGMV_SMALL_ROWS * sub;
      pc.rows = min(SGMV_SMALL_ROWS, pc.rows - SGMV_SMALL_ROWS * sub);
      if (pc.rows <= 0) return;  // uniform
    }
    if (small && tid < SGMV_SMALL_ROWS) s_tok[tid] = rec[16 + tid];
    if (table) {
      for (int i = tid; i < A.L; i += DT_THREADS) {
        s_rank[i] = A.rank[i];
        s_scale[i] = A.scale[i];
      }
    }
    if (tile >= count) return;  // uniform across the workgroup
    if (!small && tid < pc.rows) s_tok[tid] = A.sorted[pc.start + tid];
    __syncthreads();
  }
  // large pieces run as 16-row parts through the small-piece path
  const bool part = !small && rsplit > 1;
  if (part) small = true;
  pc.r = table ? s_rank[pc.lora] : A.rank[pc.lora];
  pc.scale = table ? s_scale[pc.lora] : A.scale[pc.lora];
  const int width = (((A.v_total + P - 1) / P) + 63) & ~63;
  pc.v0 = p * width;
  pc.v1 = min(pc.v0 + width, A.v_total);
  pc.tile = tile;
  pc.split = p;
  pc.nsplit = P;
  pc.xsub = part ? sub : -1;
  // a split with no columns still owes its K range to the exchange
  if (split && pc.v0 >= pc.v1 &&
      !(MODE == MODE_FUSED && XCH && (small && !part ? A.xch_small : A.xch_large)))
    return;

  const int nrk = (pc.r + 15) >> 4;
  if (MODE == MODE_EXPAND) {  // h from memory, scaled
    for (int idx = tid; idx < SGMV_TILE_ROWS * 64; idx += DT_THREADS) {
      const int row = idx >> 6, j = idx & 63;
      float v = 0.f;
      if (row < pc.rows && j < pc.r) v = A.h[(size_t)s_tok[row] * A.ldh + j] * pc.scale;
      s_h[row * HS + j] = v;
    }
  }
  run_piece<MODE, ALIGNED, NRKM, XCH>(A, pc, small, nrk, s_tok, s_part, s_h, &s_mask);

  if (MODE == MODE_SHRINK) {  // h (unscaled) of every row to memory; zeros up to R_max
    const int R = A.R_max;
    for (int idx = tid; idx < pc.rows * R; idx += DT_THREADS) {
      const int row = idx / R, j = idx - row * R;
      A.h[(size_t)s_tok[row] * A.ldh + j] = j < pc.r ? s_h[row * HS + j] : 0.f;
    }
  }
}


// Grid and dynamic LDS of a launch; the kernel arguments get the class boundary.
inline void delta_geometry(int mode, DeltaArgs& A, int& grid, size_t& lds, bool build = false) {
  const bool split = mode != MODE_SHRINK;
  // large slots: pieces, or their 16-row parts, rsplit slots per piece when the records are
  // read directly and densely numbered when built in the launch (every large piece has at
  // least 17 rows, so the parts number at most (M + 15 * large_cap) / 16)
  int large_slots = A.large_cap * A.rsplit;
  const int part_bound = (A.M + (SGMV_SMALL_ROWS - 1) * A.large_cap) / SGMV_SMALL_ROWS;
  if (build && A.rsplit > 1 && part_bound < large_slots) large_slots = part_bound;
  A.grid_large = class_grid(large_slots, split ? A.n_split_large : 1);
  grid = A.grid_large + class_grid(A.small_cap, split ? A.n_split_small : 1);
  // partial tiles of every wave (8 waves x R_pad/16 rank tiles x 1 KB); large pieces reuse
  // them for their h fragments, which fit for every rank
  lds = (size_t)DT_WAVES * (A.R_pad / 16) * 256 * sizeof(float);
  if (build && wg_build_lds_bytes(A.L) > lds) lds = wg_build_lds_bytes(A.L);  // aliases s_part
  // the h tile at SH_OFFSET, which also covers the staged shrink's ring
  if (lds < (size_t)(SH_OFFSET + SH_BYTES)) lds = (size_t)(SH_OFFSET + SH_BYTES);
  if (build && A.amajor) {
    // small slots per adapter first, then the large class, then the writer: large work is
    // rare in adapter-indexed batches, and its workgroups (which first check for it) then do
    // not put their id loads ahead of the small pieces' in the memory queues
    A.small_first = class_grid(A.L, split ? A.n_split_small : 1);
    grid = A.small_first + A.grid_large + 1;
    A.grid_writer = grid - 1;
  } else if (A.rsplit > 1) {
    // parts of large pieces (four slots per piece, most of them empty in decode-like batches)
    // after the small pieces, for the same reason
    A.small_first = class_grid(A.small_cap, split ? A.n_split_small : 1);
  }
}

}  // namespace sgmv
