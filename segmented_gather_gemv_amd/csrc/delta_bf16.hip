// bf16 multi-LoRA delta on gfx950 matrix cores.
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
#include "common.h"

namespace sgmv {

constexpr int DT_THREADS = 512;
constexpr int DT_WAVES = DT_THREADS / WAVE;
constexpr int KSTEP = 128;
constexpr int HS = 68;                // LDS row stride of the h tile (64 ranks + 4 pad floats)
constexpr int RANK_TABLE_MAX = 2048;  // pools up to this size get rank/scale staged in LDS

struct Piece {
  int lora, start, rows, r;
  float scale;
  int v0, v1;  // column range, in the concatenation of the output slices
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

// Old y of rows 4g..4g+3 of row tile rt at this lane's four columns (aligned path).
template <bool ALIGNED>
__device__ __forceinline__ void load_y(const int* s_tok, int rows, int rt, int g, int vl, int v1,
                                       const ColMap (&cm)[4], uint2 (&yv)[4]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int row = rt * 16 + 4 * g + e;
    yv[e] = make_uint2(0u, 0u);
    if (ALIGNED && row < rows && vl < v1)
      yv[e] = *reinterpret_cast<const uint2*>(cm[0].y + (size_t)s_tok[row] * (size_t)cm[0].ldy +
                                              cm[0].col);
  }
}

// y update of one row tile: yv holds the old values (aligned path), yacc the delta.
template <bool ALIGNED>
__device__ __forceinline__ void store_y(const int* s_tok, int rows, int rt, int g, int vl, int v1,
                                        const ColMap (&cm)[4], const uint2 (&yv)[4],
                                        const f32x4_t (&yacc)[4]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int row = rt * 16 + 4 * g + e;
    if (row >= rows) continue;
    const size_t tok = (size_t)s_tok[row];
    if (ALIGNED) {
      if (vl >= v1) continue;
      uint16_t* yp = cm[0].y + tok * (size_t)cm[0].ldy + cm[0].col;
      uint2 v = yv[e];
      const float d0 = bf16_bits_to_f32(v.x & 0xffffu) + yacc[0][e];
      const float d1 = bf16_bits_to_f32(v.x >> 16) + yacc[1][e];
      const float d2 = bf16_bits_to_f32(v.y & 0xffffu) + yacc[2][e];
      const float d3 = bf16_bits_to_f32(v.y >> 16) + yacc[3][e];
      v.x = f32_to_bf16_bits(d0) | (f32_to_bf16_bits(d1) << 16);
      v.y = f32_to_bf16_bits(d2) | (f32_to_bf16_bits(d3) << 16);
      *reinterpret_cast<uint2*>(yp) = v;
    } else {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (vl + q >= v1) continue;
        uint16_t* yp = cm[q].y + tok * (size_t)cm[q].ldy + cm[q].col;
        *yp = (uint16_t)f32_to_bf16_bits(bf16_bits_to_f32(*yp) + yacc[q][e]);
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

// hi and lo bf16 operand fragments of the h tile into s_pf ([row tile][rank tile of 32][hi,
// lo][lane], 16 B each). Lane (c, g) of fragment (rt, re) holds row rt*16 + c, ranks
// re*32 + 8g + 0..7; the lo part is h - hi, rounded, so hi + lo keeps about 16 bits of h.
template <int NE>
__device__ void build_fragments(int nrt, const float* s_h, u32x4_t* s_pf) {
  const int w = threadIdx.x / WAVE, lane = threadIdx.x & (WAVE - 1);
  const int c = lane & 15, g = lane >> 4;
  for (int f = w; f < nrt * NE; f += DT_WAVES) {
    const int rt = f / NE, re = f - rt * NE;
    const float* hp = s_h + (rt * 16 + c) * HS + re * 32 + 8 * g;
    u32x4_t hi, lo;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      uint32_t hb[2], lb[2];
#pragma unroll
      for (int z = 0; z < 2; ++z) {
        const float v = hp[e + z];
        hb[z] = f32_to_bf16_bits(v);
        lb[z] = f32_to_bf16_bits(v - bf16_bits_to_f32(hb[z]));
      }
      hi[e >> 1] = hb[0] | (hb[1] << 16);
      lo[e >> 1] = lb[0] | (lb[1] << 16);
    }
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

// B fragments and old y of the first PF column groups of a wave (small pieces), loaded
// before the shrink's MFMAs so their latency overlaps the shrink.
template <int NE, int PF, bool ALIGNED>
struct ExpandPrefetch {
  ColMap cm[PF][4];
  u32x4_t bq[PF][NE][4];
  uint2 yv[PF][4];
  __device__ __forceinline__ void load(const DeltaArgs& A, const uint16_t* bb, const Piece& pc,
                                       const int* s_tok, int w, int c, int g) {
#pragma unroll
    for (int f = 0; f < PF; ++f) {
      const int vl = pc.v0 + 64 * (w + DT_WAVES * f) + 4 * c;
      map_group<ALIGNED>(A, vl, cm[f]);
      load_b_group<NE>(bb, A.N_pad, pc.r, vl, pc.v1, g, cm[f], bq[f]);
      load_y<ALIGNED>(s_tok, pc.rows, 0, g, vl, pc.v1, cm[f], yv[f]);
    }
  }
};

// ---------------------------------------------------------------------------------------
// small pieces (<= 16 rows): K split across the 8 waves, expand operands prefetched
// ---------------------------------------------------------------------------------------
template <int MODE, int NRK, bool ALIGNED>
__device__ __forceinline__ void small_piece(const DeltaArgs& A, const Piece& pc, const int* s_tok, float* s_part,
                            float* s_h) {
  const int tid = threadIdx.x, w = tid / WAVE, lane = tid & (WAVE - 1);
  const int c = lane & 15, g = lane >> 4;
  // K steps whose loads are issued together, and column groups per wave whose B and y are
  // prefetched, sized so that everything in flight fits in registers
  constexpr int NSTEP = NRK == 1 ? 4 : (NRK == 2 ? 2 : 1);
  constexpr int PF = NRK == 1 ? 2 : 1;
  constexpr int NE = (NRK + 1) / 2;  // expand rank tiles of 32
  const uint16_t* bb =
      static_cast<const uint16_t*>(A.b) + (size_t)pc.lora * (A.R_pad / 8) * A.N_pad * 8;

  ExpandPrefetch<NE, PF, ALIGNED> pf;
  bool fetched = false;

  if (MODE != MODE_EXPAND) {
    f32x4_t acc[NRK];
#pragma unroll
    for (int i = 0; i < NRK; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    const bool vx = c < pc.rows;
    const uint16_t* xr =
        static_cast<const uint16_t*>(A.x) + (size_t)(vx ? s_tok[c] : 0) * (size_t)A.ldx;
    const uint16_t* ab = static_cast<const uint16_t*>(A.a) + (size_t)pc.lora * A.R_pad * A.K_pad;
    const int nch = (A.K + KSTEP - 1) / KSTEP;
    const int c0 = w * nch / DT_WAVES, c1 = (w + 1) * nch / DT_WAVES;
    for (int ch = c0; ch < c1; ch += NSTEP) {
      ShrinkSteps<NRK, NSTEP, ALIGNED> S;
      S.load(xr, vx, ab, A.K_pad, A.K, pc.r, ch, c1, c, g);
      if (MODE == MODE_FUSED && !fetched) {  // rides along the first loads
        pf.load(A, bb, pc, s_tok, w, c, g);
        fetched = true;
      }
      S.mfma(acc);
    }
    // D layout: lane (c, g) holds rows 4g..4g+3 of column c
#pragma unroll
    for (int rk = 0; rk < NRK; ++rk)
#pragma unroll
      for (int e = 0; e < 4; ++e) s_part[((w * NRK + rk) * 16 + 4 * g + e) * 16 + c] = acc[rk][e];
  }
  if (MODE != MODE_SHRINK && !fetched) pf.load(A, bb, pc, s_tok, w, c, g);
  __syncthreads();
  if (MODE != MODE_EXPAND)
    reduce_partials<NRK>(1, 1, DT_WAVES, pc.r, MODE == MODE_SHRINK ? 1.f : pc.scale, s_part, s_h);
  __syncthreads();
  if (MODE == MODE_SHRINK) return;

  u32x4_t* s_pf = reinterpret_cast<u32x4_t*>(s_part);  // free once the partials are summed
  build_fragments<NE>(1, s_h, s_pf);
  __syncthreads();
  bf16x8_t P[NE][2];
  read_fragments<NE>(s_pf, 0, lane, P);

  // prefetched groups
#pragma unroll
  for (int f = 0; f < PF; ++f) {
    const int vg = pc.v0 + 64 * (w + DT_WAVES * f);
    if (vg >= pc.v1) continue;
    f32x4_t yacc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) yacc[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    expand_mfma<NE>(P, pf.bq[f], yacc);
    store_y<ALIGNED>(s_tok, pc.rows, 0, g, vg + 4 * c, pc.v1, pf.cm[f], pf.yv[f], yacc);
  }
  // remaining groups
  for (int vg = pc.v0 + 64 * (w + DT_WAVES * PF); vg < pc.v1; vg += 64 * DT_WAVES) {
    const int vl = vg + 4 * c;
    ColMap cg[4];
    map_group<ALIGNED>(A, vl, cg);
    u32x4_t b2[NE][4];
    uint2 y2[4];
    load_b_group<NE>(bb, A.N_pad, pc.r, vl, pc.v1, g, cg, b2);
    load_y<ALIGNED>(s_tok, pc.rows, 0, g, vl, pc.v1, cg, y2);
    f32x4_t yacc[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) yacc[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    expand_mfma<NE>(P, b2, yacc);
    store_y<ALIGNED>(s_tok, pc.rows, 0, g, vl, pc.v1, cg, y2, yacc);
  }
}

// ---------------------------------------------------------------------------------------
// large pieces (17..64 rows): waves cover (row tile, K slice) pairs and stream K
// ---------------------------------------------------------------------------------------
template <int MODE, int NRK, bool ALIGNED>
__device__ __forceinline__ void large_piece(const DeltaArgs& A, const Piece& pc, const int* s_tok, float* s_part,
                            float* s_h) {
  const int tid = threadIdx.x, w = tid / WAVE, lane = tid & (WAVE - 1);
  const int c = lane & 15, g = lane >> 4;
  const int nrt = (pc.rows + 15) >> 4;  // 2..4
  const int ntp = nrt == 2 ? 2 : 4;
  const int ks = DT_WAVES / ntp;
  if (MODE != MODE_EXPAND) {
    constexpr int NSTEP = NRK <= 2 ? 2 : 1;
    const int rt = w % ntp, kslice = w / ntp;
    f32x4_t acc[NRK];
#pragma unroll
    for (int i = 0; i < NRK; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (rt < nrt) {
      const int row = rt * 16 + c;
      const bool vx = row < pc.rows;
      const uint16_t* xr =
          static_cast<const uint16_t*>(A.x) + (size_t)(vx ? s_tok[row] : 0) * (size_t)A.ldx;
      const uint16_t* ab =
          static_cast<const uint16_t*>(A.a) + (size_t)pc.lora * A.R_pad * A.K_pad;
      const int nch = (A.K + KSTEP - 1) / KSTEP;
      const int c0 = kslice * nch / ks, c1 = (kslice + 1) * nch / ks;
      for (int ch = c0; ch < c1; ch += NSTEP) {
        ShrinkSteps<NRK, NSTEP, ALIGNED> S;
        S.load(xr, vx, ab, A.K_pad, A.K, pc.r, ch, c1, c, g);
        S.mfma(acc);
      }
    }
#pragma unroll
    for (int rk = 0; rk < NRK; ++rk)
#pragma unroll
      for (int e = 0; e < 4; ++e) s_part[((w * NRK + rk) * 16 + 4 * g + e) * 16 + c] = acc[rk][e];
    __syncthreads();
    reduce_partials<NRK>(nrt, ntp, ks, pc.r, MODE == MODE_SHRINK ? 1.f : pc.scale, s_part, s_h);
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
    for (int rt = 0; rt < nrt; ++rt) {
      uint2 yv[4];
      load_y<ALIGNED>(s_tok, pc.rows, rt, g, vl, pc.v1, cm, yv);
      bf16x8_t P[NE][2];
      read_fragments<NE>(s_pf, rt, lane, P);
      f32x4_t yacc[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) yacc[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      expand_mfma<NE>(P, bq, yacc);
      store_y<ALIGNED>(s_tok, pc.rows, rt, g, vl, pc.v1, cm, yv, yacc);
    }
  }
}

template <int MODE, bool ALIGNED>
__global__ __launch_bounds__(DT_THREADS) void delta_bf16_kernel(DeltaArgs A) {
  __shared__ int s_tok[SGMV_TILE_ROWS];
  __shared__ __align__(16) float s_h[SGMV_TILE_ROWS * HS];
  __shared__ int s_rank[RANK_TABLE_MAX];
  __shared__ float s_scale[RANK_TABLE_MAX];
  // partial shrink tiles, [wave][rank tile][16][16] fp32 (R_pad/16 rank tiles); reused for
  // the expand's h fragments afterwards
  extern __shared__ __align__(16) float s_part[];

  // ---- which piece and column split (from the workgroup index alone) ----
  const bool split = MODE != MODE_SHRINK;
  bool small;
  int tile, p, P;
  if (!locate_piece(A, split, small, tile, p, P)) return;

  // ---- one round of loads: counts, the piece record, its tokens, the rank/scale table ----
  const int tid = threadIdx.x;
  const int32_t* rec = A.tiles + (size_t)(small ? A.large_cap + tile : tile) * SGMV_TILE_INTS;
  const int count = A.info[small ? 2 : 1];
  Piece pc;
  pc.lora = rec[0];
  pc.start = rec[1];
  pc.rows = rec[2];
  const bool table = A.L <= RANK_TABLE_MAX;
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
  pc.r = table ? s_rank[pc.lora] : A.rank[pc.lora];
  pc.scale = table ? s_scale[pc.lora] : A.scale[pc.lora];
  const int width = (((A.v_total + P - 1) / P) + 63) & ~63;
  pc.v0 = p * width;
  pc.v1 = min(pc.v0 + width, A.v_total);
  if (split && pc.v0 >= pc.v1) return;

  const int nrk = (pc.r + 15) >> 4;
  if (MODE == MODE_EXPAND) {  // h from memory, scaled
    for (int idx = tid; idx < SGMV_TILE_ROWS * 64; idx += DT_THREADS) {
      const int row = idx >> 6, j = idx & 63;
      float v = 0.f;
      if (row < pc.rows && j < pc.r) v = A.h[(size_t)s_tok[row] * A.ldh + j] * pc.scale;
      s_h[row * HS + j] = v;
    }
  }
#define SGMV_PIECE(FN)                                               \
  switch (nrk) {                                                     \
    case 1: FN<MODE, 1, ALIGNED>(A, pc, s_tok, s_part, s_h); break;  \
    case 2: FN<MODE, 2, ALIGNED>(A, pc, s_tok, s_part, s_h); break;  \
    case 3: FN<MODE, 3, ALIGNED>(A, pc, s_tok, s_part, s_h); break;  \
    default: FN<MODE, 4, ALIGNED>(A, pc, s_tok, s_part, s_h); break; \
  }
  if (small) {
    SGMV_PIECE(small_piece)
  } else {
    SGMV_PIECE(large_piece)
  }
#undef SGMV_PIECE

  if (MODE == MODE_SHRINK) {  // h (unscaled) of every row to memory; zeros up to R_max
    const int R = A.R_max;
    for (int idx = tid; idx < pc.rows * R; idx += DT_THREADS) {
      const int row = idx / R, j = idx - row * R;
      A.h[(size_t)s_tok[row] * A.ldh + j] = j < pc.r ? s_h[row * HS + j] : 0.f;
    }
  }
}

hipError_t launch_delta_bf16(int mode, bool aligned, DeltaArgs A, LaunchEvents ev,
                             hipStream_t stream) {
  const bool split = mode != MODE_SHRINK;
  A.grid_large = class_grid(A.large_cap, split ? A.n_split_large : 1);
  const int grid = A.grid_large + class_grid(A.small_cap, split ? A.n_split_small : 1);
  if (grid <= 0) return hipSuccess;
  const dim3 g(grid), b(DT_THREADS);
  // partial tiles of every wave; at least 16 KB, which also holds the h fragments
  const size_t lds = (size_t)DT_WAVES * (A.R_pad / 16) * 256 * sizeof(float);
#define SGMV_LAUNCH(M_, AL_) \
  hipExtLaunchKernelGGL((delta_bf16_kernel<M_, AL_>), g, b, lds, stream, ev.start, ev.stop, 0, A)
  if (mode == MODE_FUSED) {
    if (aligned) SGMV_LAUNCH(MODE_FUSED, true); else SGMV_LAUNCH(MODE_FUSED, false);
  } else if (mode == MODE_SHRINK) {
    if (aligned) SGMV_LAUNCH(MODE_SHRINK, true); else SGMV_LAUNCH(MODE_SHRINK, false);
  } else {
    if (aligned) SGMV_LAUNCH(MODE_EXPAND, true); else SGMV_LAUNCH(MODE_EXPAND, false);
  }
#undef SGMV_LAUNCH
  return hipGetLastError();
}

}  // namespace sgmv
