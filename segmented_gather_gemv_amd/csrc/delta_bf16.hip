// bf16 multi-LoRA delta on gfx950 matrix cores.
//
// One workgroup (4 waves) takes one work descriptor (a piece of <= 64 rows of one segment,
// i.e. one adapter; Ascend article 3.3) and one range of output columns:
//
//   shrink  h[rows, r] = x[rows, :] @ A[l, :r, :]^T     (Ascend article 3.2, first stage)
//   expand  y[rows, cols] += scale_l * h @ B[l, cols, :r]^T   (second stage, scatter-add)
//
// Rows are gathered through sorted_token_ids (Punica page, code section). Both contractions
// run on v_mfma_f32_16x16x32_bf16 with fp32 accumulation. h never leaves the workgroup in
// the fused kernel (Ascend article 4.3): the shrink's partial tiles are reduced in LDS and
// the scaled fp32 h is split into hi + lo bf16 parts, so the expand keeps about 16
// significant bits of h instead of 8 (the pages keep the intermediate in fp32).
//
// Shrink work split: a piece has nrt = ceil(rows/16) row tiles; the 4 waves cover
// (row tile, K slice) pairs, so a decode piece (<= 16 rows) splits K four ways and a
// prefill piece splits rows. For every K step of 128, lane (c, g) loads 64 contiguous bytes
// of x row c and of A rank row c at k = 32 g .. 32 g + 31; the four 16-byte parts feed four
// MFMAs. Any assignment of k values to MFMA slots is valid for a contraction as long as x
// and A agree, and this one keeps every lane's loads contiguous.
//
// Expand: waves take 64-column groups in turn. MFMA q of a group covers columns
// v = 4 c + q of lane column c, so a lane's four accumulators hold four adjacent columns of
// one output row and y is read and written 8 bytes at a time. B is stored in rank octets
// ([l][j/8][n][8]), so one 16-byte load is one MFMA operand fragment (8 ranks of a column).
//
// Work order: large pieces first, then small ones; each piece owns n_split workgroups along
// the columns. Workgroup IDs are remapped so that consecutive work items land on the same
// XCD (workgroup i runs on XCD i % 8): the column splits of a piece, and the pieces of one
// segment, then share x rows and A/B through one L2.
#include "common.h"

namespace sgmv {

constexpr int DT_THREADS = 256;
constexpr int DT_WAVES = DT_THREADS / WAVE;
constexpr int KSTEP = 128;
constexpr int HS = 68;  // LDS row stride of the h tile (64 ranks + 4 pad floats)

struct WorkItem {
  int lora, start, rows, v0, v1;
};

// Maps this workgroup to (piece, column range). Returns false for spare workgroups.
__device__ __forceinline__ bool decode_work(const DeltaArgs& A, bool split_cols, WorkItem& wi) {
  const int n_large = A.info[1], n_small = A.info[2];
  const int PL = split_cols ? A.n_split_large : 1;
  const int PS = split_cols ? A.n_split_small : 1;
  const int work_l = n_large * PL;
  const int work = work_l + n_small * PS;
  const int b = blockIdx.x;
  const int per = (work + 7) >> 3;
  const int slot = b >> 3;
  if (slot >= per) return false;
  const int u = (b & 7) * per + slot;
  if (u >= work) return false;
  int tile, p, P;
  if (u < work_l) {
    tile = u / PL;
    p = u - tile * PL;
    P = PL;
  } else {
    const int v = u - work_l;
    tile = A.large_cap + v / PS;
    p = v % PS;
    P = PS;
  }
  const int32_t* d = A.tiles + (size_t)tile * 4;
  wi.lora = d[0];
  wi.start = d[1];
  wi.rows = d[2];
  const int width = (((A.v_total + P - 1) / P) + 63) & ~63;
  wi.v0 = p * width;
  wi.v1 = min(wi.v0 + width, A.v_total);
  return !split_cols || wi.v0 < wi.v1;
}

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

// Shrink of one piece into s_h (fp32, [row][rank], row stride HS); columns >= r are 0.
template <int NRK, bool ALIGNED>
__device__ void shrink_piece(const DeltaArgs& A, const WorkItem& wi, int r, float mult,
                             const int* s_tok, float* s_part, float* s_h) {
  const int tid = threadIdx.x, w = tid / WAVE, lane = tid & (WAVE - 1);
  const int c = lane & 15, g = lane >> 4;
  const int nrt = (wi.rows + 15) >> 4;
  const int ntp = nrt == 1 ? 1 : (nrt == 2 ? 2 : 4);
  const int ks = DT_WAVES / ntp;
  const int rt = w % ntp, kslice = w / ntp;
  f32x4_t acc[NRK];
#pragma unroll
  for (int i = 0; i < NRK; ++i) acc[i] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  if (rt < nrt) {
    const int row = rt * 16 + c;
    const bool vx = row < wi.rows;
    const uint16_t* xr =
        static_cast<const uint16_t*>(A.x) + (size_t)(vx ? s_tok[row] : 0) * (size_t)A.ldx;
    const uint16_t* ab = static_cast<const uint16_t*>(A.a) + (size_t)wi.lora * A.R_pad * A.K_pad;
    const int nch = (A.K + KSTEP - 1) / KSTEP;
    const int c0 = kslice * nch / ks, c1 = (kslice + 1) * nch / ks;
    for (int ch = c0; ch < c1; ++ch) {
      const int kb = ch * KSTEP + 32 * g;
      u32x4_t xv[4], av[NRK][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int k = kb + 8 * i;
        xv[i] = load_x8<ALIGNED>(xr, k, A.K, vx);
#pragma unroll
        for (int rk = 0; rk < NRK; ++rk) {
          const int j = rk * 16 + c;
          av[rk][i] = (j < r && k < A.K) ? load_u32x4(ab + (size_t)j * A.K_pad + k)
                                         : u32x4_t{0u, 0u, 0u, 0u};
        }
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int rk = 0; rk < NRK; ++rk)
          acc[rk] = mfma_16x16x32_bf16(as_bf16x8(xv[i]), as_bf16x8(av[rk][i]), acc[rk]);
    }
  }
  // D layout: lane (c, g) holds rows 4g..4g+3 of column c
#pragma unroll
  for (int rk = 0; rk < NRK; ++rk)
#pragma unroll
    for (int e = 0; e < 4; ++e) s_part[((w * NRK + rk) * 16 + 4 * g + e) * 16 + c] = acc[rk][e];
  __syncthreads();
  const int ncol = NRK * 16, nrow = nrt * 16;
  for (int idx = tid; idx < nrow * ncol; idx += DT_THREADS) {
    const int row = idx / ncol, j = idx - row * ncol;
    const int rtt = row >> 4, rr = row & 15, rk = j >> 4, cc = j & 15;
    float s = 0.f;
    for (int q = 0; q < ks; ++q) s += s_part[(((q * ntp + rtt) * NRK + rk) * 16 + rr) * 16 + cc];
    s_h[row * HS + j] = j < r ? s * mult : 0.f;
  }
  __syncthreads();
}

// hi/lo bf16 operand fragments of the scaled h tile, written once to LDS (s_pf, 16-byte
// entries, [row tile][rank tile][lane]). Lane (c, g) of fragment (rt, rk) holds row
// rt*16 + c, ranks rk*16 + 8*(g&1) + 0..7: the hi part for g < 2 and the lo part
// (h - hi, rounded) for g >= 2, so one K=32 MFMA sums hi*B + lo*B over 16 ranks.
template <int NRK>
__device__ void build_fragments(const WorkItem& wi, const float* s_h, u32x4_t* s_pf) {
  const int tid = threadIdx.x, w = tid / WAVE, lane = tid & (WAVE - 1);
  const int c = lane & 15, g = lane >> 4;
  const int nrt = (wi.rows + 15) >> 4;
  for (int f = w; f < nrt * NRK; f += DT_WAVES) {
    const int rt = f / NRK, rk = f - rt * NRK;
    const float* hp = s_h + (rt * 16 + c) * HS + rk * 16 + 8 * (g & 1);
    u32x4_t pk;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      uint32_t bits[2];
#pragma unroll
      for (int z = 0; z < 2; ++z) {
        const float v = hp[e + z];
        const uint32_t hb = f32_to_bf16_bits(v);
        bits[z] = g < 2 ? hb : f32_to_bf16_bits(v - bf16_bits_to_f32(hb));
      }
      pk[e >> 1] = bits[0] | (bits[1] << 16);
    }
    s_pf[f * WAVE + lane] = pk;
  }
  __syncthreads();
}

// Expand of one piece: y[rows, cols] += h_scaled @ B^T, h fragments from s_pf.
template <int NRK, bool ALIGNED>
__device__ void expand_piece(const DeltaArgs& A, const WorkItem& wi, int r, const int* s_tok,
                             const u32x4_t* s_pf) {
  const int tid = threadIdx.x, w = tid / WAVE, lane = tid & (WAVE - 1);
  const int c = lane & 15, g = lane >> 4;
  const int nrt = (wi.rows + 15) >> 4;
  const uint16_t* bb =
      static_cast<const uint16_t*>(A.b) + (size_t)wi.lora * (A.R_pad / 8) * A.N_pad * 8;
  for (int vg = wi.v0 + 64 * w; vg < wi.v1; vg += 64 * DT_WAVES) {
    const int vl = vg + 4 * c;  // first of this lane's four columns
    ColMap cm[4];
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
    // B fragments of every rank tile for this lane's four columns, kept across row tiles
    u32x4_t bq[NRK][4];
#pragma unroll
    for (int rk = 0; rk < NRK; ++rk) {
      const int o = rk * 2 + (g & 1);
      const int live = r - 8 * o;  // live ranks in this octet
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        bq[rk][q] = (live > 0 && vl + q < wi.v1)
                        ? load_u32x4(bb + ((size_t)o * A.N_pad + cm[q].n) * 8)
                        : u32x4_t{0u, 0u, 0u, 0u};
        if (live > 0 && live < 8) {
#pragma unroll
          for (int e = 0; e < 8; ++e)
            if (e >= live) bq[rk][q][e >> 1] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
        }
      }
    }
    for (int rt = 0; rt < nrt; ++rt) {
      f32x4_t yacc[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) yacc[q] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int rk = 0; rk < NRK; ++rk) {
        const bf16x8_t P = as_bf16x8(s_pf[(rt * NRK + rk) * WAVE + lane]);
#pragma unroll
        for (int q = 0; q < 4; ++q) yacc[q] = mfma_16x16x32_bf16(P, as_bf16x8(bq[rk][q]), yacc[q]);
      }
      // y += delta; D layout: lane (c, g) holds rows 4g..4g+3 of its four columns
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = rt * 16 + 4 * g + e;
        if (row >= wi.rows) continue;
        const size_t tok = (size_t)s_tok[row];
        if (ALIGNED) {
          if (vl >= wi.v1) continue;
          uint16_t* yp = cm[0].y + tok * (size_t)cm[0].ldy + cm[0].col;
          uint2 yv = *reinterpret_cast<const uint2*>(yp);
          const float d0 = bf16_bits_to_f32(yv.x & 0xffffu) + yacc[0][e];
          const float d1 = bf16_bits_to_f32(yv.x >> 16) + yacc[1][e];
          const float d2 = bf16_bits_to_f32(yv.y & 0xffffu) + yacc[2][e];
          const float d3 = bf16_bits_to_f32(yv.y >> 16) + yacc[3][e];
          yv.x = f32_to_bf16_bits(d0) | (f32_to_bf16_bits(d1) << 16);
          yv.y = f32_to_bf16_bits(d2) | (f32_to_bf16_bits(d3) << 16);
          *reinterpret_cast<uint2*>(yp) = yv;
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (vl + q >= wi.v1) continue;
            uint16_t* yp = cm[q].y + tok * (size_t)cm[q].ldy + cm[q].col;
            *yp = (uint16_t)f32_to_bf16_bits(bf16_bits_to_f32(*yp) + yacc[q][e]);
          }
        }
      }
    }
  }
}

template <int MODE, bool ALIGNED>
__global__ __launch_bounds__(DT_THREADS) void delta_bf16_kernel(DeltaArgs A) {
  __shared__ int s_tok[SGMV_TILE_ROWS];
  __shared__ __align__(16) float s_part[DT_WAVES * 4 * 256];
  __shared__ __align__(16) float s_h[SGMV_TILE_ROWS * HS];
  WorkItem wi;
  if (!decode_work(A, MODE != MODE_SHRINK, wi)) return;
  const int r = A.rank[wi.lora];
  const float scale = A.scale[wi.lora];
  const int tid = threadIdx.x;
  if (tid < SGMV_TILE_ROWS) s_tok[tid] = tid < wi.rows ? A.sorted[wi.start + tid] : 0;
  __syncthreads();
  const int nrk = (r + 15) >> 4;

  if (MODE == MODE_EXPAND) {
    for (int idx = tid; idx < SGMV_TILE_ROWS * 64; idx += DT_THREADS) {
      const int row = idx >> 6, j = idx & 63;
      float v = 0.f;
      if (row < wi.rows && j < r) v = A.h[(size_t)s_tok[row] * A.ldh + j] * scale;
      s_h[row * HS + j] = v;
    }
    __syncthreads();
  } else {
    const float mult = MODE == MODE_SHRINK ? 1.f : scale;
    switch (nrk) {
      case 1: shrink_piece<1, ALIGNED>(A, wi, r, mult, s_tok, s_part, s_h); break;
      case 2: shrink_piece<2, ALIGNED>(A, wi, r, mult, s_tok, s_part, s_h); break;
      case 3: shrink_piece<3, ALIGNED>(A, wi, r, mult, s_tok, s_part, s_h); break;
      default: shrink_piece<4, ALIGNED>(A, wi, r, mult, s_tok, s_part, s_h); break;
    }
  }

  if (MODE == MODE_SHRINK) {
    const int R = A.R_max;
    for (int idx = tid; idx < wi.rows * R; idx += DT_THREADS) {
      const int row = idx / R, j = idx - row * R;
      A.h[(size_t)s_tok[row] * A.ldh + j] = j < r ? s_h[row * HS + j] : 0.f;
    }
    return;
  }
  u32x4_t* s_pf = reinterpret_cast<u32x4_t*>(s_part);  // s_part is free after the shrink
  switch (nrk) {
    case 1: build_fragments<1>(wi, s_h, s_pf); expand_piece<1, ALIGNED>(A, wi, r, s_tok, s_pf); break;
    case 2: build_fragments<2>(wi, s_h, s_pf); expand_piece<2, ALIGNED>(A, wi, r, s_tok, s_pf); break;
    case 3: build_fragments<3>(wi, s_h, s_pf); expand_piece<3, ALIGNED>(A, wi, r, s_tok, s_pf); break;
    default: build_fragments<4>(wi, s_h, s_pf); expand_piece<4, ALIGNED>(A, wi, r, s_tok, s_pf); break;
  }
}

hipError_t launch_delta_bf16(int mode, bool aligned, const DeltaArgs& A, int grid,
                             hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  const dim3 g(grid), b(DT_THREADS);
#define SGMV_LAUNCH(M_, AL_) hipLaunchKernelGGL((delta_bf16_kernel<M_, AL_>), g, b, 0, stream, A)
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
