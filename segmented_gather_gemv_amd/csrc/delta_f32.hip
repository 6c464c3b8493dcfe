// fp32 multi-LoRA delta on the vector ALU.
//
// Same work descriptors, column splits and workgroup mapping as the bf16 matrix-core path,
// with plain fp32 fused multiply-adds: the shrink gives each group of 16 lanes one (row,
// rank) pair at a time, its lanes splitting K (Ascend article 3.2, first stage); the expand
// gives each thread one output column, streams that column's rank octets of B and updates
// every row of the piece (second stage). Used for fp32 pools, whose products the bf16
// matrix cores cannot take; not tuned for speed.
#include "common.h"

namespace sgmv {

constexpr int F_THREADS = 256;
constexpr int F_HS = 65;  // LDS row stride of the h tile

// Expand of one piece over columns [v0, v1), one column per thread: y[tokens, col] += the
// first NR rows of the h tile (rows past `rows` are zero) times that column's ranks of B.
template <int NR>
__device__ __forceinline__ void expand_columns(const DeltaArgs& A, const float* bb,
                                               const float* s_h, const int* s_tok, int rows,
                                               int r, int v0, int v1) {
  for (int v = v0 + (int)threadIdx.x; v < v1; v += F_THREADS) {
    float* yb = static_cast<float*>(A.slices[0].y);
    int64_t ldy = A.slices[0].ldy;
    int col = v, n = A.slices[0].n_begin + v;
#pragma unroll
    for (int i = 1; i < SGMV_MAX_SLICES; ++i) {
      if (i < A.n_slices && v >= A.slices[i].v_begin) {
        yb = static_cast<float*>(A.slices[i].y);
        ldy = A.slices[i].ldy;
        col = v - A.slices[i].v_begin;
        n = A.slices[i].n_begin + col;
      }
    }
    float acc[NR];
#pragma unroll
    for (int row = 0; row < NR; ++row) acc[row] = 0.f;
    for (int j = 0; j < r; ++j) {
      const float bj = bb[((size_t)(j >> 3) * A.N_pad + n) * 8 + (j & 7)];
#pragma unroll
      for (int row = 0; row < NR; ++row) acc[row] = fmaf(s_h[row * F_HS + j], bj, acc[row]);
    }
    // the old y of 16 rows at a time, all loaded before any is stored
#pragma unroll
    for (int r0 = 0; r0 < NR; r0 += 16) {
      if (r0 >= rows) break;
      float yo[16];
#pragma unroll
      for (int i = 0; i < 16; ++i)
        yo[i] = r0 + i < rows ? yb[(size_t)s_tok[r0 + i] * (size_t)ldy + col] : 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i)
        if (r0 + i < rows) yb[(size_t)s_tok[r0 + i] * (size_t)ldy + col] = yo[i] + acc[r0 + i];
    }
  }
}

template <int MODE>
__global__ __launch_bounds__(F_THREADS) void delta_f32_kernel(DeltaArgs A) {
  __shared__ int s_tok[SGMV_TILE_ROWS];
  __shared__ float s_h[SGMV_TILE_ROWS * F_HS];
  bool small;
  int tile, p, P;
  if (!locate_piece(A, MODE != MODE_SHRINK, small, tile, p, P)) return;
  const int32_t* rec = A.tiles + (size_t)(small ? A.large_cap + tile : tile) * SGMV_TILE_INTS;
  if (tile >= A.info[small ? 2 : 1]) return;
  struct {
    int lora, start, rows, v0, v1;
  } wi;
  wi.lora = rec[0];
  wi.start = rec[1];
  wi.rows = rec[2];
  const int width = (((A.v_total + P - 1) / P) + 63) & ~63;
  wi.v0 = p * width;
  wi.v1 = min(wi.v0 + width, A.v_total);
  if (MODE != MODE_SHRINK && wi.v0 >= wi.v1) return;
  const int r = A.rank[wi.lora];
  const float scale = A.scale[wi.lora];
  const int tid = threadIdx.x;
  if (tid < SGMV_TILE_ROWS) s_tok[tid] = tid < wi.rows ? A.sorted[wi.start + tid] : 0;
  __syncthreads();

  if (MODE == MODE_EXPAND) {
    for (int idx = tid; idx < SGMV_TILE_ROWS * 64; idx += F_THREADS) {
      const int row = idx >> 6, j = idx & 63;
      float v = 0.f;
      if (row < wi.rows && j < r) v = A.h[(size_t)s_tok[row] * A.ldh + j] * scale;
      s_h[row * F_HS + j] = v;
    }
  } else {
    // four live (row, rank) pairs per wave at a time, 16 lanes each: lane l of a group takes
    // k = l, l + 16, ... (coalesced, independent loads), then a butterfly sum over the group's
    // lanes in a fixed order
    constexpr int GL = 16, GPW = WAVE / GL;
    const float mult = MODE == MODE_SHRINK ? 1.f : scale;
    const float* ab = static_cast<const float*>(A.a) + (size_t)wi.lora * A.R_pad * A.K_pad;
    for (int idx = tid; idx < SGMV_TILE_ROWS * 64; idx += F_THREADS)
      s_h[(idx >> 6) * F_HS + (idx & 63)] = 0.f;
    __syncthreads();
    const int lane = tid & (WAVE - 1), wv = tid / WAVE, sub = lane / GL, gl = lane % GL;
    const int rr = r > 0 ? r : 1, npair = wi.rows * r;
    for (int q0 = wv * GPW; q0 < npair; q0 += (F_THREADS / WAVE) * GPW) {  // wave-uniform
      const int q = q0 + sub;
      const bool live = q < npair;
      const int row = live ? q / rr : 0, j = live ? q - row * rr : 0;
      float s = 0.f;
      if (live) {
        const float* xr = static_cast<const float*>(A.x) + (size_t)s_tok[row] * (size_t)A.ldx;
        const float* ar = ab + (size_t)j * A.K_pad;
        for (int k = gl; k < A.K; k += GL) s = fmaf(xr[k], ar[k], s);
      }
#pragma unroll
      for (int off = GL / 2; off > 0; off >>= 1) s += __shfl_xor(s, off);
      if (live && gl == 0) s_h[row * F_HS + j] = s * mult;
    }
  }
  __syncthreads();

  if (MODE == MODE_SHRINK) {
    const int R = A.R_max;
    for (int idx = tid; idx < wi.rows * R; idx += F_THREADS) {
      const int row = idx / R, j = idx - row * R;
      A.h[(size_t)s_tok[row] * A.ldh + j] = j < r ? s_h[row * F_HS + j] : 0.f;
    }
    return;
  }

  const float* bb = static_cast<const float*>(A.b) + (size_t)wi.lora * (A.R_pad / 8) * A.N_pad * 8;
  if (wi.rows <= 16)  // uniform: a piece accumulates only the rows it can have
    expand_columns<16>(A, bb, s_h, s_tok, wi.rows, r, wi.v0, wi.v1);
  else if (wi.rows <= 32)
    expand_columns<32>(A, bb, s_h, s_tok, wi.rows, r, wi.v0, wi.v1);
  else
    expand_columns<SGMV_TILE_ROWS>(A, bb, s_h, s_tok, wi.rows, r, wi.v0, wi.v1);
}

hipError_t launch_delta_f32(int mode, DeltaArgs A, LaunchEvents ev, hipStream_t stream) {
  const bool split = mode != MODE_SHRINK;
  A.grid_large = class_grid(A.large_cap, split ? A.n_split_large : 1);
  const int grid = A.grid_large + class_grid(A.small_cap, split ? A.n_split_small : 1);
  if (grid <= 0) return hipSuccess;
  const dim3 g(grid), b(F_THREADS);
  if (mode == MODE_FUSED)
    hipExtLaunchKernelGGL(delta_f32_kernel<MODE_FUSED>, g, b, 0, stream, ev.start, ev.stop, 0, A);
  else if (mode == MODE_SHRINK)
    hipExtLaunchKernelGGL(delta_f32_kernel<MODE_SHRINK>, g, b, 0, stream, ev.start, ev.stop, 0, A);
  else
    hipExtLaunchKernelGGL(delta_f32_kernel<MODE_EXPAND>, g, b, 0, stream, ev.start, ev.stop, 0, A);
  return hipGetLastError();
}

}  // namespace sgmv
