// Merged weight of one adapter: W' = W + scale_l * B_l A_l (Ascend article 1.1 and 4.4: when a
// batch holds one or two long-lived adapters, the adapter can be merged into the base weight
// and the plain GEMM run instead of the unmerged delta; Punica page, SGMV section: the merged
// and unmerged forms give the same product).
//
// W is [N][ldw] with rows = outputs, as in y = x W^T. The rank-r product B_l A_l is a dense
// contraction over r, done on the matrix cores; the kernel is bound by streaming W in and W'
// out (2 * N * K elements), so each lane moves 16-byte chunks of W rows.
//
// bf16: one workgroup per 64 x 256 tile of W (8 waves: 4 row blocks of 16 x 2 halves of 128
// columns). A_l^T for the tile's 256 columns is staged in LDS ([k][rank], ranks at or past r_l
// zero), B_l comes straight from the pool's rank octets (one 16-byte load is one matrix-core
// operand fragment). Output layout of a 16x16x32 product: lane (c, g) holds rows 4g..4g+3 of
// column c. Two products per 32 columns of W, whose rows are mapped to W columns
// 8(m/4) + m%4 and 8(m/4) + 4 + m%4, give lane (c, g) the 8 consecutive W columns 8g..8g+7
// of row c: one 16-byte load and store.
// fp32: plain vector-unit FMAs, one thread per 4 columns of one row.
#include "common.h"

namespace sgmv {

namespace {

constexpr int MG_ROWS = 64, MG_COLS = 256, MG_THREADS = 512;

__device__ __forceinline__ void unpack8(u32x4_t v, float (&f)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_bits_to_f32(w[i] & 0xffffu);
    f[2 * i + 1] = bf16_bits_to_f32(w[i] >> 16);
  }
}

// RP: ranks staged per column, R_pad rounded up to 32 (one 16x16x32 product per 32 ranks)
template <int RP, bool ALIGNED>
__global__ __launch_bounds__(MG_THREADS) void merge_bf16_kernel(
    const uint16_t* w, int64_t ldw, uint16_t* w_out, int64_t ldo,
    const uint16_t* __restrict__ a, const uint16_t* __restrict__ b,
    const int32_t* __restrict__ rank, const float* __restrict__ scale, int l, int N, int K,
    int K_pad, int N_pad, int R_pad) {
  constexpr int STRIDE = RP + 8;  // LDS row of one column: RP ranks + 16 bytes of padding
  __shared__ __align__(16) uint16_t s_at[MG_COLS * STRIDE];
  const int tid = threadIdx.x, wv = tid / WAVE, lane = tid & (WAVE - 1);
  const int c = lane & 15, g = lane >> 4;
  const int n_tile = blockIdx.x * MG_ROWS, k_tile = blockIdx.y * MG_COLS;
  const int r = rank[l];
  const float s = scale[l];

  // A_l^T for columns [k_tile, k_tile + 256): thread (column pair kp, rank octet o)
  const uint16_t* al = a + (size_t)l * R_pad * K_pad;
  for (int item = tid; item < (MG_COLS / 2) * (RP / 8); item += MG_THREADS) {
    const int kp = item % (MG_COLS / 2), o = item / (MG_COLS / 2);
    const int k = k_tile + 2 * kp;
    uint32_t v[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int j = 8 * o + e;
      v[e] = (j < r && k < K_pad)
                 ? *reinterpret_cast<const uint32_t*>(al + (size_t)j * K_pad + k)
                 : 0u;
    }
    u32x4_t c0, c1;  // column k: low halves, column k + 1: high halves
    c0.x = (v[0] & 0xffffu) | (v[1] << 16);
    c0.y = (v[2] & 0xffffu) | (v[3] << 16);
    c0.z = (v[4] & 0xffffu) | (v[5] << 16);
    c0.w = (v[6] & 0xffffu) | (v[7] << 16);
    c1.x = (v[0] >> 16) | (v[1] & 0xffff0000u);
    c1.y = (v[2] >> 16) | (v[3] & 0xffff0000u);
    c1.z = (v[4] >> 16) | (v[5] & 0xffff0000u);
    c1.w = (v[6] >> 16) | (v[7] & 0xffff0000u);
    *reinterpret_cast<u32x4_t*>(s_at + (2 * kp) * STRIDE + 8 * o) = c0;
    *reinterpret_cast<u32x4_t*>(s_at + (2 * kp + 1) * STRIDE + 8 * o) = c1;
  }

  // this wave: rows n0 + [0, 16), tile columns kw + [0, 128)
  const int n0 = n_tile + 16 * (wv & 3), kw = 128 * (wv >> 2);
  const int n = n0 + c;
  const bool row_ok = n < N;

  // B_l fragments: lane (c, g) holds ranks 32 ch + 8g .. +7 of row n
  constexpr int NCH = RP / 32;
  u32x4_t bq[NCH];
  const uint16_t* bl = b + (size_t)l * (R_pad / 8) * N_pad * 8;
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) {
    const int oct = 4 * ch + g;
    u32x4_t v = {0u, 0u, 0u, 0u};
    if (row_ok && 8 * oct < r) {
      v = load_u32x4(bl + ((size_t)oct * N_pad + n) * 8);
      // ranks at or past r_l inside the octet
      const int keep = r - 8 * oct;  // >= 1
      if (keep < 8) {
        uint32_t q[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (e >= keep) q[e / 2] &= (e & 1) ? 0x0000ffffu : 0xffff0000u;
        v = u32x4_t{q[0], q[1], q[2], q[3]};
      }
    }
    bq[ch] = v;
  }

  // old W: lane (c, g) reads row n, columns k_tile + kw + 32 p + 8 g + [0, 8)
  u32x4_t wv4[4];
  float wf[4][8];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int k = k_tile + kw + 32 * p + 8 * g;
    const uint16_t* src = w + (size_t)(row_ok ? n : 0) * ldw + k;
    if (ALIGNED) {
      wv4[p] = (row_ok && k < K) ? load_u32x4(src) : u32x4_t{0u, 0u, 0u, 0u};
      unpack8(wv4[p], wf[p]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        wf[p][e] = (row_ok && k + e < K) ? bf16_bits_to_f32(src[e]) : 0.f;
    }
  }
  __syncthreads();  // s_at

  // B_l A_l on the matrix cores
  f32x4_t acc[4][2];
#pragma unroll
  for (int p = 0; p < 4; ++p) acc[p][0] = acc[p][1] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  // operand row m of the pair's two products: tile column kw + 32 p + 8 (m / 4) + m % 4 (+ 4)
  const int mcol = 8 * (c >> 2) + (c & 3);
#pragma unroll
  for (int ch = 0; ch < NCH; ++ch) {
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int col = kw + 32 * p + mcol;
      const bf16x8_t a0 = as_bf16x8(
          *reinterpret_cast<const u32x4_t*>(s_at + col * STRIDE + 32 * ch + 8 * g));
      const bf16x8_t a1 = as_bf16x8(
          *reinterpret_cast<const u32x4_t*>(s_at + (col + 4) * STRIDE + 32 * ch + 8 * g));
      acc[p][0] = mfma_16x16x32_bf16(a0, as_bf16x8(bq[ch]), acc[p][0]);
      acc[p][1] = mfma_16x16x32_bf16(a1, as_bf16x8(bq[ch]), acc[p][1]);
    }
  }

  // W' = W + scale * (B A), rounded once
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int k = k_tile + kw + 32 * p + 8 * g;
    float o[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[i] = wf[p][i] + s * acc[p][0][i];
      o[4 + i] = wf[p][4 + i] + s * acc[p][1][i];
    }
    if (!row_ok) continue;
    uint16_t* dst = w_out + (size_t)n * ldo + k;
    if (ALIGNED) {
      if (k < K) {
        const u32x4_t v = {pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]),
                           pack_bf16x2(o[4], o[5]), pack_bf16x2(o[6], o[7])};
        *reinterpret_cast<u32x4_t*>(dst) = v;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (k + e < K) dst[e] = (uint16_t)(pack_bf16x2(o[e], 0.f) & 0xffffu);
    }
  }
}

// fp32 pools: 4 consecutive columns of one row per thread, ranks summed in order
__global__ __launch_bounds__(256) void merge_f32_kernel(
    const float* w, int64_t ldw, float* w_out, int64_t ldo,
    const float* __restrict__ a, const float* __restrict__ b, const int32_t* __restrict__ rank,
    const float* __restrict__ scale, int l, int N, int K, int K_pad, int N_pad, int R_pad) {
  const int n = blockIdx.x;
  const int k0 = 4 * (blockIdx.y * blockDim.x + threadIdx.x);
  if (n >= N || k0 >= K) return;
  const int r = rank[l];
  const float s = scale[l];
  const float* al = a + (size_t)l * R_pad * K_pad;
  const float* bl = b + (size_t)l * (R_pad / 8) * N_pad * 8;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < r; ++j) {
    const float bj = bl[((size_t)(j / 8) * N_pad + n) * 8 + j % 8];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (k0 + e < K) acc[e] += bj * al[(size_t)j * K_pad + k0 + e];
  }
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (k0 + e < K) w_out[(size_t)n * ldo + k0 + e] = w[(size_t)n * ldw + k0 + e] + s * acc[e];
}

}  // namespace

hipError_t launch_merge(const void* w, int64_t ldw, void* w_out, int64_t ldo, const sgmv_pool& p,
                        int l, LaunchEvents ev, hipStream_t stream) {
  if (p.dtype == SGMV_BF16) {
    const bool aligned = p.K % 8 == 0 && ldw % 8 == 0 && ldo % 8 == 0 &&
                         (reinterpret_cast<uintptr_t>(w) % 16) == 0 &&
                         (reinterpret_cast<uintptr_t>(w_out) % 16) == 0;
    const dim3 grid((p.N + MG_ROWS - 1) / MG_ROWS, (p.K + MG_COLS - 1) / MG_COLS);
    const int rp = (p.R_pad + 31) / 32 * 32;
#define SGMV_MERGE(RP_, AL_)                                                                  \
  hipExtLaunchKernelGGL(merge_bf16_kernel<RP_, AL_>, grid, dim3(MG_THREADS), 0, stream,     \
                        ev.start, ev.stop, 0, static_cast<const uint16_t*>(w), ldw,          \
                        static_cast<uint16_t*>(w_out), ldo, static_cast<const uint16_t*>(p.a), \
                        static_cast<const uint16_t*>(p.b), p.rank, p.scale, l, p.N, p.K,      \
                        p.K_pad, p.N_pad, p.R_pad)
    if (rp == 32) {
      if (aligned) SGMV_MERGE(32, true); else SGMV_MERGE(32, false);
    } else {
      if (aligned) SGMV_MERGE(64, true); else SGMV_MERGE(64, false);
    }
#undef SGMV_MERGE
  } else {
    const dim3 grid(p.N, (p.K + 4 * 256 - 1) / (4 * 256));
    hipExtLaunchKernelGGL(merge_f32_kernel, grid, dim3(256), 0, stream, ev.start, ev.stop, 0,
                          static_cast<const float*>(w), ldw, static_cast<float*>(w_out), ldo,
                          static_cast<const float*>(p.a), static_cast<const float*>(p.b), p.rank,
                          p.scale, l, p.N, p.K, p.K_pad, p.N_pad, p.R_pad);
  }
  return hipGetLastError();
}

}  // namespace sgmv
