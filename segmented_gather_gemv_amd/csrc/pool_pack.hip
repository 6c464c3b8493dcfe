// Pool packing (load time): user-layout adapters into the library layout.
//
// Fused-LoRA page, Step 1: all adapters in one contiguous pool, A as (L, r, in) and B as
// (L, out, r). Ascend article 4.2: store the pool adapter-major with rank second and align
// K/N to hardware-friendly multiples, done once when weights are loaded rather than with a
// gather inside the kernel. Here A keeps (L, R_pad, K_pad) and B is regrouped into rank
// octets (L, R_pad/8, N_pad, 8); ranks at or past an adapter's own rank and all K/N padding
// are written as zero. Optionally each adapter's scale is folded into its B values (Ascend
// article 2.1, 3.2).
#include "common.h"

namespace sgmv {

template <typename T>
__global__ void pack_a_kernel(const T* __restrict__ a_user, T* __restrict__ a_pool,
                              const int32_t* __restrict__ rank, int R_max, int R_pad, int K,
                              int K_pad) {
  const int k = blockIdx.x * blockDim.x + threadIdx.x;
  const int j = blockIdx.y, l = blockIdx.z;
  if (k >= K_pad) return;
  T v = T(0);
  if (j < rank[l] && j < R_max && k < K) v = a_user[((size_t)l * R_max + j) * K + k];
  a_pool[((size_t)l * R_pad + j) * K_pad + k] = v;
}

// scale_l * v formed in fp32 and rounded once to the element type
__device__ __forceinline__ float fold(float v, float s) { return v * s; }
__device__ __forceinline__ uint16_t fold(uint16_t v, float s) {
  return (uint16_t)(pack_bf16x2(bf16_bits_to_f32(v) * s, 0.f) & 0xffffu);
}

// `scale` (may be null): fold each adapter's scale into its B values.
template <typename T>
__global__ void pack_b_kernel(const T* __restrict__ b_user, T* __restrict__ b_pool,
                              const int32_t* __restrict__ rank, const float* __restrict__ scale,
                              int R_max, int R_pad, int N, int N_pad) {
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  const int o = blockIdx.y, l = blockIdx.z;
  if (n >= N_pad) return;
  const int r = rank[l];
  T* dst = b_pool + (((size_t)l * (R_pad / 8) + o) * N_pad + n) * 8;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int j = 8 * o + e;
    T v = T(0);
    if (j < r && j < R_max && n < N) {
      v = b_user[((size_t)l * N + n) * R_max + j];
      if (scale != nullptr) v = fold(v, scale[l]);
    }
    dst[e] = v;
  }
}

hipError_t launch_pool_pack(const void* a_user, const void* b_user, const sgmv_pool& p,
                            bool fold_scale, hipStream_t stream) {
  const float* fs = fold_scale ? p.scale : nullptr;
  const dim3 blk(256);
  const dim3 ga((p.K_pad + 255) / 256, p.R_pad, p.L);
  const dim3 gb((p.N_pad + 255) / 256, p.R_pad / 8, p.L);
  if (p.dtype == SGMV_BF16) {
    hipLaunchKernelGGL(pack_a_kernel<uint16_t>, ga, blk, 0, stream,
                       static_cast<const uint16_t*>(a_user), static_cast<uint16_t*>(p.a), p.rank,
                       p.R_max, p.R_pad, p.K, p.K_pad);
    hipLaunchKernelGGL(pack_b_kernel<uint16_t>, gb, blk, 0, stream,
                       static_cast<const uint16_t*>(b_user), static_cast<uint16_t*>(p.b), p.rank,
                       fs, p.R_max, p.R_pad, p.N, p.N_pad);
  } else {
    hipLaunchKernelGGL(pack_a_kernel<float>, ga, blk, 0, stream, static_cast<const float*>(a_user),
                       static_cast<float*>(p.a), p.rank, p.R_max, p.R_pad, p.K, p.K_pad);
    hipLaunchKernelGGL(pack_b_kernel<float>, gb, blk, 0, stream, static_cast<const float*>(b_user),
                       static_cast<float*>(p.b), p.rank, fs, p.R_max, p.R_pad, p.N, p.N_pad);
  }
  return hipGetLastError();
}

}  // namespace sgmv
