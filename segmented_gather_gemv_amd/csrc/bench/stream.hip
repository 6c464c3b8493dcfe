// Streaming reference kernel for the benchmark (not part of the library's hot path): one
// launch reads `read_bytes` and writes `write_bytes` of device memory in 16-byte lanes, the
// byte mix of a delta launch, so that its time is the memory system's ceiling for a launch
// that moves the same bytes. Each thread issues `unroll` independent 16-byte loads before it
// uses any of them (loads in flight are what a latency-bound streaming launch needs); the
// stored values depend on every loaded one, so no load can be dropped.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

template <int U>
__global__ __launch_bounds__(1024) void stream_kernel(const u32x4_t* __restrict__ src,
                                                      int64_t n_read, u32x4_t* __restrict__ dst,
                                                      int64_t n_write) {
  const int64_t T = (int64_t)gridDim.x * blockDim.x;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  // thread t reads elements t, t + T, ..., t + (U-1) T: each load instruction of a wave
  // covers 1 KB of contiguous memory
  u32x4_t v[U];
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int64_t i = t + u * T;
    v[u] = i < n_read ? src[i] : u32x4_t{0u, 0u, 0u, 0u};
  }
  u32x4_t s = v[0];
#pragma unroll
  for (int u = 1; u < U; ++u) s ^= v[u];
  for (int64_t j = t; j < n_write; j += T) dst[j] = s + (uint32_t)j;
}

}  // namespace

extern "C" {

// Reads read_bytes from src and writes write_bytes to dst (both multiples of 16, 16-byte
// aligned device pointers) in one launch of `block` threads per workgroup (64..1024, a
// multiple of 64) and `unroll` loads in flight per thread (1, 2, 4, 8 or 16); the grid
// covers the reads. start/stop (hipEvent_t or NULL) are recorded by the kernel's own
// dispatch. Returns 0 on success, 1 on bad arguments, 2 on a failed launch.
int sgmv_bench_stream(const void* src, int64_t read_bytes, void* dst, int64_t write_bytes,
                      int32_t block, int32_t unroll, void* start, void* stop, void* stream) {
  if (!src || !dst || read_bytes <= 0 || write_bytes < 0 || read_bytes % 16 || write_bytes % 16)
    return 1;
  if (block < 64 || block > 1024 || block % 64) return 1;
  const int64_t nr = read_bytes / 16, nw = write_bytes / 16;
  const int64_t per = (int64_t)block * unroll;
  const int64_t grid = (nr + per - 1) / per;
  if (grid < 1 || grid > (1 << 30)) return 1;
  const auto* s = static_cast<const u32x4_t*>(src);
  auto* d = static_cast<u32x4_t*>(dst);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipEvent_t e0 = static_cast<hipEvent_t>(start), e1 = static_cast<hipEvent_t>(stop);
  const dim3 g((unsigned)grid), b((unsigned)block);
  switch (unroll) {
    case 1: hipExtLaunchKernelGGL(stream_kernel<1>, g, b, 0, st, e0, e1, 0, s, nr, d, nw); break;
    case 2: hipExtLaunchKernelGGL(stream_kernel<2>, g, b, 0, st, e0, e1, 0, s, nr, d, nw); break;
    case 4: hipExtLaunchKernelGGL(stream_kernel<4>, g, b, 0, st, e0, e1, 0, s, nr, d, nw); break;
    case 8: hipExtLaunchKernelGGL(stream_kernel<8>, g, b, 0, st, e0, e1, 0, s, nr, d, nw); break;
    case 16: hipExtLaunchKernelGGL(stream_kernel<16>, g, b, 0, st, e0, e1, 0, s, nr, d, nw); break;
    default: return 1;
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}  // extern "C"
