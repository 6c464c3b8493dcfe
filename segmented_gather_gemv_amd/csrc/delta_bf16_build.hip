// Fused build + delta: instantiations of the bf16 delta kernel whose workgroups first build
// the batch's segments themselves (M <= 512, ranks within one 16-rank tile), so a decode step
// needs a single launch.
#include "delta_bf16.h"

namespace sgmv {

hipError_t launch_delta_bf16_build(bool aligned, DeltaArgs A, LaunchEvents ev,
                                   hipStream_t stream) {
  int grid;
  size_t lds;
  delta_geometry(MODE_FUSED, A, grid, lds, true);
  if (grid <= 0) return hipSuccess;
  const dim3 g(grid), b(DT_THREADS);
  const int nrkm = A.R_pad / 16;
  const bool x = A.xch_small != 0 || A.xch_large != 0;
#define SGMV_LAUNCH(AL_, NR_, X_)                                                              \
  hipExtLaunchKernelGGL((delta_bf16_kernel<MODE_FUSED, AL_, NR_, X_, true>), g, b, lds, stream, \
                        ev.start, ev.stop, 0, A)
  if (nrkm != 1) return hipErrorInvalidValue;  // the caller takes two launches instead
  if (aligned) {
    if (x) SGMV_LAUNCH(true, 1, true); else SGMV_LAUNCH(true, 1, false);
  } else {  // the generic instance (any rank tile count) also serves unaligned rank-16 pools
    if (x) SGMV_LAUNCH(false, 4, true); else SGMV_LAUNCH(false, 4, false);
  }
#undef SGMV_LAUNCH
  return hipGetLastError();
}

}  // namespace sgmv

#ifdef SGMV_PHASE_STAMPS
// Profiling builds only: copies the phase stamps of the last single launches (STAMP_WGS rows
// of STAMP_SLOTS uint64 counter values, row = workgroup) to host memory. Returns 0 on success.
extern "C" int sgmv_phase_stamps(void* host, size_t bytes) {
  if (!host || bytes > sizeof(sgmv::g_phase_stamps)) return 1;
  return hipMemcpyFromSymbol(host, HIP_SYMBOL(sgmv::g_phase_stamps), bytes) == hipSuccess ? 0 : 1;
}
#endif
