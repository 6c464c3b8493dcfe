// Shrink-only and expand-only instantiations of the bf16 delta kernel.
#include "delta_bf16.h"

namespace sgmv {

hipError_t launch_delta_bf16_unfused(int mode, bool aligned, DeltaArgs A, LaunchEvents ev,
                                     hipStream_t stream) {
  int grid;
  size_t lds;
  delta_geometry(mode, A, grid, lds);
  if (grid <= 0) return hipSuccess;
  const dim3 g(grid), b(DT_THREADS);
#define SGMV_LAUNCH(M_, AL_)                                                                  \
  hipExtLaunchKernelGGL((delta_bf16_kernel<M_, AL_, 4, false, false>), g, b, lds, stream, ev.start, \
                        ev.stop, 0, A)
  if (mode == MODE_SHRINK) {
    if (aligned) SGMV_LAUNCH(MODE_SHRINK, true); else SGMV_LAUNCH(MODE_SHRINK, false);
  } else {
    if (aligned) SGMV_LAUNCH(MODE_EXPAND, true); else SGMV_LAUNCH(MODE_EXPAND, false);
  }
#undef SGMV_LAUNCH
  return hipGetLastError();
}

}  // namespace sgmv
