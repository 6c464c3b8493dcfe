// Fused-call instantiations of the bf16 delta kernel and the bf16 launch entry.
#include "delta_bf16.h"

namespace sgmv {

hipError_t launch_delta_bf16_unfused(int mode, bool aligned, DeltaArgs A, LaunchEvents ev,
                                     hipStream_t stream);

// mode: MODE_FUSED, MODE_SHRINK or MODE_EXPAND. The fused kernel is specialised on the pool's
// rank tiles (R_pad / 16: 1, 2, or up to 4) and on the K-split exchange of small pieces.
hipError_t launch_delta_bf16(int mode, bool aligned, DeltaArgs A, LaunchEvents ev,
                             hipStream_t stream) {
  if (mode != MODE_FUSED) return launch_delta_bf16_unfused(mode, aligned, A, ev, stream);
  int grid;
  size_t lds;
  delta_geometry(mode, A, grid, lds);
  if (grid <= 0) return hipSuccess;
  const dim3 g(grid), b(DT_THREADS);
  const int nrkm = A.R_pad / 16;
  const bool x = A.xch_small != 0 || A.xch_large != 0;
#define SGMV_LAUNCH(AL_, NR_, X_)                                                              \
  hipExtLaunchKernelGGL((delta_bf16_kernel<MODE_FUSED, AL_, NR_, X_, false>), g, b, lds, stream,     \
                        ev.start, ev.stop, 0, A)
  if (aligned) {
    if (nrkm == 1) {
      if (x) SGMV_LAUNCH(true, 1, true); else SGMV_LAUNCH(true, 1, false);
    } else if (nrkm == 2) {
      if (x) SGMV_LAUNCH(true, 2, true); else SGMV_LAUNCH(true, 2, false);
    } else {
      if (x) SGMV_LAUNCH(true, 4, true); else SGMV_LAUNCH(true, 4, false);
    }
  } else {
    if (x) SGMV_LAUNCH(false, 4, true); else SGMV_LAUNCH(false, 4, false);
  }
#undef SGMV_LAUNCH
  return hipGetLastError();
}

}  // namespace sgmv
