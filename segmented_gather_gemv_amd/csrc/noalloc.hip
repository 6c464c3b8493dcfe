// sgmv_lora_delta_ids_noalloc: the segment build and fused delta of sgmv_lora_delta_ids with
// the K-split exchange workspace taken from a static device array instead of the caller's
// segments object, for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid allocation).
//
// The array lives in this file. Host code never passes its name to a kernel or a copy: in
// host code the name is a host-side stand-in, not a device address. Its device address is
// looked up once per device with hipGetSymbolAddress (with that device current) and kept in
// a per-device table; kernels receive that address, exactly as they receive the caller's
// workspace in sgmv_lora_delta_ids.
//
// State across calls: the array keeps the last call's contents. Its control words (one
// arrival counter per piece slot) start at zero with the code object and every completed
// fused call advances each counter it uses by exactly 64, so every counter stays a multiple
// of 64, which is all a call needs; the two-launch path's builder also clears them. Partial
// tiles are written before they are read within one call and need no clearing. Calls that
// overlap on one GPU (different streams, or threads without ordering) share the array and
// race; order them on one stream.
#include <mutex>

#include "common.h"

namespace sgmv {
namespace {

static __device__ __align__(256) unsigned char scratch[SGMV_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[MAX_DEVICES] = {};

// Device address of `scratch` on the current device, looked up on the first call there.
hipError_t scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace
}  // namespace sgmv

using namespace sgmv;

extern "C" sgmv_status sgmv_lora_delta_ids_noalloc(const int32_t* lora_indices, const void* x,
                                                   int64_t ldx, int32_t M,
                                                   const sgmv_pool* pool,
                                                   const sgmv_segments* seg,
                                                   const sgmv_slice* out, int32_t n_slices,
                                                   void* stream) {
  if (!seg) return SGMV_EINVAL;
  const ExchangeLayout lay = exchange_layout(seg->large_cap, seg->small_cap);
  if (seg->large_cap < 0 || seg->small_cap < 0 || lay.bytes > SGMV_NOALLOC_SCRATCH_BYTES)
    return SGMV_EUNSUPPORTED;
  void* ptr = nullptr;
  if (scratch_on_current_device(&ptr) != hipSuccess) return SGMV_EHIP;
  sgmv_segments s = *seg;  // the caller's arrays, the static workspace
  s.exchange = ptr;
  s.exchange_bytes = SGMV_NOALLOC_SCRATCH_BYTES;
  return sgmv_lora_delta_ids_ex(lora_indices, x, ldx, M, pool, &s, out, n_slices, nullptr,
                                stream);
}
