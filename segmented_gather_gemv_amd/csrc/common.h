// Shared device definitions for the libsgmv HIP kernels (gfx950, wave64).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sgmv.h"
#include "workspace.h"

namespace sgmv {

constexpr int WAVE = 64;

// Eight bf16 values: one MFMA 16x16x32 operand fragment per lane.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t v) { return __uint_as_float(v << 16); }

// Two floats as packed bf16, the first in the low half: one gfx950 conversion instruction,
// rounding to nearest even (NaN stays NaN; checked bit for bit against the integer
// round-to-nearest-even on 16.8M fp32 patterns, denormals and ties included).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ f32x4_t mfma_16x16x32_bf16(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ u32x4_t load_u32x4(const void* p) {
  return *reinterpret_cast<const u32x4_t*>(p);
}

__device__ __forceinline__ uint64_t lanemask_lt(int lane) { return (1ull << lane) - 1ull; }

// Per-call kernel arguments shared by the delta kernels (passed by value).
struct SliceArg {
  void* y;
  int64_t ldy;
  int32_t n_begin;  // first pool column
  int32_t v_begin;  // first column in the concatenation of all slices
  int32_t n_len;
};

struct DeltaArgs {
  const void* x;
  int64_t ldx;
  float* h;          // shrink output / expand input (unfused paths)
  int64_t ldh;
  const void* a;     // pool A [L][R_pad][K_pad]
  const void* b;     // pool B [L][R_pad/8][N_pad][8]
  const int32_t* rank;
  const float* scale;
  int32_t R_max, R_pad, K, K_pad, N_pad;
  int32_t L;
  const int32_t* sorted;  // sorted_token_ids
  const int32_t* tiles;   // work descriptor records (SGMV_TILE_INTS ints each)
  const int32_t* info;    // {num_segments, n_large, n_small, status}
  int32_t large_cap, small_cap;
  int32_t n_split_large;  // workgroups across output columns per large piece
  int32_t n_split_small;  // ... per small piece
  int32_t grid_large;     // workgroups [0, grid_large) take large pieces, the rest small ones
                          // (unless small_first)
  int32_t n_slices;
  int32_t v_total;        // sum of slice widths
  int32_t rsplit;         // 4: large pieces run as 16-row parts (small batches), else 1
  // K-split exchange (fused calls): control words indexed like the records, partial tiles
  // of small and of large pieces (layout in workspace.h)
  int32_t* xctl;
  float* xpart_small;
  float* xpart_large;
  int32_t xch_small, xch_large;  // nonzero: that piece class splits its shrink over K
  int32_t xwait;                 // small pieces' wait bound in 10 ns ticks; < 0: no wait
  int32_t xwait_large;
  // fused build + delta launch: per-token adapter ids, and the segment arrays that workgroup 0
  // writes as the device builder would
  const int32_t* ids;
  int32_t M, chunk, seg_cap;
  // adapter-major small pieces: without chunking and with L <= small_cap, small-piece slot
  // t holds adapter t's small piece (its tokens found by one ballot per wave, no sort), and
  // workgroup grid_writer builds and writes the segment arrays
  int32_t amajor, grid_writer;
  // nonzero: workgroups [0, small_first) take small pieces, the next grid_large large ones
  int32_t small_first;
  int32_t spec;  // with amajor: A and B of a small piece loaded before its tokens are known
  int32_t *w_sorted, *w_indptr, *w_seg_lora, *w_tiles, *w_info;
  SliceArg slices[SGMV_MAX_SLICES];
};

enum Mode { MODE_FUSED = 0, MODE_SHRINK = 1, MODE_EXPAND = 2 };

// Optional events recorded by a kernel's own dispatch (start and end of execution).
struct LaunchEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};

// Piece and column split of this workgroup, from its index alone. Workgroups
// [0, grid_large) take large pieces, the rest small ones (with small_first, the small class
// comes first and has small_first workgroups, a multiple of 8); within a class, piece i runs on
// XCD i % 8 (workgroup b runs on XCD b % 8) and its P column splits on consecutive slots of
// that XCD. Returns false for a workgroup past the class capacity. With `blocked_large`, a
// large piece's `tile` is only its cyclic slot, to be turned into the piece by blocked_tile
// once the piece count is known (then no capacity check is made here).
__device__ __forceinline__ bool locate_piece(const DeltaArgs& A, bool split, bool& small,
                                             int& tile, int& p, int& P,
                                             bool blocked_large = false) {
  int b = blockIdx.x;
  if (A.small_first) {
    small = b < A.small_first;
    if (!small) b -= A.small_first;
  } else {
    small = b >= A.grid_large;
    if (small) b -= A.grid_large;
  }
  P = split ? (small ? A.n_split_small : A.n_split_large) : 1;
  const int slot = b >> 3;
  const int q = slot / P;
  tile = q * 8 + (b & 7);
  p = slot - q * P;
  if (!small && blocked_large) return true;
  return tile < (small ? A.small_cap : A.large_cap);
}

// Large pieces dealt to the XCDs in blocks: XCD x takes pieces [x * per, (x + 1) * per),
// per = ceil(n / 8). The pieces of one adapter are consecutive, so they share an XCD's L2 for
// A and B instead of every XCD fetching them. `c` is the cyclic slot q * 8 + x from
// locate_piece, n the number of large pieces; returns the piece, or -1 if the slot has none.
__device__ __forceinline__ int blocked_tile(int c, int n) {
  const int per = (n + 7) >> 3;
  const int q = c >> 3, t = (c & 7) * per + q;
  return (q < per && t < n) ? t : -1;
}

// Workgroups for one class of pieces: 8 XCDs x P splits x ceil(cap / 8) pieces per XCD.
inline int class_grid(int cap, int P) { return 8 * P * ((cap + 7) / 8); }

}  // namespace sgmv
