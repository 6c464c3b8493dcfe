// Layout of the fused call's exchange workspace (plain C++, shared by host and device code).
#pragma once

#include <stdint.h>

#include "sgmv.h"

namespace sgmv {

// Exchange workspace of the fused call:
//   control words [large_cap + small_cap][XCH_CTL_INTS] int32, indexed like the descriptor
//     records (large pieces first); word 0 is the piece's arrival counter, the rest reserved
//     and kept zero; padded to 256 bytes;
//   small-piece partial tiles [small_cap][SGMV_EXCHANGE_MAX_SPLITS][16][64] fp32;
//   large-piece partial tiles [large_cap][SGMV_EXCHANGE_MAX_SPLITS_LARGE][64][64] fp32.
constexpr int XCH_CTL_INTS = 16;
constexpr int64_t XCH_SMALL_TILE = 16 * 64;  // floats per small partial tile
constexpr int64_t XCH_LARGE_TILE = 64 * 64;  // floats per large partial tile

struct ExchangeLayout {
  int64_t small_off, large_off, bytes;  // byte offsets of the partial regions, total size
};

inline ExchangeLayout exchange_layout(int32_t large_cap, int32_t small_cap) {
  ExchangeLayout x;
  x.small_off = ((int64_t)(large_cap + small_cap) * XCH_CTL_INTS * 4 + 255) / 256 * 256;
  x.large_off = x.small_off + (int64_t)small_cap * SGMV_EXCHANGE_MAX_SPLITS * XCH_SMALL_TILE * 4;
  x.bytes = x.large_off + (int64_t)large_cap * SGMV_EXCHANGE_MAX_SPLITS_LARGE * XCH_LARGE_TILE * 4;
  return x;
}

}  // namespace sgmv
