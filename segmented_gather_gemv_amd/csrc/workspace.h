// Layout of the fused call's exchange workspace (plain C++, shared by host and device code).
#pragma once

#include <stdint.h>

#include "sgmv.h"

namespace sgmv {

// Exchange workspace of the fused call: [small_cap][XCH_CTL_INTS] int32 control words (word 0
// is the piece's arrival counter, the rest are reserved and kept zero) padded to 256 bytes,
// then
// [small_cap][SGMV_EXCHANGE_MAX_SPLITS][16][64] fp32 partial tiles.
constexpr int XCH_CTL_INTS = 16;
constexpr int64_t XCH_TILE_FLOATS = 16 * 64;
inline int64_t exchange_counter_bytes(int32_t small_cap) {
  return ((int64_t)small_cap * XCH_CTL_INTS * 4 + 255) / 256 * 256;
}
inline int64_t exchange_bytes(int32_t small_cap) {
  return exchange_counter_bytes(small_cap) +
         (int64_t)small_cap * SGMV_EXCHANGE_MAX_SPLITS * XCH_TILE_FLOATS * 4;
}

}  // namespace sgmv
