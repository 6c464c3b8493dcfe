// Grouping cache layout (plain C++, shared by host and device code).
#pragma once

#include <stdint.h>

#include "sgmv.h"

namespace sgmv {

// Header {CACHE_TAG, M, L, chunk_size}, then the M ids of the last build made with the
// cache. An all-zero cache is empty (no valid tag).
constexpr int32_t CACHE_TAG = 0x53474331;
static_assert(SGMV_CACHE_HEADER == 4, "cache header layout");

}  // namespace sgmv
