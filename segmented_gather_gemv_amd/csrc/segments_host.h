// Host segment builder (plain C++); see segments_host.cpp.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "sgmv.h"
#include "workspace.h"

namespace sgmv {

// Fills sorted[M], indptr[S+1], seg_lora[S], tiles and info[4] (host memory).
// Returns SGMV_OK, SGMV_EBADID or SGMV_ECAPACITY.
int host_build_segments(const int32_t* ids, int32_t M, int32_t L, int32_t C, int32_t* sorted,
                        int32_t* indptr, int32_t* seg_lora, int32_t* tiles, int32_t* info,
                        int32_t seg_cap, int32_t large_cap, int32_t small_cap);

// Upper bounds on segments, large and small work descriptors.
void segment_capacities(int32_t M, int32_t L, int32_t C, int32_t* seg_cap, int32_t* large_cap,
                        int32_t* small_cap);

}  // namespace sgmv
