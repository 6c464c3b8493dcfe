// Host segment builder: a stable counting sort of tokens by adapter.
//
// Punica page ("III. Punica: Multi-Tenant LoRA Serving"), code section: tokens are reordered
// by adapter and optionally cut into fixed-size chunks, each chunk one segment with one
// adapter; batching-effect section: the boundary array s. Ascend article 3.3: compact
// descriptors (start row, row count, adapter index) prepared once per step on the host.
//
// Buckets follow the order in which adapters first appear among the tokens; tokens ascend
// inside a bucket; id -1 tokens form the tail. Work descriptors are the pieces of at most
// SGMV_TILE_ROWS rows of each segment (compact descriptors: adapter, start row, row count),
// small pieces carrying their token ids. This is plain C++ with no HIP dependency.
#include "segments_host.h"

#include <vector>

namespace sgmv {

int host_build_segments(const int32_t* ids, int32_t M, int32_t L, int32_t C, int32_t* sorted,
                        int32_t* indptr, int32_t* seg_lora, int32_t* tiles, int32_t* info,
                        int32_t seg_cap, int32_t large_cap, int32_t small_cap) {
  for (int32_t t = 0; t < M; ++t) {
    if (ids[t] < -1 || ids[t] >= L) return SGMV_EBADID;
  }
  const int32_t NK = L + 1;  // key L stands for "no adapter"
  std::vector<int32_t> count(NK, 0), base(NK, 0);
  std::vector<int32_t> order;  // adapters by first appearance
  order.reserve(M < L ? M : L);
  for (int32_t t = 0; t < M; ++t) {
    const int32_t key = ids[t] < 0 ? L : ids[t];
    if (key < L && count[key] == 0) order.push_back(key);
    ++count[key];
  }
  int32_t off = 0;
  for (int32_t l : order) {
    base[l] = off;
    off += count[l];
  }
  const int32_t n_lora = off;
  base[L] = n_lora;
  // stable scatter
  std::vector<int32_t> pos(base);
  for (int32_t t = 0; t < M; ++t) {
    const int32_t key = ids[t] < 0 ? L : ids[t];
    sorted[pos[key]++] = t;
  }
  // segments, optionally chunked per bucket
  int32_t S = 0;
  for (int32_t l : order) {
    const int32_t c = count[l];
    const int32_t pieces = C > 0 ? (c + C - 1) / C : 1;
    for (int32_t i = 0; i < pieces; ++i) {
      if (S >= seg_cap) return SGMV_ECAPACITY;
      indptr[S] = base[l] + (C > 0 ? i * C : 0);
      seg_lora[S] = l;
      ++S;
    }
  }
  indptr[S] = n_lora;
  // work descriptors: pieces of at most SGMV_TILE_ROWS rows per segment
  int32_t nl = 0, ns = 0;
  for (int32_t s = 0; s < S; ++s) {
    const int32_t end = indptr[s + 1];
    for (int32_t start = indptr[s]; start < end; start += SGMV_TILE_ROWS) {
      const int32_t rows = end - start < SGMV_TILE_ROWS ? end - start : SGMV_TILE_ROWS;
      int32_t* d;
      const bool small = rows <= SGMV_SMALL_ROWS;
      if (small) {
        if (ns >= small_cap) return SGMV_ECAPACITY;
        d = tiles + (size_t)(large_cap + ns++) * SGMV_TILE_INTS;
      } else {
        if (nl >= large_cap) return SGMV_ECAPACITY;
        d = tiles + (size_t)(nl++) * SGMV_TILE_INTS;
      }
      d[0] = seg_lora[s];
      d[1] = start;
      d[2] = rows;
      d[3] = s;
      for (int i = 4; i < 16; ++i) d[i] = 0;
      for (int i = 0; i < 16; ++i) d[16 + i] = (small && i < rows) ? sorted[start + i] : -1;
    }
  }
  info[0] = S;
  info[1] = nl;
  info[2] = ns;
  info[3] = SGMV_OK;
  return SGMV_OK;
}

void segment_capacities(int32_t M, int32_t L, int32_t C, int32_t* seg_cap, int32_t* large_cap,
                        int32_t* small_cap) {
  int64_t s = M < L ? M : L;
  if (C > 0) {
    s += M / C;
    if (s > M) s = M;
  }
  *seg_cap = (int32_t)s;
  *large_cap = M / (SGMV_SMALL_ROWS + 1);
  *small_cap = (int32_t)s;
}

}  // namespace sgmv
