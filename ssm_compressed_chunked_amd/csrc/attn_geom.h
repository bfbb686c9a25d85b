// Row geometry of the chunk-aware mask, shared by the attention kernels (pith.science review of
// "Attamba: Attending To Multi-Token States", "What carries the argument": M_train Eq. 5, M_test
// Eq. 7, window Eq. 8).
//
// Query row i of a sequence [s0, s1) whose first chunk is c0 sees two contiguous key ranges:
// the boundary states of chunks c0 .. c0 + E - 1 (those that end before w) and the per-token
// keys at positions w .. i, with w = max(s0, i - L + 1) (i + 1 when L = 0) and, under M_train,
// w = min(w, start of i's chunk). Both w and E are non-decreasing in i.
#pragma once
#include "kernels.h"

namespace attamba {

struct RowGeom {
  int w;   // first band position
  int E;   // visible boundary states
};

__device__ __forceinline__ RowGeom row_geom(const AttnParams& p, int i, int s0, int s1, int c0) {
  RowGeom g;
  int w = i - p.L + 1;
  if (w < s0) w = s0;
  if (p.train) {
    const int cs = p.chunk_cu[p.token_chunk[i]];
    if (cs < w) w = cs;
  }
  g.w = w;
  g.E = (w < s1) ? p.token_chunk[w] - c0 : p.token_chunk[s1 - 1] + 1 - c0;
  return g;
}

}  // namespace attamba
