// The greedy accept walk of one round, done by one wavefront (paper §3.2 Def. 1;
// App. B.1, proof of Theorem 1): from the root row, with y the row's greedy
// token (or its draw), commit y and descend while the row has a child carrying
// y, else emit y as the next root and stop.  Lane c holds row c's parent and
// token; a child lookup is one ballot.  Shared by the walk kernel and the LM
// head's merge kernel, whose last work-group to finish walks every round.
#pragma once

#include "common.h"
#include "kernels.h"

namespace glance {

struct WalkArgs {
  const int32_t* parent = nullptr;
  const int32_t* token = nullptr;
  const int32_t* n_valid = nullptr;
  int nseq = 0;
  int n_rows = 0;
  int L = 0;
  float gap_flag = 0.f;
  int32_t* n_accept = nullptr;
  int32_t* out_tokens = nullptr;
  int32_t* path_rows = nullptr;
  int32_t* flagged = nullptr;
};

// Sequence s's walk over rows [s * n_rows, (s + 1) * n_rows) with the rows'
// greedy tokens `pick` and top-2 gaps `gap`; called by all 64 lanes of a wave.
__device__ __forceinline__ void walk_round(const WalkArgs& w, const int32_t* __restrict__ pick,
                                           const float* __restrict__ gap, int s) {
  const int lane = lane_id();
  const int n_rows = w.n_rows, L = w.L;
  const size_t rb = static_cast<size_t>(s) * n_rows;
  // every load issued at once (rows below n_rows exist whatever n_valid is); the
  // rows past n_valid are masked afterwards
  const int li = lane < n_rows ? lane : 0;
  const int nv = w.n_valid[s];
  const int ld_parent = w.parent[rb + li];
  const int ld_token = w.token[rb + li];
  const int ld_arg = pick[rb + li];
  const float ld_gap = gap[rb + li];
  const bool mine = lane < nv && lane < n_rows;
  const int my_parent = mine ? ld_parent : -2;
  const int my_token = mine ? ld_token : -2;
  const int my_arg = mine ? ld_arg : -1;
  const float my_gap = mine ? ld_gap : INFINITY;
  int r = 0, a = 0, flag = 0;
  for (;;) {
    const int y = __shfl(my_arg, r, kWave);
    const float gp = __shfl(my_gap, r, kWave);
    if (w.gap_flag > 0.f && gp <= w.gap_flag) flag = 1;
    if (lane == 0) {
      w.out_tokens[static_cast<size_t>(s) * (L + 1) + a] = y;
      w.path_rows[static_cast<size_t>(s) * (L + 1) + a] = r;
    }
    const unsigned long long hit = __ballot(lane > 0 && my_parent == r && my_token == y);
    if (hit == 0ull || a >= L) break;
    r = __ffsll(static_cast<long long>(hit)) - 1;
    ++a;
  }
  for (int k = a + 1 + lane; k <= L; k += kWave) {
    w.out_tokens[static_cast<size_t>(s) * (L + 1) + k] = -1;
    w.path_rows[static_cast<size_t>(s) * (L + 1) + k] = -1;
  }
  if (lane == 0) {
    w.n_accept[s] = a;
    w.flagged[s] = flag;
  }
}

}  // namespace glance
