// Block tables of the block-aligned sort, written by the align kernel's
// extra workgroups: for block gb (rank r, block b) of one wave, the
// weight row and expert of the segment covering it (or -1 past the rank's
// padded end), and the padding sentinel P in its rows past the segment's
// real rows.  [AlignSort]: every expert's share is padded to the grouped
// GEMM's block, so a block lies inside one segment.
#pragma once
#include "lbt_internal.h"

namespace lbt {

__device__ __forceinline__ void align_blocks(const int32_t* __restrict__ plan, const Dims& d,
                                             long long gb, int32_t* __restrict__ sorted_ids,
                                             int32_t* __restrict__ block_wrow,
                                             int32_t* __restrict__ block_expert) {
  const PlanLayout& pl = d.pl;
  const int r = (int)(gb / d.n_blocks);
  const int b = (int)(gb - (long long)r * d.n_blocks);
  const int lane = lane_id();
  const int nrp = plan[pl.n_rows_padded + r];
  const int ns = min(max(plan[pl.n_seg + r], 1), pl.max_seg);   // clamped against a corrupt blob
  const int row0 = b * d.blk;
  if (row0 >= nrp) {
    if (lane == 0) {
      block_wrow[gb] = -1;
      block_expert[gb] = -1;
    }
    return;
  }
  // the last segment starting at or before row0: count the starts <= row0
  // (non-decreasing) with the wave's lanes loading them side by side
  const int32_t* starts = plan + pl.seg_start + (long long)r * (pl.max_seg + 1);
  int nle = 0;
  for (int i0 = 0; i0 < ns; i0 += kWave) {
    const int i = i0 + lane;
    nle += __popcll(__ballot(i < ns && starts[i] <= row0));
  }
  const int s = max(nle - 1, 0);
  const long long si = (long long)r * pl.max_seg + s;
  if (lane == 0) {
    block_wrow[gb] = plan[pl.seg_wrow + si];
    block_expert[gb] = plan[pl.seg_expert + si];
  }
  const int real_end = starts[s] + plan[pl.seg_count + si];
  const int sentinel = (int)d.P;
  for (int row = max(row0, real_end) + lane; row < row0 + d.blk; row += kWave)
    sorted_ids[(long long)r * d.C + row] = sentinel;
}

}  // namespace lbt
