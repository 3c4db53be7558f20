// Launchers of the fused calls: align + dispatch in one launch for batches
// of at most 1024 tokens (align.hip), and the whole front of the step plus
// the dispatch (front.hip).  Each gives bit for bit the outputs of the
// calls it replaces.
#pragma once
#include "lbt_internal.h"

namespace lbt {

hipError_t launch_align_dispatch(const Dims& d, const int32_t* ids, const int32_t* work,
                                 const int32_t* plan, const uint16_t* x, int32_t* slot,
                                 int32_t* sorted_ids, int32_t* block_wrow, int32_t* block_expert,
                                 uint16_t* recv, int32_t* status, hipStream_t st);
hipError_t launch_front_dispatch(const Dims& d, const float* logits, const float* bias,
                                 int32_t* ids, float* gates, int32_t* work, int32_t* counts,
                                 int32_t* plan, int32_t* slot, int32_t* sorted_ids,
                                 int32_t* block_wrow, int32_t* block_expert, const uint16_t* x,
                                 uint16_t* recv, int32_t* status, hipStream_t st);

}  // namespace lbt
