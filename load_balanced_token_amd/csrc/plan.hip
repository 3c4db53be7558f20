// The online balancing plan: one workgroup turns the load matrix into the
// replica segments and per-rank segment tables, entirely on the device.
//
// [MoonEP-GR] sections "Η βασική υπόσχεση του MoonEP: σταθερό φορτίο S × K"
// (each rank receives exactly S*K; a few temporary expert copies, planned
// online from the current router output) and "Το memory contract ..."
// (weight rows 0..E-1 are the ranks' experts, E..E+B-1 local prefetch
// slots, the grouped GEMM finds experts by row index and consumes the
// planner's cu_seqlens; replicas beyond the slots are read from home).
// [UltraEP] section "その仕組みは高速なエキスパート複製に依存する" (the
// planner runs fully on the GPU, no host round trip inside a layer;
// replicas exist only when given work).
//
// The rule: rank r keeps min(L_r, S*K) of its pairs, the first ones of its
// home stream; the overflow of every expert (experts ascending) and the
// deficit of every rank (ranks ascending) are laid on one line, and each
// non-empty overlap is a replica segment ("piece").  The workgroup sums the
// load matrix, one wave then builds the whole plan in LDS with DPP prefix
// sums and binary searches (no workgroup barriers on the critical path),
// and the workgroup writes the blob.  E <= 512 experts, R <= 512 ranks.
#include "plan_core.h"

namespace lbt {

__global__ __launch_bounds__(kPlanThreads) void k_plan(const int32_t* __restrict__ counts, Dims d,
                                                      int32_t* __restrict__ plan,
                                                      int32_t* __restrict__ status) {
  __shared__ PlanSmem m;
  const int E = d.E, R = d.R;
  // T_e = column sums of the load matrix
  if (threadIdx.x < 8) m.sStat[threadIdx.x] = 0;
  for (int e = threadIdx.x; e < E; e += kPlanThreads) {
    int s = 0;
    for (int r0 = 0; r0 < R; r0 += 8) {      // eight independent loads in flight
      int v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = r0 + i < R ? counts[(long long)(r0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) s += v[i];
    }
    m.sT[e] = s;
    m.sX[e] = s;
  }
  __syncthreads();
  plan_core(d, m, plan, status);
}

hipError_t launch_plan(const Dims& d, const int32_t* counts, int32_t* plan, int32_t* status,
                       hipStream_t st) {
  hipLaunchKernelGGL(k_plan, dim3(1), dim3(kPlanThreads), 0, st, counts, d, plan, status);
  return hipGetLastError();
}

}  // namespace lbt
