// Route, load histogram and fixed-rule plan of a small batch in one launch.
//
// A decode step routes a few tokens; each kernel of the path then costs its
// fixed launch-to-end time, and the plan waits on the load matrix that the
// route just wrote.  For batches of at most 32 tokens one workgroup of 1024
// threads routes every token (the route's eight waves), keeps every 32-token
// sub-tile's expert histogram in LDS, writes the tile offsets and the load
// matrix, and plans from the column sums it already holds -- the outputs of
// lbt_route_topk followed by lbt_plan_balance, from one launch.
//
// [MoonEP-GR] section "Online planning, zero copy και στατικά σχήματα" (the
// plan is made online from the current router output, on the GPU, with no
// host round trip); [UltraEP] section "その仕組みは高速なエキスパート複製に依存する"
// (the exact post-routing load matrix is the planner's input).
#include <limits.h>

#include "plan_core.h"
#include "route_core.h"

namespace lbt {

constexpr int kFrontHist = 16384;   // [sub-tile][E] ints

static bool front_fits(const Dims& d) {
  return d.N >= 1 && d.N <= kRouteTokens && (long long)d.n_sub * d.E <= kFrontHist;
}

template <int V, bool FULL>
__global__ __launch_bounds__(kPlanThreads) void k_route_plan(
    const float* __restrict__ logits, const float* __restrict__ bias, Dims d, int vec,
    int32_t* __restrict__ ids, float* __restrict__ gates, int32_t* __restrict__ work,
    int32_t* __restrict__ counts, int32_t* __restrict__ plan, int32_t* __restrict__ status) {
  __shared__ RouteScratch rs;
  __shared__ int hist[kFrontHist];     // [sub-tile][E]
  __shared__ PlanSmem m;
  const int E = d.E, ns = d.n_sub, S = d.S, spr = d.spr, tpr = d.tpr;
  for (int i = threadIdx.x; i < ns * E; i += kPlanThreads) hist[i] = 0;
  if (threadIdx.x < 12) m.sStat[threadIdx.x] = 0;
  route_span<V, FULL>(logits, bias, d, vec, 0, d.N, ids, gates, rs, [&](long long t, int id) {
    const int r = (int)(t / S), j = (int)(t - (long long)r * S) / kSubTokens;
    atomicAdd(&hist[(r * spr + j) * E + id], 1);
  });
  __syncthreads();
  // per expert: the tile offsets align reads, the load matrix, and T_e
  int32_t* base = work + work_tile_base(d);
  for (int e = threadIdx.x; e < E; e += kPlanThreads) {
    int run = 0;
    for (int r = 0; r < d.R; ++r) {
      int sum = 0;
      for (int j = 0; j < spr; ++j) {
        const int c = hist[(r * spr + j) * E + e];
        if (j % kSubTiles == 0) base[(long long)(r * tpr + j / kSubTiles) * E + e] = run;
        run += c;
        sum += c;
      }
      counts[(long long)r * E + e] = sum;
    }
    m.sT[e] = run;
    m.sX[e] = run;
  }
  __syncthreads();
  plan_core<false>(d, m, d.SK, counts, nullptr, plan, status);
}

hipError_t launch_route_plan(const Dims& d, const float* logits, const float* bias, int32_t* ids,
                             float* gates, int32_t* work, int32_t* counts, int32_t* plan,
                             int32_t* status, hipStream_t st) {
  if (!front_fits(d)) {
    hipError_t e = launch_route_and_scan(d, logits, bias, ids, gates, work, counts, st);
    if (e == hipSuccess) e = launch_plan(d, counts, plan, status, st);
    return e;
  }
  const int vec = route_vec(logits, d.E);
  const dim3 grid(1), block(kPlanThreads);
  const int V = (d.E + kRowLanes - 1) / kRowLanes;
#define LBT_FRONT(VV)                                                                      \
  do {                                                                                     \
    if (d.E == kRowLanes * (VV))                                                           \
      hipLaunchKernelGGL((k_route_plan<VV, true>), grid, block, 0, st, logits, bias, d,    \
                         vec, ids, gates, work, counts, plan, status);                     \
    else                                                                                   \
      hipLaunchKernelGGL((k_route_plan<VV, false>), grid, block, 0, st, logits, bias, d,   \
                         vec, ids, gates, work, counts, plan, status);                     \
  } while (0)
  if (V <= 1) LBT_FRONT(1);
  else if (V <= 2) LBT_FRONT(2);
  else if (V <= 4) LBT_FRONT(4);
  else if (V <= 8) LBT_FRONT(8);
  else if (V <= 16) LBT_FRONT(16);
  else if (V <= 24) LBT_FRONT(24);
  else LBT_FRONT(32);
#undef LBT_FRONT
  return hipGetLastError();
}

}  // namespace lbt
