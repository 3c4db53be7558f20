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
// The fixed rule: rank r keeps min(L_r, S*K) of its pairs, the first ones of
// its home stream; the overflow of every expert (experts ascending) and the
// deficit of every rank (ranks ascending) are laid on one line, and each
// non-empty overlap is a replica segment ("piece").  The quota rule (below)
// searches a threshold and sheds from the hottest experts first.  The plan
// body lives in plan_core.h.  E <= 512 experts, R <= 512 ranks.
#include <limits.h>

#include "plan_core.h"

namespace lbt {

// T_e = column sums of the load matrix into sT and sX (all threads of the
// workgroup; eight independent loads in flight per thread).
template <int NT>
__device__ __forceinline__ void column_sums(const int32_t* __restrict__ counts, int E, int R,
                                            int* sT, int* sX) {
  for (int e = threadIdx.x; e < E; e += NT) {
    int s = 0;
    for (int r0 = 0; r0 < R; r0 += 8) {
      int v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = r0 + i < R ? counts[(long long)(r0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) s += v[i];
    }
    sT[e] = s;
    if (sX != nullptr) sX[e] = s;
  }
}

// Position of expert e in its rank's shedding order: load descending, ties
// to the lower index.
__device__ __forceinline__ int hot_position(const int* sT, int e, int nh) {
  const int r0 = (e / nh) * nh, T = sT[e];
  int pos = 0;
  for (int x = r0; x < r0 + nh; ++x) {
    const int Tx = sT[x];
    pos += (Tx > T) || (Tx == T && x < e);
  }
  return pos;
}

__global__ __launch_bounds__(kPlanThreads) void k_plan(const int32_t* __restrict__ counts, Dims d,
                                                      int32_t* __restrict__ plan,
                                                      int32_t* __restrict__ status) {
  __shared__ PlanSmem m;
  if (threadIdx.x < 12) m.sStat[threadIdx.x] = 0;
  column_sums<kPlanThreads>(counts, d.E, d.R, m.sT, m.sX);
  // the threshold-search region is unused by this rule; keep every word defined
  for (int i = threadIdx.x; i < d.pl.search_groups; i += kPlanThreads) plan[d.pl.search + i] = 0;
  __syncthreads();
  plan_core<false>(d, m, d.SK, plan, status);
}

// ---- quota plan: threshold search ------------------------------------------
//
// [UltraEP] section "その仕組みは高速なエキスパート複製に依存する": the runtime
// searches a target workload threshold keeping every rank under it within
// the replica slots.  Replica needs are not monotone in the threshold, so
// every candidate tau in [S*K, min(max_r L_r, tau_max)] is checked, one
// candidate per thread across the grid, and the smallest that qualifies wins.
//
// For one tau the check needs no per-expert pass: the overflow of rank r is
// the first L_r - tau pairs of its shedding order, so with SQ = inclusive
// prefix of the loads in that order, the experts an overflow interval
// [a, b) of rank r touches are indices upper_bound(SQ_r, a) ..
// upper_bound(SQ_r, b-1).  Deficit ranks (ascending) consume the overflow
// line rank by rank; each rank's replica count is the number of experts its
// interval touches.  Cost per candidate: O(R) steps plus two binary searches
// per (deficit rank, overflowing rank) contact.

struct SearchSmem {
  int sT[kMaxE];
  int sQ[kMaxE + 1];    // loads in shedding order, then inclusive prefix within each rank
  int sL[kMaxR];
  int sRed[kSearchThreads / kWave + 1];
};

// Whether threshold tau puts at most B replica segments on every rank.
__device__ __forceinline__ bool tau_fits(int tau, const int* sQ, const int* sL, int R, int nh,
                                         int B) {
  int ro = 0;
  while (ro < R && sL[ro] <= tau) ++ro;
  int off = 0;   // consumed part of rank ro's overflow
  for (int d = 0; d < R && ro < R; ++d) {
    int cap = tau - sL[d];
    if (cap <= 0) continue;
    int cnt = 0;
    while (cap > 0 && ro < R) {
      const int ov = sL[ro] - tau;
      const int take = min(cap, ov - off);
      const int* q = sQ + ro * nh;
      cnt += upper_bound(q, nh, off + take - 1) - upper_bound(q, nh, off) + 1;
      off += take;
      cap -= take;
      if (off == ov) {
        off = 0;
        ++ro;
        while (ro < R && sL[ro] <= tau) ++ro;
      }
    }
    if (cnt > B) return false;
  }
  return true;
}

__global__ __launch_bounds__(kSearchThreads) void k_tau_search(const int32_t* __restrict__ counts,
                                                               Dims d, int32_t* __restrict__ plan) {
  __shared__ SearchSmem m;
  const int E = d.E, R = d.R, nh = d.nh, tid = threadIdx.x;
  column_sums<kSearchThreads>(counts, E, R, m.sT, nullptr);
  __syncthreads();
  for (int e = tid; e < E; e += kSearchThreads) {
    const int r0 = (e / nh) * nh;
    m.sQ[r0 + hot_position(m.sT, e, nh)] = m.sT[e];
  }
  __syncthreads();
  // inclusive prefix within each rank block: exclusive scan over all, then
  // rebase on the rank's first entry
  block_excl_scan<kSearchThreads, kMaxE / kSearchThreads>(m.sQ, E, m.sRed);
  int maxL = 0;
  for (int r = tid; r < R; r += kSearchThreads) {
    const int base = m.sQ[r * nh];
    m.sL[r] = m.sQ[(r + 1) * nh] - base;
    maxL = max(maxL, m.sL[r]);
  }
  __syncthreads();
  // turn exclusive prefixes into per-rank inclusive ones (each thread its own
  // entries; the rank bases are read before any entry is rewritten)
  int incl[kMaxE / kSearchThreads];
#pragma unroll
  for (int i = 0; i < kMaxE / kSearchThreads; ++i) {
    const int g = tid + i * kSearchThreads;
    incl[i] = g < E ? m.sQ[g + 1] - m.sQ[(g / nh) * nh] : 0;
  }
  maxL = wave_max(maxL);
  if (lane_id() == 0) m.sRed[wave_id()] = maxL;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kMaxE / kSearchThreads; ++i) {
    const int g = tid + i * kSearchThreads;
    if (g < E) m.sQ[g] = incl[i];
  }
  maxL = 0;
  for (int w = 0; w < kSearchThreads / kWave; ++w) maxL = max(maxL, m.sRed[w]);
  __syncthreads();

  const int hi = min(maxL, d.tau_max);
  const int stride = gridDim.x * kSearchThreads;
  int best = INT_MAX;
  for (int tau = d.SK + blockIdx.x * kSearchThreads + tid; tau <= hi; tau += stride) {
    if (tau_fits(tau, m.sQ, m.sL, R, nh, d.B)) {
      best = tau;
      break;
    }
  }
  // workgroup minimum
  for (int o = 32; o > 0; o >>= 1) best = min(best, __shfl_xor(best, o, kWave));
  if (lane_id() == 0) m.sRed[wave_id()] = best;
  __syncthreads();
  if (tid == 0) {
    int b = INT_MAX;
    for (int w = 0; w < kSearchThreads / kWave; ++w) b = min(b, m.sRed[w]);
    plan[d.pl.search + blockIdx.x] = b;
  }
}

// ---- quota plan: the plan at the chosen threshold ---------------------------
__global__ __launch_bounds__(kPlanThreads) void k_plan_quota(const int32_t* __restrict__ counts,
                                                            Dims d, int32_t* __restrict__ plan,
                                                            int32_t* __restrict__ status) {
  __shared__ PlanSmem m;
  const int E = d.E, nh = d.nh, tid = threadIdx.x;
  if (tid < 12) m.sStat[tid] = tid == 10 ? INT_MAX : 0;   // [10]: smallest qualifying tau
  column_sums<kPlanThreads>(counts, E, d.R, m.sT, m.sX);
  __syncthreads();
  for (int e = tid; e < E; e += kPlanThreads) {
    const int g = (e / nh) * nh + hot_position(m.sT, e, nh);
    m.sLam[e] = g;
    m.sPerm[g] = e;
  }
  int best = INT_MAX;
  for (int i = tid; i < d.pl.search_groups; i += kPlanThreads) best = min(best, plan[d.pl.search + i]);
  for (int o = 32; o > 0; o >>= 1) best = min(best, __shfl_xor(best, o, kWave));
  if (lane_id() == 0 && best != INT_MAX) atomicMin(&m.sStat[10], best);
  __syncthreads();
  const int tau = m.sStat[10] == INT_MAX ? d.tau_max : m.sStat[10];
  plan_core<true>(d, m, tau, plan, status);
}

hipError_t launch_plan(const Dims& d, const int32_t* counts, int32_t* plan, int32_t* status,
                       hipStream_t st) {
  hipLaunchKernelGGL(k_plan, dim3(1), dim3(kPlanThreads), 0, st, counts, d, plan, status);
  return hipGetLastError();
}

hipError_t launch_plan_quota(const Dims& d, const int32_t* counts, int32_t* plan, int32_t* status,
                             hipStream_t st) {
  hipLaunchKernelGGL(k_tau_search, dim3(d.pl.search_groups), dim3(kSearchThreads), 0, st, counts,
                     d, plan);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k_plan_quota, dim3(1), dim3(kPlanThreads), 0, st, counts, d, plan, status);
  return hipGetLastError();
}

}  // namespace lbt
