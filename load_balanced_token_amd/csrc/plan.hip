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
// workgroup; eight independent loads in flight per thread); with sCnt, the
// matrix itself is kept in LDS too.
template <int NT>
__device__ __forceinline__ void column_sums(const int32_t* __restrict__ counts, int E, int R,
                                            int* sT, int* sX, int* sCnt = nullptr) {
  for (int e = threadIdx.x; e < E; e += NT) {
    int s = 0;
    for (int r0 = 0; r0 < R; r0 += 8) {
      int v[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = r0 + i < R ? counts[(long long)(r0 + i) * E + e] : 0;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        s += v[i];
        if (sCnt != nullptr && r0 + i < R) sCnt[(r0 + i) * E + e] = v[i];
      }
    }
    sT[e] = s;
    if (sX != nullptr) sX[e] = s;
  }
}

// Position of expert e in its rank's shedding order: load descending, ties
// to the lower index.
__device__ __forceinline__ int hot_position(const int* sT, int e, const Dims& d) {
  const int nh = d.nh, r0 = div_nh(e, d) * nh, T = sT[e];
  int pos = 0;
#pragma unroll 8
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
  __syncthreads();
  plan_core<false>(d, m, d.SK, counts, nullptr, plan, status);
}

// ---- quota plan ---------------------------------------------------------------
//
// [UltraEP] section "その仕組みは高速なエキスパート複製に依存する": the runtime
// searches a target workload threshold keeping every rank under it within
// the replica slots, then a quota planner decides which hot experts get
// copies, where, and how many tokens each takes.  Replica needs are not
// monotone in the threshold, so the smallest qualifying tau in
// [S*K, min(max_r L_r, tau_max)] is found by checking candidates in
// ascending batches of 1024, one per thread, stopping at the first batch
// that holds one.  With the slot counts the pages use, tau = S*K qualifies
// and one batch suffices.
//
// For one tau the check needs no per-expert pass: the overflow of rank r is
// the first L_r - tau pairs of its shedding order, so with Q = inclusive
// prefix of the loads in that order, expert j of rank r holds overflow
// positions [Q_r[j-1], Q_r[j]).  Deficit ranks (ascending) consume the
// overflow line rank by rank; a deficit rank's replica count is the number
// of experts its interval touches.  A cursor on the expert holding the next
// unconsumed position only moves forward, so one candidate costs O(R) steps
// plus one step per replica segment.

// Whether threshold tau puts at most B replica segments on every rank.
__device__ __forceinline__ bool tau_fits(int tau, const int* sQ, const int* sL, int R, int nh,
                                         int B) {
  int ro = 0;
  while (ro < R && sL[ro] <= tau) ++ro;
  int off = 0;   // consumed part of rank ro's overflow
  int ei = 0;    // expert (shedding order) holding position off
  for (int d = 0; d < R && ro < R; ++d) {
    int cap = tau - sL[d];
    if (cap <= 0) continue;
    int cnt = 0;
    while (cap > 0 && ro < R) {
      const int ov = sL[ro] - tau;
      const int take = min(cap, ov - off);
      const int end = off + take;
      const int* q = sQ + ro * nh;
      int ej = ei;                      // expert holding end - 1
      while (ej < nh - 1 && q[ej] < end) ++ej;
      cnt += ej - ei + 1;
      off = end;
      cap -= take;
      if (off == ov) {
        off = 0;
        ei = 0;
        ++ro;
        while (ro < R && sL[ro] <= tau) ++ro;
      } else {
        ei = q[ej] == end ? ej + 1 : ej;
      }
    }
    if (cnt > B) return false;
  }
  return true;
}

// The same check for one tau by one wave, lanes over ranks (R <= 64): the
// overflow, expert-count and deficit offsets of every rank come from wave
// prefix sums; a deficit rank's interval [a, b) on the line touches experts
// N(a) .. N(b-1), N(x) = index along the line of the expert holding x, found
// by a search over the ranks' overflow offsets and one inside the rank.
// Returns the same value in every lane.  ov_off / nv_off: R + 1 ints of LDS
// owned by the wave.
__device__ __forceinline__ bool tau_fits_wave(int tau, const int* sQ, const int* sL, int R, int nh,
                                              int B, int* ov_off, int* nv_off) {
  const int r = lane_id();
  const int L = r < R ? sL[r] : 0;
  const int ov = r < R ? max(L - tau, 0) : 0;
  const int df = r < R ? max(tau - L, 0) : 0;
  // experts of rank r that shed anything: those holding positions [0, ov)
  const int nv = ov > 0 ? upper_bound(sQ + r * nh, nh, ov - 1) + 1 : 0;
  const int ov_in = wave_incl_scan_dpp(ov), nv_in = wave_incl_scan_dpp(nv);
  const int df_ex = wave_incl_scan_dpp(df) - df;
  const int tot = __builtin_amdgcn_readlane(ov_in, kWave - 1);
  if (r < R) {
    ov_off[r] = ov_in - ov;
    nv_off[r] = nv_in - nv;
  }
  if (r == 0) ov_off[R] = tot;
  __builtin_amdgcn_wave_barrier();
  auto line_expert = [&](int x) {       // index along the line of the expert holding x
    const int rx = upper_bound(ov_off, R, x) - 1;
    return nv_off[rx] + upper_bound(sQ + rx * nh, nh, x - ov_off[rx]);
  };
  const int a = df_ex, b = min(df_ex + df, tot);
  const int pieces = (df > 0 && a < b) ? line_expert(b - 1) - line_expert(a) + 1 : 0;
  const bool bad = __any(pieces > B);
  __builtin_amdgcn_wave_barrier();      // ov_off / nv_off may be rewritten next
  return !bad;
}

// The quota plan keeps the load matrix in LDS when it has at most this many
// entries (DSV3, MoonEP and decode shapes), so the locality counts of the
// blob come from LDS instead of dependent global loads.
constexpr int kQuotaCountsLds = 4096;

__global__ __launch_bounds__(kPlanThreads) void k_plan_quota(const int32_t* __restrict__ counts,
                                                            Dims d, int32_t* __restrict__ plan,
                                                            int32_t* __restrict__ status) {
  __shared__ PlanSmem m;
  __shared__ int sQ[kMaxE];     // per-rank inclusive prefix of the loads in shedding order
  __shared__ int sLr[kMaxR];    // L_r
  __shared__ int sCnt[kQuotaCountsLds];   // the load matrix, when it fits
  __shared__ int sOvOff[kPlanThreads / kWave][kWave + 1];   // per-wave scratch of the first stage
  __shared__ int sNvOff[kPlanThreads / kWave][kWave + 1];
  const int E = d.E, R = d.R, nh = d.nh, tid = threadIdx.x;
  // [10]: smallest qualifying tau, [11]: max_r L_r
  if (tid < 12) m.sStat[tid] = tid == 10 ? INT_MAX : 0;
  const bool keep = (long long)R * E <= kQuotaCountsLds;
  column_sums<kPlanThreads>(counts, E, R, m.sT, m.sX, keep ? sCnt : nullptr);
  __syncthreads();
  for (int e = tid; e < E; e += kPlanThreads) {
    const int g = div_nh(e, d) * nh + hot_position(m.sT, e, d);
    m.sLam[e] = g;
    m.sPerm[g] = e;
    m.sHx[g] = m.sT[e];
  }
  __syncthreads();
  if (wave_id() == 0) wave_excl_scan_lds<kMaxE / kWave>(m.sHx, E);
  __syncthreads();
  for (int g = tid; g < E; g += kPlanThreads) sQ[g] = m.sHx[g + 1] - m.sHx[div_nh(g, d) * nh];
  int maxL = 0;
  for (int r = tid; r < R; r += kPlanThreads) {
    sLr[r] = m.sHx[(r + 1) * nh] - m.sHx[r * nh];
    maxL = max(maxL, sLr[r]);
  }
  maxL = wave_max(maxL);
  if (lane_id() == 0 && maxL > 0) atomicMax(&m.sStat[11], maxL);
  __syncthreads();

  const int hi = min(m.sStat[11], d.tau_max);
  constexpr int kPlanWaves = kPlanThreads / kWave;
  int first = d.SK;
  if (R <= kWave) {
    // first stage: the kPlanWaves smallest candidates, one per wave (low latency)
    const int tau = d.SK + wave_id();
    if (tau <= hi && tau_fits_wave(tau, sQ, sLr, R, nh, d.B, sOvOff[wave_id()], sNvOff[wave_id()]) &&
        lane_id() == 0)
      atomicMin(&m.sStat[10], tau);
    __syncthreads();
    first = m.sStat[10] != INT_MAX ? INT_MAX : d.SK + kPlanWaves;
    __syncthreads();   // every thread has read the result before the next stage writes
  }
  // then ascending batches, one candidate per thread (high throughput)
  for (int base = first; base <= hi; base += kPlanThreads) {
    const int tau = base + tid;
    const bool ok = tau <= hi && tau_fits(tau, sQ, sLr, R, nh, d.B);
    const unsigned long long bal = __ballot(ok);
    // lanes hold ascending candidates: the lowest set lane has the wave's smallest
    if (bal != 0ull && lane_id() == __ffsll((long long)bal) - 1) atomicMin(&m.sStat[10], tau);
    __syncthreads();
    const int found = m.sStat[10];
    __syncthreads();
    if (found != INT_MAX) break;
  }
  const int tau = m.sStat[10] == INT_MAX ? d.tau_max : m.sStat[10];
  plan_core<true>(d, m, tau, counts, keep ? sCnt : nullptr, plan, status);
}

hipError_t launch_plan(const Dims& d, const int32_t* counts, int32_t* plan, int32_t* status,
                       hipStream_t st) {
  hipLaunchKernelGGL(k_plan, dim3(1), dim3(kPlanThreads), 0, st, counts, d, plan, status);
  return hipGetLastError();
}

hipError_t launch_plan_quota(const Dims& d, const int32_t* counts, int32_t* plan, int32_t* status,
                             hipStream_t st) {
  hipLaunchKernelGGL(k_plan_quota, dim3(1), dim3(kPlanThreads), 0, st, counts, d, plan, status);
  return hipGetLastError();
}

}  // namespace lbt
