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
// matrix itself is kept in LDS too.  (Splitting each column over two or
// four lanes joined by cross-lane adds, so that a lane issues fewer loads,
// measured slower on MI355X: 1.44 vs 0.88 us at 256 experts x 8 ranks.)
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

__global__ __launch_bounds__(kPlanThreads) void k_plan(const int32_t* __restrict__ counts, Dims d,
                                                      int32_t* __restrict__ plan,
                                                      int32_t* __restrict__ status) {
  __shared__ PlanSmem m;
  if (threadIdx.x < 12) m.sStat[threadIdx.x] = 0;
  column_sums<kPlanThreads>(counts, d.E, d.R, m.sT, m.sX);
  __syncthreads();
  plan_core<false>(d, m, d.SK, counts, nullptr, plan, status);
}

// Column scan and fixed-rule plan in one launch, for batches whose sub-tile
// histograms fit in LDS (n_sub * E <= kScanPlanWords; the route kernel has
// written them).  The outputs of k_tile_scan (tile offsets, load matrix)
// and of k_plan, bit for bit, one launch and one dependent global round
// trip fewer.  All threads copy the histograms into LDS with their loads in
// flight together; then one thread per expert walks its column in
// sub-tile order (ranks ascending), writing the running prefix at each
// tile's first sub-tile and each rank's sum, and leaves T_e for the plan.
__global__ __launch_bounds__(kPlanThreads) void k_scan_plan(int32_t* __restrict__ work, Dims d,
                                                           int32_t* __restrict__ counts,
                                                           int32_t* __restrict__ plan,
                                                           int32_t* __restrict__ status) {
  __shared__ PlanSmem m;
  __shared__ int sSub[kScanPlanWords];   // [sub-tile][E]
  const int E = d.E, spr = d.spr, tpr = d.tpr, tid = threadIdx.x;
  const int n = d.n_sub * E;
  if (tid < 12) m.sStat[tid] = 0;
  constexpr int kPer = kScanPlanWords / kPlanThreads;
  int v[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int i = u * kPlanThreads + tid;
    v[u] = i < n ? work[i] : 0;
  }
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    const int i = u * kPlanThreads + tid;
    if (i < n) sSub[i] = v[u];
  }
  __syncthreads();
  int32_t* base = work + work_tile_base(d);
  for (int e = tid; e < E; e += kPlanThreads) {
    int run = 0;
    for (int r = 0; r < d.R; ++r) {
      int sum = 0;
      for (int j = 0; j < spr; ++j) {
        const int c = sSub[(r * spr + j) * E + e];
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

bool scan_plan_fits(const Dims& d) {
  return d.n_sub >= 1 && (long long)d.n_sub * d.E <= kScanPlanWords;
}

hipError_t launch_scan_plan(const Dims& d, int32_t* work, int32_t* counts, int32_t* plan,
                            int32_t* status, hipStream_t st) {
  hipLaunchKernelGGL(k_scan_plan, dim3(1), dim3(kPlanThreads), 0, st, work, d, counts, plan,
                     status);
  return hipGetLastError();
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

// Row pitch of the per-rank prefixes Q_r in LDS: odd, so that lanes over
// ranks reading entry j of their rows hit different LDS banks (with the
// pitch nh = 32 of DSV3 every lane of the threshold check read one bank).
__device__ __forceinline__ int q_pitch(int nh) { return nh | 1; }

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
      const int* q = sQ + ro * q_pitch(nh);
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
// N(a) .. N(b-1), N(x) = index along the line of the expert holding x.  The
// rank holding x is the number of ranks whose overflow starts at or below
// x, less one (broadcast reads of the rank offsets, four at a time), and
// the expert inside it the number of its prefixes at or below the rest:
// independent LDS reads, so a candidate costs a handful of LDS round trips
// rather than chains of binary-search steps.  Returns the same value in
// every lane.  ov_off / nv_off: kWave ints of LDS owned by the wave, ov_off
// 16-byte aligned.
__device__ __forceinline__ bool tau_fits_wave(int tau, const int* sQ, const int* sL, int R, int nh,
                                              int B, int* ov_off, int* nv_off) {
  const int r = lane_id();
  const int L = r < R ? sL[r] : 0;
  const int ov = r < R ? max(L - tau, 0) : 0;
  const int df = r < R ? max(tau - L, 0) : 0;
  // experts of rank r that shed anything: those holding positions [0, ov),
  // i.e. the ones whose prefix is below ov and the first that reaches it
  int nv = 0;
  if (ov > 0) {
    const int* q = sQ + r * q_pitch(nh);
#pragma unroll 8
    for (int j = 0; j < nh; ++j) nv += q[j] < ov;
    ++nv;
  }
  const int ov_in = wave_incl_scan_dpp(ov), nv_in = wave_incl_scan_dpp(nv);
  const int df_ex = wave_incl_scan_dpp(df) - df;
  const int tot = __builtin_amdgcn_readlane(ov_in, kWave - 1);
  ov_off[r] = r < R ? ov_in - ov : INT_MAX;   // lanes past R pad the four-wide reads
  nv_off[r] = nv_in - nv;
  __builtin_amdgcn_wave_barrier();
  const int a = df_ex, b = min(df_ex + df, tot);
  const bool need = df > 0 && a < b;
  const int xa = a, xb = b - 1;
  int ca = 0, cb = 0;
  for (int r0 = 0; r0 < R; r0 += 4) {        // r0 + 3 < kWave since R <= kWave
    const int4 v = *reinterpret_cast<const int4*>(ov_off + r0);
    ca += (v.x <= xa) + (v.y <= xa) + (v.z <= xa) + (v.w <= xa);
    cb += (v.x <= xb) + (v.y <= xb) + (v.z <= xb) + (v.w <= xb);
  }
  // clamped so lanes without an interval still read in bounds
  const int ra = max(ca - 1, 0), rb = max(cb - 1, 0);
  const int ya = xa - ov_off[ra], yb = xb - ov_off[rb];
  const int* qa = sQ + ra * q_pitch(nh);
  const int* qb = sQ + rb * q_pitch(nh);
  int ja = 0, jb = 0;
#pragma unroll 8
  for (int j = 0; j < nh; ++j) {
    ja += qa[j] <= ya;
    jb += qb[j] <= yb;
  }
  const int pieces = need ? (nv_off[rb] + jb) - (nv_off[ra] + ja) + 1 : 0;
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
  // per-rank inclusive prefix of the loads in shedding order, rank r's row
  // at r * q_pitch(nh)
  __shared__ int sQ[kMaxE + kMaxR];
  __shared__ int sLr[kMaxR];    // L_r
  __shared__ int sCnt[kQuotaCountsLds];   // the load matrix, when it fits
  alignas(16) __shared__ int sOvOff[kPlanThreads / kWave][kWave];   // per-wave scratch of the first stage
  __shared__ int sNvOff[kPlanThreads / kWave][kWave];
  const int E = d.E, R = d.R, nh = d.nh, tid = threadIdx.x;
  __shared__ int sFound[2];   // [1]: smallest qualifying tau of the wave stage
  // [10]: smallest qualifying tau of the batches, [11]: max_r L_r
  if (tid < 12) m.sStat[tid] = tid == 10 ? INT_MAX : 0;
  if (tid < 2) sFound[tid] = INT_MAX;
  const bool keep = (long long)R * E <= kQuotaCountsLds;
  column_sums<kPlanThreads>(counts, E, R, m.sT, m.sX, keep ? sCnt : nullptr);
  __syncthreads();
  // Shedding order in one pass over each rank's loads: expert e's position
  // is the number of its rank's experts that are hotter (load descending,
  // ties to the lower index), the load ahead of it their sum, so the
  // per-rank prefix in that order needs no separate scan.  sHx[g] = the
  // load ahead of line position g within its rank (0 at the rank's first
  // position), Q_r[pos] = the same plus the load at that position.  (Four
  // lanes per expert, each comparing every fourth expert of the rank and
  // joined by quad DPP adds, measured no faster on MI355X: 1.44 vs 1.32 us
  // at DSV3.)
  int maxL = 0;
  for (int e = tid; e < E; e += kPlanThreads) {
    const int rr = div_nh(e, d), r0 = rr * nh, T = m.sT[e];
    int pos = 0, ahead = 0, L = 0;
#pragma unroll 8
    for (int x = r0; x < r0 + nh; ++x) {
      const int Tx = m.sT[x];
      const bool hot = Tx > T || (Tx == T && x < e);
      pos += hot;
      ahead += hot ? Tx : 0;
      L += Tx;
    }
    const int g = r0 + pos;
    m.sLam[e] = g;
    m.sPerm[g] = e;
    m.sHx[g] = ahead;
    sQ[rr * q_pitch(nh) + pos] = ahead + T;
    if (e == r0) sLr[rr] = L;
    maxL = max(maxL, L);
  }
  maxL = wave_max(maxL);
  if (lane_id() == 0 && maxL > 0) atomicMax(&m.sStat[11], maxL);
  __syncthreads();

  const int hi = min(m.sStat[11], d.tau_max);
  constexpr int kPlanWaves = kPlanThreads / kWave;
  int found = INT_MAX;   // smallest qualifying threshold found (uniform)
  int next = d.SK;       // first candidate not checked yet
  bool built = false;
  if (d.SK <= hi) {
    // tau = S*K first, by building its plan: it stands when the load matrix
    // is consistent and no rank takes more than B replica segments, which
    // is the check the search makes (the plan's replicas per rank are the
    // segments the search counts), so the common case -- the pages' slot
    // counts -- pays for no separate check (a one-wave check of tau = S*K
    // took 1.7 us at DSV3 before the plan; 16 candidates at once, 3.7 us)
    plan_build<true>(d, m, d.SK);
    const bool consistent = (m.sStat[4] & LBT_ST_BADCOUNT) == 0;
    if (consistent && m.sStat[9] <= d.B) {
      found = d.SK;
      built = true;
    } else if (consistent) {
      next = d.SK + 1;   // S*K checked and too many segments on some rank
    }
    __syncthreads();     // every thread has read the stats before they are rewritten
  }
  if (!built) {
    // plan_build scans T_e in place: restore it for the second build
    for (int e = tid; e < E; e += kPlanThreads) m.sX[e] = m.sT[e];
    if (R <= kWave && next <= hi) {
      // the next kPlanWaves candidates, one per wave
      const int tau = next + wave_id();
      if (tau <= hi &&
          tau_fits_wave(tau, sQ, sLr, R, nh, d.B, sOvOff[wave_id()], sNvOff[wave_id()]) &&
          lane_id() == 0)
        atomicMin(&sFound[1], tau);
      __syncthreads();
      found = sFound[1];
      next += kPlanWaves;
    }
    // then ascending batches, one candidate per thread (high throughput)
    for (int base = next; found == INT_MAX && base <= hi; base += kPlanThreads) {
      const int tau = base + tid;
      const bool ok = tau <= hi && tau_fits(tau, sQ, sLr, R, nh, d.B);
      const unsigned long long bal = __ballot(ok);
      // lanes hold ascending candidates: the lowest set lane has the wave's smallest
      if (bal != 0ull && lane_id() == __ffsll((long long)bal) - 1) atomicMin(&m.sStat[10], tau);
      __syncthreads();
      const int f = m.sStat[10];
      __syncthreads();   // every thread has read it before the next batch writes
      if (f != INT_MAX) found = f;
    }
    const int tau = found == INT_MAX ? d.tau_max : found;
    __syncthreads();     // the restored T_e is visible
    plan_build<true>(d, m, tau);
  }
  plan_write<true>(d, m, counts, keep ? sCnt : nullptr, plan, status, tid, kPlanThreads);
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
