// The front of a small batch in one launch: route, load histogram,
// fixed-rule plan and (optionally) the block-aligned sort.
//
// A decode step routes a few tokens; each kernel of the path then costs its
// fixed launch-to-end time, and each waits on what the one before wrote to
// memory.  For batches of at most 32 tokens one workgroup of 1024 threads
// routes every token (one token per wave up to 16 tokens, else four per
// wave on eight waves), keeps every 32-token sub-tile's expert histogram in
// LDS, writes the tile offsets and the load matrix, plans from the column
// sums it already holds, and -- for lbt_front -- places every pair from the
// plan still in LDS: the outputs of lbt_route_topk, lbt_plan_balance and
// lbt_align_sort from one launch.
//
// [MoonEP-GR] section "Online planning, zero copy και στατικά σχήματα" (the
// plan is made online from the current router output, on the GPU, with no
// host round trip); [UltraEP] section "その仕組みは高速なエキスパート複製に依存する"
// (the exact post-routing load matrix is the planner's input; per-token
// destinations are a lookup against cumulative quotas); [AlignSort] (pairs
// sorted by expert, each expert's share padded to the grouped GEMM's block).
#include <limits.h>

#include "fused.h"
#include "plan_core.h"
#include "route_core.h"
#include "rows.h"

namespace lbt {

constexpr int kFrontHist = 16384;   // [sub-tile][E] ints
constexpr int kFrontBlocks = 2048;  // block-table entries the one-workgroup align handles
constexpr int kFrontWaveTokens = kPlanThreads / kWave < kWaveRouteTokens ? kPlanThreads / kWave
                                                                         : kWaveRouteTokens;

static bool front_fits(const Dims& d) {
  return d.N >= 1 && d.N <= kRouteTokens && (long long)d.n_sub * d.E <= kFrontHist;
}

// lbt_front's one-workgroup path also needs its block tables to fit in LDS.
static bool front_align_fits(const Dims& d) {
  return front_fits(d) && (long long)d.R * d.n_blocks <= kFrontBlocks;
}

// The align step of a batch of at most 32 tokens from the plan still in the
// workgroup's LDS (after plan_build), by the nthr threads whose index in
// that group is wt: a pair's stable rank inside its expert is the number of
// earlier tokens holding that expert (a bit per token), its destination the
// home segment or the replica segment its overflow position falls in -- the
// same rule and row arithmetic as k_align -- and each block-table entry the
// segment covering the block's first row, whose real end goes to blk_end
// for the padding pass.  Returns the LBT_ST_* bits it raises (only
// LBT_ST_CAPACITY can arise: the route's ids are valid and distinct).  With
// store false nothing goes to global memory; sDst (if not null) receives
// every pair's row of recv, or -1.
__device__ __forceinline__ int front_place(const Dims& d, const PlanSmem& m, const uint32_t* tmask,
                                           const RouteScratch& rs, int* blk_end,
                                           int32_t* __restrict__ slot,
                                           int32_t* __restrict__ sorted_ids,
                                           int32_t* __restrict__ block_wrow,
                                           int32_t* __restrict__ block_expert, const int wt,
                                           const int nthr, const bool store = true,
                                           int* sDst = nullptr) {
  const int E = d.E, K = d.K, R = d.R, nh = d.nh, C = d.C, blk = d.blk, B = d.B;
  const int nP = m.sStat[5], totOv = m.sStat[6];
  int flags = 0;
  // pairs: pair f = wt, wt + nthr, ... (N * K <= 32 * 64)
  for (int f = wt; f < d.N * K; f += nthr) {
    const int t = f / K, k = f - t * K;
    const int e = rs.s_id[t / kRowsPerWave][t % kRowsPerWave][k];
    const int q = __popc(tmask[e] & ((1u << t) - 1u));
    const int h = m.sH[e];
    int dd, row;
    bool ok = true;
    if (q < h) {
      dd = div_nh(e, d);
      const int fb = dd * nh + m.sRep[dd];
      row = m.sF[fb + (e - dd * nh)] - m.sF[fb] + q;
    } else {
      const int o = m.sO[e] + (q - h);
      const int g = upper_bound(m.sPl, nP, o) - 1;
      ok = o < totOv && g >= 0 && m.sPe[g] == e;
      dd = ok ? m.sPd[g] : 0;
      const int fb = dd * nh + m.sRep[dd];
      row = ok ? m.sF[fb + nh + m.sPj[g]] - m.sF[fb] + (o - m.sPl[g]) : 0;
    }
    if (!ok || row >= C || row < 0 || dd < 0 || dd >= R) {
      flags |= LBT_ST_CAPACITY;
      if (store) slot[f] = -1;
      if (sDst != nullptr) sDst[f] = -1;
      continue;
    }
    const long long dst = (long long)dd * C + row;
    if (store) {
      slot[f] = (int)dst;
      sorted_ids[dst] = f;
    }
    if (sDst != nullptr) sDst[f] = (int)dst;
  }
  if (!store) return flags;
  // block tables: one block per thread, its segment's real end kept in LDS
  const long long nblk = (long long)R * d.n_blocks;
  // (blocks from the group's last thread down, pairs from its first up: a
  // decode step's 64 pairs and 64 blocks run on two waves side by side)
  for (long long gb = nthr - 1 - wt; gb < nblk; gb += nthr) {
    const int r = (int)(gb / d.n_blocks), b = (int)(gb - (long long)r * d.n_blocks);
    const int fb = r * nh + m.sRep[r];
    const int nseg = nh + m.sRep[r + 1] - m.sRep[r];
    const int nrp = m.sF[fb + nseg] - m.sF[fb];
    const int row0 = b * blk;
    int ex = -1, wr = -1, real_end = row0 + blk;   // past the padded end: no sentinel
    if (row0 < nrp) {
      // the last segment of rank r starting at or before row0
      int lo = 0, hi = nseg;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (m.sF[fb + mid] - m.sF[fb] <= row0) lo = mid + 1; else hi = mid;
      }
      const int sg = lo - 1;
      int cnt;
      if (sg < nh) {
        ex = r * nh + sg;
        wr = ex;
        cnt = m.sH[ex];
      } else {
        const int j = sg - nh, g = m.sRep[r] + j;
        ex = m.sPe[g];
        wr = j < B ? E + j : ex;
        cnt = m.sPc[g];
      }
      real_end = max(row0, m.sF[fb + sg] - m.sF[fb] + cnt);
    }
    block_wrow[gb] = wr;
    block_expert[gb] = ex;
    if (gb < kFrontBlocks) blk_end[gb] = real_end;
  }
  return flags;
}

// The padding sentinels of the one-workgroup align (after front_place and a
// workgroup barrier): every row of every block, side by side, all threads.
__device__ __forceinline__ void front_sentinels(const Dims& d, const int* blk_end,
                                                int32_t* __restrict__ sorted_ids) {
  const int C = d.C, blk = d.blk;
  const long long nblk = (long long)d.R * d.n_blocks;
  const long long nrows = nblk * blk;
  // C = n_blocks * blk, so row i of the flat [R][C] table is row i % blk of
  // block i / blk.  With blk a multiple of 4 and a 16-byte aligned table,
  // four rows share a block and a block's padding is mostly whole 16-byte
  // groups: one store per four sentinels (the stores, not the LDS reads,
  // are what this pass costs).
  if (blk % 4 == 0 && (reinterpret_cast<uintptr_t>(sorted_ids) & 15) == 0) {
    const int sent = (int)d.P;
    for (long long q = threadIdx.x; q < nrows / 4; q += kPlanThreads) {
      const long long i0 = 4 * q;
      const long long gb = i0 / blk;
      if (gb >= kFrontBlocks) continue;
      const int row_b = (int)(gb - gb / d.n_blocks * d.n_blocks) * blk + (int)(i0 - gb * blk);
      const int end = blk_end[gb];
      if (row_b >= end) {
        *reinterpret_cast<int4*>(sorted_ids + i0) = make_int4(sent, sent, sent, sent);
      } else if (row_b + 4 > end) {
        for (int t = end - row_b; t < 4; ++t) sorted_ids[i0 + t] = sent;
      }
    }
    return;
  }
  for (long long i = threadIdx.x; i < nrows; i += kPlanThreads) {
    const long long gb = i / blk;
    const int row = (int)(i - gb * blk);
    const int row_b = (int)(gb - gb / d.n_blocks * d.n_blocks) * blk + row;   // row within the rank
    const int end = gb < kFrontBlocks ? blk_end[gb] : 0;
    if (gb < kFrontBlocks && row_b >= end)
      sorted_ids[(gb / d.n_blocks) * C + row_b] = (int)d.P;
  }
}

// MOVE (ALIGN, at most kFrontWaveTokens tokens): the dispatch fused in.
// The grid has one workgroup per token; every workgroup routes, plans and
// places the whole batch (the same integer plan and placement in each), the
// first one alone writes the outputs, and workgroup t then copies token t's
// row x[t] to its K rows of recv.  One launch for the front and the
// dispatch, whose outputs it gives bit for bit.
template <int V, bool FULL, bool ALIGN, bool MOVE>
__global__ __launch_bounds__(kPlanThreads) void k_route_plan(
    const float* __restrict__ logits, const float* __restrict__ bias, Dims d, int vec,
    int32_t* __restrict__ ids, float* __restrict__ gates, int32_t* __restrict__ work,
    int32_t* __restrict__ counts, int32_t* __restrict__ plan, int32_t* __restrict__ slot,
    int32_t* __restrict__ sorted_ids, int32_t* __restrict__ block_wrow,
    int32_t* __restrict__ block_expert, int32_t* __restrict__ status,
    const u32x4* __restrict__ x, u32x4* __restrict__ recv) {
  static_assert(!MOVE || ALIGN, "the fused dispatch needs the placement");
  const bool lead = !MOVE || blockIdx.x == 0;     // the workgroup that writes the outputs
  __shared__ RouteScratch rs;
  __shared__ int hist[kFrontHist];     // [sub-tile][E]
  __shared__ uint32_t tmask[kMaxE];    // per expert: the tokens holding it (ALIGN)
  __shared__ int blk_end[kFrontBlocks]; // per block: first padding row (ALIGN)
  __shared__ int sFlags;
  __shared__ PlanSmem m;
  const int E = d.E, ns = d.n_sub, S = d.S, spr = d.spr, tpr = d.tpr;
  for (int i = threadIdx.x; i < ns * E; i += kPlanThreads) hist[i] = 0;
  if (ALIGN)
    for (int e = threadIdx.x; e < E; e += kPlanThreads) tmask[e] = 0u;
  if (threadIdx.x < 12) m.sStat[threadIdx.x] = 0;
  if (threadIdx.x == 0) sFlags = 0;
  // MOVE: the first chunk of this workgroup's token row, loaded now so that
  // its latency hides under the route and the plan
  u32x4 x0 = {0u, 0u, 0u, 0u};
  if constexpr (MOVE) {
    if ((int)threadIdx.x < d.H / 8) x0 = x[(long long)blockIdx.x * (d.H / 8) + threadIdx.x];
  }
  auto add = [&](long long t, int id) {
    const int r = (int)(t / S), j = (int)(t - (long long)r * S) / kSubTokens;
    atomicAdd(&hist[(r * spr + j) * E + id], 1);
    if (ALIGN) atomicOr(&tmask[id], 1u << (int)t);
  };
  // up to 16 tokens: one per wave (a lane sorts a quarter of the keys);
  // else four per wave on the route's eight waves
  if (d.N <= kFrontWaveTokens)
    route_wave<V, FULL>(logits, bias, d, vec, d.N, ids, gates, rs, add, lead);
  else
    route_span<V, FULL>(logits, bias, d, vec, 0, d.N, ids, gates, rs, add);
  __syncthreads();
  // per expert: T_e, the plan's input (LDS only)
  for (int e = threadIdx.x; e < E; e += kPlanThreads) {
    int run = 0;
#pragma unroll 8
    for (int i = 0; i < ns; ++i) run += hist[i * E + e];
    m.sT[e] = run;
    m.sX[e] = run;
  }
  __syncthreads();
  // the tile offsets align reads and the load matrix, written by waves
  // 1.. while wave 0 builds the plan (their stores are off the plan's
  // critical path; decode S=1: 1.0 us of the kernel before)
  if (lead && (int)threadIdx.x >= kWave) {
    int32_t* base = work + work_tile_base(d);
    for (int e = threadIdx.x - kWave; e < E; e += kPlanThreads - kWave) {
      int run = 0;
#pragma unroll 8
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
    }
  }
  if constexpr (!ALIGN) {
    plan_core<false>(d, m, d.SK, counts, nullptr, plan, status);
  } else {
    // The plan in LDS, then two halves side by side: one writes the blob
    // (its store issue and LDS round trips), the other places the pairs
    // and writes the block tables; then everyone writes the padding
    // sentinels.  The status word is written once, after the align step.
    plan_build<false>(d, m, d.SK);
    // MOVE: every pair's row lands in LDS; the histograms are dead after
    // plan_build's closing barrier, so their space holds it
    int* sDst = MOVE ? hist : nullptr;
    constexpr int kHalf = kPlanThreads / 2;
    if ((int)threadIdx.x >= kHalf) {
      if (lead)
        plan_write<false>(d, m, counts, nullptr, plan, nullptr, (int)threadIdx.x - kHalf, kHalf);
    } else {
      const int fl = front_place(d, m, tmask, rs, blk_end, slot, sorted_ids, block_wrow,
                                 block_expert, (int)threadIdx.x, kHalf, lead, sDst);
      if (fl) atomicOr(&sFlags, fl);
    }
    __syncthreads();
    if (lead) {
      front_sentinels(d, blk_end, sorted_ids);
      if (threadIdx.x == 0 && status != nullptr) *status = m.sStat[4] | sFlags;
    }
    if constexpr (MOVE) {
      const int t = blockIdx.x, K = d.K, H8 = d.H / 8;
      const u32x4* src = x + (long long)t * H8;
      for (int c = threadIdx.x; c < H8; c += kPlanThreads) {
        const u32x4 v = c < kPlanThreads ? x0 : src[c];
        for (int k = 0; k < K; ++k) {
          const int dst = sDst[t * K + k];
          if (dst >= 0) recv[(long long)dst * H8 + c] = v;
        }
      }
    }
  }
}

// One small-batch launch: route + plan (ALIGN false) or route + plan +
// align (ALIGN true), and with MOVE the dispatch too (one workgroup per
// token, x and recv given).
template <bool ALIGN, bool MOVE = false>
static void launch_front_small(const Dims& d, const float* logits, const float* bias,
                               int32_t* ids, float* gates, int32_t* work, int32_t* counts,
                               int32_t* plan, int32_t* slot, int32_t* sorted_ids,
                               int32_t* block_wrow, int32_t* block_expert, int32_t* status,
                               hipStream_t st, const uint16_t* x = nullptr,
                               uint16_t* recv = nullptr) {
  const int vec = route_vec(logits, d.E);
  const dim3 grid(MOVE ? d.N : 1), block(kPlanThreads);
  const int V = (d.E + kRowLanes - 1) / kRowLanes;
  const u32x4* xv = reinterpret_cast<const u32x4*>(x);
  u32x4* rv = reinterpret_cast<u32x4*>(recv);
#define LBT_FRONT(VV)                                                                      \
  do {                                                                                     \
    if (d.E == kRowLanes * (VV))                                                           \
      hipLaunchKernelGGL((k_route_plan<VV, true, ALIGN, MOVE>), grid, block, 0, st,        \
                         logits, bias, d, vec, ids, gates, work, counts, plan, slot,       \
                         sorted_ids, block_wrow, block_expert, status, xv, rv);            \
    else                                                                                   \
      hipLaunchKernelGGL((k_route_plan<VV, false, ALIGN, MOVE>), grid, block, 0, st,       \
                         logits, bias, d, vec, ids, gates, work, counts, plan, slot,       \
                         sorted_ids, block_wrow, block_expert, status, xv, rv);            \
  } while (0)
  if (V <= 1) LBT_FRONT(1);
  else if (V <= 2) LBT_FRONT(2);
  else if (V <= 4) LBT_FRONT(4);
  else if (V <= 8) LBT_FRONT(8);
  else if (V <= 16) LBT_FRONT(16);
  else if (V <= 24) LBT_FRONT(24);
  else LBT_FRONT(32);
#undef LBT_FRONT
}

hipError_t launch_route_plan(const Dims& d, const float* logits, const float* bias, int32_t* ids,
                             float* gates, int32_t* work, int32_t* counts, int32_t* plan,
                             int32_t* status, hipStream_t st) {
  if (!front_fits(d)) {
    if (scan_plan_fits(d)) {   // mid-size batch: route, then column scan + plan in one launch
      hipError_t e = launch_route(d, logits, bias, ids, gates, work, st);
      if (e == hipSuccess) e = launch_scan_plan(d, work, counts, plan, status, st);
      return e;
    }
    hipError_t e = launch_route_and_scan(d, logits, bias, ids, gates, work, counts, st);
    if (e == hipSuccess) e = launch_plan(d, counts, plan, status, st);
    return e;
  }
  launch_front_small<false>(d, logits, bias, ids, gates, work, counts, plan, nullptr, nullptr,
                            nullptr, nullptr, status, st);
  return hipGetLastError();
}

hipError_t launch_front(const Dims& d, const float* logits, const float* bias, int32_t* ids,
                        float* gates, int32_t* work, int32_t* counts, int32_t* plan,
                        int32_t* slot, int32_t* sorted_ids, int32_t* block_wrow,
                        int32_t* block_expert, int32_t* status, hipStream_t st) {
  if (!front_align_fits(d)) {
    hipError_t e;
    if (!front_fits(d) && scan_plan_fits(d)) {   // mid-size batch: scan + plan in one launch
      e = launch_route(d, logits, bias, ids, gates, work, st);
      if (e == hipSuccess) e = launch_scan_plan(d, work, counts, plan, status, st);
    } else {
      e = launch_route_and_scan(d, logits, bias, ids, gates, work, counts, st);
      if (e == hipSuccess) e = launch_plan(d, counts, plan, status, st);
    }
    if (e == hipSuccess)
      e = launch_align(d, ids, work, plan, slot, sorted_ids, block_wrow, block_expert, status, st);
    return e;
  }
  launch_front_small<true>(d, logits, bias, ids, gates, work, counts, plan, slot, sorted_ids,
                           block_wrow, block_expert, status, st);
  return hipGetLastError();
}

// The front and the dispatch: batches of at most 16 tokens the
// one-workgroup front takes run it with the dispatch fused in (one launch,
// one workgroup per token); up to 32 tokens the front, then the dispatch;
// batches past 32 tokens whose sub-tile histograms fit
// 8192 words route, then scan and plan in one launch, then align and
// dispatch in one launch (three launches where lbt_front and lbt_dispatch
// make five); others make the launches of the separate calls, with align
// and dispatch fused up to 1024 tokens.
hipError_t launch_front_dispatch(const Dims& d, const float* logits, const float* bias,
                                 int32_t* ids, float* gates, int32_t* work, int32_t* counts,
                                 int32_t* plan, int32_t* slot, int32_t* sorted_ids,
                                 int32_t* block_wrow, int32_t* block_expert, const uint16_t* x,
                                 uint16_t* recv, int32_t* status, hipStream_t st) {
  if (front_align_fits(d) && d.N <= kFrontWaveTokens) {
    launch_front_small<true, true>(d, logits, bias, ids, gates, work, counts, plan, slot,
                                   sorted_ids, block_wrow, block_expert, status, st, x, recv);
    return hipGetLastError();
  }
  if (front_align_fits(d)) {
    launch_front_small<true>(d, logits, bias, ids, gates, work, counts, plan, slot, sorted_ids,
                             block_wrow, block_expert, status, st);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) e = launch_dispatch(d, x, slot, recv, st);
    return e;
  }
  hipError_t e;
  if (!front_fits(d) && scan_plan_fits(d)) {
    e = launch_route(d, logits, bias, ids, gates, work, st);
    if (e == hipSuccess) e = launch_scan_plan(d, work, counts, plan, status, st);
  } else {
    e = launch_route_and_scan(d, logits, bias, ids, gates, work, counts, st);
    if (e == hipSuccess) e = launch_plan(d, counts, plan, status, st);
  }
  if (e == hipSuccess)
    e = launch_align_dispatch(d, ids, work, plan, x, slot, sorted_ids, block_wrow, block_expert,
                              recv, status, st);
  return e;
}

}  // namespace lbt
