// The online balancing plan: one workgroup turns the per-expert loads into
// the replica segments and per-rank segment tables, entirely on the device.
// The plan body as a device function; the plan kernels wrap it.
//
// [MoonEP-GR] sections "Η βασική υπόσχεση του MoonEP: σταθερό φορτίο S × K"
// (each rank receives exactly S*K; a few temporary expert copies, planned
// online from the current router output) and "Το memory contract ..."
// (weight rows 0..E-1 are the ranks' experts, E..E+B-1 local prefetch
// slots, the grouped GEMM finds experts by row index and consumes the
// planner's cu_seqlens; replicas beyond the slots are read from home).
// [UltraEP] section "その仕組みは高速なエキスパート複製に依存する" (the
// planner runs fully on the GPU, no host round trip inside a layer;
// replicas exist only when given work; a quota planner decides which hot
// experts get copies).
//
// At threshold tau, rank r keeps min(L_r, tau) of its pairs.  Which pairs
// overflow: the fixed rule (tau = S*K) sheds the tail of the home stream
// (experts ascending); the quota rule sheds from the hottest experts first
// (load descending, ties to the lower index).  The overflow of every expert
// (in line order: experts ascending, or rank by rank in shedding order) and
// the deficit tau - min(L_r, tau) of every rank (ranks ascending) are laid on
// one line, and each non-empty overlap is a replica segment ("piece").  The
// workgroup sums the load matrix, one wave then builds the whole plan in LDS
// with DPP prefix sums and binary searches (no workgroup barriers on the
// critical path), and the workgroup writes the blob.  E <= 512, R <= 512.
#pragma once
#include "lbt_internal.h"

namespace lbt {

constexpr int kPlanThreads = 1024;

// Column scan + fixed-rule plan in one launch (plan.hip), after
// launch_route, for batches with n_sub * E <= kScanPlanWords
// (scan_plan_fits).
constexpr int kScanPlanWords = 8192;
bool scan_plan_fits(const Dims& d);
hipError_t launch_scan_plan(const Dims& d, int32_t* work, int32_t* counts, int32_t* plan,
                            int32_t* status, hipStream_t st);
// The pieces per line position are counted one of three ways, by size:
// with at most kDirectCompares (deficit rank, position) pairs per lane,
// both ends of every position by register-broadcast counting; with at most
// kLinearDeficits deficit ranks, one broadcast count per position serving
// both ends; else one binary search per position.  Measured on MI355X
// (that phase alone): DSV3, 7 deficit ranks x 4 positions per lane: 0.96 us
// (both ends) vs 1.20 (one count) vs 1.68 (two searches); Kimi-K3, about 25
// x 8: 2.7 (one count) vs 3.8 (both ends) vs 4.7; WideEP, about 49 deficit
// ranks: 2.7 (one search) vs 3.4 (two searches) vs 4.7 (counting).
constexpr int kLinearDeficits = 32;
constexpr int kDirectCompares = 64;

// c rounded up to a multiple of blk (a mask when blk is a power of two).
__device__ __forceinline__ int pad_to(int c, int blk) {
  if ((blk & (blk - 1)) == 0) return (c + blk - 1) & -blk;
  return ((c + blk - 1) / blk) * blk;
}

// LDS of the plan.  The arrays scanned by one wave hold 64*CMAX + 1 ints
// (CMAX chunks per lane) and start on 16 bytes.
struct PlanSmem {
  int sT[kMaxE + 1];                    // T_e
  alignas(16) int sX[kMaxE + 1];        // exclusive prefix of T over e
  int sH[kMaxE];                        // h_e
  alignas(16) int sO[kMaxE + 1];        // o_e, then exclusive prefix O_e
  alignas(16) int sNp[kMaxE + 1];       // pieces of expert e, then exclusive prefix
  int sDlo[kMaxE];                      // compact index of e's first deficit rank
  int sL[kMaxR];                        // L_r
  int sDef[kMaxR];                      // def_r
  alignas(16) int sD[kMaxR + 1];        // exclusive prefix D_r
  alignas(16) int sCidx[kMaxR + 1];     // compact index among deficit ranks
  int sDl[kMaxR];                       // compact index -> rank
  int sDc[kMaxR];                       // compact index -> D of that deficit rank (strictly increasing)
  int sLb[kMaxE + 1];                   // deficit starts below O_g (line position g); [E]: below the overflow total
  alignas(16) int sRep[kMaxR + 1];      // replicas per rank, then first piece of rank
  int sPe[kMaxPieces], sPd[kMaxPieces], sPc[kMaxPieces], sPl[kMaxPieces],
      sPj[kMaxPieces], sPg[kMaxPieces];
  alignas(16) int sF[kMaxE + kMaxPieces + 1];  // flat segment padded lengths -> starts
  int sLam[kMaxE];                      // quota rule: line position of expert e inside its rank block
  int sPerm[kMaxE];                     // quota rule: expert at line position
  int sHx[kMaxE];                       // quota rule: load ahead of line position g in its rank
  // max_T, max_L, over ranks, over experts, status, nP, totOv, Ptot, tau, max replicas
  int sStat[12];
};

// Pieces per line position (sNp) and the compact index of each position's
// first deficit rank (sDlo), by the one wave that builds the plan.  With
// c(x) = number of deficit starts at or below x, the overflow [O_g, O_g +
// o_g) of line position g meets compact deficit ranks c(O_g) - 1 ..
// c(O_g + o_g - 1) - 1.  Since O_g + o_g = O_{g+1}, the upper end is the
// number of starts below O_{g+1}, so one count per position serves both
// ends: c(O_g) counted, then reduced by one where O_g is itself a start.
// NQ positions per lane (g = lane + i * 64).
template <int NQ, bool HOT>
__device__ __forceinline__ void count_pieces(PlanSmem& m, const int E, const int nDef,
                                             const bool consistent, const int lane) {
  int x[NQ], ub[NQ];
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    const int g = lane + i * kWave;
    x[i] = g < E ? m.sO[g] : INT_MIN;    // starts are >= 0: empty slots count nothing
    ub[i] = 0;
  }
  const int tot = m.sO[E];               // the overflow total
  if (nDef * NQ <= kDirectCompares) {
    // very few: count both ends of every position directly, two compares
    // per (deficit rank, position) and no second pass
    const int dcv = lane < nDef ? m.sDc[lane] : 0;
    int xhi[NQ], chi[NQ];
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int g = lane + i * kWave;
      const int o = g < E ? m.sT[HOT ? m.sPerm[g] : g] - m.sH[HOT ? m.sPerm[g] : g] : 0;
      xhi[i] = g < E ? x[i] + o - 1 : INT_MIN;
      chi[i] = 0;
    }
    for (int c = 0; c < nDef; ++c) {
      const int dc = __builtin_amdgcn_readlane(dcv, c);
#pragma unroll
      for (int i = 0; i < NQ; ++i) {
        ub[i] += dc <= x[i];
        chi[i] += dc <= xhi[i];
      }
    }
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int g = lane + i * kWave;
      if (g < E) {
        const bool has = consistent && xhi[i] >= x[i];
        m.sNp[g] = has ? chi[i] - ub[i] + 1 : 0;
        if (has) m.sDlo[g] = ub[i] - 1;
      }
    }
    return;
  }
  if (nDef <= kLinearDeficits) {
    // few deficit ranks: lane c holds start c; every lane counts the starts
    // at or below its positions, one register broadcast per deficit rank
    const int dcv = lane < nDef ? m.sDc[lane] : 0;
    int below_tot = 0;
    for (int c = 0; c < nDef; ++c) {
      const int dc = __builtin_amdgcn_readlane(dcv, c);
#pragma unroll
      for (int i = 0; i < NQ; ++i) ub[i] += dc <= x[i];
      below_tot += dc < tot;
    }
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int g = lane + i * kWave;
      const int prev = __shfl(dcv, ub[i] > 0 ? ub[i] - 1 : 0, kWave);
      if (g < E) m.sLb[g] = ub[i] - (ub[i] > 0 && prev == x[i]);
    }
    if (lane == 0) m.sLb[E] = below_tot;
  } else {
#pragma unroll
    for (int i = 0; i < NQ; ++i) {
      const int g = lane + i * kWave;
      if (g < E) {
        ub[i] = upper_bound(m.sDc, nDef, x[i]);
        m.sLb[g] = ub[i] - (ub[i] > 0 && m.sDc[ub[i] - 1] == x[i]);
      }
    }
    if (lane == 0) {
      const int u = upper_bound(m.sDc, nDef, tot);
      m.sLb[E] = u - (u > 0 && m.sDc[u - 1] == tot);
    }
  }
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    const int g = lane + i * kWave;
    if (g < E) {
      const int e = HOT ? m.sPerm[g] : g;
      const bool has = consistent && m.sT[e] - m.sH[e] > 0;
      m.sNp[g] = has ? m.sLb[g + 1] - ub[i] + 1 : 0;
      if (has) m.sDlo[g] = ub[i] - 1;
    }
  }
}

// Per expert (NQ per lane, e = lane + 64 i): the home keep h_e into sH and
// the overflow o_e into sO at its line position, from the exclusive prefix
// of T (sX) -- the fixed rule keeps the first tau pairs of the rank's home
// stream, the quota rule sheds L_r - tau from the hottest experts first:
// o_e = clamp(L_r - tau - HP_e, 0, T_e) with HP_e the load of the experts
// hotter than e in its rank.  Loads are unconditional (clamped index) so the
// unrolled iterations overlap; stores are guarded.
template <int NQ, bool HOT>
__device__ __forceinline__ void keep_and_overflow(PlanSmem& m, const Dims& d, const int tau,
                                                  const bool consistent, const int lane,
                                                  int& maxT, int& nOverE) {
  const int E = d.E, nh = d.nh;
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    const int e = lane + i * kWave;
    const bool in = e < E;
    const int ec = in ? e : 0;
    const int r0 = div_nh(ec, d) * nh;      // first expert of e's rank
    const int T = m.sT[ec];
    int h;
    if (HOT) {
      const int L = m.sX[r0 + nh] - m.sX[r0];
      const int HP = m.sHx[m.sLam[ec]];
      h = T - min(max(L - tau - HP, 0), T);
    } else {
      const int Pe = m.sX[ec] - m.sX[r0];    // position in the rank's home stream
      h = min(max(tau - Pe, 0), T);
    }
    if (!consistent) h = 0;
    if (in) {
      m.sH[e] = h;
      m.sO[HOT ? m.sLam[e] : e] = consistent ? T - h : 0;
      maxT = max(maxT, T);
      nOverE += (consistent && T - h > 0);
    }
  }
}

// The padded home-segment lengths into the flat segment list: rank r's
// entries start at r*nh + (replicas of earlier ranks), home experts first.
template <int NQ>
__device__ __forceinline__ void home_lengths(PlanSmem& m, const Dims& d, const int lane) {
  const int E = d.E, nh = d.nh;
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    const int e = lane + i * kWave;
    const int ec = e < E ? e : 0;
    const int r = div_nh(ec, d);
    const int len = pad_to(m.sH[ec], d.blk);
    const int at = r * nh + m.sRep[r] + (ec - r * nh);
    if (e < E) m.sF[at] = len;
  }
}

// The plan in LDS from T_e (in m.sT and m.sX, written and made visible by a
// workgroup barrier before the call; for HOT also m.sLam, m.sPerm and m.sHx
// = the load ahead of each line position within its rank) at threshold
// tau.  Called by all 1024 threads; wave 0 does the work, and the closing
// workgroup barrier makes the plan visible to every wave.
template <bool HOT>
__device__ __forceinline__ void plan_build(const Dims& d, PlanSmem& m, const int tau) {
  auto& sT = m.sT; auto& sX = m.sX; auto& sH = m.sH; auto& sO = m.sO; auto& sNp = m.sNp;
  auto& sDlo = m.sDlo; auto& sL = m.sL; auto& sDef = m.sDef; auto& sD = m.sD;
  auto& sCidx = m.sCidx; auto& sDl = m.sDl; auto& sDc = m.sDc; auto& sRep = m.sRep;
  auto& sPe = m.sPe;
  auto& sPd = m.sPd; auto& sPc = m.sPc; auto& sPl = m.sPl; auto& sPj = m.sPj; auto& sF = m.sF;
  auto& sPg = m.sPg;
  auto& sStat = m.sStat;
  auto& sPerm = m.sPerm;
  // expert at line position g (identity for the fixed rule)
  auto perm = [&](int g) { return HOT ? sPerm[g] : g; };
  const int tid = threadIdx.x;
  const int E = d.E, R = d.R, nh = d.nh, SK = d.SK, blk = d.blk, C = d.C;

  // 2. wave 0 alone: the plan, with wave-level scans and no barriers
  if (tid < kWave) {
    const int lane = tid;
    const int Ptot = wave_excl_scan_lds<kMaxE / kWave>(sX, E);
    const bool consistent = (long long)Ptot == (long long)R * SK;
    int maxT = 0, nOverE = 0;
    if (E <= 4 * kWave) keep_and_overflow<4, HOT>(m, d, tau, consistent, lane, maxT, nOverE);
    else keep_and_overflow<kMaxE / kWave, HOT>(m, d, tau, consistent, lane, maxT, nOverE);
    int maxL = 0, nOverR = 0;
    if (R <= kWave) {
      // lane r holds rank r: the deficit prefix D and the compact deficit
      // index come straight from register scans
      const int r = lane;
      const int rc = r < R ? r : 0;
      const int L = r < R ? sX[(rc + 1) * nh] - sX[rc * nh] : 0;
      const int def = (r < R && consistent) ? tau - min(L, tau) : 0;
      const int has = def > 0;
      const int d_in = wave_incl_scan_dpp(def), c_in = wave_incl_scan_dpp(has);
      const int d_tot = __builtin_amdgcn_readlane(d_in, kWave - 1);
      const int c_tot = __builtin_amdgcn_readlane(c_in, kWave - 1);
      if (r < R) {
        sL[r] = L;
        sDef[r] = def;
        sD[r] = d_in - def;
        sCidx[r] = c_in - has;
        sRep[r] = 0;
      }
      if (r == 0) {
        sD[R] = d_tot;
        sCidx[R] = c_tot;
      }
      if (has) {
        sDl[c_in - 1] = r;
        sDc[c_in - 1] = d_in - def;
      }
      maxL = L;
      nOverR = r < R && L > tau;
    } else {
      for (int r = lane; r < R; r += kWave) {
        const int L = sX[(r + 1) * nh] - sX[r * nh];
        const int def = consistent ? tau - min(L, tau) : 0;
        sL[r] = L;
        sDef[r] = def;
        sD[r] = def;
        sCidx[r] = def > 0;
        sRep[r] = 0;
        maxL = max(maxL, L);
        nOverR += (L > tau);
      }
      __builtin_amdgcn_wave_barrier();
      wave_excl_scan_lds<kMaxR / kWave>(sD, R);
      wave_excl_scan_lds<kMaxR / kWave>(sCidx, R);
      for (int r = lane; r < R; r += kWave)
        if (sDef[r] > 0) {
          sDl[sCidx[r]] = r;
          sDc[sCidx[r]] = sD[r];
        }
    }
    __builtin_amdgcn_wave_barrier();
    const int totOv = wave_excl_scan_lds<kMaxE / kWave>(sO, E);
    const int nDef = sCidx[R];
    if (E <= 4 * kWave) count_pieces<4, HOT>(m, E, nDef, consistent, lane);
    else count_pieces<kMaxE / kWave, HOT>(m, E, nDef, consistent, lane);
    __builtin_amdgcn_wave_barrier();
    const int nP = wave_excl_scan_lds<kMaxE / kWave>(sNp, E);
    // line position of every piece: each position lists its own pieces
    // (few per position), so a piece finds its position by one LDS read
    // instead of a search over all E positions
    for (int g0 = lane; g0 < E; g0 += kWave)
      for (int g = sNp[g0]; g < sNp[g0 + 1]; ++g) sPg[g] = g0;
    __builtin_amdgcn_wave_barrier();
    // one lane per replica segment ("piece"), in line order
    for (int g = lane; g < nP; g += kWave) {
      const int ge = sPg[g];                       // line position of the piece's expert
      const int e = perm(ge);
      const int jj = g - sNp[ge];
      const int dd = sDl[sDlo[ge] + jj];
      const int Oe = sO[ge], o = sT[e] - sH[e];
      const int lo = max(Oe, sD[dd]);
      const int hi = min(Oe + o, sD[dd] + sDef[dd]);
      sPe[g] = e;
      sPd[g] = dd;
      sPc[g] = hi - lo;
      sPl[g] = lo;
      atomicAdd(&sRep[dd], 1);
    }
    __builtin_amdgcn_wave_barrier();
    wave_excl_scan_lds<kMaxR / kWave>(sRep, R);   // first piece of each rank
    // flat segment list: rank r's E/R home experts, then its pieces
    for (int g = lane; g < nP; g += kWave) {
      const int dd = sPd[g];
      const int jj = g - sRep[dd];
      sPj[g] = jj;
      sF[dd * nh + sRep[dd] + nh + jj] = pad_to(sPc[g], blk);
    }
    if (E <= 4 * kWave) home_lengths<4>(m, d, lane);
    else home_lengths<kMaxE / kWave>(m, d, lane);
    __builtin_amdgcn_wave_barrier();
    wave_excl_scan_lds<(kMaxE + kMaxPieces) / kWave>(sF, E + nP);
    // wave-wide reductions of the statistics
    maxT = wave_max(maxT);
    maxL = wave_max(maxL);
    nOverE = wave_sum(nOverE);
    nOverR = wave_sum(nOverR);
    // replicas and padded rows per rank: the capacity check
    int maxRep = 0;
    bool over_cap = false;
    for (int r = lane; r < R; r += kWave) {
      maxRep = max(maxRep, sRep[r + 1] - sRep[r]);
      over_cap = over_cap || sF[(r + 1) * nh + sRep[r + 1]] - sF[r * nh + sRep[r]] > C;
    }
    maxRep = wave_max(maxRep);
    over_cap = __any(over_cap);
    if (lane == 0) {
      sStat[8] = tau;
      sStat[9] = maxRep;
      sStat[0] = maxT;
      sStat[1] = maxL;
      sStat[2] = nOverR;
      sStat[3] = nOverE;
      sStat[4] = (consistent ? 0 : LBT_ST_BADCOUNT) | (over_cap ? LBT_ST_CAPACITY : 0);
      sStat[5] = nP;
      sStat[6] = totOv;
      sStat[7] = Ptot;
    }
  }
  __syncthreads();
}

// The header, *status and the blob from the plan in LDS (after plan_build),
// by the nthr threads (a multiple of 64) whose index in that group is wt.
// The locality counts (HOT) read the load matrix from sCnt when given (an
// LDS copy), else from counts.
template <bool HOT>
__device__ __forceinline__ void plan_write(const Dims& d, const PlanSmem& m,
                                           const int32_t* __restrict__ counts, const int* sCnt,
                                           int32_t* __restrict__ plan,
                                           int32_t* __restrict__ status, const int wt,
                                           const int nthr) {
  auto count_of = [&](int r, int e) {
    return sCnt != nullptr ? sCnt[r * d.E + e] : counts[(long long)r * d.E + e];
  };
  auto& sT = m.sT; auto& sH = m.sH; auto& sO = m.sO; auto& sL = m.sL; auto& sDef = m.sDef;
  auto& sD = m.sD; auto& sCidx = m.sCidx; auto& sRep = m.sRep; auto& sPe = m.sPe;
  auto& sPd = m.sPd; auto& sPc = m.sPc; auto& sPl = m.sPl; auto& sPj = m.sPj; auto& sF = m.sF;
  auto& sStat = m.sStat; auto& sLam = m.sLam;
  auto lam = [&](int e) { return HOT ? sLam[e] : e; };
  const int E = d.E, R = d.R, nh = d.nh, B = d.B;
  const PlanLayout pl = d.pl;
  const int ms = pl.max_seg;
  // rank r's flat entries are [fb(r), fb(r+1)) with fb(r) = r*nh + sRep[r]
  const int nP = sStat[5];
  int32_t* P = plan;

  // the header and the status word: everything they hold is in LDS already,
  // so no further barrier (which would also wait for the blob's stores)
  if (wt == 0) {
    const int st = sStat[4];
    P[pl.hdr + LBT_HDR_N_PIECES] = nP;
    P[pl.hdr + LBT_HDR_MAX_T] = sStat[0];
    P[pl.hdr + LBT_HDR_MAX_L] = sStat[1];
    P[pl.hdr + LBT_HDR_TOTAL_OVERFLOW] = sStat[6];
    P[pl.hdr + LBT_HDR_N_DEFICIT_RANKS] = sCidx[R];
    P[pl.hdr + LBT_HDR_N_OVERFLOW_RANKS] = sStat[2];
    P[pl.hdr + LBT_HDR_N_OVERFLOW_EXPERTS] = sStat[3];
    P[pl.hdr + LBT_HDR_STATUS] = st;
    P[pl.hdr + LBT_HDR_P] = sStat[7];
    P[pl.hdr + LBT_HDR_TAU] = sStat[8];
    P[pl.hdr + LBT_HDR_MAX_REPLICAS] = sStat[9];
    P[pl.hdr + LBT_HDR_FEASIBLE] = sStat[9] <= B ? 1 : 0;
    P[pl.hdr + LBT_HDR_LOCAL] = HOT ? 1 : 0;
    for (int i = LBT_HDR_LOCAL + 1; i < LBT_HDR_WORDS; ++i) P[pl.hdr + i] = 0;
    if (status != nullptr) *status = st;
  }

  for (int e = wt; e < E; e += nthr) {
    const int r = div_nh(e, d);
    const int fb = r * nh + sRep[r];
    P[pl.T + e] = sT[e];
    P[pl.h + e] = sH[e];
    // quota rule: the part of the home quota its own rank's tokens take
    P[pl.home_local + e] = HOT ? min(sH[e], count_of(r, e)) : 0;
    P[pl.O + e] = sO[lam(e)];
    P[pl.home_row + e] = sF[fb + (e - r * nh)] - sF[fb];
  }
  for (int r = wt; r < R; r += nthr) {
    const int fb = r * nh + sRep[r];
    const int fe = (r + 1) * nh + sRep[r + 1];
    const int nrep = sRep[r + 1] - sRep[r];
    const int nrp = sF[fe] - sF[fb];
    P[pl.L + r] = sL[r];
    P[pl.def + r] = sDef[r];
    P[pl.D + r] = sD[r];
    P[pl.n_seg + r] = nh + nrep;
    P[pl.n_rows_padded + r] = nrp;
    P[pl.n_slots + r] = min(nrep, B);
    P[pl.n_remote + r] = nrep - min(nrep, B);
  }
  if (wt == 0) P[pl.D + R] = sD[R];
  // segment tables, one rank per wave at a time, entries across the lanes.
  // Ranks go to the waves from the last one down (the first waves also
  // write the per-expert arrays and the pieces), and each lane handles
  // kSegUnroll entries per trip with every LDS read issued before the
  // stores, so a trip waits for one LDS round trip instead of one per
  // 64 entries (DSV3: 256 entries per rank).
  constexpr int kSegUnroll = 4;
  const int nw = nthr / kWave;
  for (int r = nw - 1 - wt / kWave; r < R; r += nw) {
    const int rep0 = sRep[r], nrep = sRep[r + 1] - rep0;
    const int fb = r * nh + rep0;
    const int nseg = nh + nrep;
    const int f0 = sF[fb];
    const long long row = (long long)r * ms;
    const long long row1 = (long long)r * (ms + 1);
    for (int s0 = lane_id(); s0 <= ms; s0 += kSegUnroll * kWave) {
      int ex[kSegUnroll], wr[kSegUnroll], cnt[kSegUnroll], st[kSegUnroll];
#pragma unroll
      for (int u = 0; u < kSegUnroll; ++u) {
        const int s = s0 + u * kWave;
        ex[u] = -1;
        wr[u] = -1;
        cnt[u] = 0;
        if (s < nh) {
          ex[u] = r * nh + s;
          wr[u] = ex[u];
          cnt[u] = sH[ex[u]];
        } else if (s < nseg) {
          const int g = rep0 + (s - nh);
          ex[u] = sPe[g];
          cnt[u] = sPc[g];
          wr[u] = (s - nh < B) ? E + (s - nh) : ex[u];
        }
        st[u] = sF[fb + min(s, nseg)];
      }
#pragma unroll
      for (int u = 0; u < kSegUnroll; ++u) {
        const int s = s0 + u * kWave;
        if (s < ms) {
          P[pl.seg_expert + row + s] = ex[u];
          P[pl.seg_wrow + row + s] = wr[u];
          P[pl.seg_count + row + s] = cnt[u];
        }
        if (s <= ms) P[pl.seg_start + row1 + s] = st[u] - f0;
      }
    }
  }
  for (int g = wt; g < pl.max_pieces; g += nthr) {
    int ex = -1, dd = -1, cnt = 0, line = -1, row = -1, wrow = -1, loc = 0;
    if (g < nP) {
      ex = sPe[g];
      dd = sPd[g];
      cnt = sPc[g];
      line = sPl[g];
      const int fb = dd * nh + sRep[dd];
      row = sF[fb + nh + sPj[g]] - sF[fb];
      wrow = sPj[g] < B ? E + sPj[g] : ex;
      if (HOT) loc = min(cnt, count_of(dd, ex));   // its own rank's tokens
    }
    P[pl.piece_local + g] = loc;
    P[pl.piece_wrow + g] = wrow;
    P[pl.piece_expert + g] = ex;
    P[pl.piece_rank + g] = dd;
    P[pl.piece_count + g] = cnt;
    P[pl.piece_line + g] = line;
    P[pl.piece_row + g] = row;
  }
}

// plan_build then plan_write by the whole workgroup: the plan from T_e at
// threshold tau, with the blob and *status written.
template <bool HOT>
__device__ __forceinline__ void plan_core(const Dims& d, PlanSmem& m, const int tau,
                                          const int32_t* __restrict__ counts,
                                          const int* sCnt, int32_t* __restrict__ plan,
                                          int32_t* __restrict__ status) {
  plan_build<HOT>(d, m, tau);
  plan_write<HOT>(d, m, counts, sCnt, plan, status, (int)threadIdx.x, kPlanThreads);
}

}  // namespace lbt
