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
// Up to this many deficit ranks the per-expert piece counts come from a
// register-broadcast count (cost grows with the deficit ranks); above it,
// from binary searches (cost grows with their logarithm).  Measured on
// MI355X: 7 deficit ranks 0.96 vs 1.68 us, about 25 3.8 vs 4.7 us, about
// 49 4.7 vs 3.6 us.
constexpr int kLinearDeficits = 32;

__device__ __forceinline__ int pad_to(int c, int blk) { return ((c + blk - 1) / blk) * blk; }

// LDS of the plan.
struct PlanSmem {
  int sT[kMaxE + 1];      // T_e
  int sX[kMaxE + 1];      // exclusive prefix of T over e
  int sH[kMaxE];          // h_e
  int sO[kMaxE + 1];      // o_e, then exclusive prefix O_e
  int sNp[kMaxE + 1];     // pieces of expert e, then exclusive prefix
  int sDlo[kMaxE];        // compact index of e's first deficit rank
  int sL[kMaxR];          // L_r
  int sDef[kMaxR];        // def_r
  int sD[kMaxR + 1];      // exclusive prefix D_r
  int sCidx[kMaxR + 1];   // compact index among deficit ranks
  int sDl[kMaxR];         // compact index -> rank
  int sDc[kMaxR];         // compact index -> D of that deficit rank (strictly increasing)
  int sRep[kMaxR + 1];    // replicas per rank, then first piece of rank
  int sPe[kMaxPieces], sPd[kMaxPieces], sPc[kMaxPieces], sPl[kMaxPieces],
      sPj[kMaxPieces];
  int sF[kMaxE + kMaxPieces + 1];  // flat segment padded lengths -> starts
  int sLam[kMaxE];        // quota rule: line position of expert e inside its rank block
  int sPerm[kMaxE];       // quota rule: expert at line position
  int sHx[kMaxE + 1];     // quota rule: loads in line order, then exclusive prefix
  // max_T, max_L, over ranks, over experts, status, nP, totOv, Ptot, tau, max replicas
  int sStat[12];

};

// The plan from T_e (in m.sT and m.sX, written and made visible by a
// workgroup barrier before the call; for HOT also m.sLam, m.sPerm and m.sHx
// = exclusive prefix of the loads in line order) at threshold tau; 1024
// threads; writes the whole blob and *status.
template <bool HOT>
__device__ __forceinline__ void plan_core(const Dims& d, PlanSmem& m, const int tau,
                                          int32_t* __restrict__ plan,
                                          int32_t* __restrict__ status) {
  auto& sT = m.sT; auto& sX = m.sX; auto& sH = m.sH; auto& sO = m.sO; auto& sNp = m.sNp;
  auto& sDlo = m.sDlo; auto& sL = m.sL; auto& sDef = m.sDef; auto& sD = m.sD;
  auto& sCidx = m.sCidx; auto& sDl = m.sDl; auto& sDc = m.sDc; auto& sRep = m.sRep;
  auto& sPe = m.sPe;
  auto& sPd = m.sPd; auto& sPc = m.sPc; auto& sPl = m.sPl; auto& sPj = m.sPj; auto& sF = m.sF;
  auto& sStat = m.sStat;
  auto& sLam = m.sLam; auto& sPerm = m.sPerm; auto& sHx = m.sHx;
  // line position of expert e, expert at line position g (identity for the fixed rule)
  auto lam = [&](int e) { return HOT ? sLam[e] : e; };
  auto perm = [&](int g) { return HOT ? sPerm[g] : g; };
  const int tid = threadIdx.x;
  const int E = d.E, R = d.R, nh = d.nh, SK = d.SK, B = d.B, blk = d.blk, C = d.C;
  const PlanLayout pl = d.pl;
  const int ms = pl.max_seg;

  // 2. wave 0 alone: the plan, with wave-level scans and no barriers
  if (tid < kWave) {
    const int lane = tid;
    const int Ptot = wave_excl_scan_lds<kMaxE / kWave>(sX, E);
    const bool consistent = (long long)Ptot == (long long)R * SK;
    int maxT = 0, nOverE = 0;
    for (int e = lane; e < E; e += kWave) {
      const int r = e / nh;
      const int T = sT[e];
      int h;
      if (HOT) {
        // shed L_r - tau from the hottest experts: o_e = clamp(L_r - tau - HP_e, 0, T_e)
        // with HP_e the load of the experts hotter than e in its rank
        const int L = sX[(r + 1) * nh] - sX[r * nh];
        const int HP = sHx[sLam[e]] - sHx[r * nh];
        h = T - min(max(L - tau - HP, 0), T);
      } else {
        const int Pe = sX[e] - sX[r * nh];      // position in r's home stream
        h = min(max(tau - Pe, 0), T);
      }
      if (!consistent) h = 0;
      sH[e] = h;
      sO[lam(e)] = consistent ? T - h : 0;
      maxT = max(maxT, T);
      nOverE += (consistent && T - h > 0);
    }
    int maxL = 0, nOverR = 0;
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
    const int totOv = wave_excl_scan_lds<kMaxE / kWave>(sO, E);
    wave_excl_scan_lds<kMaxR / kWave>(sD, R);
    wave_excl_scan_lds<kMaxR / kWave>(sCidx, R);
    for (int r = lane; r < R; r += kWave)
      if (sDef[r] > 0) {
        sDl[sCidx[r]] = r;
        sDc[sCidx[r]] = sD[r];
      }
    __builtin_amdgcn_wave_barrier();
    // Pieces of the expert at line position g: its overflow [O, O + o)
    // meets the deficit ranks from the one holding O to the one holding
    // O + o - 1.  With c(x) = number of deficit ranks starting at or below
    // x, those are compact indices c(O) - 1 .. c(O + o - 1) - 1.
    const int nDef = sCidx[R];
    if (nDef <= kLinearDeficits) {
      // few deficit ranks: lane c holds start c, and every lane counts the
      // starts at or below its experts' first and last overflow positions,
      // one register broadcast per deficit rank (no LDS in the loop)
      const int dcv = lane < nDef ? sDc[lane] : 0;
      for (int g0 = 0; g0 < E; g0 += 4 * kWave) {
        int xlo[4], xhi[4], clo[4], chi[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int g = g0 + lane + i * kWave;
          const int o = g < E ? sT[perm(g)] - sH[perm(g)] : 0;
          xlo[i] = g < E ? sO[g] : -1;      // empty slots count nothing
          xhi[i] = g < E ? xlo[i] + o - 1 : -2;
          clo[i] = 0;
          chi[i] = 0;
        }
        for (int c = 0; c < nDef; ++c) {
          const int dc = __builtin_amdgcn_readlane(dcv, c);
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            clo[i] += dc <= xlo[i];
            chi[i] += dc <= xhi[i];
          }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int g = g0 + lane + i * kWave;
          if (g < E) {
            const bool has = consistent && xhi[i] >= xlo[i];
            sNp[g] = has ? chi[i] - clo[i] + 1 : 0;
            if (has) sDlo[g] = clo[i] - 1;
          }
        }
      }
    } else {
      for (int g = lane; g < E; g += kWave) {     // line position g, expert perm(g)
        const int e = perm(g);
        const int o = sT[e] - sH[e];
        int np = 0;
        if (consistent && o > 0) {
          const int Oe = sO[g];
          const int clo = upper_bound(sDc, nDef, Oe);
          const int chi = upper_bound(sDc, nDef, Oe + o - 1);
          np = chi - clo + 1;
          sDlo[g] = clo - 1;
        }
        sNp[g] = np;
      }
    }
    __builtin_amdgcn_wave_barrier();
    const int nP = wave_excl_scan_lds<kMaxE / kWave>(sNp, E);
    // one lane per replica segment ("piece"), in line order
    for (int g = lane; g < nP; g += kWave) {
      const int ge = upper_bound(sNp, E, g) - 1;   // line position of the piece's expert
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
    for (int e = lane; e < E; e += kWave) {
      const int r = e / nh;
      sF[r * nh + sRep[r] + (e - r * nh)] = pad_to(sH[e], blk);
    }
    __builtin_amdgcn_wave_barrier();
    wave_excl_scan_lds<(kMaxE + kMaxPieces) / kWave>(sF, E + nP);
    // wave-wide reductions of the statistics
    for (int o = 32; o > 0; o >>= 1) {
      maxT = max(maxT, __shfl_xor(maxT, o, kWave));
      maxL = max(maxL, __shfl_xor(maxL, o, kWave));
      nOverE += __shfl_xor(nOverE, o, kWave);
      nOverR += __shfl_xor(nOverR, o, kWave);
    }
    int maxRep = 0;
    for (int r = lane; r < R; r += kWave) maxRep = max(maxRep, sRep[r + 1] - sRep[r]);
    maxRep = wave_max(maxRep);
    if (lane == 0) {
      sStat[8] = tau;
      sStat[9] = maxRep;
      sStat[0] = maxT;
      sStat[1] = maxL;
      sStat[2] = nOverR;
      sStat[3] = nOverE;
      sStat[4] = consistent ? 0 : LBT_ST_BADCOUNT;
      sStat[5] = nP;
      sStat[6] = totOv;
      sStat[7] = Ptot;
    }
  }
  __syncthreads();
  // rank r's flat entries are [fb(r), fb(r+1)) with fb(r) = r*nh + sRep[r]
  const int nP = sStat[5];

  // 3. every wave: write the blob from LDS
  int32_t* P = plan;
  for (int e = tid; e < E; e += kPlanThreads) {
    const int r = e / nh;
    const int fb = r * nh + sRep[r];
    P[pl.T + e] = sT[e];
    P[pl.h + e] = sH[e];
    P[pl.O + e] = sO[lam(e)];
    P[pl.home_row + e] = sF[fb + (e - r * nh)] - sF[fb];
  }
  int capflag = 0;
  for (int r = tid; r < R; r += kPlanThreads) {
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
    if (nrp > C) capflag = LBT_ST_CAPACITY;
  }
  if (capflag) atomicOr(&sStat[4], capflag);
  if (tid == 0) P[pl.D + R] = sD[R];
  // segment tables, one rank per wave at a time, entries across the lanes
  constexpr int kPlanWaves = kPlanThreads / kWave;
  for (int r = wave_id(); r < R; r += kPlanWaves) {
    const int rep0 = sRep[r], nrep = sRep[r + 1] - rep0;
    const int fb = r * nh + rep0;
    const int nseg = nh + nrep;
    const int f0 = sF[fb];
    const long long row = (long long)r * ms;
    for (int s = lane_id(); s < ms; s += kWave) {
      int ex = -1, wr = -1, cnt = 0;
      if (s < nh) {
        ex = r * nh + s;
        wr = ex;
        cnt = sH[ex];
      } else if (s < nseg) {
        const int g = rep0 + (s - nh);
        ex = sPe[g];
        cnt = sPc[g];
        wr = (s - nh < B) ? E + (s - nh) : ex;
      }
      P[pl.seg_expert + row + s] = ex;
      P[pl.seg_wrow + row + s] = wr;
      P[pl.seg_count + row + s] = cnt;
    }
    const long long row1 = (long long)r * (ms + 1);
    for (int s = lane_id(); s <= ms; s += kWave)
      P[pl.seg_start + row1 + s] = (s < nseg ? sF[fb + s] : sF[fb + nseg]) - f0;
  }
  for (int g = tid; g < pl.max_pieces; g += kPlanThreads) {
    int ex = -1, dd = -1, cnt = 0, line = -1, row = -1, wrow = -1;
    if (g < nP) {
      ex = sPe[g];
      dd = sPd[g];
      cnt = sPc[g];
      line = sPl[g];
      const int fb = dd * nh + sRep[dd];
      row = sF[fb + nh + sPj[g]] - sF[fb];
      wrow = sPj[g] < B ? E + sPj[g] : ex;
    }
    P[pl.piece_wrow + g] = wrow;
    P[pl.piece_expert + g] = ex;
    P[pl.piece_rank + g] = dd;
    P[pl.piece_count + g] = cnt;
    P[pl.piece_line + g] = line;
    P[pl.piece_row + g] = row;
  }
  __syncthreads();
  if (tid == 0) {
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
    for (int i = LBT_HDR_FEASIBLE + 1; i < LBT_HDR_WORDS; ++i) P[pl.hdr + i] = 0;
    if (status != nullptr) *status = st;
  }
}

}  // namespace lbt
