// MoE Align & Sort under the balancing plan: the destination row of every
// (token, expert) pair, the inverse map, and the per-block weight-row table.
//
// [AlignSort]: pairs are sorted by expert id with each expert's share padded
// to the grouped GEMM's block; the permutation records source -> target.
// The prior kernel there computes aligned offsets in one block, then
// scatters; here the offsets come from the plan and the per-tile prefix
// counts, so every tile of 128 tokens works independently.
// [UltraEP] section "その仕組みは高速なエキスパート複製に依存する": per-token
// destinations are a local lookup against cumulative quotas, and under a
// quota plan tokens first use the capacity of their own rank's instance of
// their expert (the locality step): pair rank among its rank's pairs of e
// below that instance's local count -> that instance; otherwise its rank
// among the pairs left after the local step picks the home's or a piece's
// share of the rest.
//
// Stable rank of a pair inside its expert: q = (pairs of e in earlier tiles,
// from the column scan) + (pairs of e in earlier 32-token sub-tiles of this
// tile) + popcount of the sub-tile's bit mask of tokens holding e below this
// token.  A token holds K distinct experts, so ranks by token order equal
// ranks by flat index f = t*K + k.
#include "align_core.h"

namespace lbt {

// Threads per token.  Measured on MI355X (align alone, in the step):
// 1 / 2 / 4 / 8 threads per token took DSV3 15.7 / 11.6 / 9.5 / 8.9 us and
// Kimi-K3 62 / 49 / 37 / 36 us; 4 keeps every thread busy for K = 4 and 8.
constexpr int kAlignTPT = 4;
constexpr int kAlignThreads = kTileTokens * kAlignTPT;
constexpr int kBlockWaves = kAlignThreads / kWave;   // blocks handled per workgroup

// Thread tid serves token tid % kTileTokens of the tile and its pairs
// k = part, part + TPT, ... with part = tid / kTileTokens.
template <int TPT>
__global__ __launch_bounds__(kTileTokens * TPT) void k_align(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ work,
    const int32_t* __restrict__ plan, Dims d, int32_t* __restrict__ slot,
    int32_t* __restrict__ sorted_ids, int32_t* __restrict__ block_wrow,
    int32_t* __restrict__ block_expert, int32_t* __restrict__ status) {
  constexpr int NT = kTileTokens * TPT;
  if ((int)blockIdx.x >= d.n_tiles) {
    const long long gb = (long long)(blockIdx.x - d.n_tiles) * (NT / kWave) + wave_id();
    if (gb < (long long)d.R * d.n_blocks) align_blocks(plan, d, gb, sorted_ids, block_wrow, block_expert);
    return;
  }
  // LDS, carved to the shape (align_lds_bytes): per expert sH, sO, sHome,
  // sBase and, for the locality step of quota plans, sHL (home local
  // count), sSrc0 (pairs of e from ranks below this tile's rank r), sPN
  // (first piece << 16 | piece count), sLocCap / sLocRow (r's own instance
  // of e: quota its tokens take, start row), sLP (local pairs of instances
  // on ranks <= r); the sub-tile masks and prefix counts; per piece sPl,
  // sPd, sPr, sPe, sPc, sPLoc (local count) and sRem (start of its share of
  // the pairs left after the local step).
  extern __shared__ int smem[];
  const int Ea = d.E, Pa = d.pl.max_pieces;
  int* sH = smem;
  int* sO = sH + Ea;
  int* sHome = sO + Ea;
  int* sBase = sHome + Ea;
  int* sHL = sBase + Ea;
  int* sSrc0 = sHL + Ea;
  int* sPN = sSrc0 + Ea;
  int* sLocCap = sPN + Ea;
  int* sLocRow = sLocCap + Ea;
  int* sLP = sLocRow + Ea;
  uint32_t* sMask = reinterpret_cast<uint32_t*>(sLP + Ea);   // [kSubTiles][E]
  int* sSub = reinterpret_cast<int*>(sMask + kSubTiles * Ea); // [kSubTiles][E]
  int* sPl = sSub + kSubTiles * Ea;
  int* sPd = sPl + Pa;
  int* sPr = sPd + Pa;
  int* sPe = sPr + Pa;
  int* sPc = sPe + Pa;
  int* sPLoc = sPc + Pa;
  int* sRem = sPLoc + Pa;

  const PlanLayout& pl = d.pl;
  const int E = d.E, K = d.K, C = d.C, nh = d.nh;
  const int tile = blockIdx.x;
  const int r = tile / d.tpr, j = tile - r * d.tpr;
  const int t0 = r * d.S + j * kTileTokens;
  const int len = min(kTileTokens, d.S - j * kTileTokens);
  const int nP = min(plan[pl.hdr + LBT_HDR_N_PIECES], pl.max_pieces);
  const int totOv = plan[pl.hdr + LBT_HDR_TOTAL_OVERFLOW];
  const bool local = plan[pl.hdr + LBT_HDR_LOCAL] != 0;
  const int32_t* tbase = work + work_tile_base(d) + (long long)tile * E;
  const int32_t* rbase = work + work_tile_base(d) + (long long)r * d.tpr * E;   // rank r's first tile
  const int tid = threadIdx.x;
  const int ti = tid % kTileTokens, part = tid / kTileTokens;
  const long long t = (long long)t0 + ti;

  // the thread's first kPre expert ids (k = part + j * TPT), loaded before
  // the plan so that the two latencies overlap (for K <= 8 no id is read
  // twice)
  constexpr int kPre = (8 + TPT - 1) / TPT;
  int idp[kPre];
#pragma unroll
  for (int j = 0; j < kPre; ++j) {
    const int k = part + j * TPT;
    idp[j] = (ti < len && k < K) ? ids[t * K + k] : -1;
  }

  for (int e = tid; e < E; e += NT) {
    sH[e] = plan[pl.h + e];
    sO[e] = plan[pl.O + e];
    sHome[e] = plan[pl.home_row + e];
    sBase[e] = tbase[e];
    sHL[e] = plan[pl.home_local + e];
    sSrc0[e] = rbase[e];
#pragma unroll
    for (int s = 0; s < kSubTiles; ++s) sMask[s * E + e] = 0u;
  }
  // the whole piece table (entries past nP are unused), so that these loads
  // do not wait for the piece count
  for (int g = tid; g < pl.max_pieces; g += NT) {
    sPl[g] = plan[pl.piece_line + g];
    sPd[g] = plan[pl.piece_rank + g];
    sPr[g] = plan[pl.piece_row + g];
    sPe[g] = plan[pl.piece_expert + g];
    sPc[g] = plan[pl.piece_count + g];
    sPLoc[g] = plan[pl.piece_local + g];
  }
  __syncthreads();

  if (local) {
    // per expert: walk its instances (home, then its pieces in line order)
    for (int e = tid; e < E; e += NT) {
      const int he = e / nh;
      int cap = 0, row0 = 0, lp = 0;
      if (he == r) {
        cap = sHL[e];
        row0 = sHome[e];
      }
      if (he <= r) lp += sHL[e];
      int rs = sH[e] - sHL[e];                 // the home's share of the remaining pairs
      const int p0 = upper_bound(sPl, nP, sO[e]) - 1;   // the piece holding O_e, if e's
      int np = 0;
      if (p0 >= 0 && sPe[p0] == e) {
        for (int g = p0; g < nP && sPe[g] == e; ++g, ++np) {
          const int dg = sPd[g];
          if (dg == r) {
            cap = sPLoc[g];
            row0 = sPr[g];
          }
          if (dg <= r) lp += sPLoc[g];
          sRem[g] = rs;
          rs += sPc[g] - sPLoc[g];
        }
      }
      sPN[e] = (max(p0, 0) << 16) | np;   // p0 < max_pieces <= 1024, np <= max_pieces
      sLocCap[e] = cap;
      sLocRow[e] = row0;
      sLP[e] = lp;
    }
  }

  int flags = 0;
  const int sub = ti / kSubTokens;
  const uint32_t bit = 1u << (ti % kSubTokens);
  auto mark = [&](int e) {
    if (e < 0 || e >= E) return;
    const uint32_t old = atomicOr(&sMask[sub * E + e], bit);
    if (old & bit) flags |= LBT_ST_DUPID;
  };
  if (ti < len) {
#pragma unroll
    for (int j = 0; j < kPre; ++j)
      if (part + j * TPT < K) mark(idp[j]);
    for (int k = part + kPre * TPT; k < K; k += TPT) mark(ids[t * K + k]);
  }
  __syncthreads();
  for (int e = tid; e < E; e += NT) {
    int run = 0;
#pragma unroll
    for (int s = 0; s < kSubTiles; ++s) {
      sSub[s * E + e] = run;
      run += __popc(sMask[s * E + e]);
    }
  }
  __syncthreads();

  auto place = [&](int k, int e) {
    const long long f = t * K + k;
    if (e < 0 || e >= E) {
      flags |= LBT_ST_BADID;
      slot[f] = -1;
      return;
    }
    const int q = sBase[e] + sSub[sub * E + e] + __popc(sMask[sub * E + e] & (bit - 1u));
    const int h = sH[e];
    int dd, row;
    bool ok = true;
    if (local) {
      const int qs = q - sSrc0[e];             // rank of the pair among e's pairs from rank r
      if (qs < sLocCap[e]) {                   // taken by r's own instance of e
        dd = r;
        row = sLocRow[e] + qs;
      } else {
        const int qr = q - sLP[e];             // rank among the pairs left after the local step
        const int hrem = h - sHL[e];
        if (qr < hrem) {
          dd = e / nh;
          row = sHome[e] + sHL[e] + qr;
        } else {
          // the last of e's pieces whose share starts at or below qr
          const int p0 = sPN[e] >> 16, np = sPN[e] & 0xFFFF;
          int lo = 0, hi = np;
          while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (sRem[p0 + mid] <= qr) lo = mid + 1; else hi = mid;
          }
          const int g = p0 + lo - 1;
          ok = lo > 0 && qr < sRem[g] + (sPc[g] - sPLoc[g]);
          dd = ok ? sPd[g] : 0;
          row = ok ? sPr[g] + sPLoc[g] + (qr - sRem[g]) : 0;
        }
      }
    } else if (q < h) {
      dd = e / nh;
      row = sHome[e] + q;
    } else {
      const int o = sO[e] + (q - h);
      const int g = upper_bound(sPl, nP, o) - 1;
      ok = o < totOv && g >= 0 && sPe[g] == e;
      dd = ok ? sPd[g] : 0;
      row = ok ? sPr[g] + (o - sPl[g]) : 0;
    }
    // a row past the capacity, or a rank / row a corrupt plan would give
    if (!ok || row >= C || row < 0 || dd < 0 || dd >= d.R) {
      flags |= LBT_ST_CAPACITY;
      slot[f] = -1;
      return;
    }
    const long long dst = (long long)dd * C + row;
    slot[f] = (int)dst;
    sorted_ids[dst] = (int)f;
  };
  if (ti < len) {
#pragma unroll
    for (int j = 0; j < kPre; ++j)
      if (part + j * TPT < K) place(part + j * TPT, idp[j]);
    for (int k = part + kPre * TPT; k < K; k += TPT) place(k, ids[t * K + k]);
  }
  if (flags && status != nullptr) atomicOr(status, flags);
}

// LDS of a tile workgroup: 10 per-expert arrays, the two [kSubTiles][E]
// sub-tile tables and 7 per-piece arrays; at most 64 KiB (E = 512, 1024
// pieces).
static size_t align_lds_bytes(const Dims& d) {
  return sizeof(int) * ((size_t)(10 + 2 * kSubTiles) * d.E + (size_t)7 * d.pl.max_pieces);
}

hipError_t launch_align(const Dims& d, const int32_t* ids, const int32_t* work, const int32_t* plan,
                        int32_t* slot, int32_t* sorted_ids, int32_t* block_wrow,
                        int32_t* block_expert, int32_t* status, hipStream_t st) {
  const long long nblk = (long long)d.R * d.n_blocks;
  const long long grid = d.n_tiles + (nblk + kBlockWaves - 1) / kBlockWaves;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(k_align<kAlignTPT>, dim3((unsigned)grid), dim3(kAlignThreads),
                     align_lds_bytes(d), st, ids, work, plan, d, slot, sorted_ids, block_wrow,
                     block_expert, status);
  return hipGetLastError();
}

}  // namespace lbt
