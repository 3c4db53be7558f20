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
#include "fused.h"
#include "rows.h"

namespace lbt {

// Threads of a tile workgroup.  The tile's pairs f = t0*K + p are taken in
// flat order, thread tid placing p = tid, tid + 512, ..., so consecutive
// lanes read consecutive ids and write consecutive slots.  (Measured on
// MI355X with 1 / 2 / 4 / 8 threads per token instead, each taking every
// 1st / 2nd / 4th / 8th pair of its token: DSV3 15.7 / 11.6 / 9.5 / 8.9 us,
// Kimi-K3 62 / 49 / 37 / 36 us.)
constexpr int kAlignThreads = 512;
constexpr int kBlockWaves = kAlignThreads / kWave;   // blocks handled per workgroup
// Tile workgroups the chip holds at once (256 CUs, four 512-thread
// workgroups each).
constexpr int kAlignTilesOneRound = 1024;

// MOVE: the dispatch fused in (batches of at most kMoveTokens tokens).  Each
// tile has D = min(128, S) workgroups, workgroup g of a tile handling the
// tile's token g: it builds the tile's masks and plan arrays like a tile
// workgroup, places only its token's K pairs (so every pair is still placed
// once), then copies the token's row x[t] to each of their rows of recv.
// The outputs are lbt_align_sort's and lbt_dispatch's, one launch and one
// dependent round trip (slot written, then read back) fewer.
template <int NT, bool MOVE>
__global__ __launch_bounds__(NT) void k_align(
    const int32_t* __restrict__ ids, const int32_t* __restrict__ work,
    const int32_t* __restrict__ plan, Dims d, int32_t* __restrict__ slot,
    int32_t* __restrict__ sorted_ids, int32_t* __restrict__ block_wrow,
    int32_t* __restrict__ block_expert, int32_t* __restrict__ status,
    const u32x4* __restrict__ x, u32x4* __restrict__ recv) {
  // Block-table workgroups and tile workgroups share the grid.  When the
  // tiles fit the chip in one round they go first and the short block-table
  // workgroups finish under them (DSV3: 256 tiles; dispatching the 510
  // block-table workgroups first delayed every tile by ~0.8 us).  When the
  // tiles take several rounds the block-table workgroups go first, or they
  // would start only after the last tile was dispatched (Kimi-K3: 2048
  // tiles; placed after them they ended ~3 us past the last tile).
  const long long nblk = (long long)d.R * d.n_blocks;
  const int nbw = (int)((nblk + NT / kWave - 1) / (NT / kWave));
  const int D = MOVE ? min(kTileTokens, d.S) : 1;   // workgroups per tile
  const int ntw = d.n_tiles * D;                    // tile workgroups
  const bool blocks_first = ntw > kAlignTilesOneRound;
  const int bid = (int)blockIdx.x;
  if (blocks_first ? bid < nbw : bid >= ntw) {
    const long long gb = (long long)(blocks_first ? bid : bid - ntw) * (NT / kWave) + wave_id();
    if (gb < nblk) align_blocks(plan, d, gb, sorted_ids, block_wrow, block_expert);
    return;
  }
  // LDS, carved to the shape (align_lds_bytes): per expert sH, sO, sHome,
  // sBase and, for the locality step of quota plans, sHL (home local
  // count), sSrc0 (pairs of e from ranks below this tile's rank r), sPN
  // (first piece << 16 | piece count; without the locality step, sP0: the
  // first piece), sLocCap / sLocRow (r's own instance of e: quota its tokens
  // take, start row), sLP (local pairs of instances on ranks <= r); the
  // sub-tile token masks; per piece sPl,
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
  int* sP0 = sPN;   // plans without the locality step: first replica segment of e
  uint32_t* sMask = reinterpret_cast<uint32_t*>(sLP + Ea);   // [kSubTiles][E]
  int* sPl = reinterpret_cast<int*>(sMask + kSubTiles * Ea);
  int* sPd = sPl + Pa;
  int* sPr = sPd + Pa;
  int* sPe = sPr + Pa;
  int* sPc = sPe + Pa;
  int* sPLoc = sPc + Pa;
  int* sRem = sPLoc + Pa;

  const PlanLayout& pl = d.pl;
  const int E = d.E, K = d.K, C = d.C, nh = d.nh;
  const int tw = blocks_first ? bid - nbw : bid;
  const int tile = MOVE ? tw / D : tw;
  const int tg = MOVE ? tw - tile * D : 0;          // MOVE: the workgroup's token in the tile
  const int r = tile / d.tpr, j = tile - r * d.tpr;
  const int t0 = r * d.S + j * kTileTokens;
  const int len = min(kTileTokens, d.S - j * kTileTokens);
  if (MOVE && tg >= len) return;                    // past a short tile (before any barrier)
  const int nP = min(plan[pl.hdr + LBT_HDR_N_PIECES], pl.max_pieces);
  const int totOv = plan[pl.hdr + LBT_HDR_TOTAL_OVERFLOW];
  const bool local = plan[pl.hdr + LBT_HDR_LOCAL] != 0;
  const int32_t* tbase = work + work_tile_base(d) + (long long)tile * E;
  const int32_t* rbase = work + work_tile_base(d) + (long long)r * d.tpr * E;   // rank r's first tile
  const int tid = threadIdx.x;
  const long long f0 = (long long)t0 * K;   // first pair of the tile
  const int np = len * K;                   // pairs of the tile

  // the thread's first kPre expert ids (pairs tid + j * NT), loaded before
  // the plan so that the two latencies overlap (for K <= 8 no id is read
  // twice)
  constexpr int kPre = (kTileTokens * 8 + NT - 1) / NT;
  int idp[kPre];
#pragma unroll
  for (int u = 0; u < kPre; ++u) {
    const int p = tid + u * NT;
    idp[u] = p < np ? ids[f0 + p] : -1;
  }
  // MOVE: the token's own ids (thread k < K holds pair k) and the first
  // chunks of its row, loaded now so that their latency overlaps the
  // tile's prefix work
  constexpr int kXPre = MOVE ? 2 : 1;
  const int H8 = d.H / 8;
  const u32x4* src = MOVE ? x + (long long)(t0 + tg) * H8 : nullptr;
  int own_id = -1;
  u32x4 xv[kXPre];
  if constexpr (MOVE) {
    if (tid < K) own_id = ids[f0 + tg * K + tid];
#pragma unroll
    for (int i = 0; i < kXPre; ++i) {
      const int c = tid + i * NT;
      xv[i] = c < H8 ? src[c] : u32x4{0u, 0u, 0u, 0u};
    }
  }

  for (int e = tid; e < E; e += NT) {
    sH[e] = plan[pl.h + e];
    sO[e] = plan[pl.O + e];
    sHome[e] = plan[pl.home_row + e];
    sBase[e] = tbase[e];
    sHL[e] = plan[pl.home_local + e];
    sSrc0[e] = rbase[e];
    sPN[e] = -1;
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
      const int he = div_nh(e, d);
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
  // token (within the tile) of pair p: p / K by one multiply-high
  auto token_of = [&](int p) { return d.K == 1 ? p : (int)__umulhi((uint32_t)p, d.k_magic); };
  auto mark = [&](int p, int e) {
    if (e < 0 || e >= E) return;
    const int ti = token_of(p);
    const uint32_t bit = 1u << (ti % kSubTokens);
    const uint32_t old = atomicOr(&sMask[(ti / kSubTokens) * E + e], bit);
    if (old & bit) flags |= LBT_ST_DUPID;
  };
#pragma unroll
  for (int u = 0; u < kPre; ++u) {
    const int p = tid + u * NT;
    if (p < np) mark(p, idp[u]);
  }
  for (int p = tid + kPre * NT; p < np; p += NT) mark(p, ids[f0 + p]);
  // the first replica segment of each expert (an expert's segments are
  // consecutive on the line), so a pair finds its segment by a short walk
  // over its expert's few segments instead of a search over all of them
  if (!local)
    for (int g = tid; g < nP; g += NT) {
      const int e = sPe[g];
      if (e >= 0 && e < E && (g == 0 || sPe[g - 1] != e)) sP0[e] = g;
    }
  __syncthreads();

  // the pair's row of recv (also written to slot and sorted_ids), or -1
  auto place = [&](int p, int e) -> long long {
    const long long f = f0 + p;
    if (e < 0 || e >= E) {
      flags |= LBT_ST_BADID;
      slot[f] = -1;
      return -1;
    }
    const int ti = token_of(p);
    const int sub = ti / kSubTokens;
    const uint32_t bit = 1u << (ti % kSubTokens);
    // earlier sub-tiles' pairs of e, read straight from their masks (all
    // kSubTiles loads issued together; a separate prefix pass would cost a
    // workgroup barrier)
    int q = sBase[e] + __popc(sMask[sub * E + e] & (bit - 1u));
#pragma unroll
    for (int s = 0; s < kSubTiles; ++s) q += s < sub ? __popc(sMask[s * E + e]) : 0;
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
          dd = div_nh(e, d);
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
      dd = div_nh(e, d);
      row = sHome[e] + q;
    } else {
      // the last of e's segments starting at or below its line position o
      const int o = sO[e] + (q - h);
      int g = sP0[e];
      if (g >= 0)
        while (g + 1 < nP && sPe[g + 1] == e && sPl[g + 1] <= o) ++g;
      ok = o < totOv && g >= 0 && sPl[g] <= o;
      dd = ok ? sPd[g] : 0;
      row = ok ? sPr[g] + (o - sPl[g]) : 0;
    }
    // a row past the capacity, or a rank / row a corrupt plan would give
    if (!ok || row >= C || row < 0 || dd < 0 || dd >= d.R) {
      flags |= LBT_ST_CAPACITY;
      slot[f] = -1;
      return -1;
    }
    const long long dst = (long long)dd * C + row;
    slot[f] = (int)dst;
    sorted_ids[dst] = (int)f;
    return dst;
  };
  if constexpr (MOVE) {
    // the token's K pairs, one per thread, then its row to each of them
    __shared__ long long sDst[kMaxK];
    if (tid < K) sDst[tid] = place(tg * K + tid, own_id);
    if (flags && status != nullptr) atomicOr(status, flags);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kXPre; ++i) {
      const int c = tid + i * NT;
      if (c < H8)
        for (int k = 0; k < K; ++k) {
          const long long dst = sDst[k];
          if (dst >= 0) recv[dst * H8 + c] = xv[i];
        }
    }
    for (int c = tid + kXPre * NT; c < H8; c += NT) {
      const u32x4 v = src[c];
      for (int k = 0; k < K; ++k) {
        const long long dst = sDst[k];
        if (dst >= 0) recv[dst * H8 + c] = v;
      }
    }
  } else {
#pragma unroll
    for (int u = 0; u < kPre; ++u) {
      const int p = tid + u * NT;
      if (p < np) place(p, idp[u]);
    }
    for (int p = tid + kPre * NT; p < np; p += NT) place(p, ids[f0 + p]);
    if (flags && status != nullptr) atomicOr(status, flags);
  }
}

// LDS of a tile workgroup: 10 per-expert arrays, the [kSubTiles][E]
// sub-tile token masks and 7 per-piece arrays; at most 56 KiB (E = 512,
// 1024 pieces).
static size_t align_lds_bytes(const Dims& d) {
  return sizeof(int) * ((size_t)(10 + kSubTiles) * d.E + (size_t)7 * d.pl.max_pieces);
}

hipError_t launch_align(const Dims& d, const int32_t* ids, const int32_t* work, const int32_t* plan,
                        int32_t* slot, int32_t* sorted_ids, int32_t* block_wrow,
                        int32_t* block_expert, int32_t* status, hipStream_t st) {
  const long long nblk = (long long)d.R * d.n_blocks;
  const long long grid = d.n_tiles + (nblk + kBlockWaves - 1) / kBlockWaves;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL((k_align<kAlignThreads, false>), dim3((unsigned)grid), dim3(kAlignThreads),
                     align_lds_bytes(d), st, ids, work, plan, d, slot, sorted_ids, block_wrow,
                     block_expert, status, nullptr, nullptr);
  return hipGetLastError();
}

// Batches the fused align + dispatch launch takes: one workgroup per token
// (with the tile's placement work repeated in each) pays off while the
// tokens are few; larger batches make the two launches.
constexpr int kMoveTokens = 1024;

hipError_t launch_align_dispatch(const Dims& d, const int32_t* ids, const int32_t* work,
                                 const int32_t* plan, const uint16_t* x, int32_t* slot,
                                 int32_t* sorted_ids, int32_t* block_wrow, int32_t* block_expert,
                                 uint16_t* recv, int32_t* status, hipStream_t st) {
  if (d.N < 1 || d.N > kMoveTokens) {
    hipError_t e = launch_align(d, ids, work, plan, slot, sorted_ids, block_wrow, block_expert,
                                status, st);
    if (e == hipSuccess) e = launch_dispatch(d, x, slot, recv, st);
    return e;
  }
  const long long nblk = (long long)d.R * d.n_blocks;
  const long long grid = (long long)d.n_tiles * (d.S < kTileTokens ? d.S : kTileTokens) +
                         (nblk + kBlockWaves - 1) / kBlockWaves;
  if (grid > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL((k_align<kAlignThreads, true>), dim3((unsigned)grid), dim3(kAlignThreads),
                     align_lds_bytes(d), st, ids, work, plan, d, slot, sorted_ids, block_wrow,
                     block_expert, status, reinterpret_cast<const u32x4*>(x),
                     reinterpret_cast<u32x4*>(recv));
  return hipGetLastError();
}

}  // namespace lbt
