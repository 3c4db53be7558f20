// MoE Align & Sort under the balancing plan: the destination row of every
// (token, expert) pair, the inverse map, and the per-block weight-row table.
//
// [AlignSort]: pairs are sorted by expert id with each expert's share padded
// to the grouped GEMM's block; the permutation records source -> target.
// The prior kernel there computes aligned offsets in one block, then
// scatters; here the offsets come from the plan and the per-tile prefix
// counts, so every tile of 128 tokens works independently.
// [UltraEP] section "その仕組みは高速なエキスパート複製に依存する": per-token
// destinations are a local lookup against cumulative quotas.
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
  __shared__ int sH[kMaxE], sO[kMaxE], sHome[kMaxE], sBase[kMaxE];
  __shared__ uint32_t sMask[kSubTiles][kMaxE];
  __shared__ int sSub[kSubTiles][kMaxE];
  __shared__ int sPl[kMaxPieces], sPd[kMaxPieces], sPr[kMaxPieces], sPe[kMaxPieces];

  const PlanLayout& pl = d.pl;
  const int E = d.E, K = d.K, C = d.C, nh = d.nh;
  const int tile = blockIdx.x;
  const int r = tile / d.tpr, j = tile - r * d.tpr;
  const int t0 = r * d.S + j * kTileTokens;
  const int len = min(kTileTokens, d.S - j * kTileTokens);
  const int nP = plan[pl.hdr + LBT_HDR_N_PIECES];
  const int totOv = plan[pl.hdr + LBT_HDR_TOTAL_OVERFLOW];
  const int32_t* tbase = work + work_tile_base(d) + (long long)tile * E;
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
#pragma unroll
    for (int s = 0; s < kSubTiles; ++s) sMask[s][e] = 0u;
  }
  // the whole piece table (entries past nP are unused), so that these loads
  // do not wait for the piece count
  for (int g = tid; g < pl.max_pieces; g += NT) {
    sPl[g] = plan[pl.piece_line + g];
    sPd[g] = plan[pl.piece_rank + g];
    sPr[g] = plan[pl.piece_row + g];
    sPe[g] = plan[pl.piece_expert + g];
  }
  __syncthreads();

  int flags = 0;
  const int sub = ti / kSubTokens;
  const uint32_t bit = 1u << (ti % kSubTokens);
  auto mark = [&](int e) {
    if (e < 0 || e >= E) return;
    const uint32_t old = atomicOr(&sMask[sub][e], bit);
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
      sSub[s][e] = run;
      run += __popc(sMask[s][e]);
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
    const int q = sBase[e] + sSub[sub][e] + __popc(sMask[sub][e] & (bit - 1u));
    const int h = sH[e];
    int dd, row;
    bool ok = true;
    if (q < h) {
      dd = e / nh;
      row = sHome[e] + q;
    } else {
      const int o = sO[e] + (q - h);
      const int g = upper_bound(sPl, nP, o) - 1;
      ok = o < totOv && g >= 0 && sPe[g] == e;
      dd = ok ? sPd[g] : 0;
      row = ok ? sPr[g] + (o - sPl[g]) : 0;
    }
    if (!ok || row >= C) {
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

hipError_t launch_align(const Dims& d, const int32_t* ids, const int32_t* work, const int32_t* plan,
                        int32_t* slot, int32_t* sorted_ids, int32_t* block_wrow,
                        int32_t* block_expert, int32_t* status, hipStream_t st) {
  const long long nblk = (long long)d.R * d.n_blocks;
  const long long grid = d.n_tiles + (nblk + kBlockWaves - 1) / kBlockWaves;
  if (grid == 0) return hipSuccess;
  hipLaunchKernelGGL(k_align<kAlignTPT>, dim3((unsigned)grid), dim3(kAlignThreads), 0, st, ids, work,
                     plan, d, slot, sorted_ids, block_wrow, block_expert, status);
  return hipGetLastError();
}

}  // namespace lbt
