// Internal declarations of the HIP library behind include/lbt.h (gfx950,
// wave64).  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <limits.h>
#include <stdint.h>

#include "../../include/lbt.h"

namespace lbt {

constexpr int kWave = 64;
constexpr int kTileTokens = 128;   // tokens per align tile (prefix offsets)
constexpr int kSubTokens = 32;     // tokens per histogram sub-tile (one u32 bit mask)
constexpr int kSubTiles = kTileTokens / kSubTokens;
constexpr int kMaxE = 512;
constexpr int kMaxR = 512;
constexpr int kMaxPieces = kMaxE + kMaxR;
constexpr int kMaxK = 64;

// Plan blob word offsets (mirrors lbt_sizes, 32-bit for the device).
struct PlanLayout {
  int E, R, max_seg, max_pieces;
  int hdr, T, h, O, home_row, L, def, D, n_seg, n_rows_padded, n_slots, n_remote;
  int seg_expert, seg_wrow, seg_count, seg_start;
  int piece_expert, piece_rank, piece_count, piece_line, piece_row, piece_wrow;
  int home_local, piece_local;
  int total;
};

// Everything the kernels need about a shape, derived once on the host.
struct Dims {
  int E, K, R, S, H, B, blk, score_fn, renorm;
  int nh;        // E / R home experts per rank
  uint32_t nh_magic;   // ceil(2^32 / nh) for nh >= 2: e / nh = umulhi(e, nh_magic) for e < 2^16
  uint32_t k_magic;    // ceil(2^32 / K) for K >= 2: p / K = umulhi(p, k_magic) for p < 2^16
  int N;         // R * S tokens
  long long P;   // N * K pairs
  int SK;        // S * K
  int tau_max;   // largest per-rank load a plan may give (>= SK)
  int C;         // rows per rank
  int n_blocks;  // C / blk
  int tpr;       // align tiles per rank
  int n_tiles;   // R * tpr
  int spr;       // histogram sub-tiles per rank
  int n_sub;     // R * spr
  PlanLayout pl;
};

// Host-side helpers (api.hip).
int make_dims(const lbt_shape* s, Dims* d, lbt_sizes* z);

// Launchers (one per kernel family).  Return hipError_t of the launch.
hipError_t launch_route(const Dims& d, const float* logits, const float* bias, int32_t* ids,
                        float* gates, int32_t* work, hipStream_t st);
hipError_t launch_histogram(const Dims& d, const int32_t* ids, int32_t* work, int32_t* status,
                            hipStream_t st);
hipError_t launch_tile_scan(const Dims& d, int32_t* work, int32_t* counts, hipStream_t st);
hipError_t launch_route_and_scan(const Dims& d, const float* logits, const float* bias,
                                 int32_t* ids, float* gates, int32_t* work, int32_t* counts,
                                 hipStream_t st);
hipError_t launch_plan(const Dims& d, const int32_t* counts, int32_t* plan, int32_t* status,
                       hipStream_t st);
// route + histogram + fixed-rule plan (one launch for small batches)
hipError_t launch_route_plan(const Dims& d, const float* logits, const float* bias, int32_t* ids,
                             float* gates, int32_t* work, int32_t* counts, int32_t* plan,
                             int32_t* status, hipStream_t st);
// route + histogram + fixed-rule plan + align (one launch for small batches)
hipError_t launch_front(const Dims& d, const float* logits, const float* bias, int32_t* ids,
                        float* gates, int32_t* work, int32_t* counts, int32_t* plan,
                        int32_t* slot, int32_t* sorted_ids, int32_t* block_wrow,
                        int32_t* block_expert, int32_t* status, hipStream_t st);
hipError_t launch_plan_quota(const Dims& d, const int32_t* counts, int32_t* plan,
                             int32_t* status, hipStream_t st);
hipError_t launch_align(const Dims& d, const int32_t* ids, const int32_t* work, const int32_t* plan,
                        int32_t* slot, int32_t* sorted_ids, int32_t* block_wrow,
                        int32_t* block_expert, int32_t* status, hipStream_t st);
hipError_t launch_dispatch(const Dims& d, const uint16_t* x, const int32_t* slot, uint16_t* recv,
                           hipStream_t st);
hipError_t launch_combine(const Dims& d, const uint16_t* out, const int32_t* slot,
                          const float* gates, int y_dtype, void* y, hipStream_t st);
// the align step with the library's static workspace (noalloc.hip)
bool noalloc_fits(const Dims& d);
hipError_t launch_align_noalloc(const Dims& d, const int32_t* ids, const int32_t* plan,
                                int32_t* slot, int32_t* sorted_ids, int32_t* block_wrow,
                                int32_t* block_expert, int32_t* status, hipStream_t st);
// gates == nullptr: every gate is 1 (the backward of dispatch)
hipError_t launch_prefetch(const Dims& d, const int32_t* plan, const void* weights, void* slots,
                           long long row_bytes, hipStream_t st);
hipError_t launch_reduce_grad(const Dims& d, const int32_t* plan, float* slot_grads, float* grads,
                              long long row_elems, hipStream_t st);
hipError_t launch_combine_bwd(const Dims& d, const uint16_t* out, const int32_t* slot,
                              const float* gates, int dy_dtype, const void* dy, uint16_t* d_out,
                              float* d_gates, hipStream_t st);

// Workspace layout: sub_counts [n_sub][E] (per 32-token sub-tile, sub-tile-
// major: each route workgroup writes one contiguous run) followed by
// tile_base [n_tiles][E] (per 128-token tile, tile-major, for the align
// step).  Sub-tiles and tiles
// never cross ranks; tile j of rank r holds its sub-tiles 4j .. 4j+3.
__host__ __device__ inline long long work_tile_base(const Dims& d) {
  return (long long)d.E * d.n_sub;
}

// ---- device helpers -------------------------------------------------------
__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// e / nh for 0 <= e < 2^16 by one multiply-high (exact there: the rounding
// error of the multiplier is below nh, so e times it stays below 2^32).
__device__ __forceinline__ int div_nh(int e, const Dims& d) {
  return d.nh == 1 ? e : (int)__umulhi((uint32_t)e, d.nh_magic);
}
__device__ __forceinline__ int wave_id() { return threadIdx.x / kWave; }

// Wave-wide max and sum, the same value in every lane, for a full wave: four
// DPP steps inside each 16-lane row (each lane paired with one of the
// other half of its quad, pair, half-row and row; the identity as the old
// value lets the compiler fold every move into the max or add), then the
// four row results read into scalars.  No LDS round trip.
__device__ __forceinline__ int wave_max(int x) {
  x = max(x, __builtin_amdgcn_update_dpp(INT_MIN, x, 0xB1, 0xF, 0xF, false));    // quad_perm [1,0,3,2]
  x = max(x, __builtin_amdgcn_update_dpp(INT_MIN, x, 0x4E, 0xF, 0xF, false));    // quad_perm [2,3,0,1]
  x = max(x, __builtin_amdgcn_update_dpp(INT_MIN, x, 0x141, 0xF, 0xF, false));   // row_half_mirror
  x = max(x, __builtin_amdgcn_update_dpp(INT_MIN, x, 0x140, 0xF, 0xF, false));   // row_mirror
  return max(max(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16)),
             max(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48)));
}

__device__ __forceinline__ int wave_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false);
  x += __builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, false);
  return (__builtin_amdgcn_readlane(x, 0) + __builtin_amdgcn_readlane(x, 16)) +
         (__builtin_amdgcn_readlane(x, 32) + __builtin_amdgcn_readlane(x, 48));
}

// Inclusive prefix sum across a wave64 with DPP: Hillis-Steele steps inside
// each 16-lane row (row_shr 1, 2, 4, 8; lanes without a source add 0), then
// row_bcast:15 carries rows 0 and 2 into rows 1 and 3, and row_bcast:31
// carries rows 0-1 into rows 2-3.
__device__ __forceinline__ int wave_incl_scan_dpp(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}

// Exclusive prefix sum of a[0..n) in LDS by ONE wave, n <= 64*C: lane l
// takes the contiguous chunk [l*C, l*C + C) with C fixed at compile time, so
// the chunk is read and written without branches (neighbouring words pair
// up into wide LDS accesses) and scanned in registers.  a must hold at least
// 64*C + 1 ints: entries at or past n are read as 0, entries n .. 64*C - 1
// are overwritten with the total, and a[n] receives the total, which every
// lane returns.  No workgroup barrier.
template <int C>
__device__ __forceinline__ int wave_excl_scan_chunk(int* a, int n) {
  const int lane = lane_id();
  const int lo = lane * C;
  int v[C];
#pragma unroll
  for (int i = 0; i < C; ++i) {
    const int x = a[lo + i];
    v[i] = lo + i < n ? x : 0;
  }
  int s = 0;
#pragma unroll
  for (int i = 0; i < C; ++i) s += v[i];
  const int incl = wave_incl_scan_dpp(s);
  int run = incl - s;
#pragma unroll
  for (int i = 0; i < C; ++i) {
    a[lo + i] = run;
    run += v[i];
  }
  const int total = __builtin_amdgcn_readlane(incl, kWave - 1);
  if (lane == 0) a[n] = total;   // after the chunk stores in program order
  __builtin_amdgcn_wave_barrier();
  return total;
}

// The same for n <= 64*CMAX, with the smallest chunk of 1, 2, 4, 8, 16 or
// CMAX that covers n.  a must hold at least 64*CMAX + 1 ints, and its entries
// past n are scratch (overwritten).
template <int CMAX>
__device__ __forceinline__ int wave_excl_scan_lds(int* a, int n) {
  const int c = (n + kWave - 1) / kWave;
  if (c <= 1) return wave_excl_scan_chunk<1>(a, n);
  if constexpr (CMAX >= 2) if (c <= 2) return wave_excl_scan_chunk<2>(a, n);
  if constexpr (CMAX >= 4) if (c <= 4) return wave_excl_scan_chunk<4>(a, n);
  if constexpr (CMAX >= 8) if (c <= 8) return wave_excl_scan_chunk<8>(a, n);
  if constexpr (CMAX >= 16) if (c <= 16) return wave_excl_scan_chunk<16>(a, n);
  return wave_excl_scan_chunk<CMAX>(a, n);
}

// First index in a[0..n) whose value is > x (a non-decreasing).
__device__ __forceinline__ int upper_bound(const int* a, int n, int x) {
  int lo = 0, hi = n;
  while (lo < hi) {
    const int mid = (lo + hi) >> 1;
    if (a[mid] <= x) lo = mid + 1; else hi = mid;
  }
  return lo;
}

}  // namespace lbt
