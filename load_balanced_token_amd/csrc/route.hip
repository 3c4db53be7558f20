// Router top-K with the fused per-sub-tile expert histogram, the histogram
// of caller-supplied ids, and the column scan that turns per-sub-tile counts
// into per-tile prefix offsets and the per-rank load matrix.
//
// The top-K itself is in route_core.h.
#include "route_core.h"

namespace lbt {

template <int V, bool FULL>
__global__ __launch_bounds__(kRouteThreads) void k_route(const float* __restrict__ logits,
                                                         const float* __restrict__ bias, Dims d,
                                                         int vec, int32_t* __restrict__ ids,
                                                         float* __restrict__ gates,
                                                         int32_t* __restrict__ sub_counts) {
  __shared__ RouteSmem sm;
  route_sub<V, FULL>(logits, bias, d, vec, blockIdx.x, ids, gates, sub_counts, sm);
}

// The same with the register budget of eight waves per SIMD (a few scalar
// registers spill to vector lanes), so that four 512-thread workgroups fit
// on a CU: at 32K tokens the 1024 sub-tile workgroups then run in one round
// instead of 768 plus a tail of 256 (the compiler's own allocation, 104
// scalar registers at V = 16, leaves room for seven waves).  Used for
// V <= 16; wider lanes would spill vector registers.
template <int V, bool FULL>
__global__ __launch_bounds__(kRouteThreads) __attribute__((amdgpu_waves_per_eu(8, 8)))
void k_route_o8(const float* __restrict__ logits, const float* __restrict__ bias, Dims d, int vec,
                int32_t* __restrict__ ids, float* __restrict__ gates,
                int32_t* __restrict__ sub_counts) {
  __shared__ RouteSmem sm;
  route_sub<V, FULL>(logits, bias, d, vec, blockIdx.x, ids, gates, sub_counts, sm);
}

// Histogram of caller-supplied ids, one thread per token of a sub-tile.
constexpr int kHistThreads = 64;
__global__ __launch_bounds__(kHistThreads) void k_histogram(const int32_t* __restrict__ ids, Dims d,
                                                            int32_t* __restrict__ sub_counts,
                                                            int32_t* __restrict__ status) {
  __shared__ int hist[kMaxE];
  const int E = d.E, K = d.K;
  const int sub = blockIdx.x;
  const int r = sub / d.spr, j = sub - r * d.spr;
  const int t0 = r * d.S + j * kSubTokens;
  const int len = min(kSubTokens, d.S - j * kSubTokens);
  for (int e = threadIdx.x; e < E; e += kHistThreads) hist[e] = 0;
  __syncthreads();
  int flags = 0;
  if ((int)threadIdx.x < len) {
    const long long t = (long long)t0 + threadIdx.x;
    for (int k = 0; k < K; ++k) {
      const int e = ids[t * K + k];
      if (e < 0 || e >= E) flags |= LBT_ST_BADID;
      else atomicAdd(&hist[e], 1);
    }
  }
  if (flags && status != nullptr) atomicOr(status, flags);
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kHistThreads)
    sub_counts[(long long)e * d.n_sub + sub] = hist[e];
}

// One wave per expert column (one workgroup each, so the columns spread over
// the CUs): exclusive prefix over the sub-tiles, written at each 128-token
// tile's first sub-tile (tile-major, for the align step), and per-source-rank
// sums (the load matrix) as differences of the prefix at the ranks' first
// sub-tiles (sub-tiles never cross ranks).  Each lane takes kScanPer
// consecutive sub-tiles of a batch of 64 * kScanPer, sums them in registers,
// and one wave-wide scan of the lane sums gives every lane its offset, so a
// batch costs one scan.  (Measured on MI355X, DSV3, 1024 sub-tiles per
// column: one 64-wide chunk per scan, the chunks scanned one after another
// with a carried total, took 6.3 us.)
constexpr int kScanPer = 16;

__global__ __launch_bounds__(kWave) void k_tile_scan(Dims d, int32_t* __restrict__ work,
                                                     int32_t* __restrict__ counts) {
  __shared__ int sPre[kMaxR + 1];   // prefix at each rank's first sub-tile, then the total
  const int e = blockIdx.x;
  const int lane = lane_id();
  const int ns = d.n_sub, spr = d.spr, tpr = d.tpr, E = d.E;
  const int32_t* col = work + (long long)e * ns;
  int32_t* base = work + work_tile_base(d);
  // every column starts on 16 bytes when ns is a multiple of 4 (work itself is)
  const bool vec4 = (ns & 3) == 0 && (reinterpret_cast<uintptr_t>(work) & 15) == 0;
  for (int r = lane; r <= d.R; r += kWave) sPre[r] = 0;   // ranks without tokens (S = 0) sum to 0
  __builtin_amdgcn_wave_barrier();
  int carry = 0;
  for (int c0 = 0; c0 < ns; c0 += kScanPer * kWave) {
    const int i0 = c0 + lane * kScanPer;
    int v[kScanPer];
    if (vec4 && i0 + kScanPer <= ns) {
      // 16-byte loads: a quarter of the load instructions
      const int4* c4 = reinterpret_cast<const int4*>(col + i0);
#pragma unroll
      for (int u = 0; u < kScanPer / 4; ++u) {
        const int4 q = c4[u];
        v[4 * u] = q.x;
        v[4 * u + 1] = q.y;
        v[4 * u + 2] = q.z;
        v[4 * u + 3] = q.w;
      }
    } else {
#pragma unroll
      for (int u = 0; u < kScanPer; ++u) v[u] = i0 + u < ns ? col[i0 + u] : 0;
    }
    int s = 0;
#pragma unroll
    for (int u = 0; u < kScanPer; ++u) s += v[u];
    const int incl = wave_incl_scan_dpp(s);
    int run = carry + incl - s;
    // rank and sub-tile within it of element i0 (spr > 0 whenever ns > 0)
    int r = i0 / spr, j = i0 - r * spr;
#pragma unroll
    for (int u = 0; u < kScanPer; ++u) {
      if (i0 + u < ns) {
        if (j == 0) sPre[r] = run;
        if (j % kSubTiles == 0) base[(long long)(r * tpr + j / kSubTiles) * E + e] = run;
      }
      run += v[u];
      if (++j == spr) {
        j = 0;
        ++r;
      }
    }
    carry += __builtin_amdgcn_readlane(incl, kWave - 1);
  }
  if (lane == 0) sPre[d.R] = carry;
  __builtin_amdgcn_wave_barrier();
  for (int rr = lane; rr < d.R; rr += kWave)
    counts[(long long)rr * E + e] = sPre[rr + 1] - sPre[rr];
}

hipError_t launch_route(const Dims& d, const float* logits, const float* bias, int32_t* ids,
                        float* gates, int32_t* work, hipStream_t st) {
  if (d.n_sub == 0) return hipSuccess;
  const int vec = route_vec(logits, d.E);
  const dim3 grid(d.n_sub), block(kRouteThreads);
  const int V = (d.E + kRowLanes - 1) / kRowLanes;
  // FULL: every lane holds V real experts (E = 16 V), no per-key bounds test
#define LBT_ROUTE(KERN, VV)                                                                   \
  do {                                                                                        \
    if (d.E == kRowLanes * (VV))                                                              \
      hipLaunchKernelGGL((KERN<VV, true>), grid, block, 0, st, logits, bias, d, vec, ids,     \
                         gates, work);                                                        \
    else                                                                                      \
      hipLaunchKernelGGL((KERN<VV, false>), grid, block, 0, st, logits, bias, d, vec, ids,    \
                         gates, work);                                                        \
  } while (0)
  if (V <= 1) LBT_ROUTE(k_route_o8, 1);
  else if (V <= 2) LBT_ROUTE(k_route_o8, 2);
  else if (V <= 4) LBT_ROUTE(k_route_o8, 4);
  else if (V <= 8) LBT_ROUTE(k_route_o8, 8);
  else if (V <= 16) LBT_ROUTE(k_route_o8, 16);
  else if (V <= 24) LBT_ROUTE(k_route, 24);
  else LBT_ROUTE(k_route, 32);
#undef LBT_ROUTE
  return hipGetLastError();
}

hipError_t launch_histogram(const Dims& d, const int32_t* ids, int32_t* work, int32_t* status,
                            hipStream_t st) {
  if (d.n_sub == 0) return hipSuccess;
  hipLaunchKernelGGL(k_histogram, dim3(d.n_sub), dim3(kHistThreads), 0, st, ids, d, work, status);
  return hipGetLastError();
}

hipError_t launch_tile_scan(const Dims& d, int32_t* work, int32_t* counts, hipStream_t st) {
  hipLaunchKernelGGL(k_tile_scan, dim3(d.E), dim3(kWave), 0, st, d, work, counts);
  return hipGetLastError();
}

// Small batches (1 <= N <= kSmallTokens and n_sub * E <= kSmallHist): one
// workgroup routes every token, keeps each sub-tile's histogram in LDS and
// does the scan itself, so route + scan is one launch.  Same outputs as
// k_route + k_tile_scan.  Measured on MI355X: N = 8 (decode, S = 1) route +
// scan 12.3 -> 9.9 us; at N = 128 one workgroup is slower than spreading
// the tokens over several (11.7 -> 20.3 us), so only batches that fit one
// pass take it.
constexpr int kSmallHist = 16384;
constexpr int kSmallTokens = kRouteTokens;

static bool small_batch(const Dims& d) {
  return d.N >= 1 && d.N <= kSmallTokens && (long long)d.n_sub * d.E <= kSmallHist;
}

template <int V, bool FULL>
__global__ __launch_bounds__(kRouteThreads) void k_route_small(const float* __restrict__ logits,
                                                               const float* __restrict__ bias,
                                                               Dims d, int vec,
                                                               int32_t* __restrict__ ids,
                                                               float* __restrict__ gates,
                                                               int32_t* __restrict__ work,
                                                               int32_t* __restrict__ counts) {
  __shared__ RouteScratch rs;
  __shared__ int hist[kSmallHist];     // [sub-tile][E]
  const int E = d.E, ns = d.n_sub, S = d.S, spr = d.spr, tpr = d.tpr;
  for (int i = threadIdx.x; i < ns * E; i += kRouteThreads) hist[i] = 0;
  route_span<V, FULL>(logits, bias, d, vec, 0, d.N, ids, gates, rs, [&](long long t, int id) {
    const int r = (int)(t / S), j = (int)(t - (long long)r * S) / kSubTokens;
    atomicAdd(&hist[(r * spr + j) * E + id], 1);
  });
  __syncthreads();
  // the tile prefixes align reads and the load matrix (the per-sub-tile
  // counts are an intermediate of the two-launch path and are not written)
  int32_t* base = work + work_tile_base(d);
  for (int e = threadIdx.x; e < E; e += kRouteThreads) {
    int run = 0;
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

// The whole routing step: route + scan, or the one small-batch launch.
hipError_t launch_route_and_scan(const Dims& d, const float* logits, const float* bias,
                                 int32_t* ids, float* gates, int32_t* work, int32_t* counts,
                                 hipStream_t st) {
  if (!small_batch(d)) {
    hipError_t e = launch_route(d, logits, bias, ids, gates, work, st);
    if (e == hipSuccess) e = launch_tile_scan(d, work, counts, st);
    return e;
  }
  const int vec = route_vec(logits, d.E);
  const dim3 grid(1), block(kRouteThreads);
  const int V = (d.E + kRowLanes - 1) / kRowLanes;
#define LBT_SMALL(VV)                                                                      \
  do {                                                                                     \
    if (d.E == kRowLanes * (VV))                                                           \
      hipLaunchKernelGGL((k_route_small<VV, true>), grid, block, 0, st, logits, bias, d,   \
                         vec, ids, gates, work, counts);                                   \
    else                                                                                   \
      hipLaunchKernelGGL((k_route_small<VV, false>), grid, block, 0, st, logits, bias, d,  \
                         vec, ids, gates, work, counts);                                   \
  } while (0)
  if (V <= 1) LBT_SMALL(1);
  else if (V <= 2) LBT_SMALL(2);
  else if (V <= 4) LBT_SMALL(4);
  else if (V <= 8) LBT_SMALL(8);
  else if (V <= 16) LBT_SMALL(16);
  else if (V <= 24) LBT_SMALL(24);
  else LBT_SMALL(32);
#undef LBT_SMALL
  return hipGetLastError();
}


}  // namespace lbt
