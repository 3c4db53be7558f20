// Router top-K with the fused per-sub-tile expert histogram, the histogram
// of caller-supplied ids, and the column scan that turns per-sub-tile counts
// into per-tile prefix offsets and the per-rank load matrix.
//
// The top-K itself is in route_core.h.
#include "route_core.h"
#include "rows.h"

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
    sub_counts[(long long)sub * E + e] = hist[e];
}

// The column scan, one workgroup per expert column: exclusive prefix over
// the sub-tiles, written at each 128-token tile's first sub-tile
// (tile-major, for the align step), and per-source-rank sums (the load
// matrix) as differences of the prefix at the ranks' first sub-tiles
// (sub-tiles never cross ranks).  A batch is 64 * kScanPer consecutive
// sub-tiles, kScanPer per lane: the lane sums its share in registers and
// one wave-wide scan of the lane sums gives every lane its offset.  A
// column of nb batches takes min(nb, 8) waves, each a contiguous run of
// batches: the waves' totals meet in LDS, then each wave scans its own
// batches from its offset, its first batches still in registers (so at
// Kimi-K3, eight batches per column, every load is issued up front; one
// wave walking the eight batches in turn took 26-29 us, against 4-5 at
// DSV3's one batch).
//
// The sub-tile histograms are sub-tile-major ([n_sub][E]): each route
// workgroup writes its E counts as one contiguous run (written expert-major,
// E single counts 4 KB apart, they had cost the DSV3 route ~1.7 us and the
// Kimi-K3 route ~9 us on MI355X).  A lane's loads then hit a different
// 128-byte line each, and a line holds 32 neighbouring experts: the columns
// go to the XCDs in contiguous ranges, so the 32 columns of a line are read
// through one XCD's L2.  (Measured on MI355X: a workgroup per 16 experts
// with lanes over sub-tile chunks read whole runs but spread a column's
// sub-tiles over too few CUs: DSV3 5.6 us, Kimi-K3 36 us.)
constexpr int kScanPer = 16;
constexpr int kScanBatch = kScanPer * kWave;
constexpr int kScanMaxWaves = 8;

// C columns per workgroup: C = 4 (E a multiple of 4, 16-byte aligned
// workspace, several batches per column) reads four neighbouring experts'
// counts of a sub-tile with one 16-byte load and writes their tile offsets
// with one 16-byte store, a quarter of the memory requests of one column at
// a time.
template <int C>
__global__ __launch_bounds__(kScanMaxWaves * kWave) void k_tile_scan(Dims d,
                                                                     int32_t* __restrict__ work,
                                                                     int32_t* __restrict__ counts) {
  constexpr int KEEP = C == 1 ? 2 : 1;   // batches a wave keeps in registers
  __shared__ int sPre[kMaxR + 1][C];     // prefix at each rank's first sub-tile, then the total
  __shared__ int sTot[kScanMaxWaves][C]; // each wave's total
  const int e0 = xcd_contiguous(blockIdx.x, gridDim.x) * C;
  const int lane = lane_id(), w = wave_id(), nw = blockDim.x / kWave;
  const int ns = d.n_sub, spr = d.spr, tpr = d.tpr, E = d.E;
  int32_t* base = work + work_tile_base(d);
  for (int i = threadIdx.x; i < (d.R + 1) * C; i += blockDim.x) sPre[i / C][i % C] = 0;
  const int nb = (ns + kScanBatch - 1) / kScanBatch;
  const int bpw = (nb + nw - 1) / nw;
  const int b0 = min(w * bpw, nb), b1 = min(b0 + bpw, nb);
  // a batch's values, indices clamped into the column (the loads carry no
  // branches; masked when used; ns > 0 whenever a wave has a batch)
  auto load_batch = [&](int b, int (&dst)[kScanPer][C]) {
    const int i0 = b * kScanBatch + lane * kScanPer;
#pragma unroll
    for (int u = 0; u < kScanPer; ++u) {
      const int32_t* p = work + (long long)min(i0 + u, ns - 1) * E + e0;
      if constexpr (C == 4) {
        const int4 q = *reinterpret_cast<const int4*>(p);
        dst[u][0] = q.x;
        dst[u][1] = q.y;
        dst[u][2] = q.z;
        dst[u][3] = q.w;
      } else {
        dst[u][0] = *p;
      }
    }
  };
  auto lane_sums = [&](int b, const int (&v)[kScanPer][C], int (&acc)[C]) {
    const int i0 = b * kScanBatch + lane * kScanPer;
#pragma unroll
    for (int u = 0; u < kScanPer; ++u)
#pragma unroll
      for (int c = 0; c < C; ++c) acc[c] += i0 + u < ns ? v[u][c] : 0;
  };
  int va[KEEP][kScanPer][C];
#pragma unroll
  for (int k = 0; k < KEEP; ++k)
    if (b0 + k < b1) load_batch(b0 + k, va[k]);
  // first pass: the wave's totals
  int part[C];
#pragma unroll
  for (int c = 0; c < C; ++c) part[c] = 0;
  for (int b = b0 + KEEP; b < b1; ++b) {
    int q[kScanPer][C];
    load_batch(b, q);
    lane_sums(b, q, part);
  }
#pragma unroll
  for (int k = 0; k < KEEP; ++k)
    if (b0 + k < b1) lane_sums(b0 + k, va[k], part);
#pragma unroll
  for (int c = 0; c < C; ++c) {
    const int wtot = __builtin_amdgcn_readlane(wave_incl_scan_dpp(part[c]), kWave - 1);
    if (lane == 0) sTot[w][c] = wtot;
  }
  __syncthreads();
  int carry[C];
#pragma unroll
  for (int c = 0; c < C; ++c) {
    carry[c] = 0;
    for (int x = 0; x < w; ++x) carry[c] += sTot[x][c];
  }
  // second pass: the prefix at every sub-tile of the wave's batches
  auto scan_batch = [&](int b, const int (&v)[kScanPer][C]) {
    const int i0 = b * kScanBatch + lane * kScanPer;
    int run[C], incl[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
      int s = 0;
#pragma unroll
      for (int u = 0; u < kScanPer; ++u) s += i0 + u < ns ? v[u][c] : 0;
      incl[c] = wave_incl_scan_dpp(s);
      run[c] = carry[c] + incl[c] - s;
    }
    // rank and sub-tile within it of element i0 (spr > 0 whenever ns > 0)
    int r = i0 / spr, j = i0 - r * spr;
#pragma unroll
    for (int u = 0; u < kScanPer; ++u) {
      if (i0 + u < ns) {
        if (j == 0)
#pragma unroll
          for (int c = 0; c < C; ++c) sPre[r][c] = run[c];
        if (j % kSubTiles == 0) {
          int32_t* o = base + (long long)(r * tpr + j / kSubTiles) * E + e0;
          if constexpr (C == 4)
            *reinterpret_cast<int4*>(o) = make_int4(run[0], run[1], run[2], run[3]);
          else
            *o = run[0];
        }
#pragma unroll
        for (int c = 0; c < C; ++c) run[c] += v[u][c];
      }
      if (++j == spr) {
        j = 0;
        ++r;
      }
    }
#pragma unroll
    for (int c = 0; c < C; ++c) carry[c] += __builtin_amdgcn_readlane(incl[c], kWave - 1);
  };
#pragma unroll
  for (int k = 0; k < KEEP; ++k)
    if (b0 + k < b1) scan_batch(b0 + k, va[k]);
  for (int b = b0 + KEEP; b < b1; ++b) {
    int q[kScanPer][C];
    load_batch(b, q);
    scan_batch(b, q);
  }
  if ((int)threadIdx.x < C) {
    int total = 0;
    for (int x = 0; x < nw; ++x) total += sTot[x][threadIdx.x];
    sPre[d.R][threadIdx.x] = total;
  }
  __syncthreads();
  for (int i = threadIdx.x; i < d.R * C; i += blockDim.x) {
    const int rr = i / C, c = i % C;
    counts[(long long)rr * E + e0 + c] = sPre[rr + 1][c] - sPre[rr][c];
  }
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
  const long long nb = ((long long)d.n_sub + kScanBatch - 1) / kScanBatch;
  const int nw = nb < 1 ? 1 : (nb > kScanMaxWaves ? kScanMaxWaves : (int)nb);
  // four columns per workgroup once a column has several batches (Kimi-K3,
  // eight: 23.7 -> 15.5 us on MI355X); with one batch the single columns
  // spread over more CUs (DSV3: 4.8 vs 5.0 us)
  if (nb > 1 && d.E % 4 == 0 && (reinterpret_cast<uintptr_t>(work) & 15) == 0)
    hipLaunchKernelGGL(k_tile_scan<4>, dim3(d.E / 4), dim3(nw * kWave), 0, st, d, work, counts);
  else
    hipLaunchKernelGGL(k_tile_scan<1>, dim3(d.E), dim3(nw * kWave), 0, st, d, work, counts);
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
