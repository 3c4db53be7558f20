// Router top-K with the fused per-tile expert histogram, the histogram of
// caller-supplied ids, and the column scan that turns per-tile counts into
// per-tile prefix offsets and the per-rank load matrix.
//
// Top-K: [AlignSort] -- the MoE layer routes each token to its Top-K experts
// by gate score (DeepSeek V3/R1 add a per-expert gating bias that penalises
// hot experts); the article names warp-shuffle sorting in thread-local
// registers as the faster alternative to a shared-memory radix sort.  Here
// one wave64 owns one token: lane l holds experts [l*V, l*V+V) of the row,
// and K rounds of a wave-wide max over order-preserving 32-bit keys pick
// the experts, lowest lane (= lowest expert index) winning ties.
// Load matrix: [UltraEP] section "その仕組みは高速なエキスパート複製に依存する".
#include "lbt_internal.h"

namespace lbt {

constexpr int kRouteThreads = 1024;
constexpr int kRouteWaves = kRouteThreads / kWave;

// Order-preserving map of a finite fp32 value to u32; -0.0 maps like +0.0 so
// the two tie (IEEE equality).  Every finite value maps above 0x007FFFFF.
__device__ __forceinline__ uint32_t ordered_key(float v) {
  uint32_t u = __float_as_uint(v);
  if (v == 0.0f) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// DPP lane permutations inside a 16-lane row.
constexpr int kDppQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7-i inside each 8 lanes
constexpr int kDppRowMirror = 0x140;   // lane i <-> 15-i inside each 16 lanes

template <int CTRL>
__device__ __forceinline__ int dpp(int v) {
  return __builtin_amdgcn_update_dpp(v, v, CTRL, 0xF, 0xF, false);
}

// Wave-wide max of a u32, returned as a wave-uniform value: four DPP steps
// leave every lane of a 16-lane row holding the row's max, and the four
// row maxima are combined from lanes 0, 16, 32, 48.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  int v = (int)x;
  v = (int)max((uint32_t)v, (uint32_t)dpp<kDppQuadXor1>(v));
  v = (int)max((uint32_t)v, (uint32_t)dpp<kDppQuadXor2>(v));
  v = (int)max((uint32_t)v, (uint32_t)dpp<kDppHalfMirror>(v));
  v = (int)max((uint32_t)v, (uint32_t)dpp<kDppRowMirror>(v));
  const uint32_t a = (uint32_t)__builtin_amdgcn_readlane(v, 0);
  const uint32_t b = (uint32_t)__builtin_amdgcn_readlane(v, 16);
  const uint32_t c = (uint32_t)__builtin_amdgcn_readlane(v, 32);
  const uint32_t d = (uint32_t)__builtin_amdgcn_readlane(v, 48);
  return max(max(a, b), max(c, d));
}

__device__ __forceinline__ float wave_max_f32(float x) {
  int v = __float_as_int(x);
  v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(dpp<kDppQuadXor1>(v))));
  v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(dpp<kDppQuadXor2>(v))));
  v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(dpp<kDppHalfMirror>(v))));
  v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(dpp<kDppRowMirror>(v))));
  const float a = __int_as_float(__builtin_amdgcn_readlane(v, 0));
  const float b = __int_as_float(__builtin_amdgcn_readlane(v, 16));
  const float c = __int_as_float(__builtin_amdgcn_readlane(v, 32));
  const float d = __int_as_float(__builtin_amdgcn_readlane(v, 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

__device__ __forceinline__ double wave_sum_f64(double x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, kWave);
  return x;
}

// Load lane's V logits [lane*V, lane*V+V) of one row; vec = 4, 2 or 1.
template <int V>
__device__ __forceinline__ void load_row(const float* __restrict__ row, int E, int lane, int vec,
                                         float (&raw)[V]) {
  const int e0 = lane * V;
  if constexpr (V % 4 == 0) {
    if (vec == 4) {
#pragma unroll
      for (int v = 0; v < V; v += 4) {
        float4 q = make_float4(0.f, 0.f, 0.f, 0.f);
        if (e0 + v < E) q = *reinterpret_cast<const float4*>(row + e0 + v);
        raw[v] = q.x; raw[v + 1] = q.y; raw[v + 2] = q.z; raw[v + 3] = q.w;
      }
      return;
    }
  }
  if constexpr (V % 2 == 0) {
    if (vec >= 2) {
#pragma unroll
      for (int v = 0; v < V; v += 2) {
        float2 q = make_float2(0.f, 0.f);
        if (e0 + v < E) q = *reinterpret_cast<const float2*>(row + e0 + v);
        raw[v] = q.x; raw[v + 1] = q.y;
      }
      return;
    }
  }
#pragma unroll
  for (int v = 0; v < V; ++v) raw[v] = (e0 + v < E) ? row[e0 + v] : 0.f;
}

template <int V>
__global__ __launch_bounds__(kRouteThreads) void k_route(const float* __restrict__ logits,
                                                         const float* __restrict__ bias, Dims d,
                                                         int vec, int32_t* __restrict__ ids,
                                                         float* __restrict__ gates,
                                                         int32_t* __restrict__ tile_counts) {
  __shared__ int hist[kMaxE];
  const int E = d.E, K = d.K;
  const int tile = blockIdx.x;
  const int r = tile / d.tpr, j = tile - r * d.tpr;
  const int t0 = r * d.S + j * kTileTokens;
  const int len = min(kTileTokens, d.S - j * kTileTokens);
  for (int e = threadIdx.x; e < E; e += kRouteThreads) hist[e] = 0;
  __syncthreads();

  const int lane = lane_id();
  const int e0 = lane * V;
  float b[V];
#pragma unroll
  for (int v = 0; v < V; ++v) b[v] = (bias != nullptr && e0 + v < E) ? bias[e0 + v] : 0.f;

  // every wave loads all of its tokens' rows first (one latency for all),
  // then routes them one after the other
  constexpr int TPW = kTileTokens / kRouteWaves;
  float rows[TPW][V];
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int i = wave_id() + u * kRouteWaves;
    if (i < len) load_row<V>(logits + ((long long)t0 + i) * E, E, lane, vec, rows[u]);
  }
#pragma unroll
  for (int u = 0; u < TPW; ++u) {
    const int i = wave_id() + u * kRouteWaves;
    if (i >= len) break;
    const long long t = (long long)t0 + i;
    float (&raw)[V] = rows[u];
    uint32_t key[V];
#pragma unroll
    for (int v = 0; v < V; ++v)
      key[v] = (e0 + v < E) ? ordered_key(bias != nullptr ? raw[v] + b[v] : raw[v]) : 0u;

    uint32_t taken = 0;
    int my_id = 0;
    float my_logit = 0.f;
    for (int k = 0; k < K; ++k) {
      // lane-local best untaken key; strict '>' keeps the lower expert on ties
      uint32_t best = 0;
      int bv = 0;
      float braw = 0.f;
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const bool ok = !((taken >> v) & 1u) && key[v] > best;
        best = ok ? key[v] : best;
        bv = ok ? v : bv;
        braw = ok ? raw[v] : braw;
      }
      const uint32_t wmax = wave_max_u32(best);
      const unsigned long long m = __ballot(best == wmax);
      const int win = __ffsll((long long)m) - 1;          // lowest lane = lowest expert
      const int wbv = __builtin_amdgcn_readlane(bv, win);
      const float wraw = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(braw), win));
      if (lane == win) taken |= 1u << bv;
      if (lane == k) {
        my_id = win * V + wbv;
        my_logit = wraw;
      }
    }

    double g;
    if (d.score_fn == LBT_SIGMOID) {
      g = 1.0 / (1.0 + exp(-(double)my_logit));
    } else {
      float mx = -INFINITY;
#pragma unroll
      for (int v = 0; v < V; ++v)
        if (e0 + v < E) mx = fmaxf(mx, raw[v]);
      mx = wave_max_f32(mx);
      double s = 0.0;
#pragma unroll
      for (int v = 0; v < V; ++v)
        if (e0 + v < E) s += exp((double)raw[v] - (double)mx);
      s = wave_sum_f64(s);
      g = exp((double)my_logit - (double)mx) / s;
    }
    if (d.renorm) {
      const double gs = wave_sum_f64(lane < K ? g : 0.0);
      g = g / gs;
    }
    if (lane < K) {
      ids[t * K + lane] = my_id;
      gates[t * K + lane] = (float)g;
      atomicAdd(&hist[my_id], 1);
    }
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += kRouteThreads)
    tile_counts[(long long)e * d.n_tiles + tile] = hist[e];
}

// Histogram of caller-supplied ids, one thread per token of a tile.
__global__ __launch_bounds__(kTileTokens) void k_histogram(const int32_t* __restrict__ ids, Dims d,
                                                           int32_t* __restrict__ tile_counts,
                                                           int32_t* __restrict__ status) {
  __shared__ int hist[kMaxE];
  const int E = d.E, K = d.K;
  const int tile = blockIdx.x;
  const int r = tile / d.tpr, j = tile - r * d.tpr;
  const int t0 = r * d.S + j * kTileTokens;
  const int len = min(kTileTokens, d.S - j * kTileTokens);
  for (int e = threadIdx.x; e < E; e += kTileTokens) hist[e] = 0;
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
  for (int e = threadIdx.x; e < E; e += kTileTokens)
    tile_counts[(long long)e * d.n_tiles + tile] = hist[e];
}

// One wave per expert column: exclusive prefix over tiles (written
// tile-major for the align step) and per-source-rank sums (the load matrix).
__global__ __launch_bounds__(256) void k_tile_scan(Dims d, int32_t* __restrict__ work,
                                                   int32_t* __restrict__ counts) {
  const int e = blockIdx.x * 4 + wave_id();
  if (e >= d.E) return;
  const int lane = lane_id();
  const int nt = d.n_tiles;
  const int32_t* col = work + (long long)e * nt;
  int32_t* base = work + work_tile_base(d);
  const int per = (nt + kWave - 1) / kWave;
  const int lo = min(nt, lane * per), hi = min(nt, lo + per);
  int local = 0;
  for (int t = lo; t < hi; ++t) local += col[t];
  int run = wave_incl_scan(local) - local;
  for (int t = lo; t < hi; ++t) {
    base[(long long)t * d.E + e] = run;
    run += col[t];
  }
  for (int r = lane; r < d.R; r += kWave) {
    int s = 0;
    for (int t = r * d.tpr; t < (r + 1) * d.tpr; ++t) s += col[t];
    counts[(long long)r * d.E + e] = s;
  }
}

static int route_vec(const float* p, int E) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  if ((a & 15) == 0 && (E & 3) == 0) return 4;
  if ((a & 7) == 0 && (E & 1) == 0) return 2;
  return 1;
}

hipError_t launch_route(const Dims& d, const float* logits, const float* bias, int32_t* ids,
                        float* gates, int32_t* work, hipStream_t st) {
  if (d.n_tiles == 0 || d.S == 0) return hipSuccess;
  const int vec = route_vec(logits, d.E);
  const dim3 grid(d.n_tiles), block(kRouteThreads);
  const int V = (d.E + kWave - 1) / kWave;
  if (V <= 1) hipLaunchKernelGGL(k_route<1>, grid, block, 0, st, logits, bias, d, vec, ids, gates, work);
  else if (V <= 2) hipLaunchKernelGGL(k_route<2>, grid, block, 0, st, logits, bias, d, vec, ids, gates, work);
  else if (V <= 4) hipLaunchKernelGGL(k_route<4>, grid, block, 0, st, logits, bias, d, vec, ids, gates, work);
  else if (V <= 6) hipLaunchKernelGGL(k_route<6>, grid, block, 0, st, logits, bias, d, vec, ids, gates, work);
  else hipLaunchKernelGGL(k_route<8>, grid, block, 0, st, logits, bias, d, vec, ids, gates, work);
  return hipGetLastError();
}

hipError_t launch_histogram(const Dims& d, const int32_t* ids, int32_t* work, int32_t* status,
                            hipStream_t st) {
  if (d.n_tiles == 0 || d.S == 0) return hipSuccess;
  hipLaunchKernelGGL(k_histogram, dim3(d.n_tiles), dim3(kTileTokens), 0, st, ids, d, work, status);
  return hipGetLastError();
}

hipError_t launch_tile_scan(const Dims& d, int32_t* work, int32_t* counts, hipStream_t st) {
  hipLaunchKernelGGL(k_tile_scan, dim3((d.E + 3) / 4), dim3(256), 0, st, d, work, counts);
  return hipGetLastError();
}

}  // namespace lbt
