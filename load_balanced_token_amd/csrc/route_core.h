// Router top-K over one 32-token sub-tile plus its expert histogram, as a
// device function (the route kernel is a thin wrapper around it).
//
// Top-K: [AlignSort] -- the MoE layer routes each token to its Top-K experts
// by gate score (DeepSeek V3/R1 add a per-expert gating bias that penalises
// hot experts); the article names warp-shuffle sorting in thread-local
// registers as the faster alternative to a shared-memory radix sort.  Here a
// token belongs to one 16-lane DPP row of a wave64 (four tokens per wave):
// lane j of the row holds experts [j*V, j*V+V); each of the K rounds takes
// the row-wide max of order-preserving 32-bit keys with four DPP steps and
// the lowest lane holding it (= the lowest expert index) wins.
// Load matrix: [UltraEP] section "その仕組みは高速なエキスパート複製に依存する".
#pragma once
#include "lbt_internal.h"

namespace lbt {

// One workgroup routes one 32-token sub-tile in a single pass (eight waves
// of four tokens): small batches spread over as many CUs as they have
// sub-tiles, and at 32K tokens the chip holds more resident waves than with
// 128-token workgroups taking two passes.
constexpr int kRouteThreads = 512;
constexpr int kRouteWaves = kRouteThreads / kWave;
constexpr int kRowLanes = 16;                        // lanes per token
constexpr int kRowsPerWave = kWave / kRowLanes;      // tokens per wave
constexpr int kRouteTokens = kRouteWaves * kRowsPerWave;   // tokens per pass
constexpr int kRoutePasses = kSubTokens / kRouteTokens;
static_assert(kRoutePasses * kRouteTokens == kSubTokens, "whole passes per sub-tile");

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

// Row-wide (16-lane) reductions; every lane of the row receives the result.
__device__ __forceinline__ uint32_t row_max_u32(uint32_t x) {
  int v = (int)x;
  v = (int)max((uint32_t)v, (uint32_t)dpp<kDppQuadXor1>(v));
  v = (int)max((uint32_t)v, (uint32_t)dpp<kDppQuadXor2>(v));
  v = (int)max((uint32_t)v, (uint32_t)dpp<kDppHalfMirror>(v));
  v = (int)max((uint32_t)v, (uint32_t)dpp<kDppRowMirror>(v));
  return (uint32_t)v;
}

__device__ __forceinline__ float row_max_f32(float x) {
  int v = __float_as_int(x);
  v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(dpp<kDppQuadXor1>(v))));
  v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(dpp<kDppQuadXor2>(v))));
  v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(dpp<kDppHalfMirror>(v))));
  v = __float_as_int(fmaxf(__int_as_float(v), __int_as_float(dpp<kDppRowMirror>(v))));
  return __int_as_float(v);
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double x) {
  const long long b = __double_as_longlong(x);
  const int lo = dpp<CTRL>((int)(b & 0xFFFFFFFFll));
  const int hi = dpp<CTRL>((int)(b >> 32));
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

__device__ __forceinline__ double row_sum_f64(double x) {
  x += dpp_f64<kDppQuadXor1>(x);
  x += dpp_f64<kDppQuadXor2>(x);
  x += dpp_f64<kDppHalfMirror>(x);
  x += dpp_f64<kDppRowMirror>(x);
  return x;
}

// Load lane's V logits [j*V, j*V+V) of one row (j = lane within its
// 16-lane row); vec = 4, 2 or 1 is the widest aligned load.
template <int V>
__device__ __forceinline__ void load_row(const float* __restrict__ row, int E, int e0, int vec,
                                         float (&raw)[V]) {
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

// Winners of each round: expert per wave, token row and k.
struct RouteScratch {
  int s_id[kRouteWaves][kRowsPerWave][kMaxK];
};

// The lane's best T keys among those that come after (tk, tv) in the order
// (key descending, local index ascending) -- all keys when !AFTER -- sorted
// in that order into lk/lv; unused entries hold key 0 (below every valid
// key, which is > 0x007FFFFF).  Strict '>' keeps the lower index first on
// equal keys.
template <int V, int T, bool AFTER>
__device__ __forceinline__ void build_list(const uint32_t (&key)[V], uint32_t tk, int tv,
                                           uint32_t (&lk)[T], int (&lv)[T]) {
#pragma unroll
  for (int j = 0; j < T; ++j) {
    lk[j] = 0u;
    lv[j] = 0;
  }
#pragma unroll
  for (int v = 0; v < V; ++v) {
    uint32_t x = key[v];
    if constexpr (AFTER) x = (x < tk || (x == tk && v > tv)) ? x : 0u;
    bool c[T];
#pragma unroll
    for (int j = 0; j < T; ++j) c[j] = x > lk[j];
#pragma unroll
    for (int j = T - 1; j > 0; --j) {
      lk[j] = c[j - 1] ? lk[j - 1] : (c[j] ? x : lk[j]);
      lv[j] = c[j - 1] ? lv[j - 1] : (c[j] ? v : lv[j]);
    }
    lk[0] = c[0] ? x : lk[0];
    lv[0] = c[0] ? v : lv[0];
  }
}

// LDS of one route workgroup.
struct RouteSmem {
  int hist[kMaxE];
  RouteScratch rs;
};

// Route tokens [t0, t0 + len), len <= kSubTokens, with kRouteThreads threads; for every
// chosen (token, expert) pair call hist_add(t, expert).  Contains one
// workgroup barrier (after the row loads), so state the caller set up before
// the call (a zeroed histogram) is visible to hist_add.
template <int V, typename HistAdd>
__device__ __forceinline__ void route_span(const float* __restrict__ logits,
                                           const float* __restrict__ bias, const Dims& d, int vec,
                                           int t0, int len, int32_t* __restrict__ ids,
                                           float* __restrict__ gates, RouteScratch& sm,
                                           HistAdd hist_add) {
  auto& s_id = sm.s_id;
  const int E = d.E, K = d.K;

  const int lane = lane_id(), wv = wave_id();
  const int row = lane / kRowLanes, rl = lane % kRowLanes;
  const int e0 = rl * V;

  // all rows of this wave first (one memory latency), then the rounds
  float rows[kRoutePasses][V];
#pragma unroll
  for (int u = 0; u < kRoutePasses; ++u) {
    const int i = (u * kRouteWaves + wv) * kRowsPerWave + row;
    if (i < len) {
      load_row<V>(logits + ((long long)t0 + i) * E, E, e0, vec, rows[u]);
    } else {
#pragma unroll
      for (int v = 0; v < V; ++v) rows[u][v] = 0.f;
    }
  }
  __syncthreads();   // the caller's histogram set-up is visible

#pragma unroll
  for (int u = 0; u < kRoutePasses; ++u) {
    const int i = (u * kRouteWaves + wv) * kRowsPerWave + row;
    const bool valid = i < len;
    if (!__any(valid)) continue;
    // keys only from here on: gates and the softmax re-read the row, so the
    // raw values do not stay live through the rounds
    uint32_t key[V];
    if (bias != nullptr) {
#pragma unroll
      for (int v = 0; v < V; ++v)
        key[v] = (valid && e0 + v < E) ? ordered_key(rows[u][v] + bias[e0 + v]) : 0u;
    } else {
#pragma unroll
      for (int v = 0; v < V; ++v) key[v] = (valid && e0 + v < E) ? ordered_key(rows[u][v]) : 0u;
    }
    // Each lane keeps its best T keys sorted (key desc, local index asc);
    // a round compares list heads across the row and the winner pops.  A
    // lane whose full list runs dry refills from the keys after the one it
    // gave up last, so the order of choices is exactly the K rounds of
    // "largest untaken key, lowest expert on ties".
    constexpr int T = V < 4 ? V : 4;
    uint32_t lk[T];
    int lv[T];
    build_list<V, T, false>(key, 0u, 0, lk, lv);
    bool more = V > T && lk[T - 1] != 0u;   // the lane may hold keys past its list
    for (int k = 0; k < K; ++k) {
      const uint32_t head = lk[0];
      const uint32_t rmax = row_max_u32(head);
      const bool cand = valid && head == rmax;
      const unsigned long long m = __ballot(cand);
      // candidates below this lane in the wave, minus those in lower rows
      const int below = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                  __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
      const int p1 = __popcll(m & 0xFFFFull), p2 = __popcll(m & 0xFFFFFFFFull),
                p3 = __popcll(m & 0xFFFFFFFFFFFFull);
      const int lower = row == 0 ? 0 : row == 1 ? p1 : row == 2 ? p2 : p3;
      bool dry = false;
      if (cand && below == lower) {        // lowest lane of the row = lowest expert
        const uint32_t tk = lk[0];
        const int tv = lv[0];
        s_id[wv][row][k] = e0 + tv;
#pragma unroll
        for (int j = 0; j + 1 < T; ++j) {
          lk[j] = lk[j + 1];
          lv[j] = lv[j + 1];
        }
        lk[T - 1] = 0u;
        if constexpr (V > T) {
          dry = more && lk[0] == 0u;
          if (dry) {
            lk[0] = tk;                    // remember the threshold for the refill
            lv[0] = tv;
          }
        }
      }
      if constexpr (V > T) {
        if (__any(dry)) {
          if (dry) {
            build_list<V, T, true>(key, lk[0], lv[0], lk, lv);
            more = lk[T - 1] != 0u;
          }
        }
      }
    }
    __builtin_amdgcn_wave_barrier();

    const long long t = (long long)t0 + i;
    // raw logits are read back from the row just loaded (cache hits)
    const float* lrow = logits + (valid ? t : (long long)t0) * E;
    double mx = 0.0, denom = 1.0;
    if (d.score_fn == LBT_SOFTMAX) {
      float raw[V];
      load_row<V>(lrow, E, e0, vec, raw);
      float m = -INFINITY;
#pragma unroll
      for (int v = 0; v < V; ++v)
        if (e0 + v < E) m = fmaxf(m, raw[v]);
      mx = (double)row_max_f32(m);
      double s = 0.0;
#pragma unroll
      for (int v = 0; v < V; ++v)
        if (e0 + v < E) s += exp((double)raw[v] - mx);
      denom = row_sum_f64(s);
    }
    double gsum = 1.0;
    if (d.renorm) {
      double part = 0.0;
      for (int kk = rl; kk < K; kk += kRowLanes) {
        const double lg = valid ? (double)lrow[s_id[wv][row][kk]] : 0.0;
        part += d.score_fn == LBT_SIGMOID ? 1.0 / (1.0 + exp(-lg)) : exp(lg - mx) / denom;
      }
      gsum = row_sum_f64(part);
    }
    if (valid) {
      for (int kk = rl; kk < K; kk += kRowLanes) {
        const int id = s_id[wv][row][kk];
        const double lg = (double)lrow[id];
        double g = d.score_fn == LBT_SIGMOID ? 1.0 / (1.0 + exp(-lg)) : exp(lg - mx) / denom;
        if (d.renorm) g = g / gsum;
        ids[t * K + kk] = id;
        gates[t * K + kk] = (float)g;
        hist_add(t, id);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// Route the tokens of sub-tile `sub` (kRouteThreads threads) and write its
// expert histogram to sub_counts[e][sub].
template <int V>
__device__ __forceinline__ void route_sub(const float* __restrict__ logits,
                                          const float* __restrict__ bias, const Dims& d, int vec,
                                          int sub, int32_t* __restrict__ ids,
                                          float* __restrict__ gates,
                                          int32_t* __restrict__ sub_counts, RouteSmem& sm) {
  int* hist = sm.hist;
  const int r = sub / d.spr, j = sub - r * d.spr;
  const int t0 = r * d.S + j * kSubTokens;
  const int len = min(kSubTokens, d.S - j * kSubTokens);
  for (int e = threadIdx.x; e < d.E; e += kRouteThreads) hist[e] = 0;
  route_span<V>(logits, bias, d, vec, t0, len, ids, gates, sm.rs,
                [&](long long, int id) { atomicAdd(&hist[id], 1); });
  __syncthreads();
  for (int e = threadIdx.x; e < d.E; e += kRouteThreads)
    sub_counts[(long long)e * d.n_sub + sub] = hist[e];
}

// Widest aligned logit load (floats) for rows of E floats starting at p.
static inline int route_vec(const float* p, int E) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  if ((a & 15) == 0 && (E & 3) == 0) return 4;
  if ((a & 7) == 0 && (E & 1) == 0) return 2;
  return 1;
}

}  // namespace lbt
