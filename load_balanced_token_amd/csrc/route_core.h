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

// Order-preserving map of an fp32 value (not NaN) to u32; adding +0.0 turns
// -0.0 into +0.0 so the two tie (IEEE equality).  -inf maps to 0x007FFFFF,
// every larger value above it.
__device__ __forceinline__ uint32_t ordered_key(float v) {
  const uint32_t u = __float_as_uint(v + 0.0f);
  return u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
}

// The value of an ordered key (its inverse; -0.0 comes back as +0.0).
__device__ __forceinline__ float ordered_value(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o ^ 0x80000000u) : ~o);
}

// Median of three (the compiler emits one v_med3_u32).
__device__ __forceinline__ uint32_t med3_u32(uint32_t a, uint32_t b, uint32_t c) {
  return min(max(a, b), max(min(a, b), c));
}

// Insert x into l[0..T), kept descending, so that l holds the T largest of
// the values inserted so far, repeats included: position j takes the median
// of its old value, x and the old value above it.  0 (below every ordered
// key) marks an empty entry; inserting 0 changes nothing.
template <int T>
__device__ __forceinline__ void list_insert(uint32_t (&l)[T], uint32_t x) {
#pragma unroll
  for (int j = T - 1; j > 0; --j) l[j] = med3_u32(l[j - 1], x, l[j]);
  l[0] = max(l[0], x);
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

// The same permutation with the old value set to an identity of the
// operation that consumes it (every lane of the row has a source, so the
// old value is never used): the compiler then folds the move into that
// operation as a DPP operand, one instruction per step.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_or(uint32_t v, uint32_t identity) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)identity, (int)v, CTRL, 0xF, 0xF, false);
}

// Row-wide (16-lane) reductions; every lane of the row receives the result.
__device__ __forceinline__ uint32_t row_max_u32(uint32_t x) {
  x = max(x, dpp_or<kDppQuadXor1>(x, 0u));
  x = max(x, dpp_or<kDppQuadXor2>(x, 0u));
  x = max(x, dpp_or<kDppHalfMirror>(x, 0u));
  x = max(x, dpp_or<kDppRowMirror>(x, 0u));
  return x;
}

__device__ __forceinline__ uint32_t row_min_u32(uint32_t x) {
  x = min(x, dpp_or<kDppQuadXor1>(x, 0xFFFFFFFFu));
  x = min(x, dpp_or<kDppQuadXor2>(x, 0xFFFFFFFFu));
  x = min(x, dpp_or<kDppHalfMirror>(x, 0xFFFFFFFFu));
  x = min(x, dpp_or<kDppRowMirror>(x, 0xFFFFFFFFu));
  return x;
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
// 16-lane row); vec = 4, 2 or 1 is the widest aligned load.  FULL: the row
// has 16 V logits, so no load needs a bounds test.
template <int V, bool FULL>
__device__ __forceinline__ void load_row(const float* __restrict__ row, int E, int e0, int vec,
                                         float (&raw)[V]) {
  if constexpr (V % 4 == 0) {
    if (vec == 4) {
#pragma unroll
      for (int v = 0; v < V; v += 4) {
        float4 q = make_float4(0.f, 0.f, 0.f, 0.f);
        if (FULL || e0 + v < E) q = *reinterpret_cast<const float4*>(row + e0 + v);
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
        if (FULL || e0 + v < E) q = *reinterpret_cast<const float2*>(row + e0 + v);
        raw[v] = q.x; raw[v + 1] = q.y;
      }
      return;
    }
  }
#pragma unroll
  for (int v = 0; v < V; ++v) raw[v] = (FULL || e0 + v < E) ? row[e0 + v] : 0.f;
}

// Winners of each round per wave, token row and k: the expert and the key
// bits (route_span records the winning lane and its count of earlier wins
// of the same value during the rounds, and the expert once it is known).
struct RouteScratch {
  int s_id[kRouteWaves][kRowsPerWave][kMaxK];
  uint32_t s_key[kRouteWaves][kRowsPerWave][kMaxK];
};

// The lane's best T keys among those that come after (tk, tv) in the order
// (key descending, local index ascending) -- all keys when !AFTER -- sorted
// in that order into lk/lv; unused entries hold -inf, below every key (keys
// are > -inf).  Float comparison makes -0.0 and +0.0 equal; strict '>'
// keeps the lower index first on equal keys.
template <int V, int T, bool AFTER>
__device__ __forceinline__ void build_list(const float (&key)[V], float tk, int tv, float (&lk)[T],
                                           int (&lv)[T]) {
#pragma unroll
  for (int j = 0; j < T; ++j) {
    lk[j] = -INFINITY;
    lv[j] = 0;
  }
#pragma unroll
  for (int v = 0; v < V; ++v) {
    float x = key[v];
    if constexpr (AFTER) x = (x < tk || (x == tk && v > tv)) ? x : -INFINITY;
    bool c[T];
#pragma unroll
    for (int j = 0; j < T; ++j) c[j] = x > lk[j];
    // (the keys as a median of three per position, the indices still by
    // selects, cut 47 instructions from the kernel but ran slower on MI355X:
    // DSV3 route 17.8 vs 14.3 us)
#pragma unroll
    for (int j = T - 1; j > 0; --j) {
      lk[j] = c[j - 1] ? lk[j - 1] : (c[j] ? x : lk[j]);
      lv[j] = c[j - 1] ? lv[j - 1] : (c[j] ? v : lv[j]);
    }
    lk[0] = c[0] ? x : lk[0];
    lv[0] = c[0] ? v : lv[0];
  }
}

// Tokens route_wave can hold (one RouteScratch row each).
constexpr int kWaveRouteTokens = kRouteWaves * kRowsPerWave;

// LDS of one route workgroup.
struct RouteSmem {
  int hist[kMaxE];
  RouteScratch rs;
};

// Route tokens [t0, t0 + len), len <= kSubTokens, with the first kRouteThreads
// threads of the workgroup; for every chosen (token, expert) pair call
// hist_add(t, expert).  Contains one workgroup barrier (after the row loads),
// which every thread of the workgroup meets (threads past kRouteThreads do
// nothing else), so state the caller set up before the call (a zeroed
// histogram) is visible to hist_add.
template <int V, bool FULL, typename HistAdd>
__device__ __forceinline__ void route_span(const float* __restrict__ logits,
                                           const float* __restrict__ bias, const Dims& d, int vec,
                                           int t0, int len, int32_t* __restrict__ ids,
                                           float* __restrict__ gates, RouteScratch& sm,
                                           HistAdd hist_add) {
  auto& s_id = sm.s_id;
  auto& s_okey = sm.s_key;   // ordered keys
  const int E = d.E, K = d.K;

  const int lane = lane_id(), wv = wave_id();
  const int row = lane / kRowLanes, rl = lane % kRowLanes;
  const int e0 = rl * V;

  // all rows of this wave first (one memory latency), then the rounds
  const bool active = wv < kRouteWaves;
  float rows[kRoutePasses][V];
#pragma unroll
  for (int u = 0; u < kRoutePasses; ++u) {
    const int i = (u * kRouteWaves + wv) * kRowsPerWave + row;
    if (active && i < len) {
      load_row<V, FULL>(logits + ((long long)t0 + i) * E, E, e0, vec, rows[u]);
    } else {
#pragma unroll
      for (int v = 0; v < V; ++v) rows[u][v] = 0.f;
    }
  }
  __syncthreads();   // the caller's histogram set-up is visible
  if (!active) return;

#pragma unroll
  for (int u = 0; u < kRoutePasses; ++u) {
    const int i = (u * kRouteWaves + wv) * kRowsPerWave + row;
    const bool valid = i < len;
    if (!__any(valid)) continue;
    // Keys as order-preserving u32 (equal floats, -0.0 and +0.0 included,
    // give equal keys); 0 stands for "no expert" past E.  The raw values do
    // not stay live through the rounds: the gates and the softmax re-read
    // the row.
    uint32_t ok[V];
#pragma unroll
    for (int v = 0; v < V; ++v) {
      const float x = bias != nullptr ? rows[u][v] + bias[e0 + v] : rows[u][v];
      ok[v] = (FULL || e0 + v < E) ? ordered_key(x) : 0u;
    }
    // Each lane keeps its best T key values sorted, without their experts;
    // a round compares list heads across the row, the lowest lane holding
    // the largest wins and pops its head.  A lane whose full list runs dry
    // refills from the values after the ones it gave up.  Which expert a
    // win was is settled after the rounds: a lane's equal keys are taken in
    // expert order, so its i-th win of a value is the i-th of its experts
    // holding that value.  Together this is exactly K rounds of "largest
    // untaken key, lowest expert on ties".
    constexpr int T = V < 4 ? V : 4;
    uint32_t l[T];
#pragma unroll
    for (int j = 0; j < T; ++j) l[j] = 0u;
#pragma unroll
    for (int v = 0; v < V; ++v) list_insert<T>(l, ok[v]);
    bool more = V > T && l[T - 1] != 0u;   // the lane may hold keys past its list
    uint32_t last = 0u;                     // the value it gave up last
    int eq = 0;                             // its wins of that value so far
    for (int k = 0; k < K; ++k) {
      const uint32_t head = l[0];
      const uint32_t rmax = row_max_u32(head);
      const bool cand = valid && head == rmax;
      // the lowest candidate lane of the row holds the lowest expert
      const uint32_t first = row_min_u32(cand ? (uint32_t)rl : (uint32_t)kRowLanes);
      const bool win = cand && (uint32_t)rl == first;
      if (win) {
        eq = head == last ? eq + 1 : 1;
        last = head;
        s_id[wv][row][k] = (eq - 1) * kRowLanes + rl;
        s_okey[wv][row][k] = head;
#pragma unroll
        for (int j = 0; j + 1 < T; ++j) l[j] = l[j + 1];
        l[T - 1] = 0u;
      }
      if constexpr (V > T) {
        const bool dry = win && more && l[0] == 0u;
        if (__any(dry)) {
          if (dry) {
            // every key below `last`, and those equal to it past the first
            // `eq` in expert order (rare)
            int seen = 0;
#pragma unroll
            for (int v = 0; v < V; ++v) {
              const bool same = ok[v] == last;
              list_insert<T>(l, (ok[v] < last || (same && seen >= eq)) ? ok[v] : 0u);
              seen += same ? 1 : 0;
            }
            more = l[T - 1] != 0u;
          }
        }
      }
    }
    __builtin_amdgcn_wave_barrier();

    const long long t = (long long)t0 + i;
    const float* lrow = logits + (valid ? t : (long long)t0) * E;
    // Winner kk's expert: with (lane wl, its wins of the value before this
    // one) recorded in the round, the matching key among lane wl's experts,
    // read back from the row just loaded (cache hits).
    auto expert_of = [&](int kk) -> int {
      const int code = s_id[wv][row][kk];
      const int wl = code % kRowLanes, occ = code / kRowLanes;
      const float xv = ordered_value(s_okey[wv][row][kk]);
      const int w0 = wl * V;
      float kv[V];
      load_row<V, FULL>(lrow, E, w0, vec, kv);
      if (bias != nullptr) {
#pragma unroll
        for (int v = 0; v < V; ++v) kv[v] += (FULL || w0 + v < E) ? bias[w0 + v] : 0.f;
      }
      int at = 0;
      if (occ == 0) {
#pragma unroll
        for (int v = V - 1; v >= 0; --v)
          if ((FULL || w0 + v < E) && kv[v] == xv) at = v;
      } else {
        int seen = 0;
#pragma unroll
        for (int v = 0; v < V; ++v) {
          const bool same = (FULL || w0 + v < E) && kv[v] == xv;
          if (same && seen == occ) at = v;
          seen += same ? 1 : 0;
        }
      }
      return w0 + at;
    };
    const bool raw_keys = bias == nullptr;
    double mx = 0.0, denom = 1.0;
    if (d.score_fn == LBT_SOFTMAX) {
      float raw[V];
      load_row<V, FULL>(lrow, E, e0, vec, raw);
#pragma unroll
      for (int v = 0; v < V; ++v) raw[v] = (FULL || e0 + v < E) ? raw[v] : -INFINITY;
      float m = -INFINITY;
#pragma unroll
      for (int v = 0; v < V; ++v) m = fmaxf(m, raw[v]);
      mx = (double)row_max_f32(m);
      double s = 0.0;
#pragma unroll
      for (int v = 0; v < V; ++v)
        if (FULL || e0 + v < E) s += exp((double)raw[v] - mx);
      denom = row_sum_f64(s);
    }
    auto score = [&](double lg) -> double {
      return d.score_fn == LBT_SIGMOID ? 1.0 / (1.0 + exp(-lg)) : exp(lg - mx) / denom;
    };
    // the logit of winner kk, expert id: without a selection bias the key
    // is the logit (-0.0 comes back as +0.0, which scores the same)
    auto logit_of = [&](int kk, int id) -> double {
      return raw_keys ? (double)ordered_value(s_okey[wv][row][kk]) : (double)lrow[id];
    };
    if (K <= kRowLanes) {
      // one choice per lane: its score serves both the row sum and the gate
      const bool mine = valid && rl < K;
      int id = 0;
      double g = 0.0;
      if (mine) {
        id = expert_of(rl);
        g = score(logit_of(rl, id));
      }
      if (d.renorm) g = g / row_sum_f64(g);
      if (mine) {
        s_id[wv][row][rl] = id;   // the expert, for callers that read the winners back
        ids[t * K + rl] = id;
        gates[t * K + rl] = (float)g;
        hist_add(t, id);
      }
    } else {
      if (valid)
        for (int kk = rl; kk < K; kk += kRowLanes) s_id[wv][row][kk] = expert_of(kk);
      __builtin_amdgcn_wave_barrier();
      double gsum = 1.0;
      if (d.renorm) {
        double part = 0.0;
        for (int kk = rl; kk < K; kk += kRowLanes)
          part += valid ? score(logit_of(kk, s_id[wv][row][kk])) : 0.0;
        gsum = row_sum_f64(part);
      }
      if (valid) {
        for (int kk = rl; kk < K; kk += kRowLanes) {
          const int id = s_id[wv][row][kk];
          double g = score(logit_of(kk, id));
          if (d.renorm) g = g / gsum;
          ids[t * K + kk] = id;
          gates[t * K + kk] = (float)g;
          hist_add(t, id);
        }
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
}

// Route tokens [0, N) of a small batch, one token per wave (N <= the
// caller's waves and N <= kWaveRouteTokens, the winners' scratch rows;
// every thread of the workgroup calls this, and like
// route_span it contains one workgroup barrier, after the row loads).  Lane
// l holds experts [l*W, l*W + W), W = ceil(V / 4) for the 16-lane layout's V,
// so a lane sorts a quarter of the keys route_span's lanes sort.  A round
// takes the wave-wide max of the list heads (row max by DPP, then the four
// rows' maxima by readlane) and the lowest lane holding it (first set bit
// of a ballot), i.e. the same "largest untaken key, lowest expert on ties".
// The gates are computed by lanes 0..15 exactly as route_span's row lanes
// compute them (same 16-lane layout of the row for the softmax, same
// assignment of k to lanes, same order of additions), so ids and gates are
// bit for bit route_span's.  With store false the ids and gates are not
// written (the winners still reach sm.s_id and hist_add).
template <int V, bool FULL, typename HistAdd>
__device__ __forceinline__ void route_wave(const float* __restrict__ logits,
                                           const float* __restrict__ bias, const Dims& d, int vec,
                                           int N, int32_t* __restrict__ ids,
                                           float* __restrict__ gates, RouteScratch& sm,
                                           HistAdd hist_add, const bool store = true) {
  constexpr int W = (V + 3) / 4;
  constexpr bool FULLW = FULL && V % 4 == 0;   // E = 16 V = 64 W
  const int E = d.E, K = d.K;
  const int lane = lane_id(), t = wave_id();
  const int e0 = lane * W;
  const bool valid = t < N;
  auto& s_id = sm.s_id[t / kRowsPerWave][t % kRowsPerWave];
  auto& s_key = sm.s_key[t / kRowsPerWave][t % kRowsPerWave];
  float raw[W];
  if (valid) {
    load_row<W, FULLW>(logits + (long long)t * E, E, e0, vec, raw);
  } else {
#pragma unroll
    for (int v = 0; v < W; ++v) raw[v] = 0.f;
  }
  __syncthreads();   // the caller's histogram set-up is visible
  if (!valid) return;
  float key[W];
#pragma unroll
  for (int v = 0; v < W; ++v) {
    const bool in = FULLW || e0 + v < E;
    key[v] = in ? (bias != nullptr ? raw[v] + bias[e0 + v] : raw[v]) : -INFINITY;
  }
  constexpr int T = W < 4 ? W : 4;
  float lk[T];
  int lv[T];
  build_list<W, T, false>(key, 0.f, 0, lk, lv);
  bool more = W > T && lk[T - 1] != -INFINITY;
  for (int k = 0; k < K; ++k) {
    const uint32_t head = ordered_key(lk[0]);
    const uint32_t rmax = row_max_u32(head);
    const uint32_t m01 = max((uint32_t)__builtin_amdgcn_readlane((int)rmax, 0),
                             (uint32_t)__builtin_amdgcn_readlane((int)rmax, 16));
    const uint32_t m23 = max((uint32_t)__builtin_amdgcn_readlane((int)rmax, 32),
                             (uint32_t)__builtin_amdgcn_readlane((int)rmax, 48));
    const uint32_t wmax = max(m01, m23);
    const unsigned long long bal = __ballot(head == wmax);
    const bool win = lane == __ffsll((long long)bal) - 1;
    const float tk = lk[0];
    const int tv = lv[0];
    if (win) {
      s_id[k] = e0 + tv;
      s_key[k] = __float_as_uint(tk);
#pragma unroll
      for (int j = 0; j + 1 < T; ++j) {
        lk[j] = lk[j + 1];
        lv[j] = lv[j + 1];
      }
      lk[T - 1] = -INFINITY;
    }
    if constexpr (W > T) {
      const bool dry = win && more && lk[0] == -INFINITY;
      if (__any(dry)) {
        if (dry) {
          build_list<W, T, true>(key, tk, tv, lk, lv);
          more = lk[T - 1] != -INFINITY;
        }
      }
    }
  }
  __builtin_amdgcn_wave_barrier();
  // gates: lanes 0..15 as the 16 lanes of route_span's row
  if (lane >= kRowLanes) return;
  const int rl = lane;
  const float* lrow = logits + (long long)t * E;
  const bool raw_keys = bias == nullptr;
  auto logit_of = [&](int kk) -> double {
    return raw_keys ? (double)__uint_as_float(s_key[kk]) : (double)lrow[s_id[kk]];
  };
  double mx = 0.0, denom = 1.0;
  if (d.score_fn == LBT_SOFTMAX) {
    float r16[V];
    load_row<V, FULL>(lrow, E, rl * V, vec, r16);
#pragma unroll
    for (int v = 0; v < V; ++v) r16[v] = (FULL || rl * V + v < E) ? r16[v] : -INFINITY;
    float m = -INFINITY;
#pragma unroll
    for (int v = 0; v < V; ++v) m = fmaxf(m, r16[v]);
    mx = (double)row_max_f32(m);
    double sacc = 0.0;
#pragma unroll
    for (int v = 0; v < V; ++v)
      if (FULL || rl * V + v < E) sacc += exp((double)r16[v] - mx);
    denom = row_sum_f64(sacc);
  }
  auto score = [&](double lg) -> double {
    return d.score_fn == LBT_SIGMOID ? 1.0 / (1.0 + exp(-lg)) : exp(lg - mx) / denom;
  };
  if (K <= kRowLanes) {
    double g = rl < K ? score(logit_of(rl)) : 0.0;
    if (d.renorm) g = g / row_sum_f64(g);
    if (rl < K) {
      const int id = s_id[rl];
      if (store) {
        ids[(long long)t * K + rl] = id;
        gates[(long long)t * K + rl] = (float)g;
      }
      hist_add((long long)t, id);
    }
    return;
  }
  double gsum = 1.0;
  if (d.renorm) {
    double part = 0.0;
    for (int kk = rl; kk < K; kk += kRowLanes) part += score(logit_of(kk));
    gsum = row_sum_f64(part);
  }
  for (int kk = rl; kk < K; kk += kRowLanes) {
    const int id = s_id[kk];
    double g = score(logit_of(kk));
    if (d.renorm) g = g / gsum;
    if (store) {
      ids[(long long)t * K + kk] = id;
      gates[(long long)t * K + kk] = (float)g;
    }
    hist_add((long long)t, id);
  }
}

// Route the tokens of sub-tile `sub` (kRouteThreads threads) and write its
// expert histogram to sub_counts[sub][e] (one contiguous run).
template <int V, bool FULL>
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
  route_span<V, FULL>(logits, bias, d, vec, t0, len, ids, gates, sm.rs,
                [&](long long, int id) { atomicAdd(&hist[id], 1); });
  __syncthreads();
  for (int e = threadIdx.x; e < d.E; e += kRouteThreads)
    sub_counts[(long long)sub * d.E + e] = hist[e];
}

// Widest aligned logit load (floats) for rows of E floats starting at p.
static inline int route_vec(const float* p, int E) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  if ((a & 15) == 0 && (E & 3) == 0) return 4;
  if ((a & 7) == 0 && (E & 1) == 0) return 2;
  return 1;
}

}  // namespace lbt
