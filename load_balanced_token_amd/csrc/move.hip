// Zero-copy dispatch and the inverse combine: the HBM-bound row movement.
//
// [MoonEP-GR] section "Online planning, zero copy και στατικά σχήματα":
// tokens are written straight to their final positions, grouped by expert,
// in a static S*K-shaped buffer whose views the caller gets, with no copy
// from a communication buffer to a user buffer.  Combine returns expert
// results to their source tokens ([MoonEP-GR] evaluation checklist;
// [UltraEP] tokens return after expert compute).
//
// One workgroup per token row (H = 7168: dispatch 896 threads x 1 chunk of
// 16 bytes, combine 224 threads x 8 groups of 8 bytes): short-lived waves
// with all their loads in flight measured fastest on MI355X for both the
// write-heavy dispatch and the read-heavy combine.
#include "rows.h"

namespace lbt {

// Dispatch: one token per workgroup; per pass thread j moves the 16-byte
// chunks base + j + i*blockDim (i < CH) of the row: loaded once, stored K
// times.  One pass covers rows up to 2048 chunks (H = 16384).
template <int CH, int KT, bool FULL>
__global__ __launch_bounds__(1024) void k_dispatch(const u32x4* __restrict__ x,
                                                   const int32_t* __restrict__ slot,
                                                   u32x4* __restrict__ recv, int N, int Krt, int H8,
                                                   long long n_rows) {
  // KT > 0: K fixed at compile time, all destination rows read up front
  const int K = KT > 0 ? KT : Krt;
  const int t = xcd_contiguous(blockIdx.x, gridDim.x);
  const int nthr = blockDim.x;
  const u32x4* src = x + (long long)t * H8;
  const int32_t* sl = slot + (long long)t * K;
  int sk[KT > 0 ? KT : 1];
  if constexpr (KT > 0) {
#pragma unroll
    for (int k = 0; k < KT; ++k) sk[k] = sl[k];
  }
  for (int base = 0; base < H8; base += CH * nthr) {
    u32x4 v[CH];
    uint32_t off[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int c = base + threadIdx.x + j * nthr;
      off[j] = (uint32_t)c * 16u;
      if (FULL || c < H8) v[j] = *at_bytes<u32x4>(src, off[j]);
    }
#pragma unroll
    for (int k = 0; k < K; ++k) {
      const int s = KT > 0 ? sk[KT > 0 ? k : 0] : sl[k];
      if (s < 0 || (long long)s >= n_rows) continue;
      u32x4* dst = recv + (long long)s * H8;
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        const int c = base + threadIdx.x + j * nthr;
        if (FULL || c < H8) *at_bytes<u32x4>(dst, off[j]) = v[j];
      }
    }
  }
}

// acc[0..3] += g * (4 bf16 values), one fused multiply-add each
__device__ __forceinline__ void fma4(float (&a)[4], float g, const u32x2& v) {
  a[0] = fmaf(g, bf16_lo(v.x), a[0]);
  a[1] = fmaf(g, bf16_hi(v.x), a[1]);
  a[2] = fmaf(g, bf16_lo(v.y), a[2]);
  a[3] = fmaf(g, bf16_hi(v.y), a[3]);
}


// Combine: one token per workgroup; per pass thread j owns the groups of 4
// bf16 values base + j + i*blockDim (i < GPT).  Loads are 8 bytes per lane,
// so a lane's 4 fp32 results are 16 contiguous bytes and every store
// instruction writes whole cache lines.  The K source rows are loaded in one
// group of KT (or groups of 8 when K is not a compile-time constant), all in
// flight before the first multiply-add, and accumulated in ascending k.
// One pass covers rows up to H = 8192 (512 threads x 4 groups of 4).  UNIT:
// every gate is 1 (the backward of dispatch, a plain K-row sum).
constexpr int kCombineMaxThreads = 512;

template <int GPT, bool BF16, int KT, bool FULL, bool UNIT = false>
__global__ __launch_bounds__(kCombineMaxThreads) void k_combine(const u32x2* __restrict__ out,
                                                  const int32_t* __restrict__ slot,
                                                  const float* __restrict__ gates, int N, int Krt,
                                                  int G4, long long n_rows, void* __restrict__ y) {
  constexpr int G = KT > 0 ? KT : 8;
  const int K = KT > 0 ? KT : Krt;
  const int t = blockIdx.x;
  const int nthr = blockDim.x;
  const int32_t* sl = slot + (long long)t * K;
  const float* gt = UNIT ? nullptr : gates + (long long)t * K;
  for (int base = 0; base < G4; base += GPT * nthr) {
    float acc[GPT][4];
#pragma unroll
    for (int i = 0; i < GPT; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) acc[i][q] = 0.f;
    for (int k0 = 0; k0 < K; k0 += G) {
      int s[G];
      float g[G];
      bool use[G];
#pragma unroll
      for (int kk = 0; kk < G; ++kk) {
        const int k = k0 + kk;
        s[kk] = k < K ? sl[k] : -1;
        use[kk] = s[kk] >= 0 && (long long)s[kk] < n_rows;   // k < K and the pair fit
        g[kk] = use[kk] ? (UNIT ? 1.f : gt[k]) : 0.f;
      }
      // every load is issued before the first multiply-add; an unused k reads
      // row 0 (always present) and is skipped below
      u32x2 v[G][GPT];
#pragma unroll
      for (int kk = 0; kk < G; ++kk) {
        const u32x2* src = out + (long long)(use[kk] ? s[kk] : 0) * G4;
#pragma unroll
        for (int i = 0; i < GPT; ++i) {
          const int q = base + threadIdx.x + i * nthr;
          v[kk][i] = (FULL || q < G4)
                         ? __builtin_nontemporal_load(at_bytes<u32x2>(src, (uint32_t)q * 8u))
                         : u32x2{0u, 0u};
        }
      }
      bool all_used = true;
#pragma unroll
      for (int kk = 0; kk < G; ++kk) all_used = all_used && use[kk];
      if (all_used) {          // the usual case: one straight run of multiply-adds
#pragma unroll
        for (int i = 0; i < GPT; ++i)
#pragma unroll
          for (int kk = 0; kk < G; ++kk) fma4(acc[i], g[kk], v[kk][i]);
      } else {
#pragma unroll
        for (int i = 0; i < GPT; ++i)
#pragma unroll
          for (int kk = 0; kk < G; ++kk)
            if (use[kk]) fma4(acc[i], g[kk], v[kk][i]);
      }
    }
#pragma unroll
    for (int i = 0; i < GPT; ++i) {
      const int q = base + threadIdx.x + i * nthr;
      if (!FULL && q >= G4) continue;
      if constexpr (BF16) {
        const u32x2 o{to_bf16(acc[i][0]) | (to_bf16(acc[i][1]) << 16),
                      to_bf16(acc[i][2]) | (to_bf16(acc[i][3]) << 16)};
        __builtin_nontemporal_store(
            o, at_bytes<u32x2>(reinterpret_cast<u32x2*>(y) + (long long)t * G4, (uint32_t)q * 8u));
      } else {
        __builtin_nontemporal_store(
            f32x4{acc[i][0], acc[i][1], acc[i][2], acc[i][3]},
            at_bytes<f32x4>(reinterpret_cast<f32x4*>(y) + (long long)t * G4, (uint32_t)q * 16u));
      }
    }
  }
}

// Dispatch specialised for one row width (THR threads x CH chunks of 16
// bytes, THR * CH == the row's chunks) and K = KT; same stores as k_dispatch.
template <int THR, int CH, int KT>
__global__ __launch_bounds__(THR) void k_dispatch_w(const u32x4* __restrict__ x,
                                                    const int32_t* __restrict__ slot,
                                                    u32x4* __restrict__ recv, long long n_rows) {
  constexpr int H8 = THR * CH;
  const int t = xcd_contiguous(blockIdx.x, gridDim.x);
  const u32x4* src = x + (long long)t * H8;
  int s[KT];
#pragma unroll
  for (int k = 0; k < KT; ++k) s[k] = slot[(long long)t * KT + k];
  u32x4 v[CH];
#pragma unroll
  for (int j = 0; j < CH; ++j) v[j] = src[threadIdx.x + j * THR];
#pragma unroll
  for (int k = 0; k < KT; ++k) {
    if (s[k] < 0 || (long long)s[k] >= n_rows) continue;
    u32x4* dst = recv + (long long)s[k] * H8;
#pragma unroll
    for (int j = 0; j < CH; ++j) dst[threadIdx.x + j * THR] = v[j];
  }
}

// Combine specialised for one row width (G4C groups of 4 bf16, THR threads x
// GPT groups each, THR * GPT == G4C) and K = KT.  Same arithmetic and order
// as k_combine.  With the width fixed at compile time this form measured
// ~5% faster on MI355X at H = 7168.  A token holding a slot that did not fit
// (slot < 0, capacity overflow) takes the checked path.
template <int THR, int GPT, int KT, bool BF16, bool UNIT = false>
__global__ __launch_bounds__(THR) void k_combine_w(const u32x2* __restrict__ out,
                                                   const int32_t* __restrict__ slot,
                                                   const float* __restrict__ gates,
                                                   long long n_rows, void* __restrict__ y) {
  constexpr int G4 = THR * GPT;
  const int t = blockIdx.x;
  int s[KT];
  float g[KT];
  bool all_used = true;
#pragma unroll
  for (int k = 0; k < KT; ++k) {
    s[k] = slot[(long long)t * KT + k];
    g[k] = UNIT ? 1.f : gates[(long long)t * KT + k];
    all_used = all_used && s[k] >= 0 && (long long)s[k] < n_rows;
  }
  float acc[GPT][4];
#pragma unroll
  for (int i = 0; i < GPT; ++i)
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[i][q] = 0.f;
  if (all_used) {
    u32x2 v[KT][GPT];
#pragma unroll
    for (int k = 0; k < KT; ++k)
#pragma unroll
      for (int i = 0; i < GPT; ++i) {
        const int q = threadIdx.x + i * THR;
        v[k][i] = q < G4 ? __builtin_nontemporal_load(out + (long long)s[k] * G4 + q)
                         : u32x2{0u, 0u};
      }
#pragma unroll
    for (int i = 0; i < GPT; ++i)
#pragma unroll
      for (int k = 0; k < KT; ++k) fma4(acc[i], g[k], v[k][i]);
  } else {
#pragma unroll
    for (int k = 0; k < KT; ++k) {
      if (!(s[k] >= 0 && (long long)s[k] < n_rows)) continue;
#pragma unroll
      for (int i = 0; i < GPT; ++i) {
        const int q = threadIdx.x + i * THR;
        fma4(acc[i], g[k], out[(long long)s[k] * G4 + q]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < GPT; ++i) {
    const int q = threadIdx.x + i * THR;
    if constexpr (BF16) {
      const u32x2 o{to_bf16(acc[i][0]) | (to_bf16(acc[i][1]) << 16),
                    to_bf16(acc[i][2]) | (to_bf16(acc[i][3]) << 16)};
      __builtin_nontemporal_store(o, reinterpret_cast<u32x2*>(y) + (long long)t * G4 + q);
    } else {
      __builtin_nontemporal_store(f32x4{acc[i][0], acc[i][1], acc[i][2], acc[i][3]},
                                  reinterpret_cast<f32x4*>(y) + (long long)t * G4 + q);
    }
  }
}

// Small batches (at most kColsTokens tokens): one wave per (token, 64
// consecutive pieces of its row), so that a few tokens still spread over many
// CUs instead of keeping a handful of workgroups busy.  Same stores as
// k_dispatch: lane c of slice y moves chunk y*64 + c of the row to all K
// destinations.
constexpr int kColsTokens = 256;
constexpr int kMaxGridY = 65535;   // largest grid y dimension

template <int KT>
__global__ __launch_bounds__(kWave) void k_dispatch_cols(const u32x4* __restrict__ x,
                                                         const int32_t* __restrict__ slot,
                                                         u32x4* __restrict__ recv, int Krt,
                                                         int H8, long long n_rows) {
  const int K = KT > 0 ? KT : Krt;
  const int t = blockIdx.x;
  const int c = blockIdx.y * kWave + threadIdx.x;
  if (c >= H8) return;
  const u32x4 v = x[(long long)t * H8 + c];
  const int32_t* sl = slot + (long long)t * K;
#pragma unroll
  for (int k = 0; k < K; ++k) {
    const int s = sl[k];
    if (s >= 0 && (long long)s < n_rows) recv[(long long)s * H8 + c] = v;
  }
}

// Combine of a small batch, one wave per (token, 64 groups of 4 values):
// the same multiply-adds as k_combine in the same ascending-k order, so the
// results are bit-identical.  The K rows are loaded in groups of KT (or 8
// when K is not a compile-time constant) before the group's multiply-adds.
template <int KT, bool BF16, bool UNIT>
__global__ __launch_bounds__(kWave) void k_combine_cols(const u32x2* __restrict__ out,
                                                        const int32_t* __restrict__ slot,
                                                        const float* __restrict__ gates, int Krt,
                                                        int G4, long long n_rows,
                                                        void* __restrict__ y) {
  constexpr int G = KT > 0 ? KT : 8;
  const int K = KT > 0 ? KT : Krt;
  const int t = blockIdx.x;
  const int q = blockIdx.y * kWave + threadIdx.x;
  if (q >= G4) return;
  const int32_t* sl = slot + (long long)t * K;
  const float* gt = UNIT ? nullptr : gates + (long long)t * K;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int k0 = 0; k0 < K; k0 += G) {
    int s[G];
    bool use[G];
    u32x2 v[G];
#pragma unroll
    for (int kk = 0; kk < G; ++kk) {
      s[kk] = k0 + kk < K ? sl[k0 + kk] : -1;
      use[kk] = s[kk] >= 0 && (long long)s[kk] < n_rows;   // the same for the whole wave
      v[kk] = use[kk] ? __builtin_nontemporal_load(out + (long long)s[kk] * G4 + q) : u32x2{0u, 0u};
    }
#pragma unroll
    for (int kk = 0; kk < G; ++kk)
      if (use[kk]) fma4(acc, UNIT ? 1.f : gt[k0 + kk], v[kk]);
  }
  if constexpr (BF16) {
    const u32x2 o{to_bf16(acc[0]) | (to_bf16(acc[1]) << 16),
                  to_bf16(acc[2]) | (to_bf16(acc[3]) << 16)};
    __builtin_nontemporal_store(o, reinterpret_cast<u32x2*>(y) + (long long)t * G4 + q);
  } else {
    __builtin_nontemporal_store(f32x4{acc[0], acc[1], acc[2], acc[3]},
                                reinterpret_cast<f32x4*>(y) + (long long)t * G4 + q);
  }
}

// Threads of a row workgroup: enough for `per` pieces each, a multiple of
// 64, at most `cap` (wider rows take several passes).
static int row_threads(int pieces, int per, int cap) {
  int thr = (pieces + per - 1) / per;
  thr = ((thr + kWave - 1) / kWave) * kWave;
  return thr > cap ? cap : thr;
}

template <int KT>
static void launch_dispatch_t(const Dims& d, const u32x4* x, const int32_t* slot, u32x4* recv,
                              hipStream_t st) {
  const int H8 = d.H / 8;
  const int thr = row_threads(H8, 2, 1024);
  const dim3 grid(d.N), block(thr);
  const long long n_rows = (long long)d.R * d.C;
  if (H8 % (2 * thr) == 0)   // every pass fills every lane: no per-lane bounds checks
    hipLaunchKernelGGL((k_dispatch<2, KT, true>), grid, block, 0, st, x, slot, recv, d.N, d.K, H8, n_rows);
  else
    hipLaunchKernelGGL((k_dispatch<2, KT, false>), grid, block, 0, st, x, slot, recv, d.N, d.K, H8, n_rows);
}

hipError_t launch_dispatch(const Dims& d, const uint16_t* x, const int32_t* slot, uint16_t* recv,
                           hipStream_t st) {
  if (d.N == 0) return hipSuccess;
  const u32x4* xs = reinterpret_cast<const u32x4*>(x);
  u32x4* rv = reinterpret_cast<u32x4*>(recv);
  const long long n_rows = (long long)d.R * d.C;
  if (d.N <= kColsTokens && d.H / 8 <= kWave * kMaxGridY) {
    const int H8 = d.H / 8;
    const dim3 grid(d.N, (H8 + kWave - 1) / kWave), block(kWave);
    switch (d.K) {
      case 2: hipLaunchKernelGGL(k_dispatch_cols<2>, grid, block, 0, st, xs, slot, rv, d.K, H8, n_rows); break;
      case 4: hipLaunchKernelGGL(k_dispatch_cols<4>, grid, block, 0, st, xs, slot, rv, d.K, H8, n_rows); break;
      case 8: hipLaunchKernelGGL(k_dispatch_cols<8>, grid, block, 0, st, xs, slot, rv, d.K, H8, n_rows); break;
      default: hipLaunchKernelGGL(k_dispatch_cols<0>, grid, block, 0, st, xs, slot, rv, d.K, H8, n_rows); break;
    }
    return hipGetLastError();
  }
  if (d.H == 7168 && d.K == 8) {   // DeepSeek-V3 / Kimi-K2 hidden size
    hipLaunchKernelGGL((k_dispatch_w<896, 1, 8>), dim3(d.N), dim3(896), 0, st, xs, slot, rv,
                       n_rows);
    return hipGetLastError();
  }
  switch (d.K) {
    case 2: launch_dispatch_t<2>(d, xs, slot, rv, st); break;
    case 4: launch_dispatch_t<4>(d, xs, slot, rv, st); break;
    case 8: launch_dispatch_t<8>(d, xs, slot, rv, st); break;
    default: launch_dispatch_t<0>(d, xs, slot, rv, st); break;
  }
  return hipGetLastError();
}

template <bool BF16, int KT, bool UNIT>
static void launch_combine_t(const Dims& d, const u32x2* o, const int32_t* slot, const float* gates,
                             void* y, hipStream_t st) {
  const int G4 = d.H / 4;
  const int thr = row_threads(G4, 4, kCombineMaxThreads);
  const dim3 grid(d.N), block(thr);
  const long long n_rows = (long long)d.R * d.C;
  if (G4 % (4 * thr) == 0)   // every pass fills every lane: no per-lane bounds checks
    hipLaunchKernelGGL((k_combine<4, BF16, KT, true, UNIT>), grid, block, 0, st, o, slot, gates, d.N, d.K, G4, n_rows, y);
  else
    hipLaunchKernelGGL((k_combine<4, BF16, KT, false, UNIT>), grid, block, 0, st, o, slot, gates, d.N, d.K, G4, n_rows, y);
}

template <bool BF16, bool UNIT>
static void launch_combine_k(const Dims& d, const u32x2* o, const int32_t* slot, const float* gates,
                             void* y, hipStream_t st) {
  if (d.N <= kColsTokens && d.H / 4 <= kWave * kMaxGridY) {
    const int G4 = d.H / 4;
    const long long n_rows = (long long)d.R * d.C;
    const dim3 grid(d.N, (G4 + kWave - 1) / kWave), block(kWave);
    switch (d.K) {
      case 2: hipLaunchKernelGGL((k_combine_cols<2, BF16, UNIT>), grid, block, 0, st, o, slot, gates, d.K, G4, n_rows, y); break;
      case 4: hipLaunchKernelGGL((k_combine_cols<4, BF16, UNIT>), grid, block, 0, st, o, slot, gates, d.K, G4, n_rows, y); break;
      case 8: hipLaunchKernelGGL((k_combine_cols<8, BF16, UNIT>), grid, block, 0, st, o, slot, gates, d.K, G4, n_rows, y); break;
      default: hipLaunchKernelGGL((k_combine_cols<0, BF16, UNIT>), grid, block, 0, st, o, slot, gates, d.K, G4, n_rows, y); break;
    }
    return;
  }
  if (d.H == 7168 && d.K == 8) {   // DeepSeek-V3 / Kimi-K2 hidden size
    hipLaunchKernelGGL((k_combine_w<224, 8, 8, BF16, UNIT>), dim3(d.N), dim3(224), 0, st, o, slot,
                       gates, (long long)d.R * d.C, y);
    return;
  }
  switch (d.K) {
    case 2: launch_combine_t<BF16, 2, UNIT>(d, o, slot, gates, y, st); break;
    case 4: launch_combine_t<BF16, 4, UNIT>(d, o, slot, gates, y, st); break;
    case 8: launch_combine_t<BF16, 8, UNIT>(d, o, slot, gates, y, st); break;
    default: launch_combine_t<BF16, 0, UNIT>(d, o, slot, gates, y, st); break;
  }
}

hipError_t launch_combine(const Dims& d, const uint16_t* out, const int32_t* slot,
                          const float* gates, int y_dtype, void* y, hipStream_t st) {
  if (d.N == 0) return hipSuccess;
  const u32x2* o = reinterpret_cast<const u32x2*>(out);
  const bool unit = gates == nullptr;
  if (y_dtype == LBT_Y_BF16) {
    if (unit) launch_combine_k<true, true>(d, o, slot, gates, y, st);
    else launch_combine_k<true, false>(d, o, slot, gates, y, st);
  } else {
    if (unit) launch_combine_k<false, true>(d, o, slot, gates, y, st);
    else launch_combine_k<false, false>(d, o, slot, gates, y, st);
  }
  return hipGetLastError();
}

}  // namespace lbt
