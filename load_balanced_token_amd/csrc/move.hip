// Zero-copy dispatch and the inverse combine: the HBM-bound row movement.
//
// [MoonEP-GR] section "Online planning, zero copy και στατικά σχήματα":
// tokens are written straight to their final positions, grouped by expert,
// in a static S*K-shaped buffer whose views the caller gets, with no copy
// from a communication buffer to a user buffer.  Combine returns expert
// results to their source tokens ([MoonEP-GR] evaluation checklist;
// [UltraEP] tokens return after expert compute).
//
// One wave64 per token row: dispatch reads the row once in 16-byte pieces
// (CH per lane) and stores it K times; combine gathers the K rows and
// accumulates gate * value in fp32, ascending k, with fused multiply-add.
#include "lbt_internal.h"

namespace lbt {

// Native clang vector types: the nontemporal builtins take these, not
// HIP_vector_type.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMoveThreads = 256;
constexpr int kMoveWaves = kMoveThreads / kWave;

template <int CH>
__global__ __launch_bounds__(kMoveThreads) void k_dispatch(const u32x4* __restrict__ x,
                                                          const int32_t* __restrict__ slot,
                                                          u32x4* __restrict__ recv, int N, int K,
                                                          int H8, long long n_rows) {
  const int t = blockIdx.x * kMoveWaves + wave_id();
  if (t >= N) return;
  const int lane = lane_id();
  const u32x4* src = x + (long long)t * H8;
  const int32_t* sl = slot + (long long)t * K;
  for (int base = 0; base < H8; base += CH * kWave) {
    u32x4 v[CH];
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = base + i * kWave + lane;
      if (c < H8) v[i] = __builtin_nontemporal_load(src + c);
    }
    for (int k = 0; k < K; ++k) {
      const int s = sl[k];
      if (s < 0 || (long long)s >= n_rows) continue;
      u32x4* dst = recv + (long long)s * H8;
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const int c = base + i * kWave + lane;
        if (c < H8) __builtin_nontemporal_store(v[i], dst + c);
      }
    }
  }
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t to_bf16(float f) {
  const uint32_t u = __float_as_uint(f);
  if (f != f) return 0x7FC0u;
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ void fma8(float (&a)[8], float g, const u32x4& v) {
  a[0] = fmaf(g, bf16_lo(v.x), a[0]);
  a[1] = fmaf(g, bf16_hi(v.x), a[1]);
  a[2] = fmaf(g, bf16_lo(v.y), a[2]);
  a[3] = fmaf(g, bf16_hi(v.y), a[3]);
  a[4] = fmaf(g, bf16_lo(v.z), a[4]);
  a[5] = fmaf(g, bf16_hi(v.z), a[5]);
  a[6] = fmaf(g, bf16_lo(v.w), a[6]);
  a[7] = fmaf(g, bf16_hi(v.w), a[7]);
}

template <int CH, bool BF16>
__global__ __launch_bounds__(kMoveThreads) void k_combine(const u32x4* __restrict__ out,
                                                         const int32_t* __restrict__ slot,
                                                         const float* __restrict__ gates, int N,
                                                         int K, int H8, long long n_rows,
                                                         void* __restrict__ y) {
  const int t = blockIdx.x * kMoveWaves + wave_id();
  if (t >= N) return;
  const int lane = lane_id();
  const int32_t* sl = slot + (long long)t * K;
  const float* gt = gates + (long long)t * K;
  for (int base = 0; base < H8; base += CH * kWave) {
    float acc[CH][8];
#pragma unroll
    for (int i = 0; i < CH; ++i)
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[i][q] = 0.f;
    for (int k = 0; k < K; ++k) {
      const int s = sl[k];
      if (s < 0 || (long long)s >= n_rows) continue;
      const float g = gt[k];
      const u32x4* src = out + (long long)s * H8;
      u32x4 v[CH];
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const int c = base + i * kWave + lane;
        v[i] = c < H8 ? __builtin_nontemporal_load(src + c) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int i = 0; i < CH; ++i) fma8(acc[i], g, v[i]);
    }
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int c = base + i * kWave + lane;
      if (c >= H8) continue;
      if constexpr (BF16) {
        u32x4 o;
        o.x = to_bf16(acc[i][0]) | (to_bf16(acc[i][1]) << 16);
        o.y = to_bf16(acc[i][2]) | (to_bf16(acc[i][3]) << 16);
        o.z = to_bf16(acc[i][4]) | (to_bf16(acc[i][5]) << 16);
        o.w = to_bf16(acc[i][6]) | (to_bf16(acc[i][7]) << 16);
        __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(y) + (long long)t * H8 + c);
      } else {
        f32x4* yp = reinterpret_cast<f32x4*>(y) + ((long long)t * H8 + c) * 2;
        __builtin_nontemporal_store(f32x4{acc[i][0], acc[i][1], acc[i][2], acc[i][3]}, yp);
        __builtin_nontemporal_store(f32x4{acc[i][4], acc[i][5], acc[i][6], acc[i][7]}, yp + 1);
      }
    }
  }
}

// Chunks per lane: the smallest instantiated count covering the row, else 16
// with several passes.
static int pick_ch(int H8) {
  const int need = (H8 + kWave - 1) / kWave;
  if (need <= 1) return 1;
  if (need <= 2) return 2;
  if (need <= 4) return 4;
  if (need <= 8) return 8;
  if (need <= 14) return 14;
  return 16;
}

hipError_t launch_dispatch(const Dims& d, const uint16_t* x, const int32_t* slot, uint16_t* recv,
                           hipStream_t st) {
  if (d.N == 0) return hipSuccess;
  const int H8 = d.H / 8;
  const long long n_rows = (long long)d.R * d.C;
  const dim3 grid((d.N + kMoveWaves - 1) / kMoveWaves), block(kMoveThreads);
  const u32x4* xs = reinterpret_cast<const u32x4*>(x);
  u32x4* rv = reinterpret_cast<u32x4*>(recv);
  switch (pick_ch(H8)) {
    case 1: hipLaunchKernelGGL(k_dispatch<1>, grid, block, 0, st, xs, slot, rv, d.N, d.K, H8, n_rows); break;
    case 2: hipLaunchKernelGGL(k_dispatch<2>, grid, block, 0, st, xs, slot, rv, d.N, d.K, H8, n_rows); break;
    case 4: hipLaunchKernelGGL(k_dispatch<4>, grid, block, 0, st, xs, slot, rv, d.N, d.K, H8, n_rows); break;
    case 8: hipLaunchKernelGGL(k_dispatch<8>, grid, block, 0, st, xs, slot, rv, d.N, d.K, H8, n_rows); break;
    case 14: hipLaunchKernelGGL(k_dispatch<14>, grid, block, 0, st, xs, slot, rv, d.N, d.K, H8, n_rows); break;
    default: hipLaunchKernelGGL(k_dispatch<16>, grid, block, 0, st, xs, slot, rv, d.N, d.K, H8, n_rows); break;
  }
  return hipGetLastError();
}

template <bool BF16>
static void launch_combine_t(const Dims& d, const u32x4* o, const int32_t* slot, const float* gates,
                             void* y, hipStream_t st) {
  const int H8 = d.H / 8;
  const long long n_rows = (long long)d.R * d.C;
  const dim3 grid((d.N + kMoveWaves - 1) / kMoveWaves), block(kMoveThreads);
  switch (pick_ch(H8)) {
    case 1: hipLaunchKernelGGL((k_combine<1, BF16>), grid, block, 0, st, o, slot, gates, d.N, d.K, H8, n_rows, y); break;
    case 2: hipLaunchKernelGGL((k_combine<2, BF16>), grid, block, 0, st, o, slot, gates, d.N, d.K, H8, n_rows, y); break;
    case 4: hipLaunchKernelGGL((k_combine<4, BF16>), grid, block, 0, st, o, slot, gates, d.N, d.K, H8, n_rows, y); break;
    case 8: hipLaunchKernelGGL((k_combine<8, BF16>), grid, block, 0, st, o, slot, gates, d.N, d.K, H8, n_rows, y); break;
    case 14: hipLaunchKernelGGL((k_combine<14, BF16>), grid, block, 0, st, o, slot, gates, d.N, d.K, H8, n_rows, y); break;
    default: hipLaunchKernelGGL((k_combine<16, BF16>), grid, block, 0, st, o, slot, gates, d.N, d.K, H8, n_rows, y); break;
  }
}

hipError_t launch_combine(const Dims& d, const uint16_t* out, const int32_t* slot,
                          const float* gates, int y_dtype, void* y, hipStream_t st) {
  if (d.N == 0) return hipSuccess;
  const u32x4* o = reinterpret_cast<const u32x4*>(out);
  if (y_dtype == LBT_Y_BF16) launch_combine_t<true>(d, o, slot, gates, y, st);
  else launch_combine_t<false>(d, o, slot, gates, y, st);
  return hipGetLastError();
}

}  // namespace lbt
