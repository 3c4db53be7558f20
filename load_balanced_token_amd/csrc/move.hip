// Zero-copy dispatch and the inverse combine: the HBM-bound row movement.
//
// [MoonEP-GR] section "Online planning, zero copy και στατικά σχήματα":
// tokens are written straight to their final positions, grouped by expert,
// in a static S*K-shaped buffer whose views the caller gets, with no copy
// from a communication buffer to a user buffer.  Combine returns expert
// results to their source tokens ([MoonEP-GR] evaluation checklist;
// [UltraEP] tokens return after expert compute).
//
// One workgroup per token row (H = 7168: dispatch 448 threads x 2 chunks of
// 16 bytes, combine 896 threads x 1 chunk): short-lived waves with all their
// loads in flight measured fastest on MI355X for both the write-heavy
// dispatch and the read-heavy combine.
#include "lbt_internal.h"

namespace lbt {

// Native clang vector types: the nontemporal builtins take these, not
// HIP_vector_type.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));


// Workgroup i runs on XCD i % 8; give each XCD a contiguous range of tokens
// so that one XCD's L2 sees neighbouring rows.  A bijection on [0, G).
__device__ __forceinline__ int xcd_contiguous(int i, int G) {
  const int q = G / 8, rem = G % 8, x = i % 8, pos = i / 8;
  return x * q + min(x, rem) + pos;
}

// Dispatch: one token per workgroup; per pass thread j moves the 16-byte
// chunks base + j + i*blockDim (i < CH) of the row: loaded once, stored K
// times.  One pass covers rows up to 2048 chunks (H = 16384).
template <int CH>
__global__ __launch_bounds__(1024) void k_dispatch(const u32x4* __restrict__ x,
                                                   const int32_t* __restrict__ slot,
                                                   u32x4* __restrict__ recv, int N, int K, int H8,
                                                   long long n_rows) {
  const int t = xcd_contiguous(blockIdx.x, gridDim.x);
  const int nthr = blockDim.x;
  const u32x4* src = x + (long long)t * H8;
  const int32_t* sl = slot + (long long)t * K;
  for (int base = 0; base < H8; base += CH * nthr) {
    u32x4 v[CH];
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int c = base + threadIdx.x + j * nthr;
      if (c < H8) v[j] = src[c];
    }
    for (int k = 0; k < K; ++k) {
      const int s = sl[k];
      if (s < 0 || (long long)s >= n_rows) continue;
      u32x4* dst = recv + (long long)s * H8;
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        const int c = base + threadIdx.x + j * nthr;
        if (c < H8) dst[c] = v[j];
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

// Combine: one token per workgroup; per pass thread j owns the 16-byte
// chunks base + j + i*blockDim (i < CH).  The K source rows are loaded in
// groups of 8 (all loads of a group in flight before the first multiply-add)
// and accumulated over k in ascending order.  One pass covers rows up to
// 1024 chunks (H = 8192).
template <int CH, bool BF16>
__global__ __launch_bounds__(1024) void k_combine(const u32x4* __restrict__ out,
                                                  const int32_t* __restrict__ slot,
                                                  const float* __restrict__ gates, int N, int K,
                                                  int H8, long long n_rows, void* __restrict__ y) {
  constexpr int G = 8;
  __shared__ float s_stage[1024 * 8];   // fp32 outputs of the workgroup's chunks
  const int t = blockIdx.x;
  const int nthr = blockDim.x;
  const int32_t* sl = slot + (long long)t * K;
  const float* gt = gates + (long long)t * K;
  for (int base = 0; base < H8; base += CH * nthr) {
    float acc[CH][8];
#pragma unroll
    for (int j = 0; j < CH; ++j)
#pragma unroll
      for (int q = 0; q < 8; ++q) acc[j][q] = 0.f;
    for (int k0 = 0; k0 < K; k0 += G) {
      u32x4 v[G][CH];
      float g[G];
      bool use[G];
#pragma unroll
      for (int kk = 0; kk < G; ++kk) {
        const int k = k0 + kk;
        const int s = k < K ? sl[k] : -1;
        const bool ok = s >= 0 && (long long)s < n_rows;
        use[kk] = ok;
        g[kk] = ok ? gt[k] : 0.f;
        const u32x4* src = out + (long long)(ok ? s : 0) * H8;
#pragma unroll
        for (int j = 0; j < CH; ++j) {
          const int c = base + threadIdx.x + j * nthr;
          v[kk][j] = (ok && c < H8) ? __builtin_nontemporal_load(src + c) : u32x4{0u, 0u, 0u, 0u};
        }
      }
#pragma unroll
      for (int kk = 0; kk < G; ++kk) {
        if (!use[kk]) continue;   // k >= K, or a slot that did not fit
#pragma unroll
        for (int j = 0; j < CH; ++j) fma8(acc[j], g[kk], v[kk][j]);
      }
    }
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int c = base + threadIdx.x + j * nthr;
      if constexpr (BF16) {
        if (c >= H8) continue;
        u32x4 o;
        o.x = to_bf16(acc[j][0]) | (to_bf16(acc[j][1]) << 16);
        o.y = to_bf16(acc[j][2]) | (to_bf16(acc[j][3]) << 16);
        o.z = to_bf16(acc[j][4]) | (to_bf16(acc[j][5]) << 16);
        o.w = to_bf16(acc[j][6]) | (to_bf16(acc[j][7]) << 16);
        __builtin_nontemporal_store(o, reinterpret_cast<u32x4*>(y) + (long long)t * H8 + c);
      } else {
        // The wave's 64 chunks are 512 consecutive fp32 outputs; regroup them
        // through LDS so each store instruction writes 1 KB contiguously
        // (lane l's own 32 bytes would leave every line half-written).
        f32x4* stage = reinterpret_cast<f32x4*>(s_stage) + wave_id() * 2 * kWave;
        const int lane = lane_id();
        stage[2 * lane] = f32x4{acc[j][0], acc[j][1], acc[j][2], acc[j][3]};
        stage[2 * lane + 1] = f32x4{acc[j][4], acc[j][5], acc[j][6], acc[j][7]};
        __builtin_amdgcn_wave_barrier();
        const f32x4 lo = stage[lane], hi = stage[kWave + lane];
        __builtin_amdgcn_wave_barrier();
        // chunk c0 = first chunk of this wave; its fp32 outputs start at 8*c0
        const int c0 = c - lane;
        f32x4* yp = reinterpret_cast<f32x4*>(y) + ((long long)t * H8 + c0) * 2;
        if (c0 + lane / 2 < H8) __builtin_nontemporal_store(lo, yp + lane);
        if (c0 + kWave / 2 + lane / 2 < H8) __builtin_nontemporal_store(hi, yp + kWave + lane);
      }
    }
  }
}

// Threads of a row workgroup: enough for `per` chunks each, a multiple of
// 64, at most 1024 (wider rows take several passes).
static int row_threads(int H8, int per) {
  int thr = (H8 + per - 1) / per;
  thr = ((thr + kWave - 1) / kWave) * kWave;
  return thr > 1024 ? 1024 : thr;
}

hipError_t launch_dispatch(const Dims& d, const uint16_t* x, const int32_t* slot, uint16_t* recv,
                           hipStream_t st) {
  if (d.N == 0) return hipSuccess;
  const int H8 = d.H / 8;
  const long long n_rows = (long long)d.R * d.C;
  hipLaunchKernelGGL(k_dispatch<2>, dim3(d.N), dim3(row_threads(H8, 2)), 0, st,
                     reinterpret_cast<const u32x4*>(x), slot, reinterpret_cast<u32x4*>(recv), d.N,
                     d.K, H8, n_rows);
  return hipGetLastError();
}

hipError_t launch_combine(const Dims& d, const uint16_t* out, const int32_t* slot,
                          const float* gates, int y_dtype, void* y, hipStream_t st) {
  if (d.N == 0) return hipSuccess;
  const int H8 = d.H / 8;
  const long long n_rows = (long long)d.R * d.C;
  const u32x4* o = reinterpret_cast<const u32x4*>(out);
  const dim3 grid(d.N), block(row_threads(H8, 1));
  if (y_dtype == LBT_Y_BF16)
    hipLaunchKernelGGL((k_combine<1, true>), grid, block, 0, st, o, slot, gates, d.N, d.K, H8, n_rows, y);
  else
    hipLaunchKernelGGL((k_combine<1, false>), grid, block, 0, st, o, slot, gates, d.N, d.K, H8, n_rows, y);
  return hipGetLastError();
}

}  // namespace lbt
