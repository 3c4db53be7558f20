// The training side of the path on one GPU: replica weight prefetch into the
// prefetch slots, the backward of combine (expert-output and gate
// gradients), and reduce_grad (replica weight gradients folded into their
// home experts).  The backward of dispatch is the combine kernel with unit
// gates (move.hip).
//
// [MoonEP-GR] sections "Το memory contract ..." (one contiguous [E+B, H, H']
// weight tensor per expert projection; rows E..E+B-1 are the rank's local
// prefetch slots; the pool is process-global) and "Τι συμβαίνει στους
// gradients κατά την εκπαίδευση" (fp32 gradients laid out like the weights;
// prefetched slots write to a separate reduce buffer [R, B, H, H'];
// reduce_grad adds them into the home parameter gradients and clears them).
// [AlignSort] (the gradient of unpermute is a permute).
//
// All three kernels are HBM-bound streams.  Prefetch reads each rank's
// slotted replicas from its segment table (n_slots, seg_expert); reduce_grad
// walks the replica-segment table (piece_*), whose weight-row column marks
// the slotted replicas; every index taken from the plan is bounds-checked
// before it addresses memory.
#include "rows.h"

namespace lbt {

constexpr int kCopyThreads = 256;
constexpr int kRedUnroll = 4;                                       // float4 per thread
constexpr long long kRedTile = (long long)kCopyThreads * kRedUnroll * 4;       // 4096 floats
constexpr int kStreamGroups = 2048;                                 // persistent grid
constexpr int kMaxSlots = 1024;                                     // slots per rank (B) held in LDS

// ---- prefetch -----------------------------------------------------------------
// Grid (4 KiB tile of a weight row, rank r): the workgroup copies that tile
// of every slotted replica of rank r -- slot j < n_slots[r] holds the
// expert at entry E/R + j of r's segment table -- one 16-byte chunk per
// thread per slot, two slots in flight.  Sized without the slot count
// (unknown on the host), a rank with few slots costs only short
// workgroups.  Measured on MI355X against the earlier persistent grid of
// 32 KiB items: DSV3 418 -> 405 us, Kimi-K3 607 -> 549 us.
constexpr int kPrefetchTile = 4096;
constexpr int kPrefetchUnroll = 2;

__global__ __launch_bounds__(kCopyThreads) void k_prefetch(const int32_t* __restrict__ plan, Dims d,
                                                           const char* __restrict__ weights,
                                                           char* __restrict__ slots,
                                                           long long row_bytes) {
  __shared__ int sE[kMaxSlots];
  const PlanLayout pl = d.pl;
  const int r = blockIdx.y;
  const int n = min(max(plan[pl.n_slots + r], 0), min(d.B, pl.max_seg - d.nh));
  for (int j = threadIdx.x; j < n; j += kCopyThreads)
    sE[j] = plan[pl.seg_expert + (long long)r * pl.max_seg + d.nh + j];
  __syncthreads();
  const long long off = (long long)blockIdx.x * kPrefetchTile + threadIdx.x * 16;
  if (off + 16 > row_bytes) return;
  for (int j0 = 0; j0 < n; j0 += kPrefetchUnroll) {
    u32x4 v[kPrefetchUnroll];
#pragma unroll
    for (int u = 0; u < kPrefetchUnroll; ++u) {
      const int e = j0 + u < n ? sE[j0 + u] : -1;
      if (e >= 0 && e < d.E) v[u] = *at_bytes<u32x4>(weights + (long long)e * row_bytes, off);
    }
#pragma unroll
    for (int u = 0; u < kPrefetchUnroll; ++u) {
      const int e = j0 + u < n ? sE[j0 + u] : -1;
      if (e >= 0 && e < d.E)
        *at_bytes<u32x4>(slots + ((long long)r * d.B + j0 + u) * row_bytes, off) = v[u];
    }
  }
}

hipError_t launch_prefetch(const Dims& d, const int32_t* plan, const void* weights, void* slots,
                           long long row_bytes, hipStream_t st) {
  if (d.B == 0 || d.R == 0) return hipSuccess;
  const long long tiles = (row_bytes + kPrefetchTile - 1) / kPrefetchTile;
  if (tiles > 0x7FFFFFFFLL) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_prefetch, dim3((unsigned)tiles, (unsigned)d.R), dim3(kCopyThreads), 0, st,
                     plan, d, static_cast<const char*>(weights), static_cast<char*>(slots),
                     row_bytes);
  return hipGetLastError();
}

// ---- reduce_grad --------------------------------------------------------------
// Work item = (replica segment g that starts its expert's run on the line,
// tile of 4096 floats).  The run's slotted segments are added to the home
// gradient in line order and cleared; a run with no slotted segment writes
// nothing.
__global__ __launch_bounds__(kCopyThreads) void k_reduce_grad(const int32_t* __restrict__ plan,
                                                              Dims d, float* __restrict__ slot_grads,
                                                              float* __restrict__ grads,
                                                              long long row_elems, long long tiles) {
  const PlanLayout pl = d.pl;
  const int nP = min(plan[pl.hdr + LBT_HDR_N_PIECES], pl.max_pieces);
  const long long items = (long long)nP * tiles;
  for (long long it = blockIdx.x; it < items; it += gridDim.x) {
    const int g = (int)(it / tiles);
    const long long off = (it - (long long)g * tiles) * kRedTile;
    const int e = plan[pl.piece_expert + g];
    if (e < 0 || e >= d.E) continue;
    if (g > 0 && plan[pl.piece_expert + g - 1] == e) continue;   // not the first of its run
    const long long n = min(kRedTile, row_elems - off);
    float* home = grads + (long long)e * row_elems + off;
    f32x4 acc[kRedUnroll];
#pragma unroll
    for (int u = 0; u < kRedUnroll; ++u) {
      const uint32_t q = (uint32_t)(u * kCopyThreads + threadIdx.x) * 4u;
      acc[u] = q < n ? *at_bytes<f32x4>(home, q * 4u) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    bool any = false;
    for (int p = g; p < nP && plan[pl.piece_expert + p] == e; ++p) {
      const int j = plan[pl.piece_wrow + p] - d.E;
      const int r = plan[pl.piece_rank + p];
      if (j < 0 || j >= d.B || r < 0 || r >= d.R) continue;       // remote: no slot
      float* sg = slot_grads + ((long long)r * d.B + j) * row_elems + off;
#pragma unroll
      for (int u = 0; u < kRedUnroll; ++u) {
        const uint32_t q = (uint32_t)(u * kCopyThreads + threadIdx.x) * 4u;
        if (q < n) {
          acc[u] += *at_bytes<f32x4>(sg, q * 4u);
          *at_bytes<f32x4>(sg, q * 4u) = f32x4{0.f, 0.f, 0.f, 0.f};
        }
      }
      any = true;
    }
    if (!any) continue;
#pragma unroll
    for (int u = 0; u < kRedUnroll; ++u) {
      const uint32_t q = (uint32_t)(u * kCopyThreads + threadIdx.x) * 4u;
      if (q < n) *at_bytes<f32x4>(home, q * 4u) = acc[u];
    }
  }
}

hipError_t launch_reduce_grad(const Dims& d, const int32_t* plan, float* slot_grads, float* grads,
                              long long row_elems, hipStream_t st) {
  if (d.B == 0) return hipSuccess;
  const long long tiles = (row_elems + kRedTile - 1) / kRedTile;
  const long long items = (long long)d.pl.max_pieces * tiles;
  const int grid = (int)(items < kStreamGroups ? items : kStreamGroups);
  hipLaunchKernelGGL(k_reduce_grad, dim3(grid), dim3(kCopyThreads), 0, st, plan, d, slot_grads,
                     grads, row_elems, tiles);
  return hipGetLastError();
}

// ---- combine backward ---------------------------------------------------------
// One token per workgroup, 8 elements (16 bytes of bf16) per chunk, chunks
// c = base + threadIdx.x + i*THR.  For each of the token's pairs, in groups
// of G: the expert-output gradient row g * dy (fp32 product, bf16 nearest
// even) is written to the pair's row, and the gate gradient <dy, out row> is
// accumulated in fp64 per thread, reduced over the workgroup (waves in
// order) and rounded once to fp32.
template <int CH, int KT, bool DYB>
__global__ __launch_bounds__(1024) void k_combine_bwd(const u32x4* __restrict__ out,
                                                      const int32_t* __restrict__ slot,
                                                      const float* __restrict__ gates,
                                                      const void* __restrict__ dy,
                                                      u32x4* __restrict__ d_out,
                                                      float* __restrict__ d_gates, int Krt, int H8,
                                                      long long n_rows) {
  constexpr int G = KT > 0 ? KT : 8;
  __shared__ double red[1024 / kWave][G];
  const int K = KT > 0 ? KT : Krt;
  const int t = blockIdx.x;
  const int nthr = blockDim.x, nw = nthr / kWave;
  const int32_t* sl = slot + (long long)t * K;
  const float* gt = gates + (long long)t * K;
  for (int k0 = 0; k0 < K; k0 += G) {
    int s[G];
    float g[G];
    double part[G];
#pragma unroll
    for (int kk = 0; kk < G; ++kk) {
      const int k = k0 + kk;
      s[kk] = k < K ? sl[k] : -1;
      if (!(s[kk] >= 0 && (long long)s[kk] < n_rows)) s[kk] = -1;
      g[kk] = s[kk] >= 0 ? gt[k] : 0.f;
      part[kk] = 0.0;
    }
    for (int base = 0; base < H8; base += CH * nthr) {
#pragma unroll
      for (int i = 0; i < CH; ++i) {
        const int c = base + threadIdx.x + i * nthr;
        if (c >= H8) continue;
        float v[8];
        if constexpr (DYB) {
          const u32x4 w = reinterpret_cast<const u32x4*>(dy)[(long long)t * H8 + c];
          v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
          v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z); v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
        } else {
          const f32x4* p = reinterpret_cast<const f32x4*>(dy) + ((long long)t * H8 + c) * 2;
          const f32x4 a = p[0], b = p[1];
          v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
          v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
        }
        u32x4 o[G];
#pragma unroll
        for (int kk = 0; kk < G; ++kk)
          o[kk] = s[kk] >= 0 ? __builtin_nontemporal_load(out + (long long)s[kk] * H8 + c)
                             : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int kk = 0; kk < G; ++kk) {
          if (s[kk] < 0) continue;
          const u32x4 w = o[kk];
          const float ov[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                               bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
          double acc = part[kk];
#pragma unroll
          for (int q = 0; q < 8; ++q) acc = fma((double)v[q], (double)ov[q], acc);
          part[kk] = acc;
          u32x4 r;
          r.x = to_bf16(g[kk] * v[0]) | (to_bf16(g[kk] * v[1]) << 16);
          r.y = to_bf16(g[kk] * v[2]) | (to_bf16(g[kk] * v[3]) << 16);
          r.z = to_bf16(g[kk] * v[4]) | (to_bf16(g[kk] * v[5]) << 16);
          r.w = to_bf16(g[kk] * v[6]) | (to_bf16(g[kk] * v[7]) << 16);
          d_out[(long long)s[kk] * H8 + c] = r;
        }
      }
    }
    // workgroup sums of the fp64 partials, waves in order
#pragma unroll
    for (int kk = 0; kk < G; ++kk) {
      double x = part[kk];
      for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, kWave);
      if (lane_id() == 0) red[wave_id()][kk] = x;
    }
    __syncthreads();
    if (threadIdx.x < G && k0 + (int)threadIdx.x < K) {
      const int k = k0 + threadIdx.x;
      const int sk = sl[k];
      double x = 0.0;
      for (int w = 0; w < nw; ++w) x += red[w][threadIdx.x];
      d_gates[(long long)t * K + k] = (sk >= 0 && (long long)sk < n_rows) ? (float)x : 0.f;
    }
    __syncthreads();
  }
}

// Threads for one row of H8 chunks: CH chunks each, a multiple of 64, <= 1024.
static int bwd_threads(int H8, int CH) {
  int thr = (H8 + CH - 1) / CH;
  thr = ((thr + kWave - 1) / kWave) * kWave;
  return thr > 1024 ? 1024 : thr;
}

template <bool DYB, int KT>
static void launch_combine_bwd_t(const Dims& d, const u32x4* o, const int32_t* slot,
                                 const float* gates, const void* dy, u32x4* d_out, float* d_gates,
                                 hipStream_t st) {
  const int H8 = d.H / 8;
  hipLaunchKernelGGL((k_combine_bwd<2, KT, DYB>), dim3(d.N), dim3(bwd_threads(H8, 2)), 0, st, o,
                     slot, gates, dy, d_out, d_gates, d.K, H8, (long long)d.R * d.C);
}

template <bool DYB>
static void launch_combine_bwd_k(const Dims& d, const u32x4* o, const int32_t* slot,
                                 const float* gates, const void* dy, u32x4* d_out, float* d_gates,
                                 hipStream_t st) {
  switch (d.K) {
    case 2: launch_combine_bwd_t<DYB, 2>(d, o, slot, gates, dy, d_out, d_gates, st); break;
    case 4: launch_combine_bwd_t<DYB, 4>(d, o, slot, gates, dy, d_out, d_gates, st); break;
    case 8: launch_combine_bwd_t<DYB, 8>(d, o, slot, gates, dy, d_out, d_gates, st); break;
    default: launch_combine_bwd_t<DYB, 0>(d, o, slot, gates, dy, d_out, d_gates, st); break;
  }
}

hipError_t launch_combine_bwd(const Dims& d, const uint16_t* out, const int32_t* slot,
                              const float* gates, int dy_dtype, const void* dy, uint16_t* d_out,
                              float* d_gates, hipStream_t st) {
  if (d.N == 0) return hipSuccess;
  const u32x4* o = reinterpret_cast<const u32x4*>(out);
  u32x4* dout = reinterpret_cast<u32x4*>(d_out);
  if (dy_dtype == LBT_Y_BF16) launch_combine_bwd_k<true>(d, o, slot, gates, dy, dout, d_gates, st);
  else launch_combine_bwd_k<false>(d, o, slot, gates, dy, dout, d_gates, st);
  return hipGetLastError();
}

}  // namespace lbt
