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
// All three kernels are HBM-bound streams.  Prefetch and reduce_grad walk
// the replica-segment table (piece_*), whose weight-row column marks the
// slotted replicas, grouped by expert so that each home row is read once;
// every index taken from the plan is bounds-checked before it addresses
// memory.
#include "rows.h"

namespace lbt {

constexpr int kCopyThreads = 256;
constexpr int kCopyWaves = kCopyThreads / kWave;

// ---- the slotted replicas, grouped by expert --------------------------------
// Replica segments are in line order, and an expert's overflow is one
// interval of the line, so all segments of one expert are consecutive: a
// "run".  A segment is slotted when its weight row is E + j with j < B.  The
// first slotted segment of each run is its head; the workgroup of rank y
// handles the heads that lie on rank y.  Every index taken from the plan is
// checked before it addresses memory.
struct SlotRuns {
  int pe[kMaxPieces], pr[kMaxPieces], pw[kMaxPieces];
  int head[kMaxPieces];
  int wcnt[kCopyWaves];
};

__device__ __forceinline__ bool slotted(const SlotRuns& s, int p, const Dims& d) {
  const int w = s.pw[p], r = s.pr[p], e = s.pe[p];
  return w >= d.E && w < d.E + d.B && r >= 0 && r < d.R && e >= 0 && e < d.E;
}

// Load the segment table and list, in ascending segment order, the heads on
// rank y (the same list in every workgroup of rank y).  Returns the head
// count; *nP_out receives the number of segments.
__device__ __forceinline__ int slotted_heads(const int32_t* __restrict__ plan, const Dims& d, int y,
                                             SlotRuns& s, int* nP_out) {
  const PlanLayout& pl = d.pl;
  const int mp = pl.max_pieces;
  const int nP = min(max(plan[pl.hdr + LBT_HDR_N_PIECES], 0), mp);
  for (int g = threadIdx.x; g < mp; g += kCopyThreads) {   // every entry: no wait on nP
    s.pe[g] = plan[pl.piece_expert + g];
    s.pr[g] = plan[pl.piece_rank + g];
    s.pw[g] = plan[pl.piece_wrow + g];
  }
  __syncthreads();
  int n = 0;
  for (int g0 = 0; g0 < nP; g0 += kCopyThreads) {
    const int g = g0 + threadIdx.x;
    bool h = g < nP && s.pr[g] == y && slotted(s, g, d);
    if (h) {
      const int e = s.pe[g];
      for (int p = g - 1; p >= 0 && s.pe[p] == e; --p)
        if (slotted(s, p, d)) {
          h = false;
          break;
        }
    }
    const unsigned long long m = __ballot(h);
    if (lane_id() == 0) s.wcnt[wave_id()] = __popcll(m);
    __syncthreads();
    int before = n, total = 0;
#pragma unroll
    for (int w = 0; w < kCopyWaves; ++w) {
      before += w < wave_id() ? s.wcnt[w] : 0;
      total += s.wcnt[w];
    }
    if (h)
      s.head[before + __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u))] = g;
    n += total;
    __syncthreads();
  }
  *nP_out = nP;
  return n;
}

// ---- prefetch -----------------------------------------------------------------
// Grid (4 KiB tile of a weight row, rank y * subs + sub): the workgroup takes
// heads sub, sub + subs, ... of rank y; for each it reads the tile of the
// expert's home row once (16 bytes per thread) and stores it into every
// slotted segment of the run, so a home row replicated on several ranks is
// read once.  One 16-byte chunk per thread per head: short-lived waves with
// one load each are the fastest copy shape measured on MI355X.
constexpr int kPrefetchTile = kCopyThreads * 16;

__global__ __launch_bounds__(kCopyThreads) void k_prefetch(const int32_t* __restrict__ plan, Dims d,
                                                           int subs,
                                                           const char* __restrict__ weights,
                                                           char* __restrict__ slots,
                                                           long long row_bytes) {
  __shared__ SlotRuns s;
  const int y = blockIdx.y / subs, sub = blockIdx.y - y * subs;
  int nP;
  const int nh = slotted_heads(plan, d, y, s, &nP);
  const long long tile0 = (long long)blockIdx.x * kPrefetchTile;
  const uint32_t lo = threadIdx.x * 16u;
  if (tile0 + lo + 16 > row_bytes) return;
  for (int i = sub; i < nh; i += 2 * subs) {
    const int h0 = s.head[i];
    const int h1 = i + subs < nh ? s.head[i + subs] : -1;
    const u32x4 v0 = *at_bytes<u32x4>(weights + (long long)s.pe[h0] * row_bytes + tile0, lo);
    u32x4 v1 = {0u, 0u, 0u, 0u};
    if (h1 >= 0) v1 = *at_bytes<u32x4>(weights + (long long)s.pe[h1] * row_bytes + tile0, lo);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int h = u == 0 ? h0 : h1;
      if (h < 0) continue;
      const int e = s.pe[h];
      for (int p = h; p < nP && s.pe[p] == e; ++p) {
        if (!slotted(s, p, d)) continue;
        char* dst = slots + ((long long)s.pr[p] * d.B + (s.pw[p] - d.E)) * row_bytes + tile0;
        *at_bytes<u32x4>(dst, lo) = u == 0 ? v0 : v1;
      }
    }
  }
}

// Workgroups per (tile, rank).  More than one spreads a rank's heads over
// several workgroups, but every workgroup pays the segment-table prologue:
// measured on MI355X (DSV3, 38 slots) with 8 per rank, prefetch 565 us and
// reduce_grad 1886 us against about 400 and 1710 with one.
static int copy_subs(const Dims&) { return 1; }

hipError_t launch_prefetch(const Dims& d, const int32_t* plan, const void* weights, void* slots,
                           long long row_bytes, hipStream_t st) {
  if (d.B == 0 || d.R == 0) return hipSuccess;
  const long long tiles = (row_bytes + kPrefetchTile - 1) / kPrefetchTile;
  const int subs = copy_subs(d);
  if (tiles > 0x7FFFFFFFLL || (long long)d.R * subs > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_prefetch, dim3((unsigned)tiles, (unsigned)(d.R * subs)), dim3(kCopyThreads),
                     0, st, plan, d, subs, static_cast<const char*>(weights),
                     static_cast<char*>(slots), row_bytes);
  return hipGetLastError();
}

// ---- reduce_grad --------------------------------------------------------------
// Grid (tile of 1024 floats, rank y * subs + sub), heads taken as in the
// prefetch: for each expert run, the tile of the home gradient and of the
// run's slotted segments (up to kRedBatch at a time, all loads in flight)
// are loaded, added in line order (one fp32 addition each, so the result is
// the oracle's bit for bit), the slots cleared and the sum stored.
constexpr long long kRedTile = (long long)kCopyThreads * 4;   // floats
constexpr int kRedBatch = 4;

__global__ __launch_bounds__(kCopyThreads) void k_reduce_grad(const int32_t* __restrict__ plan,
                                                              Dims d, int subs,
                                                              float* __restrict__ slot_grads,
                                                              float* __restrict__ grads,
                                                              long long row_elems) {
  __shared__ SlotRuns s;
  const int y = blockIdx.y / subs, sub = blockIdx.y - y * subs;
  int nP;
  const int nh = slotted_heads(plan, d, y, s, &nP);
  const long long tile0 = (long long)blockIdx.x * kRedTile;
  const uint32_t lo = threadIdx.x * 16u;
  if (tile0 + threadIdx.x * 4 + 4 > row_elems) return;
  for (int i = sub; i < nh; i += subs) {
    const int h = s.head[i];
    const int e = s.pe[h];
    float* home = grads + (long long)e * row_elems + tile0;
    f32x4 acc = *at_bytes<f32x4>(home, lo);
    int p = h;
    while (p < nP && s.pe[p] == e) {
      float* sg[kRedBatch];
      int n = 0;
      for (; p < nP && s.pe[p] == e && n < kRedBatch; ++p)
        if (slotted(s, p, d))
          sg[n++] = slot_grads + ((long long)s.pr[p] * d.B + (s.pw[p] - d.E)) * row_elems + tile0;
      f32x4 v[kRedBatch];
#pragma unroll
      for (int u = 0; u < kRedBatch; ++u)
        if (u < n) v[u] = *at_bytes<f32x4>(sg[u], lo);
#pragma unroll
      for (int u = 0; u < kRedBatch; ++u)
        if (u < n) {
          acc += v[u];
          *at_bytes<f32x4>(sg[u], lo) = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
    *at_bytes<f32x4>(home, lo) = acc;
  }
}

hipError_t launch_reduce_grad(const Dims& d, const int32_t* plan, float* slot_grads, float* grads,
                              long long row_elems, hipStream_t st) {
  if (d.B == 0 || d.R == 0) return hipSuccess;
  const long long tiles = (row_elems + kRedTile - 1) / kRedTile;
  const int subs = copy_subs(d);
  if (tiles > 0x7FFFFFFFLL || (long long)d.R * subs > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_reduce_grad, dim3((unsigned)tiles, (unsigned)(d.R * subs)),
                     dim3(kCopyThreads), 0, st, plan, d, subs, slot_grads, grads, row_elems);
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
