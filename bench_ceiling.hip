// Reference HBM streams for bench.py --ceilings: what plain reads, writes
// and copies reach on this GPU, in the shapes measured fastest on MI355X
// (one 16-byte access per thread: reads in 1024-thread workgroups with
// non-temporal loads, writes and copies in 256-thread workgroups), plus
// the copy with non-temporal loads, the fastest copy shape measured.  The
// plain copy is also the known-size kernel the HBM traffic counters are
// calibrated on.  They
// bound the row-movement kernels: dispatch and prefetch are copies with
// fan-out, combine and reduce_grad mostly reads.  Measurement support for
// the benchmark, not part of the path.
#include <hip/hip_runtime.h>
#include <stdint.h>

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(1024) void k_read(const u32x4* __restrict__ p, long long n,
                                               u32x4* __restrict__ sink) {
  const long long i = (long long)blockIdx.x * 1024 + threadIdx.x;
  if (i >= n) return;
  const u32x4 v = __builtin_nontemporal_load(p + i);
  // a store no real data triggers keeps the load from being removed
  if (v.x == 0x9E3779B9u && v.y == 0x7F4A7C15u && v.z == 0xF39CC060u) sink[0] = v;
}

__global__ __launch_bounds__(256) void k_write(u32x4* __restrict__ p, long long n) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = u32x4{1u, 2u, 3u, 4u};
}

__global__ __launch_bounds__(256) void k_copy(const u32x4* __restrict__ s, u32x4* __restrict__ d,
                                              long long n) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i < n) d[i] = s[i];
}

__global__ __launch_bounds__(256) void k_copy_nt(const u32x4* __restrict__ s,
                                                 u32x4* __restrict__ d, long long n) {
  const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
  if (i < n) d[i] = __builtin_nontemporal_load(s + i);
}

// kind 0: read `bytes` at a (b: 16-byte sink); 1: write `bytes` at a;
// 2: copy `bytes` from a to b; 3: the same copy with non-temporal loads.
// bytes a multiple of 16, pointers 16-byte
// aligned.  0 on success, -1 for bad arguments, -2 for a failed launch.
extern "C" int hbm_stream(int kind, void* a, void* b, long long bytes, void* stream) {
  if (a == nullptr || bytes <= 0 || bytes % 16 != 0 || (kind != 1 && b == nullptr)) return -1;
  const long long n = bytes / 16;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  if (kind == 0) {
    hipLaunchKernelGGL(k_read, dim3((unsigned)((n + 1023) / 1024)), dim3(1024), 0, st,
                       static_cast<const u32x4*>(a), n, static_cast<u32x4*>(b));
  } else if (kind == 1) {
    hipLaunchKernelGGL(k_write, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                       static_cast<u32x4*>(a), n);
  } else if (kind == 2) {
    hipLaunchKernelGGL(k_copy, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                       static_cast<const u32x4*>(a), static_cast<u32x4*>(b), n);
  } else if (kind == 3) {
    hipLaunchKernelGGL(k_copy_nt, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st,
                       static_cast<const u32x4*>(a), static_cast<u32x4*>(b), n);
  } else {
    return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -2;
}
