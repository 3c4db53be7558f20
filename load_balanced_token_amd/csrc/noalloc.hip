// lbt_align_sort_noalloc: the block-aligned sort from expert ids and a plan,
// with its workspace (the per-sub-tile expert histogram, the per-tile
// prefix offsets and the load matrix) in a file-scope device array instead
// of a caller buffer.  For callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// allocation).  The same kernels as lbt_histogram followed by lbt_align_sort.
#include <mutex>

#include "lbt_internal.h"

namespace lbt {

// Words of the array: E * (R * ceil(S / 32) + R * ceil(S / 128)) + R * E must
// fit.  16 MiB holds the Kimi-K3 prefill shape (E = 384, R = 32, S = 8192:
// 3.95 M words).
constexpr long long kNoAllocWords = 4LL << 20;

// Each GPU the library runs on holds its own copy until the process ends.
static __device__ __align__(256) int32_t scratch[kNoAllocWords];

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static int32_t* g_scratch_ptr[kMaxDevices];   // the array's device address, per device

// Device address of the array on the current device, looked up once per
// device with that device current.  hipSuccess or the lookup's error.
static hipError_t scratch_of_current_device(int32_t** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = static_cast<int32_t*>(p);
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

long long noalloc_words(const Dims& d) {
  return (long long)d.E * (d.n_sub + d.n_tiles) + (long long)d.R * d.E;
}

hipError_t launch_align_noalloc(const Dims& d, const int32_t* ids, const int32_t* plan,
                                int32_t* slot, int32_t* sorted_ids, int32_t* block_wrow,
                                int32_t* block_expert, int32_t* status, hipStream_t st) {
  int32_t* work = nullptr;
  hipError_t e = scratch_of_current_device(&work);
  if (e != hipSuccess) return e;
  // every word the align step reads is written first: the histogram writes
  // every (expert, sub-tile) count, the scan every tile offset and count
  int32_t* counts = work + (long long)d.E * (d.n_sub + d.n_tiles);
  e = launch_histogram(d, ids, work, status, st);
  if (e == hipSuccess) e = launch_tile_scan(d, work, counts, st);
  if (e == hipSuccess)
    e = launch_align(d, ids, work, plan, slot, sorted_ids, block_wrow, block_expert, status, st);
  return e;
}

bool noalloc_fits(const Dims& d) { return noalloc_words(d) <= kNoAllocWords; }

}  // namespace lbt
