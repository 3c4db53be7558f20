// Host side of the C ABI in include/lbt.h: argument checks, derived sizes,
// the plan-blob layout and kernel launches.  Nothing here allocates memory
// or synchronises with the device.
#include <string.h>

#include "fused.h"
#include "lbt_internal.h"

namespace lbt {

static bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

int make_dims(const lbt_shape* s, Dims* d, lbt_sizes* z) {
  if (s == nullptr) return LBT_EINVAL;
  const long long E = s->E, K = s->K, R = s->R, S = s->S, H = s->H, B = s->B, blk = s->blk;
  if (E < 1 || R < 1 || K < 1 || S < 0 || H < 8 || B < 0 || blk < 1 || s->cap < 0)
    return LBT_EINVAL;
  if (E % R != 0 || K > E || H % 8 != 0) return LBT_EINVAL;
  if (s->score_fn != LBT_SOFTMAX && s->score_fn != LBT_SIGMOID) return LBT_EINVAL;
  if (s->renorm != 0 && s->renorm != 1) return LBT_EINVAL;
  if (E > kMaxE || R > kMaxR || K > kMaxK || blk > 1024) return LBT_EUNSUPPORTED;
  if (s->cap % blk != 0) return LBT_EINVAL;

  const long long nh = E / R, N = R * S, P = N * K, SK = S * K;
  if (s->tau_max != 0 && (s->tau_max < SK || s->tau_max >= (1 << 30))) return LBT_EINVAL;
  const long long tmax = s->tau_max != 0 ? s->tau_max : SK;
  long long C = s->cap;
  if (C == 0) {
    const long long need = tmax + (E < tmax ? E : tmax) * (blk - 1);
    C = (need + blk - 1) / blk * blk;
    if (C == 0) C = blk;
  }
  const long long tpr = (S + kTileTokens - 1) / kTileTokens;
  const long long nt = R * tpr;
  const long long spr = (S + kSubTokens - 1) / kSubTokens;
  if (P >= (1LL << 31) || R * C >= (1LL << 31) || N * H / 8 >= (1LL << 40)) return LBT_EUNSUPPORTED;
  if (SK >= (1LL << 30)) return LBT_EUNSUPPORTED;

  const long long ms = nh + ((E - nh) < tmax ? (E - nh) : tmax);

  const long long mp = E + R;
  PlanLayout pl;
  long long off = 0;
  auto take = [&](long long n) { const long long o = off; off += n; return (int)o; };
  pl.E = (int)E;
  pl.R = (int)R;
  pl.max_seg = (int)ms;
  pl.max_pieces = (int)mp;
  pl.hdr = take(LBT_HDR_WORDS);
  pl.T = take(E);
  pl.h = take(E);
  pl.O = take(E);
  pl.home_row = take(E);
  pl.L = take(R);
  pl.def = take(R);
  pl.D = take(R + 1);
  pl.n_seg = take(R);
  pl.n_rows_padded = take(R);
  pl.n_slots = take(R);
  pl.n_remote = take(R);
  pl.seg_expert = take(R * ms);
  pl.seg_wrow = take(R * ms);
  pl.seg_count = take(R * ms);
  pl.seg_start = take(R * (ms + 1));
  pl.piece_expert = take(mp);
  pl.piece_rank = take(mp);
  pl.piece_count = take(mp);
  pl.piece_line = take(mp);
  pl.piece_row = take(mp);
  pl.piece_wrow = take(mp);
  pl.home_local = take(E);
  pl.piece_local = take(mp);
  pl.total = (int)off;

  if (d != nullptr) {
    d->E = (int)E; d->K = (int)K; d->R = (int)R; d->S = (int)S; d->H = (int)H; d->B = (int)B;
    d->blk = (int)blk; d->score_fn = s->score_fn; d->renorm = s->renorm;
    d->nh = (int)nh;
    d->nh_magic = nh >= 2 ? (uint32_t)(((1ULL << 32) + nh - 1) / nh) : 0u;
    d->k_magic = K >= 2 ? (uint32_t)(((1ULL << 32) + K - 1) / K) : 0u;
    d->N = (int)N; d->P = P; d->SK = (int)SK; d->tau_max = (int)tmax; d->C = (int)C;
    d->n_blocks = (int)(C / blk); d->tpr = (int)tpr; d->n_tiles = (int)nt;
    d->spr = (int)spr; d->n_sub = (int)(R * spr); d->pl = pl;
  }
  if (z != nullptr) {
    memset(z, 0, sizeof(*z));
    z->N = N; z->P = P; z->SK = SK; z->C = C; z->n_blocks = C / blk;
    z->tile_tokens = kTileTokens; z->tiles_per_rank = tpr; z->n_tiles = nt;
    z->work_words = E * (R * spr + nt);
    z->max_seg = ms; z->max_pieces = mp; z->plan_words = off;
    z->off_hdr = pl.hdr; z->off_T = pl.T; z->off_h = pl.h; z->off_O = pl.O;
    z->off_home_row = pl.home_row; z->off_L = pl.L; z->off_def = pl.def; z->off_D = pl.D;
    z->off_n_seg = pl.n_seg; z->off_n_rows_padded = pl.n_rows_padded;
    z->off_n_slots = pl.n_slots; z->off_n_remote = pl.n_remote;
    z->off_seg_expert = pl.seg_expert; z->off_seg_wrow = pl.seg_wrow;
    z->off_seg_count = pl.seg_count; z->off_seg_start = pl.seg_start;
    z->off_piece_expert = pl.piece_expert; z->off_piece_rank = pl.piece_rank;
    z->off_piece_count = pl.piece_count; z->off_piece_line = pl.piece_line;
    z->off_piece_row = pl.piece_row;
    z->off_piece_wrow = pl.piece_wrow;
    z->off_home_local = pl.home_local;
    z->off_piece_local = pl.piece_local;
  }
  return LBT_OK;
}

// The HIP error behind this thread's most recent LBT_EHIP.
static thread_local hipError_t g_last_hip_error = hipSuccess;

static int hip_rc(hipError_t e) {
  if (e == hipSuccess) return LBT_OK;
  g_last_hip_error = e;
  return LBT_EHIP;
}

// Clear the calling thread's HIP last-error state before a call's first
// launch, so that the launchers' hipGetLastError() checks see only errors
// raised by this call's own launches, never one left by an earlier HIP call
// of the application.
static hipStream_t begin_launches(void* stream) {
  (void)hipGetLastError();
  return static_cast<hipStream_t>(stream);
}

}  // namespace lbt

using namespace lbt;

extern "C" {

int lbt_version(void) { return LBT_VERSION; }

const char* lbt_last_hip_error(void) { return hipGetErrorName(g_last_hip_error); }

const char* lbt_strerror(int code) {
  switch (code) {
    case LBT_OK: return "ok";
    case LBT_EINVAL: return "invalid argument (dimension, null or misaligned pointer)";
    case LBT_EHIP: return "HIP kernel launch failed";
    case LBT_EUNSUPPORTED: return "shape outside the supported limits";
    default: return "unknown error";
  }
}

int lbt_query_sizes(const lbt_shape* s, lbt_sizes* out) {
  if (out == nullptr) return LBT_EINVAL;
  return make_dims(s, nullptr, out);
}

int lbt_route_topk(const lbt_shape* s, const float* logits, const float* sel_bias, int32_t* ids,
                   float* gates, int32_t* counts, int32_t* work, void* stream) {
  Dims d;
  const int rc = make_dims(s, &d, nullptr);
  if (rc) return rc;
  if (counts == nullptr || (d.N > 0 && (!logits || !ids || !gates || !work))) return LBT_EINVAL;
  const hipStream_t st = begin_launches(stream);
  return hip_rc(launch_route_and_scan(d, logits, sel_bias, ids, gates, work, counts, st));
}

int lbt_histogram(const lbt_shape* s, const int32_t* ids, int32_t* counts, int32_t* work,
                  int32_t* status, void* stream) {
  Dims d;
  const int rc = make_dims(s, &d, nullptr);
  if (rc) return rc;
  if (counts == nullptr || (d.N > 0 && (!ids || !work))) return LBT_EINVAL;
  const hipStream_t st = begin_launches(stream);
  hipError_t e = launch_histogram(d, ids, work, status, st);
  if (e == hipSuccess) e = launch_tile_scan(d, work, counts, st);
  return hip_rc(e);
}

int lbt_plan_balance(const lbt_shape* s, const int32_t* counts, int32_t* plan, int32_t* status,
                     void* stream) {
  Dims d;
  const int rc = make_dims(s, &d, nullptr);
  if (rc) return rc;
  if (!counts || !plan) return LBT_EINVAL;
  return hip_rc(launch_plan(d, counts, plan, status, begin_launches(stream)));
}

int lbt_plan_quota(const lbt_shape* s, const int32_t* counts, int32_t* plan, int32_t* status,
                   void* stream) {
  Dims d;
  const int rc = make_dims(s, &d, nullptr);
  if (rc) return rc;
  if (!counts || !plan) return LBT_EINVAL;
  return hip_rc(launch_plan_quota(d, counts, plan, status, begin_launches(stream)));
}

int lbt_route_plan(const lbt_shape* s, const float* logits, const float* sel_bias, int32_t* ids,
                   float* gates, int32_t* counts, int32_t* work, int32_t* plan, int32_t* status,
                   void* stream) {
  Dims d;
  const int rc = make_dims(s, &d, nullptr);
  if (rc) return rc;
  if (counts == nullptr || plan == nullptr ||
      (d.N > 0 && (!logits || !ids || !gates || !work)))
    return LBT_EINVAL;
  const hipStream_t st = begin_launches(stream);
  return hip_rc(launch_route_plan(d, logits, sel_bias, ids, gates, work, counts, plan, status, st));
}

int lbt_front(const lbt_shape* s, const float* logits, const float* sel_bias, int32_t* ids,
              float* gates, int32_t* counts, int32_t* work, int32_t* plan, int32_t* slot,
              int32_t* sorted_ids, int32_t* block_wrow, int32_t* block_expert, int32_t* status,
              void* stream) {
  Dims d;
  const int rc = make_dims(s, &d, nullptr);
  if (rc) return rc;
  if (counts == nullptr || plan == nullptr || !sorted_ids || !block_wrow || !block_expert ||
      (d.N > 0 && (!logits || !ids || !gates || !work || !slot)))
    return LBT_EINVAL;
  const hipStream_t st = begin_launches(stream);
  return hip_rc(launch_front(d, logits, sel_bias, ids, gates, work, counts, plan, slot,
                             sorted_ids, block_wrow, block_expert, status, st));
}

int lbt_align_sort(const lbt_shape* s, const int32_t* ids, const int32_t* work, const int32_t* plan,
                   int32_t* slot, int32_t* sorted_ids, int32_t* block_wrow, int32_t* block_expert,
                   int32_t* status, void* stream) {
  Dims d;
  const int rc = make_dims(s, &d, nullptr);
  if (rc) return rc;
  if (!plan || !sorted_ids || !block_wrow || !block_expert) return LBT_EINVAL;
  if (d.N > 0 && (!ids || !work || !slot)) return LBT_EINVAL;
  return hip_rc(launch_align(d, ids, work, plan, slot, sorted_ids, block_wrow, block_expert, status,
                             begin_launches(stream)));
}

int lbt_align_dispatch(const lbt_shape* s, const int32_t* ids, const int32_t* work,
                       const int32_t* plan, const uint16_t* x, int32_t* slot, int32_t* sorted_ids,
                       int32_t* block_wrow, int32_t* block_expert, uint16_t* recv,
                       int32_t* status, void* stream) {
  Dims d;
  const int rc = make_dims(s, &d, nullptr);
  if (rc) return rc;
  if (!plan || !sorted_ids || !block_wrow || !block_expert) return LBT_EINVAL;
  if (d.N > 0 && (!ids || !work || !slot || !x || !recv || !aligned16(x) || !aligned16(recv)))
    return LBT_EINVAL;
  return hip_rc(launch_align_dispatch(d, ids, work, plan, x, slot, sorted_ids, block_wrow,
                                      block_expert, recv, status, begin_launches(stream)));
}

int lbt_front_dispatch(const lbt_shape* s, const float* logits, const float* sel_bias,
                       int32_t* ids, float* gates, int32_t* counts, int32_t* work, int32_t* plan,
                       int32_t* slot, int32_t* sorted_ids, int32_t* block_wrow,
                       int32_t* block_expert, const uint16_t* x, uint16_t* recv,
                       int32_t* status, void* stream) {
  Dims d;
  const int rc = make_dims(s, &d, nullptr);
  if (rc) return rc;
  if (counts == nullptr || plan == nullptr || !sorted_ids || !block_wrow || !block_expert ||
      (d.N > 0 && (!logits || !ids || !gates || !work || !slot || !x || !recv ||
                   !aligned16(x) || !aligned16(recv))))
    return LBT_EINVAL;
  return hip_rc(launch_front_dispatch(d, logits, sel_bias, ids, gates, work, counts, plan, slot,
                                      sorted_ids, block_wrow, block_expert, x, recv, status,
                                      begin_launches(stream)));
}

int lbt_align_sort_noalloc(const lbt_shape* s, const int32_t* ids, const int32_t* plan,
                           int32_t* slot, int32_t* sorted_ids, int32_t* block_wrow,
                           int32_t* block_expert, int32_t* status, void* stream) {
  Dims d;
  const int rc = make_dims(s, &d, nullptr);
  if (rc) return rc;
  if (!plan || !sorted_ids || !block_wrow || !block_expert) return LBT_EINVAL;
  if (d.N > 0 && (!ids || !slot)) return LBT_EINVAL;
  if (!noalloc_fits(d)) return LBT_EUNSUPPORTED;
  return hip_rc(launch_align_noalloc(d, ids, plan, slot, sorted_ids, block_wrow, block_expert,
                                     status, begin_launches(stream)));
}

int lbt_dispatch(const lbt_shape* s, const uint16_t* x, const int32_t* slot, uint16_t* recv,
                 void* stream) {
  Dims d;
  const int rc = make_dims(s, &d, nullptr);
  if (rc) return rc;
  if (d.N > 0 && (!x || !slot || !recv || !aligned16(x) || !aligned16(recv))) return LBT_EINVAL;
  return hip_rc(launch_dispatch(d, x, slot, recv, begin_launches(stream)));
}

int lbt_combine(const lbt_shape* s, const uint16_t* out, const int32_t* slot, const float* gates,
                int32_t y_dtype, void* y, void* stream) {
  Dims d;
  const int rc = make_dims(s, &d, nullptr);
  if (rc) return rc;
  if (y_dtype != LBT_Y_F32 && y_dtype != LBT_Y_BF16) return LBT_EINVAL;
  if (d.N > 0 && (!out || !slot || !gates || !y || !aligned16(out) || !aligned16(y)))
    return LBT_EINVAL;
  return hip_rc(launch_combine(d, out, slot, gates, y_dtype, y, begin_launches(stream)));
}

int lbt_prefetch_weights(const lbt_shape* s, const int32_t* plan, const void* weights, void* slots,
                         int64_t row_bytes, void* stream) {
  Dims d;
  const int rc = make_dims(s, &d, nullptr);
  if (rc) return rc;
  if (!plan || row_bytes <= 0 || row_bytes % 16 != 0) return LBT_EINVAL;
  if (d.B > 0 && (!weights || !slots || !aligned16(weights) || !aligned16(slots))) return LBT_EINVAL;
  return hip_rc(launch_prefetch(d, plan, weights, slots, row_bytes, begin_launches(stream)));
}

int lbt_reduce_grad(const lbt_shape* s, const int32_t* plan, float* slot_grads, float* grads,
                    int64_t row_elems, void* stream) {
  Dims d;
  const int rc = make_dims(s, &d, nullptr);
  if (rc) return rc;
  if (!plan || row_elems <= 0 || row_elems % 4 != 0) return LBT_EINVAL;
  if (d.B > 0 && (!slot_grads || !grads || !aligned16(slot_grads) || !aligned16(grads)))
    return LBT_EINVAL;
  return hip_rc(launch_reduce_grad(d, plan, slot_grads, grads, row_elems,
                                   begin_launches(stream)));
}

int lbt_combine_bwd(const lbt_shape* s, const uint16_t* out, const int32_t* slot,
                    const float* gates, int32_t dy_dtype, const void* dy, uint16_t* d_out,
                    float* d_gates, void* stream) {
  Dims d;
  const int rc = make_dims(s, &d, nullptr);
  if (rc) return rc;
  if (dy_dtype != LBT_Y_F32 && dy_dtype != LBT_Y_BF16) return LBT_EINVAL;
  if (d.N > 0 && (!out || !slot || !gates || !dy || !d_out || !d_gates || !aligned16(out) ||
                  !aligned16(dy) || !aligned16(d_out)))
    return LBT_EINVAL;
  return hip_rc(launch_combine_bwd(d, out, slot, gates, dy_dtype, dy, d_out, d_gates,
                                   begin_launches(stream)));
}

int lbt_dispatch_bwd(const lbt_shape* s, const uint16_t* d_recv, const int32_t* slot,
                     int32_t dx_dtype, void* dx, void* stream) {
  Dims d;
  const int rc = make_dims(s, &d, nullptr);
  if (rc) return rc;
  if (dx_dtype != LBT_Y_F32 && dx_dtype != LBT_Y_BF16) return LBT_EINVAL;
  if (d.N > 0 && (!d_recv || !slot || !dx || !aligned16(d_recv) || !aligned16(dx)))
    return LBT_EINVAL;
  return hip_rc(launch_combine(d, d_recv, slot, nullptr, dx_dtype, dx,
                               begin_launches(stream)));
}

}  // extern "C"
