/*
 * lbt.h -- C ABI of the load-balanced MoE token path on one MI355X (gfx950).
 *
 * The path: router top-K -> per-expert token histogram -> online
 * redundant-expert balancing plan giving every (virtual) rank exactly S*K
 * token slots -> block-aligned sort (MoE Align & Sort) -> zero-copy dispatch
 * into static per-rank buffers -> inverse combine.  All R expert-parallel
 * ranks are logical partitions of one device buffer.
 *
 * Sources (page title, then section):
 *   [MoonEP-GR] TWO DOTS, "MoonEP: πώς η εξισορρόπηση των AI experts αλλάζει
 *               την υποδομή των MoE μοντέλων"
 *   [MoonEP-FR] hamidun.com, "Moonshot AI открыла код MoonEP ..."
 *   [UltraEP]   remio.ai, "Xiaohongshuと北京大学がUltraEPを発表、静的MoE負荷分散に挑戦"
 *   [AlignSort] 新智元 article on SGLang's MoE Align & Sort kernel
 *
 * Conventions shared by every call
 *   - Every data pointer is a DEVICE pointer owned by the caller; the
 *     library allocates nothing and keeps no state between calls.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the
 *     default stream) and never synchronises the host.
 *   - Arguments are checked on the host: a call returns LBT_OK (0) or a
 *     negative LBT_E* code and then launches nothing.  LBT_EHIP reports a
 *     failed launch of this call: the calling thread's HIP last-error state
 *     is cleared before the call's first launch, so an error left by an
 *     earlier HIP call is never reported as this call's; kernels the call
 *     queued before the failing launch stay queued, later ones are not
 *     launched.  Data-dependent problems (inconsistent counts, an id
 *     out of range, a rank needing more rows than the capacity) are reported
 *     through the device status word (LBT_ST_* bits) that plan_balance
 *     writes and align_sort / histogram OR into; the caller reads it when it
 *     wants to.
 *   - Sizes of every buffer come from lbt_query_sizes().
 *   - Integer outputs are bit-for-bit deterministic (no order-dependent
 *     atomics feed them).
 *
 * Notation: N = R*S tokens, P = N*K (token, expert) pairs, flat pair index
 * f = t*K + k, SK = S*K slots per rank, E/R home experts per rank (rank r
 * owns experts [r*E/R, (r+1)*E/R)), token t comes from source rank t / S,
 * C = static rows per rank of the receive buffer.
 */
#ifndef LBT_H
#define LBT_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LBT_VERSION 4

/* return codes */
#define LBT_OK 0
#define LBT_EINVAL (-1)      /* bad dimension, null or misaligned pointer */
#define LBT_EHIP (-2)        /* a kernel launch failed */
#define LBT_EUNSUPPORTED (-3)/* shape outside the supported limits below */

/* device status bits */
#define LBT_ST_BADCOUNT 1    /* the load matrix does not sum to R*S*K */
#define LBT_ST_CAPACITY 2    /* a rank needs more than C rows; pairs that do not fit get slot -1 */
#define LBT_ST_BADID 4       /* an expert id outside [0, E) was skipped */
#define LBT_ST_DUPID 8       /* a token names the same expert twice */

/* gate score function */
#define LBT_SOFTMAX 0
#define LBT_SIGMOID 1

/* combine output type */
#define LBT_Y_F32 0
#define LBT_Y_BF16 1

/* Supported limits: 1 <= R <= E <= 512, E % R == 0, 1 <= K <= min(E, 64),
 * S >= 0, H >= 8 with H % 8 == 0, B >= 0, 1 <= blk <= 1024, cap % blk == 0,
 * tau_max == 0 or S*K <= tau_max < 2^30, R*C and P below 2^31. */
typedef struct lbt_shape {
  int32_t E;        /* routed experts */
  int32_t K;        /* experts per token */
  int32_t R;        /* expert-parallel ranks (logical partitions) */
  int32_t S;        /* tokens per rank */
  int32_t H;        /* hidden size (bf16 elements per row) */
  int32_t B;        /* prefetch slots per rank (weight rows E..E+B-1) */
  int32_t blk;      /* alignment block of the grouped GEMM */
  int32_t score_fn; /* LBT_SOFTMAX or LBT_SIGMOID */
  int32_t renorm;   /* 1: gates renormalised over the K chosen */
  int32_t cap;      /* rows per rank of recv; 0 = worst case (always enough) */
  int32_t tau_max;  /* largest per-rank load a plan may give a rank; 0 = S*K
                       (exact balance).  Sizes C and bounds lbt_plan_quota's
                       threshold search; lbt_plan_balance always uses S*K. */
} lbt_shape;

/* Sizes (elements unless stated) and plan-blob word offsets. */
typedef struct lbt_sizes {
  int64_t N, P, SK;
  int64_t C;              /* rows per rank of recv / out */
  int64_t n_blocks;       /* C / blk blocks per rank */
  int64_t tile_tokens;    /* tokens per align tile (tiles never cross ranks) */
  int64_t tiles_per_rank; /* ceil(S / tile_tokens) */
  int64_t n_tiles;        /* R * tiles_per_rank */
  int64_t work_words;     /* int32 words of the route/histogram workspace */
  int64_t max_seg;        /* segment-table entries per rank: E/R + min(E - E/R, tau_max) */
  int64_t max_pieces;     /* replica-segment table entries: E + R */
  int64_t plan_words;     /* int32 words of the plan blob */
  /* plan blob layout: word offsets of each int32 field */
  int64_t off_hdr;        /* [16] see LBT_HDR_* */
  int64_t off_T;          /* [E]  T_e = pairs routed to expert e */
  int64_t off_h;          /* [E]  pairs of e kept on its home rank */
  int64_t off_O;          /* [E]  start of e's overflow o_e = T_e - h_e on the line */
  int64_t off_home_row;   /* [E]  padded start row of e's home segment */
  int64_t off_L;          /* [R]  L_r = load of rank r's home experts */
  int64_t off_def;        /* [R]  def_r = tau - min(L_r, tau), tau = LBT_HDR_TAU */
  int64_t off_D;          /* [R+1] exclusive prefix of def_r (D[R] = total) */
  int64_t off_n_seg;      /* [R]  used segment-table entries: E/R + replicas */
  int64_t off_n_rows_padded; /* [R] padded rows used by rank r (<= C) */
  int64_t off_n_slots;    /* [R]  replicas held in prefetch slots (<= B) */
  int64_t off_n_remote;   /* [R]  replicas read from their home rank */
  int64_t off_seg_expert; /* [R][max_seg] logical expert, -1 when unused */
  int64_t off_seg_wrow;   /* [R][max_seg] weight row ([E+B] pool), -1 when unused */
  int64_t off_seg_count;  /* [R][max_seg] real rows, 0 when unused */
  int64_t off_seg_start;  /* [R][max_seg+1] padded starts = cu_seqlens; unused
                             entries and entry max_seg hold n_rows_padded[r] */
  int64_t off_piece_expert; /* [max_pieces] replica segments in line order */
  int64_t off_piece_rank;   /*   destination rank d */
  int64_t off_piece_count;  /*   pairs */
  int64_t off_piece_line;   /*   start on the shared overflow/deficit line */
  int64_t off_piece_row;    /*   padded start row on rank d */
  int64_t off_piece_wrow;   /*   weight row: E + j for prefetch slot j, else the expert (remote) */
  int64_t off_home_local;   /* [E] of e's home quota h_e, the pairs whose token comes from e's
                               home rank (quota plans; 0 under lbt_plan_balance) */
  int64_t off_piece_local;  /* [max_pieces] of each replica segment's count, the pairs whose
                               token comes from its rank d (quota plans; 0 otherwise) */
} lbt_sizes;

/* plan header words */
#define LBT_HDR_N_PIECES 0
#define LBT_HDR_MAX_T 1       /* max_e T_e  (max_vio = MAX_T*E/P - 1) */
#define LBT_HDR_MAX_L 2       /* max_r L_r  (rank imbalance = MAX_L/SK - 1) */
#define LBT_HDR_TOTAL_OVERFLOW 3
#define LBT_HDR_N_DEFICIT_RANKS 4
#define LBT_HDR_N_OVERFLOW_RANKS 5
#define LBT_HDR_N_OVERFLOW_EXPERTS 6
#define LBT_HDR_STATUS 7      /* LBT_ST_* bits raised by the plan */
#define LBT_HDR_P 8           /* sum of the load matrix */
#define LBT_HDR_TAU 9         /* per-rank load threshold the plan used (S*K for plan_balance) */
#define LBT_HDR_MAX_REPLICAS 10 /* most replica segments on one rank */
#define LBT_HDR_FEASIBLE 11   /* 1 when no rank holds more than B replicas (no remote reads) */
#define LBT_HDR_LOCAL 12      /* 1: align places pairs with the locality step (lbt_plan_quota) */
#define LBT_HDR_WORDS 16

/* Fill *out for shape *s.  Pure host function.  LBT_EINVAL/LBT_EUNSUPPORTED
 * when the shape is outside the limits above. */
int lbt_query_sizes(const lbt_shape* s, lbt_sizes* out);

/* Router top-K and the expert histogram of every 32-token sub-tile (one
 * launch), then the per-rank load matrix and per-tile prefix offsets (a
 * second launch; batches of at most 32 tokens do both in one).
 * [AlignSort] (the MoE layer gates each token to its Top-K experts by gate
 * score, DeepSeek's gating bias steering the choice); [UltraEP] section
 * "その仕組みは高速なエキスパート複製に依存する" (the exact post-routing load
 * matrix, per source rank and logical expert).
 *   logits   [N, E] fp32 row-major, finite (no NaN)
 *   sel_bias [E] fp32 or NULL; the key is the fp32 sum logits + sel_bias
 *   ids      [N, K] int32 out: the K largest keys, descending, ties to the
 *            lower expert index (-0.0 ties +0.0)
 *   gates    [N, K] fp32 out: sigmoid(logit) or softmax over the E raw
 *            logits (the bias only steers selection), evaluated in fp64 and
 *            rounded once; optionally renormalised over the K chosen
 *   counts   [R, E] int32 out: the load matrix
 *   work     [work_words] int32 scratch the align step reads back; keep it
 *            alive and unmodified until lbt_align_sort has run */
int lbt_route_topk(const lbt_shape* s, const float* logits, const float* sel_bias,
                   int32_t* ids, float* gates, int32_t* counts, int32_t* work, void* stream);

/* The histogram step alone, for expert ids the caller already has (each
 * token's K ids distinct, in [0, E)).  Same outputs as lbt_route_topk's
 * counts/work.  Ids out of range are skipped and raise LBT_ST_BADID in
 * *status when status is not NULL. */
int lbt_histogram(const lbt_shape* s, const int32_t* ids, int32_t* counts, int32_t* work,
                  int32_t* status, void* stream);

/* Balancing plan from the load matrix; one workgroup, no host round trip.
 * [MoonEP-GR] sections "Η βασική υπόσχεση του MoonEP: σταθερό φορτίο S × K"
 * and "Το memory contract ..."; [UltraEP] "その仕組みは...".  Rule: rank r
 * keeps min(L_r, S*K) pairs -- the first ones of its home stream (experts
 * ascending, pairs by ascending f); overflow segments (experts ascending)
 * fill deficit ranks in ascending order; every non-empty overlap is one
 * replica segment; on its rank the first B replica segments take prefetch
 * slots (weight rows E..E+B-1), later ones are remote (weight row = expert,
 * read from home).  Segment table of rank r: its E/R home experts, then its
 * replicas in line order; counts padded to blk; starts = cu_seqlens.
 *   counts [R, E] int32 in
 *   plan   [plan_words] int32 out, layout in lbt_sizes (every word written)
 *   status int32 out (may be NULL): set to the plan's LBT_ST_* bits */
int lbt_plan_balance(const lbt_shape* s, const int32_t* counts, int32_t* plan, int32_t* status,
                     void* stream);

/* Route, histogram and fixed-rule plan in one call: the outputs of
 * lbt_route_topk (ids, gates, counts, work) followed by lbt_plan_balance
 * (plan, status), bit for bit.  [MoonEP-GR] section "Online planning, zero
 * copy και στατικά σχήματα" (the plan is made online from the current router
 * output, on the GPU, with no host round trip).  Batches of at most 32
 * tokens (with R * ceil(S / 32) * E <= 16384) run as one workgroup that
 * keeps the load matrix in LDS and plans from it -- one launch where the
 * two calls make two.  Larger batches whose sub-tile histograms fit in
 * 8192 words (R * ceil(S / 32) * E <= 8192) route, then run the column scan
 * and the plan as one launch; others make the same launches as the two
 * calls.  Arguments as for the two calls; plan [plan_words] int32 out,
 * status int32 out (may be NULL). */
int lbt_route_plan(const lbt_shape* s, const float* logits, const float* sel_bias, int32_t* ids,
                   float* gates, int32_t* counts, int32_t* work, int32_t* plan, int32_t* status,
                   void* stream);

/* The front of the step in one call: route, histogram, fixed-rule plan and
 * block-aligned sort -- the outputs of lbt_route_topk, lbt_plan_balance and
 * lbt_align_sort, bit for bit (status: the plan's bits ORed with the align
 * step's).  Batches of at most 32 tokens (with R * ceil(S / 32) * E <=
 * 16384 and R * C / blk <= 2048) run as one workgroup that keeps the
 * routing, the load matrix and the plan in LDS and places every pair from
 * them -- one launch where the three calls make three.  Batches past 32
 * tokens with R * ceil(S / 32) * E <= 8192 make three launches (route;
 * column scan and plan; align); others make the same launches as the three
 * calls.  [MoonEP-GR] section "Online planning, zero copy και στατικά
 * σχήματα"; [AlignSort]; [UltraEP] section "その仕組みは...".  Arguments as
 * for the three calls. */
int lbt_front(const lbt_shape* s, const float* logits, const float* sel_bias, int32_t* ids,
              float* gates, int32_t* counts, int32_t* work, int32_t* plan, int32_t* slot,
              int32_t* sorted_ids, int32_t* block_wrow, int32_t* block_expert, int32_t* status,
              void* stream);

/* Quota plan with a searched threshold: same blob layout and meaning as
 * lbt_plan_balance, so lbt_align_sort, lbt_dispatch and lbt_combine take it
 * unchanged.  [UltraEP] section "その仕組みは高速なエキスパート複製に依存する"
 * (from the exact load matrix, search a workload threshold that keeps every
 * rank under it within the replica slots; a quota-driven planner decides
 * which hot experts get copies, where, and how many tokens each instance
 * takes; replicas only where there is work; fully on the GPU).  Rule at
 * threshold tau: an overloaded rank keeps tau pairs and sheds the rest from
 * its hottest experts first (load descending, ties to the lower index); the
 * overflow line lists experts rank by
 * rank in that order; deficit ranks (def_r = tau - min(L_r, tau)) fill in
 * ascending order, one replica segment per overlap.  tau is the smallest
 * integer in [S*K, min(max_r L_r, tau_max)] for which no rank holds more than
 * B replica segments (candidates checked in ascending batches of 1024 in
 * parallel, stopping at the first batch holding one); when none qualifies,
 * tau = tau_max and replicas beyond B are remote (LBT_HDR_FEASIBLE = 0).
 * Every rank then holds at most tau pairs.  Locality (same section: tokens
 * use local instances' capacity before the rest of the demand goes
 * elsewhere): the blob sets LBT_HDR_LOCAL and records, per instance, how
 * many of its quota come from its own rank (home_local, piece_local), and
 * lbt_align_sort places pairs accordingly.  One workgroup, one launch.
 *   counts [R, E] int32 in
 *   plan   [plan_words] int32 out (LBT_HDR_TAU holds the threshold)
 *   status int32 out (may be NULL) */
int lbt_plan_quota(const lbt_shape* s, const int32_t* counts, int32_t* plan, int32_t* status,
                   void* stream);

/* Block-aligned sort: destination row of every pair.  [AlignSort] (pairs
 * sorted by expert, each expert's share padded to the GEMM block; the
 * permutation records source -> destination); [UltraEP] (per-token
 * destinations by lookup against cumulative quotas).  For pair f with
 * expert e and q = #{f' < f : ids[f'] = e}: q < h_e -> home rank of e, row
 * home_row[e] + q; else o = O_e + q - h_e lies in one replica segment
 * (d, line, row) -> rank d, row + o - line.  With LBT_HDR_LOCAL set (quota
 * plans) the instances of e -- its home, then its replica segments in line
 * order -- first take, up to their quota, the earliest pairs of e whose
 * token comes from their own rank; the other pairs, by ascending f, fill the
 * remaining quotas in instance order; a segment lists its local pairs
 * first, then the others, each by ascending f.
 *   ids        [N, K] int32 in (the ids the histogram counted)
 *   work       the workspace filled by lbt_route_topk / lbt_histogram
 *   plan       the blob from lbt_plan_balance or lbt_plan_quota
 *   slot       [P] int32 out: d*C + row, or -1 if it did not fit the capacity
 *   sorted_ids [R*C] int32 out: row -> f; padding rows below a rank's
 *              n_rows_padded hold P; rows at or past it are not written
 *   block_wrow, block_expert [R, C/blk] int32 out: weight row / expert of
 *              the segment covering each block, -1 past n_rows_padded
 *   status     int32 in/out (may be NULL): LBT_ST_* bits ORed in */
int lbt_align_sort(const lbt_shape* s, const int32_t* ids, const int32_t* work,
                   const int32_t* plan, int32_t* slot, int32_t* sorted_ids,
                   int32_t* block_wrow, int32_t* block_expert, int32_t* status, void* stream);

/* lbt_histogram followed by lbt_align_sort without a workspace argument,
 * for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation).  The
 * workspace -- per-sub-tile expert counts, per-tile prefix offsets and the
 * load matrix -- lives in a static device array of 16 MiB that each GPU the
 * library runs on holds until the process ends; the call allocates nothing
 * and writes every word of it that it reads.  Shapes needing more than
 * 4 Mi words, E * (R * ceil(S/32) + R * ceil(S/128)) + R * E, return
 * LBT_EUNSUPPORTED (the Kimi-K3 prefill shape needs 3.95 Mi).  Every call on
 * one GPU shares that GPU's array: calls that overlap on one GPU (on
 * different streams, or from different threads) race and must be ordered
 * by the caller.  Arguments and outputs as for lbt_align_sort (ids as for
 * lbt_histogram: out-of-range ids raise LBT_ST_BADID in *status). */
int lbt_align_sort_noalloc(const lbt_shape* s, const int32_t* ids, const int32_t* plan,
                           int32_t* slot, int32_t* sorted_ids, int32_t* block_wrow,
                           int32_t* block_expert, int32_t* status, void* stream);

/* Zero-copy dispatch: recv[slot[f]] = x[f / K], a bit copy of each bf16
 * row, straight into its final expert-grouped row of the static per-rank
 * buffer ([MoonEP-GR] "Online planning, zero copy και στατικά σχήματα").
 * Padding rows and rows past n_rows_padded are not touched.  Views into
 * recv stay valid until the next dispatch into the same buffer.
 *   x    [N, H] bf16 bits, 16-byte aligned
 *   slot [P] int32 (entries < 0 skipped)
 *   recv [R*C, H] bf16 bits, 16-byte aligned */
int lbt_dispatch(const lbt_shape* s, const uint16_t* x, const int32_t* slot, uint16_t* recv,
                 void* stream);

/* lbt_align_sort followed by lbt_dispatch in one call: every output of the
 * two (slot, sorted_ids, block tables, status, recv rows) bit for bit.
 * [AlignSort] (a pair's target row is its expert-grouped, block-padded
 * position); [MoonEP-GR] "Online planning, zero copy και στατικά σχήματα"
 * (each row written once, straight into its final row).  Batches of 1 to
 * 1024 tokens run as one launch: one workgroup per token places that
 * token's K pairs, repeating its 128-token tile's prefix work, and copies
 * the token's row to their rows; larger batches make the launches of the
 * two calls.  Any plan (either planner, with or without the locality
 * step).  Arguments as for the two calls; x [N, H] and recv [R*C, H] bf16
 * bits, 16-byte aligned. */
int lbt_align_dispatch(const lbt_shape* s, const int32_t* ids, const int32_t* work,
                       const int32_t* plan, const uint16_t* x, int32_t* slot, int32_t* sorted_ids,
                       int32_t* block_wrow, int32_t* block_expert, uint16_t* recv,
                       int32_t* status, void* stream);

/* lbt_front followed by lbt_dispatch in one call (the fixed-rule front of
 * the step and the zero-copy dispatch): the outputs of the two, bit for
 * bit.  Batches of at most 16 tokens that lbt_front runs as one workgroup
 * make one launch (one workgroup per token, each computing the whole front;
 * the first writes its outputs, each copies its token's row); up to 32
 * tokens, the front's launch and the dispatch; batches past 32 tokens with R * ceil(S / 32) * E <= 8192 make
 * three launches (route; column scan and plan; align and dispatch); other
 * batches make the launches of the separate calls, with align and dispatch
 * as in lbt_align_dispatch.  [MoonEP-GR] "Online planning, zero copy και
 * στατικά σχήματα"; [AlignSort]; [UltraEP] "その仕組みは...".  Arguments as
 * for lbt_front and lbt_dispatch. */
int lbt_front_dispatch(const lbt_shape* s, const float* logits, const float* sel_bias,
                       int32_t* ids, float* gates, int32_t* counts, int32_t* work, int32_t* plan,
                       int32_t* slot, int32_t* sorted_ids, int32_t* block_wrow,
                       int32_t* block_expert, const uint16_t* x, uint16_t* recv,
                       int32_t* status, void* stream);

/* Combine, the inverse of dispatch: y[t] = sum_k gates[t,k] * out[slot[t*K+k]]
 * with fp32 accumulation in ascending k (fused multiply-add), from the
 * expert outputs laid out like recv ([MoonEP-GR]: combine returns expert
 * results to the source tokens).
 *   out   [R*C, H] bf16 bits, 16-byte aligned
 *   slot  [P] int32 (entries < 0 contribute nothing)
 *   gates [N, K] fp32
 *   y     [N, H] fp32 (LBT_Y_F32) or bf16 bits rounded to nearest even
 *         (LBT_Y_BF16), 16-byte aligned */
int lbt_combine(const lbt_shape* s, const uint16_t* out, const int32_t* slot, const float* gates,
                int32_t y_dtype, void* y, void* stream);

/* Replica weight prefetch: copy each slotted replica's home weights into its
 * rank's prefetch slot.  [MoonEP-GR] section "Το memory contract ..." (one
 * contiguous [E+B, H, H'] weight tensor per expert projection: rows 0..E-1
 * the ranks' experts, rows E..E+B-1 the rank's local prefetch slots, found by
 * row index; the pool is process-global, shared by the layers; replicas
 * beyond the slots read home weights).  For every replica segment of the plan
 * with weight row E + j on rank d: slots[d][j] = weights[expert], a bit copy
 * streamed in 4 KiB tiles.  Slots the plan does not use are not written.
 *   plan      blob from lbt_plan_balance / lbt_plan_quota
 *   weights   [E][row_bytes] home weight rows (rows 0..E-1 of the pool), 16-byte aligned
 *   slots     [R][B][row_bytes] each rank's prefetch slots, 16-byte aligned
 *   row_bytes bytes of one expert's weights (H * H' * element size), a
 *             positive multiple of 16 */
int lbt_prefetch_weights(const lbt_shape* s, const int32_t* plan, const void* weights, void* slots,
                         int64_t row_bytes, void* stream);

/* Fold the replicas' weight gradients into their home experts' gradients
 * and clear the used slots.  [MoonEP-GR] section "Τι συμβαίνει στους
 * gradients κατά την εκπαίδευση" (fp32 gradients laid out like the weights;
 * prefetched slots write to a separate reduce buffer, seen over the ranks as
 * [R, B, H, H']; reduce_grad adds the slots of each rank's own experts into
 * the parameter gradient and clears them before the next micro-batch).  For
 * every expert, its slotted replicas are added in line order (ascending
 * rank), one fp32 addition each; remote replicas hold no slot.
 *   plan       blob from lbt_plan_balance / lbt_plan_quota
 *   slot_grads [R][B][row_elems] fp32, in/out (used slots set to 0)
 *   grads      [E][row_elems] fp32 home gradients, in/out
 *   row_elems  elements of one expert's gradient, a positive multiple of 4;
 *              both pointers 16-byte aligned */
int lbt_reduce_grad(const lbt_shape* s, const int32_t* plan, float* slot_grads, float* grads,
                    int64_t row_elems, void* stream);

/* Backward of combine.  [AlignSort] (permute records source -> destination;
 * the gradient of unpermute is a permute); [MoonEP-GR] (combine inverts the
 * zero-copy dispatch).  For pair f = t*K + k with row s = slot[f] >= 0:
 *   d_out[s]     = bf16(g[f] * dy[t])   fp32 product, rounded to nearest even
 *   d_gates[f]   = sum_h dy[t,h] * out[s,h], accumulated in fp64, rounded once
 * Pairs with slot < 0 get d_gates = 0 and write no row.
 *   out     [R*C, H] bf16 expert outputs (as combine read them), 16-byte aligned
 *   dy      [N, H] fp32 (LBT_Y_F32) or bf16 (LBT_Y_BF16), 16-byte aligned
 *   d_out   [R*C, H] bf16 out: only rows some pair maps to are written
 *   d_gates [N, K] fp32 out */
int lbt_combine_bwd(const lbt_shape* s, const uint16_t* out, const int32_t* slot,
                    const float* gates, int32_t dy_dtype, const void* dy, uint16_t* d_out,
                    float* d_gates, void* stream);

/* Backward of dispatch: dx[t] = sum_k d_recv[slot[t*K+k]] in ascending k,
 * fp32 accumulation (combine with every gate 1); slot < 0 contributes
 * nothing.  dx fp32 (LBT_Y_F32) or bf16 rounded to nearest even
 * (LBT_Y_BF16); d_recv and dx 16-byte aligned. */
int lbt_dispatch_bwd(const lbt_shape* s, const uint16_t* d_recv, const int32_t* slot,
                     int32_t dx_dtype, void* dx, void* stream);

/* Text for a return code. */
const char* lbt_strerror(int code);

/* Name of the HIP error behind the calling thread's most recent LBT_EHIP
 * (for example "hipErrorInvalidHandle"), or "hipSuccess" if that thread has
 * had none.  The string is static; the call launches nothing. */
const char* lbt_last_hip_error(void);

/* LBT_VERSION of the built library. */
int lbt_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LBT_H */
