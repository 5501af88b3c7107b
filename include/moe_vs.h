/*
 * moe_vs.h -- C ABI of the MI355X (gfx950) MoE variable-size grouped GEMM.
 *
 * One launch computes Y_e = X_e W_e for every expert e, where K and N are shared
 * and the row count m_e of each expert is data-dependent, may be zero, and sums
 * to T*k.  Pages the operations follow:
 *   [GG]   "Grouped GEMM for MoE, in depth" (aicassindra.com)
 *   [CARD] "grouped-gemm-moe" (model card of a published grouped GEMM kernel)
 *   [NOTE] "Grouped GEMM" (scholia-log study notes)
 *
 * Conventions shared by every call:
 *   - Every array argument is a DEVICE pointer unless stated otherwise; arrays
 *     are dense, row-major, with unit last stride.  The caller owns every
 *     buffer; no pointer is retained after a call returns.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the default
 *     stream).  No call synchronises with the device, reads device data back to
 *     the host, or allocates/frees device memory, so the whole layer can be
 *     captured in a HIP graph ([GG] "Problem descriptors and the tile
 *     scheduler": the schedule is computed on the device; "Failure modes": no
 *     host sync per layer).
 *   - Argument errors that the host can see (NULL pointers, sizes, dtypes,
 *     alignment, workspace size) return a nonzero MOE_ERR_* code BEFORE anything
 *     is launched.  A failed launch returns MOE_ERR_HIP.  Errors that depend on
 *     device data are never trapped: they are counted in the schedule's status
 *     words (see moe_schedule).
 *   - An assignment is one (token t, slot j) entry of expert_ids [T, k]; it is
 *     numbered s = t*k + j.
 *   - Expert weights are stored (E, N, K) like nn.Linear ([GG] "Data layout,
 *     offsets and alignment"): the forward product of a row x is x W[e]^T.
 *   - Offsets are int32 END offsets: offsets[e] = one past the last row of
 *     group e, so counts [3,0,5] give offsets [3,3,8] ([GG] "Data layout,
 *     offsets and alignment").  Empty groups are legal.
 *   - dtype codes: MOE_F32 (float) or MOE_BF16 (bfloat16 bit patterns).  The
 *     bf16 path multiplies on the matrix cores with fp32 accumulation; the fp32
 *     path is exact fp32 (no reduced-precision products) ([CARD] "How it works").
 *   - Sizes: every input tensor handed to a call must be smaller than 2^31
 *     bytes (x, dY, each expert's weight slice and the saved gate/up values
 *     are addressed with 32-bit offsets); E <= 1024; 1 <= k <= 64.  The
 *     outputs y, dX, dW and a grouped GEMM's out take 64-bit addresses and
 *     may be larger, except under the ranked combine (moe_set_combine), which
 *     reads y / dX back with 32-bit offsets: a launch that would use it on an
 *     output of 2^31 bytes or more returns MOE_ERR_LIMIT when the ranked
 *     combine is forced and takes the atomic combine otherwise.
 */
#ifndef MOE_VS_H
#define MOE_VS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------- */
#define MOE_OK 0
#define MOE_ERR_NULL 1      /* a required pointer is NULL                          */
#define MOE_ERR_SHAPE 2     /* a size is out of range or sizes are inconsistent    */
#define MOE_ERR_DTYPE 3     /* unsupported dtype or dtype combination              */
#define MOE_ERR_ALIGN 4     /* a pointer is not aligned as the call requires       */
#define MOE_ERR_WORKSPACE 5 /* workspace NULL or smaller than the query returned   */
#define MOE_ERR_HIP 6       /* the HIP runtime reported an error at launch         */
#define MOE_ERR_LIMIT 7     /* a size exceeds a documented library limit          */

/* ---- dtype and layout codes --------------------------------------------- */
#define MOE_F32 0
#define MOE_BF16 1
#define MOE_LAYOUT_CONTIGUOUS 0 /* rows of all experts concatenated (training / prefill) */
#define MOE_LAYOUT_MASKED 1     /* fixed capacity slots per expert (decode)               */

/* Row-block prefixes are kept for these tile heights (index i -> 32 << i). */
#define MOE_NUM_BM 4

/*
 * Routing schedule: a host-side descriptor filled by moe_build_schedule.  All
 * array members point into the caller's device workspace.  The descriptor is
 * plain data: copy it freely; it stays valid as long as the workspace does.
 *
 * Contiguous layout ([GG] "Data layout, offsets and alignment"; [CARD] "How it
 * works"): the assignments are sorted stably by expert, so row r (0 <= r <
 * offsets[E-1]) of the virtual sorted matrix is assignment row_to_assign[r];
 * rows of expert e are [offsets[e]-counts[e], offsets[e]) and come in ascending
 * assignment order.  Rows at or past offsets[E-1] (only when some ids are out
 * of range) hold -1 / weight 0.
 *
 * Masked layout ([NOTE] section 5): expert e owns the `capacity` rows
 * [e*capacity, (e+1)*capacity); its j-th assignment (ascending s) sits in row
 * e*capacity + j when j < capacity and is dropped otherwise; counts[e] =
 * min(m_e, capacity) valid rows form a prefix; empty slots hold -1 / weight 0.
 */
typedef struct moe_schedule {
  int64_t T;        /* tokens                                                */
  int64_t S;        /* assignments T*k                                       */
  int64_t R;        /* rows of the row maps: S (contiguous) or E*capacity    */
  int32_t k;        /* experts per token                                     */
  int32_t E;        /* experts                                               */
  int32_t layout;   /* MOE_LAYOUT_*                                          */
  int32_t capacity; /* masked: slots per expert; contiguous: 0               */
  int32_t *counts;        /* [E]  rows per expert (masked: min(m_e, capacity))  */
  int32_t *offsets;       /* [E]  END offsets = inclusive prefix sum of counts  */
  int32_t *block_start;   /* [MOE_NUM_BM][E+1] exclusive prefix of
                             ceil(counts[e] / BM) for BM = 32, 64, 128, 256;
                             entry E is the total number of row blocks          */
  int32_t *expert_order;  /* [E]  experts by descending count (ties: lower id)  */
  int32_t *row_to_assign; /* [R]  assignment s of each row, or -1               */
  int32_t *row_to_token;  /* [R]  token s / k of each row, or -1                */
  float *row_weight;      /* [R]  routing weight of each row (1 when no weights
                             were given), 0 for an empty row                    */
  int32_t *status;        /* [2]  {#assignments with expert id outside [0, E),
                                   #assignments dropped over capacity}          */
  /* Rank-ordered view (contiguous layout, k <= 8 and k*E <= 1024, and built
   * only when the combine setting in force at build time can use it:
   * MOE_COMBINE_RANKED, or MOE_COMBINE_AUTO with k = 1; otherwise phases = 0
   * and the pointers are NULL; the workspace size does not depend on it).  The rank of an assignment is the
   * number of valid assignments of the same token in earlier slots; the rows
   * are sorted stably by (rank, expert), so for each rank p the rows of rank p
   * form E consecutive groups (group p*E + e: rank p routed to expert e) and
   * every token has at most one row of each rank.  A token with no valid
   * assignment has one row of rank 0 in expert 0's group, with weight 0 and
   * assignment -1, so every token has exactly one rank-0 row.  The fused
   * kernels use it to combine the k contributions to an output row without
   * atomics: rank 0 stores, rank p > 0 adds to what ranks < p wrote. */
  int32_t phases;              /* k when built, else 0                           */
  int32_t *phase_counts;       /* [k*E] rows of each (rank, expert) group        */
  int32_t *phase_offsets;      /* [k*E] END offsets of those groups              */
  int32_t *phase_block_start;  /* [MOE_NUM_BM][k*E+1] their row-block prefixes  */
  int32_t *phase_row_to_assign;/* [S]  assignment of each row, or -1            */
  int32_t *phase_row_to_token; /* [S]  token of each row, or -1 past the end    */
  float *phase_row_weight;     /* [S]  routing weight (1 without weights; 0 for
                                  the row of a token with no valid assignment)  */
  int32_t *phase_sync;         /* [8*64 + 2] completion counters of the ranked
                                  combine (zeroed by the build, left zeroed by
                                  each ranked launch); word 8*64 + 1 counts
                                  waits that gave up (0 unless a ranked launch
                                  did not get every compute unit)               */
  int32_t weighted;            /* 1 when the build was given topk_weights; 0
                                  when every row weight is 1 (the kernels then
                                  skip the multiplications by the weight)      */
  int32_t *dw_queue;           /* [2] work-queue counters of the weight
                                  gradient: zeroed by the build, left zeroed by
                                  each launch.  Weight-gradient launches that
                                  use the same schedule must not overlap in
                                  time (they share these counters)             */
} moe_schedule;

/* Bytes of device workspace moe_build_schedule needs (256-byte aligned
 * internally).  Returns 0 for invalid sizes. */
size_t moe_schedule_workspace_bytes(int64_t T, int32_t k, int32_t E, int32_t layout,
                                    int32_t capacity);

/*
 * Build the routing schedule on the device: per-expert counts (bincount), END
 * offsets (int32 inclusive scan), the row-block/tile prefix, a stable counting
 * sort by expert giving row -> assignment, row -> token and the per-row
 * routing weight, and (masked layout) the fixed-capacity slots.
 * [GG] "Data layout, offsets and alignment" (argsort(stable), bincount, int32
 * cumsum); [GG] "Problem descriptors and the tile scheduler" (tiles per group,
 * prefix, total, on the device); [CARD] "How it works" (row -> token map,
 * per-row weight, tile layout); [NOTE] 4.1 permute and section 5 masked layout.
 *
 *   expert_ids   [T, k] int32 device; ids outside [0, E) are excluded from every
 *                group and counted in status[0].
 *   topk_weights [T, k] float device, or NULL for weight 1.
 *   layout       MOE_LAYOUT_CONTIGUOUS (capacity ignored) or MOE_LAYOUT_MASKED
 *                (1 <= capacity <= 65536; E*capacity < 2^31).
 *   workspace    device buffer of at least moe_schedule_workspace_bytes(...)
 *                bytes, 256-byte aligned; owned by the caller; holds every
 *                array of the schedule.
 *   sched        HOST pointer; filled on return (before the device work ends).
 * Requires T >= 1, 1 <= k <= 64, 1 <= E <= 1024, T*k < 2^31.
 */
int moe_build_schedule(const int32_t *expert_ids, const float *topk_weights, int64_t T,
                       int32_t k, int32_t E, int32_t layout, int32_t capacity,
                       void *workspace, size_t workspace_bytes, moe_schedule *sched,
                       void *stream);

/*
 * moe_build_schedule for callers that cannot allocate device memory at all
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  It builds the same schedule, bit for bit, into `workspace`,
 * but the per-block count tables the build needs on the way are kept in a
 * static device array of the library (192 KiB per GPU, held until the process
 * ends) instead of at the end of the workspace.  Nothing is allocated or freed.
 *   Arguments and results as for moe_build_schedule, except workspace_bytes:
 *   moe_schedule_workspace_bytes(...) always suffices; the call needs that
 *   size less the tables' share (256-byte aligned), and returns
 *   MOE_ERR_WORKSPACE below it.
 *   Returns MOE_ERR_LIMIT if the tables would not fit the static array (not
 *   reachable within the size limits above: the tables hold at most 3 * 16384
 *   ints) and MOE_ERR_HIP if the array's device address cannot be obtained.
 * Every call on one GPU uses that GPU's one array: calls that overlap in time
 * on the same GPU (on different streams, or from several host threads without
 * ordering) race and may build wrong schedules; calls ordered on one stream
 * are safe.  The array needs no clearing: each build writes every entry it
 * reads.
 */
int moe_build_schedule_noalloc(const int32_t *expert_ids, const float *topk_weights, int64_t T,
                               int32_t k, int32_t E, int32_t layout, int32_t capacity,
                               void *workspace, size_t workspace_bytes, moe_schedule *sched,
                               void *stream);

/*
 * Bare variable-size grouped GEMM, rows already grouped by expert ([GG] "Problem
 * descriptors and the tile scheduler"; [CARD] "How it works", the kernel with
 * the permutation maps omitted):
 *     C[r, n] = sum_k A[r, k] * W[e(r), n, k]   for r < offsets[E-1],
 * where e(r) is the group whose row range holds r.  Rows r >= offsets[E-1] of C
 * are not written.  One persistent launch covers every group; the tile space is
 * derived on the device from `offsets`.
 *   A [M, K], W [E, N, K] in `dtype`; offsets [E] int32 END offsets,
 *   non-decreasing, offsets[E-1] <= M; C [M, N] in `out_dtype`.
 *   dtype MOE_F32 -> out_dtype MOE_F32; dtype MOE_BF16 -> MOE_BF16 or MOE_F32.
 *   M may be 0 (nothing is launched).  Any K, N >= 1 (tails are guarded).
 */
int grouped_gemm(const void *A, const void *W, const int32_t *offsets, void *C, int64_t M,
                 int64_t K, int64_t N, int32_t E, int32_t dtype, int32_t out_dtype,
                 void *stream);

/*
 * Fused MoE forward ([CARD] intro and "How it works"): activation rows are
 * gathered through row -> token as they are loaded, each tile multiplies by its
 * expert's weights, and each result is scaled by its routing weight and added
 * atomically into the token's output row, so neither the [S, K] permuted input
 * nor the [S, N] expanded output is stored:
 *     y[t, n] = sum_j w[t, j] * sum_k x[t, k] * W[ids[t, j], n, k].
 * Works on both layouts (masked = the decode path; tiles with no valid rows
 * skip their weights).
 *   x [T, K] and W [E, N, K] in `dtype`; sched from moe_build_schedule;
 *   y [T, N] float, OVERWRITTEN (zeroed by the call, then accumulated).
 * With dtype MOE_F32 and k <= 2 the result is bitwise reproducible.
 */
int moe_fused_fwd(const void *x, const void *W, const moe_schedule *sched, float *y,
                  int64_t K, int64_t N, int32_t dtype, void *stream);

/*
 * Fused MoE forward on 8-bit operands with scales that travel with each group
 * ([GG] "Choosing an implementation": FP8 brings per-group or per-block scale
 * factors that must accompany every group):
 *     y[t, n] = sum_j w[t, j] * x_scale[t] * w_scale[e, n]
 *               * sum_k q(x_q[t, k]) * q(W_q[e, n, k]),   e = ids[t, j],
 * where q(.) is the value of an E4M3 code (1 sign, 4 exponent bits with bias
 * 7, 3 mantissa bits, subnormals, no infinities, 0x7F / 0xFF = NaN, largest
 * finite 448).  The products run on the matrix cores' 8-bit path with fp32
 * accumulation; the scales are applied to the fp32 result.
 *   x_q [T, K] and W_q [E, N, K] uint8 codes, 16-byte aligned; K a multiple
 *   of 16 (MOE_ERR_SHAPE otherwise); x_scale [T] and w_scale [E, N] float.
 *   sched from moe_build_schedule (either layout); y [T, N] float,
 *   OVERWRITTEN (zeroed by the call, then accumulated).
 */
int moe_fused_fwd_fp8(const void *x_q, const float *x_scale, const void *W_q,
                      const float *w_scale, const moe_schedule *sched, float *y, int64_t K,
                      int64_t N, void *stream);

/*
 * Fused MoE forward on 8-bit operands with per-block scales ([GG] "Choosing
 * an implementation": FP8 brings per-group or per-block scale factors; this
 * is the per-block form the gfx950 matrix cores apply themselves): every run
 * of 32 consecutive reduction elements of a token row and of an expert weight
 * row carries a power-of-two scale, an E8M0 code c with value 2^(c - 127):
 *     y[t, n] = sum_j w[t, j] * sum_b 2^(x_bs[t, b] - 127) * 2^(w_bs[e, n, b] - 127)
 *               * sum_{k in block b} q(x_q[t, k]) * q(W_q[e, n, k]),  e = ids[t, j],
 * with q(.) the E4M3 value as in moe_fused_fwd_fp8.
 *   x_q [T, K], W_q [E, N, K] uint8 codes (16-byte aligned); x_bs [T, K/32],
 *   w_bs [E, N, K/32] uint8 E8M0 codes (4-byte aligned); K a multiple of 128
 *   (MOE_ERR_SHAPE otherwise).  sched from moe_build_schedule (either
 *   layout); y [T, N] float, OVERWRITTEN.
 */
int moe_fused_fwd_mx(const void *x_q, const uint8_t *x_bs, const void *W_q, const uint8_t *w_bs,
                     const moe_schedule *sched, float *y, int64_t K, int64_t N, void *stream);

/*
 * Gated expert FFN forward ([GG] "Choosing an implementation": the gate and up
 * projections run as one grouped GEMM over a weight with twice the output
 * rows, with the activation in that GEMM's epilogue; the down projection is
 * the fused forward above applied to the activation):
 *     h[r, f] = silu(g) * u,  g = sum_k x[t_r, k] W_gu[e_r, f, k],
 *                             u = sum_k x[t_r, k] W_gu[e_r, F + f, k],
 *     y[t, n] = sum_j w[t, j] * sum_f h[r(t,j), f] * W_down[ids[t, j], n, f],
 * with silu(z) = z / (1 + exp(-z)), r the schedule row of an assignment, t_r,
 * e_r its token and expert.
 *   x [T, K], W_gu [E, 2F, K] (rows 0..F-1 gate, F..2F-1 up) and
 *   W_down [E, N, F] in `dtype` (MOE_BF16 or MOE_F32).  bf16 with K, F and N
 *   multiples of 8 runs on the matrix cores (x, W_gu, W_down, h and gu then
 *   16-byte aligned); fp32, or bf16 with other sizes, runs on the vector ALUs
 *   with exact fp32 products (element alignment only, any sizes).
 *   h [sched->R, F] in `dtype`, written for every valid row of the schedule in
 *   schedule row order (kept for a backward pass); rows of empty masked slots
 *   and rows at or past offsets[E-1] are left untouched.  h is rounded to
 *   `dtype` before the down projection.
 *   gu [sched->R, 2F] float or NULL: when given, the gate values g (columns
 *   0..F-1) and up values u (F..2F-1) of every valid row as accumulated (fp32),
 *   which moe_gated_ffn_bwd needs; same rows as h.
 *   y [T, N] float, OVERWRITTEN (zeroed by the call, then accumulated).
 * Three launches on `stream`: the gated up-projection, the zeroing of y and
 * the down projection.
 */
int moe_gated_ffn_fwd(const void *x, const void *W_gu, const void *W_down,
                      const moe_schedule *sched, void *h, void *gu, float *y, int64_t K,
                      int64_t F, int64_t N, int32_t dtype, void *stream);

/* Bytes of device workspace moe_gated_ffn_bwd needs (its [R, 2F] gradient of
 * the gate/up values, sized for either dtype); 0 for invalid arguments. */
size_t moe_gated_ffn_bwd_workspace_bytes(const moe_schedule *sched, int64_t F);

/*
 * Gated expert FFN backward for L = sum(dY * y) with y from moe_gated_ffn_fwd
 * (the chain rule through the down projection, the SiLU gate and the doubled
 * up-projection; [GG] "The backward pass" for the grouped products):
 *   dh[r]      = w_r * dY[t_r] W_down[e_r]                       (per row)
 *   dgu[r]     = (dh * u * silu'(g) | dh * silu(g)),  silu'(g) = s (1 + g (1 - s)),
 *                s = 1 / (1 + exp(-g)), with g, u the saved gate / up values
 *   dX[t]      = sum over the token's rows of dgu[r] W_gu[e_r]
 *   dW_gu[e]   = sum over rows of e of dgu[r]^T x[t_r]
 *   dW_down[e] = sum over rows of e of (w_r dY[t_r])^T h[r]   (0 for empty experts)
 *   d_topk[t, j] = dY[t] . (h[r] W_down[e]^T), the unweighted down output.
 *   dY [T, N], x [T, K], W_gu [E, 2F, K], W_down [E, N, F] and h [R, F] in
 *   `dtype`, gu [R, 2F] float (h and gu saved by the forward with the same
 *   schedule); on the matrix-core path (bf16, K, F, N multiples of 8) all
 *   16-byte aligned, as are dW_gu and dW_down; else element alignment.
 *   dX [T, K] float, dW_gu [E, 2F, K] and dW_down [E, N, F] in `dtype`,
 *   d_topk [T, k] float: each OVERWRITTEN, or NULL to skip.
 *   workspace: moe_gated_ffn_bwd_workspace_bytes(sched, F) bytes, 256-byte
 *   aligned (required when dX or dW_gu is asked for).
 * Up to four launches on `stream` (matrix cores): dW_down (which zeroes dX and
 * d_topk on the side; a fill launch when dW_down is NULL), the per-row dh /
 * dgu / d_topk kernel, dX, dW_gu; the vector-ALU path zeroes with a fill
 * launch first.  The routing weight enters through dh, so dX and dW_gu take
 * dgu unweighted.
 */
int moe_gated_ffn_bwd(const void *dY, const void *x, const void *W_gu, const void *W_down,
                      const moe_schedule *sched, const void *gu, const void *h, float *dX,
                      void *dW_gu, void *dW_down, float *d_topk, int64_t K, int64_t F, int64_t N,
                      int32_t dtype, void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of device workspace moe_fused_bwd needs for these sizes (may be 0). */
size_t moe_fused_bwd_workspace_bytes(const moe_schedule *sched, int64_t K, int64_t N,
                                     int32_t dtype);

/*
 * Fused MoE backward for L = sum(dY * y) ([GG] "The backward pass"; [CARD]
 * "How it works"):
 *   dX[t, k]     = sum_j w[t,j] * sum_n dY[t, n] * W[ids[t,j], n, k]
 *                  (the fused forward run on dY with each expert's weights
 *                  transposed; gather on load, weighted atomic scatter);
 *   dW[e, n, k]  = sum over assignments s routed to e of
 *                  w_s * dY[t_s, n] * x[t_s, k]   (a per-expert A^T B reduction
 *                  whose reduction length m_e varies; written for EVERY expert,
 *                  exactly 0 for an expert with no rows);
 *   d_topk[t, j] = sum_n dY[t, n] * Z[s, n], Z[s] = x[t] W[ids[t,j]]^T (the
 *                  product of assignment s before its weight is applied).
 *   dY [T, N], x [T, K], W [E, N, K] in `dtype`.
 *   dX [T, K] float or NULL (skip); OVERWRITTEN.
 *   dW [E, N, K] in `dtype` or NULL (skip); OVERWRITTEN; 16-byte aligned for
 *   bf16 (4-byte for fp32).
 *   d_topk [T, k] float or NULL (skip); OVERWRITTEN.  Rows of empty masked
 *   slots contribute nothing; dropped assignments get 0.
 *   W may be NULL only when dX and d_topk are both NULL.
 *   workspace: device buffer of moe_fused_bwd_workspace_bytes(...) bytes (may
 *   be NULL when that is 0).
 */
int moe_fused_bwd(const void *dY, const void *x, const void *W, const moe_schedule *sched,
                  float *dX, void *dW, float *d_topk, int64_t K, int64_t N, int32_t dtype,
                  void *workspace, size_t workspace_bytes, void *stream);

/*
 * Export the flat tile space the grouped kernels walk for an output of N
 * columns with tiles of BM x BN ([GG] "Problem descriptors and the tile
 * scheduler"): tiles[e] = ceil(counts[e]/BM) * ceil(N/BN) (masked layout:
 * ceil(capacity/BM) * ceil(N/BN)), tile_start = exclusive prefix, total, and
 * the owner of every tile, found with the same device code the kernels use
 * (upper bound of the tile index in tile_start, minus one).
 *   BM in {32, 64, 128, 256}; BN >= 1.
 *   tile_start [E] int32, total [1] int32, owner [owner_capacity] int32 (device);
 *   owners of tiles >= owner_capacity are not written.
 */
int moe_tile_map(const moe_schedule *sched, int64_t N, int32_t BM, int32_t BN,
                 int32_t *tile_start, int32_t *total, int32_t *owner, int64_t owner_capacity,
                 void *stream);

/*
 * Tile height of the routed kernels (the fused forward, the gated FFN and the
 * input gradient), a process-wide setting read at each launch ([GG] "Worked
 * example: tile counts under skew": shorter tiles waste fewer rows of small
 * groups, taller ones reuse each weight tile more).
 *   rows  0   = chosen on the device at each launch from the schedule's
 *               row-block totals (the default; no host read-back);
 *         128 or 256 = that height for every routed launch until changed.
 * Returns MOE_ERR_SHAPE (and changes nothing) for any other value.  Results
 * do not depend on the setting beyond floating-point summation order.
 */
int moe_set_tile_rows(int32_t rows);

/*
 * How the fused forward and the input gradient combine the k contributions to
 * a token's output row (a process-wide setting read at each call):
 *   MOE_COMBINE_AUTO   (default) chosen per call from the sizes alone;
 *   MOE_COMBINE_ATOMIC the output is zeroed, then one launch adds every
 *                      routing-weighted product into it atomically ([CARD]
 *                      "How it works": scatter-combine on store);
 *   MOE_COMBINE_RANKED one launch over the schedule's rank-ordered view (see
 *                      moe_schedule), tiles in rank order: rank 0 stores
 *                      w * product, rank p adds w * product to what ranks < p
 *                      stored, with plain loads and stores (a rank holds at
 *                      most one row per token); no zero fill and no atomics.
 *                      Used only where the schedule has the view (phases > 0)
 *                      and the matrix-core path runs; otherwise atomic.
 * The ranked combine is one launch over all ranks: a tile of rank p > 0 waits
 * (in the device) until every rank p-1 tile of its output column block has
 * stored, so launches that use the same schedule's rank-ordered view must not
 * run concurrently (its completion counters live in the schedule).  It needs
 * every compute unit for its persistent workgroups; a wait that does not end
 * within about half a second gives up and is counted in phase_sync (results
 * are then wrong, the call still returns).  Output column blocks (256 wide)
 * at most 64.  The fp32 sum for a token follows rank order (deterministic).
 * The setting in force when a schedule is built also decides whether the
 * schedule carries the rank-ordered view (see moe_schedule): set
 * MOE_COMBINE_RANKED before building a schedule meant for ranked launches.
 * Returns MOE_ERR_SHAPE for an unknown mode.
 */
#define MOE_COMBINE_AUTO 0
#define MOE_COMBINE_ATOMIC 1
#define MOE_COMBINE_RANKED 2
int moe_set_combine(int32_t mode);

/*
 * Kernel timing for benchmarks.  While enabled, the library brackets every
 * kernel it launches with a pair of HIP events recorded on that launch's own
 * stream and keeps them per kernel family.  Families: "build_schedule",
 * "fill_zero", "grouped_gemm", "fused_fwd", "bwd_dx", "bwd_dw", "tile_map",
 * "gated_up", "gated_down", "fused_fwd_fp8", "gated_bwd_dw_down",
 * "gated_bwd_dh", "gated_bwd_dx", "gated_bwd_dw_gu", "fused_fwd_mx".
 *   moe_timing_enable(1) clears earlier records and starts recording;
 *   moe_timing_enable(0) stops recording (records are kept).
 *   moe_timing_read waits for the recorded events of `family` and returns the
 *   summed duration in milliseconds and the number of launches.  Returns
 *   MOE_ERR_SHAPE for an unknown family, MOE_ERR_HIP on an event failure.
 * Recording creates HIP events (host-side objects); it is meant for benchmark
 * runs, not for graph capture.
 */
int moe_timing_enable(int enable);
int moe_timing_read(const char *family, double *total_ms, int64_t *launches);

/* Human-readable text of a status code (static storage). */
const char *moe_status_string(int status);

/* Library version string (static storage). */
const char *moe_version(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_VS_H */
