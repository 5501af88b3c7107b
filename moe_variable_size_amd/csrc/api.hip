// C ABI of the MoE grouped GEMM library: host-side validation and dispatch.
//
// Every entry point checks its arguments completely before it launches
// anything, so a nonzero return means nothing was enqueued.  Nothing here
// synchronises, reads device memory back or allocates: the whole layer can be
// captured in a HIP graph ([GG] "Failure modes": no host sync per layer;
// [GG] = "Grouped GEMM for MoE, in depth").
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "common.hpp"

namespace moe {

int device_cu_count() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cache[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev] = n;
  }
  return cache[dev];
}

namespace {

constexpr int64_t kMax32 = (int64_t)1 << 31;

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

struct WsLayout {
  size_t counts, offsets, bstart, order, status, queue, r2a, r2t, rw;
  size_t pcounts, poffsets, pbstart, pr2a, pr2t, prw, psync;  // rank-ordered view (0 sizes if absent)
  size_t scratch, total;
  bool ranked;
};

WsLayout ws_layout(int64_t S, int64_t R, int E, int k, int layout) {
  WsLayout l;
  l.ranked = rank_order_supported(layout, k, E);
  const int64_t kE = l.ranked ? (int64_t)k * E : 0;
  const int64_t PR = l.ranked ? S + kRowPad : 0;
  size_t o = 0;
  l.counts = o;  o = align256(o + sizeof(int32_t) * E);
  l.offsets = o; o = align256(o + sizeof(int32_t) * E);
  l.bstart = o;  o = align256(o + sizeof(int32_t) * MOE_NUM_BM * (E + 1));
  l.order = o;   o = align256(o + sizeof(int32_t) * E);
  l.status = o;  o = align256(o + sizeof(int32_t) * 2);
  l.queue = o;   o = align256(o + sizeof(int32_t) * 2);
  // row arrays carry kRowPad spare entries: kernels read row data a stage
  // (32 rows) at a time and may read past the last row (values ignored)
  l.r2a = o;     o = align256(o + sizeof(int32_t) * (R + kRowPad));
  l.r2t = o;     o = align256(o + sizeof(int32_t) * (R + kRowPad));
  l.rw = o;      o = align256(o + sizeof(float) * (R + kRowPad));
  l.pcounts = o;  o = align256(o + sizeof(int32_t) * kE);
  l.poffsets = o; o = align256(o + sizeof(int32_t) * kE);
  l.pbstart = o;  o = align256(o + sizeof(int32_t) * (l.ranked ? MOE_NUM_BM * (kE + 1) : 0));
  l.pr2a = o;     o = align256(o + sizeof(int32_t) * PR);
  l.pr2t = o;     o = align256(o + sizeof(int32_t) * PR);
  l.prw = o;      o = align256(o + sizeof(float) * PR);
  l.psync = o;    o = align256(o + sizeof(int32_t) * (l.ranked ? kRankSyncInts : 0));
  l.scratch = o;  o = align256(o + schedule_scratch_bytes(S, E, k, l.ranked));  // block tables
  l.total = o;
  return l;
}

int check_sizes(int64_t T, int32_t k, int32_t E, int32_t layout, int32_t capacity, int64_t *R) {
  if (T < 1 || k < 1 || k > 64 || E < 1) return MOE_ERR_SHAPE;
  if (E > kMaxExperts) return MOE_ERR_LIMIT;
  if (T * k >= kMax32) return MOE_ERR_LIMIT;
  if (layout == MOE_LAYOUT_CONTIGUOUS) {
    *R = T * k;
  } else if (layout == MOE_LAYOUT_MASKED) {
    if (capacity < 1 || capacity > 65536) return MOE_ERR_SHAPE;
    if ((int64_t)E * capacity >= kMax32) return MOE_ERR_LIMIT;
    *R = (int64_t)E * capacity;
  } else {
    return MOE_ERR_SHAPE;
  }
  return MOE_OK;
}

int check_sched(const moe_schedule *s) {
  if (!s || !s->counts || !s->offsets || !s->block_start || !s->expert_order ||
      !s->row_to_assign || !s->row_to_token || !s->row_weight || !s->status || !s->dw_queue)
    return MOE_ERR_NULL;
  int64_t R = 0;
  int rc = check_sizes(s->T, s->k, s->E, s->layout, s->capacity, &R);
  if (rc) return rc;
  if (R != s->R || s->S != s->T * s->k) return MOE_ERR_SHAPE;
  if (s->phases != 0) {
    if (s->phases != s->k || !rank_order_supported(s->layout, s->k, s->E)) return MOE_ERR_SHAPE;
    if (!s->phase_counts || !s->phase_offsets || !s->phase_block_start ||
        !s->phase_row_to_assign || !s->phase_row_to_token || !s->phase_row_weight ||
        !s->phase_sync)
      return MOE_ERR_NULL;
  }
  return MOE_OK;
}

int check_dtype_dims(int32_t dtype, int64_t K, int64_t N) {
  if (dtype != MOE_F32 && dtype != MOE_BF16) return MOE_ERR_DTYPE;
  if (K < 1 || N < 1) return MOE_ERR_SHAPE;
  if (K >= kMax32 || N >= kMax32) return MOE_ERR_LIMIT;
  return MOE_OK;
}

size_t esize(int32_t dtype) { return dtype == MOE_F32 ? 4 : 2; }

// byte size of an [rows, cols] tensor must stay below 2^31 (32-bit offsets)
bool fits(int64_t rows, int64_t cols, int32_t dtype) {
  return (double)rows * (double)cols * (double)esize(dtype) < (double)kMax32;
}

// ---- combine of the k contributions to an output row -----------------------
std::atomic<int> g_combine{MOE_COMBINE_AUTO};

// Whether a scattering launch over this schedule uses the ranked combine (one
// launch over the rank-ordered view: rank 0 stores, later ranks wait for the
// earlier ones and add; no atomics, no zero fill) rather than atomic adds into
// a zeroed output.  The automatic choice is the atomic combine except for a
// forward with one slot per token (k = 1: a single rank, only stores, no
// waits): measured on MI355X, the waits and read-backs of later ranks cost
// more than the atomic adds they replace (T = 4096, K = N = 2048, E = 8 top-2:
// forward 105-109 against 104-107 us, input gradient 229-236 against 125-129 us).
// Whether a schedule built now gets the rank-ordered view: only when a launch
// under the present combine setting can use it (the second sort job costs
// about a fifth of the build).
bool rank_view_wanted(int k) {
  const int mode = g_combine.load(std::memory_order_relaxed);
  return mode == MOE_COMBINE_RANKED || (mode == MOE_COMBINE_AUTO && k == 1);
}

// The ranked combine reads earlier ranks' values back through 32-bit buffer
// offsets, so its output must stay below 2^31 bytes: the automatic choice
// takes the atomic combine (64-bit addresses, any size) for a larger output,
// and a launch with the ranked combine forced refuses it (MOE_ERR_LIMIT).
bool use_ranked(const moe_schedule &s, int64_t out_cols, bool input_grad) {
  if (s.phases == 0 || (out_cols + 255) / 256 > kRankSyncCols) return false;
  const int mode = g_combine.load(std::memory_order_relaxed);
  if (mode == MOE_COMBINE_ATOMIC) return false;
  if (mode == MOE_COMBINE_RANKED) return true;
  return !input_grad && s.k == 1 && fits(s.T, out_cols, MOE_F32);
}

// The gated FFN's products take the matrix cores for bf16 with K, F and N
// multiples of 8 (both of its GEMM shapes then fit them).
bool gated_mfma(int32_t dtype, int64_t K, int64_t F, int64_t N) {
  return dtype == MOE_BF16 && mfma_supported((int)K, (int)(2 * F)) &&
         mfma_supported((int)F, (int)N);
}

// ---- kernel timing (benchmarks only) ---------------------------------------
const char *const kFamilies[] = {"build_schedule", "fill_zero", "grouped_gemm", "fused_fwd",
                                 "bwd_dx", "bwd_dw", "tile_map", "gated_up", "gated_down",
                                 "fused_fwd_fp8", "gated_bwd_dw_down", "gated_bwd_dh",
                                 "gated_bwd_dx", "gated_bwd_dw_gu", "fused_fwd_mx"};
constexpr int kNumFamilies = sizeof(kFamilies) / sizeof(kFamilies[0]);

struct Timing {
  std::mutex mu;
  bool on = false;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> ev[kNumFamilies];
};
Timing &timing() {
  static Timing t;
  return t;
}

int family_index(const char *name) {
  for (int i = 0; i < kNumFamilies; ++i)
    if (strcmp(name, kFamilies[i]) == 0) return i;
  return -1;
}

// Launch `f` (returning hipError_t) bracketed by events when timing is on.
template <typename F>
hipError_t timed(int fam, hipStream_t st, F &&f) {
  Timing &t = timing();
  if (!t.on) return f();
  // an event failure only drops this launch's record; the launch still runs
  hipEvent_t a = nullptr, b = nullptr;
  if (hipEventCreate(&a) != hipSuccess) return f();
  if (hipEventCreate(&b) != hipSuccess) {
    (void)hipEventDestroy(a);
    return f();
  }
  const bool ra = hipEventRecord(a, st) == hipSuccess;
  const hipError_t e = f();
  const bool rb = ra && hipEventRecord(b, st) == hipSuccess;
  if (!rb) {
    (void)hipEventDestroy(a);
    (void)hipEventDestroy(b);
    return e;
  }
  std::lock_guard<std::mutex> g(t.mu);
  t.ev[fam].emplace_back(a, b);
  return e;
}

enum { F_SCHED = 0, F_FILL, F_BARE, F_FWD, F_DX, F_DW, F_TILEMAP, F_GATED_UP, F_GATED_DOWN,
       F_FWD_FP8, F_GB_DWD, F_GB_DH, F_GB_DX, F_GB_DWGU, F_FWD_MX };

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" {

const char *moe_version(void) { return "moe_vs 0.1.0 gfx950"; }

const char *moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "a size is out of range or sizes are inconsistent";
    case MOE_ERR_DTYPE: return "unsupported dtype";
    case MOE_ERR_ALIGN: return "a pointer is not aligned as required";
    case MOE_ERR_WORKSPACE: return "workspace NULL or too small";
    case MOE_ERR_HIP: return "HIP runtime error at launch";
    case MOE_ERR_LIMIT: return "a size exceeds a library limit";
    default: return "unknown status";
  }
}

size_t moe_schedule_workspace_bytes(int64_t T, int32_t k, int32_t E, int32_t layout,
                                    int32_t capacity) {
  int64_t R = 0;
  if (check_sizes(T, k, E, layout, capacity, &R)) return 0;
  return ws_layout(T * k, R, E, k, layout).total;
}

}  // extern "C"

namespace moe {
namespace {
// The schedule build of both entry points: the schedule's arrays go into
// `workspace`; the block tables into `tables` (static_tables) or behind the
// arrays in the workspace.
int build_schedule(const int32_t *expert_ids, const float *topk_weights, int64_t T, int32_t k,
                   int32_t E, int32_t layout, int32_t capacity, void *workspace,
                   size_t workspace_bytes, moe_schedule *sched, void *stream, bool static_tables) {
  if (!expert_ids || !sched) return MOE_ERR_NULL;
  int64_t R = 0;
  int rc = check_sizes(T, k, E, layout, capacity, &R);
  if (rc) return rc;
  if (!aligned(expert_ids, 4) || (topk_weights && !aligned(topk_weights, 4))) return MOE_ERR_ALIGN;
  const WsLayout l = ws_layout(T * k, R, E, k, layout);
  if (!workspace || workspace_bytes < (static_tables ? l.scratch : l.total))
    return MOE_ERR_WORKSPACE;
  if (!aligned(workspace, 256)) return MOE_ERR_ALIGN;
  char *w = (char *)workspace;
  int32_t *tables = (int32_t *)(w + l.scratch);
  if (static_tables) {
    size_t cap = 0;
    if (static_schedule_scratch(&tables, &cap) != hipSuccess) return MOE_ERR_HIP;
    if (schedule_scratch_bytes(T * k, E, k, l.ranked) > cap) return MOE_ERR_LIMIT;
  }
  moe_schedule s;
  memset(&s, 0, sizeof(s));
  s.T = T;
  s.S = T * k;
  s.R = R;
  s.k = k;
  s.E = E;
  s.layout = layout;
  s.capacity = layout == MOE_LAYOUT_MASKED ? capacity : 0;
  s.weighted = topk_weights ? 1 : 0;
  s.counts = (int32_t *)(w + l.counts);
  s.offsets = (int32_t *)(w + l.offsets);
  s.block_start = (int32_t *)(w + l.bstart);
  s.expert_order = (int32_t *)(w + l.order);
  s.status = (int32_t *)(w + l.status);
  s.dw_queue = (int32_t *)(w + l.queue);
  s.row_to_assign = (int32_t *)(w + l.r2a);
  s.row_to_token = (int32_t *)(w + l.r2t);
  s.row_weight = (float *)(w + l.rw);
  if (l.ranked && rank_view_wanted(k)) {
    s.phases = k;
    s.phase_counts = (int32_t *)(w + l.pcounts);
    s.phase_offsets = (int32_t *)(w + l.poffsets);
    s.phase_block_start = (int32_t *)(w + l.pbstart);
    s.phase_row_to_assign = (int32_t *)(w + l.pr2a);
    s.phase_row_to_token = (int32_t *)(w + l.pr2t);
    s.phase_row_weight = (float *)(w + l.prw);
    s.phase_sync = (int32_t *)(w + l.psync);
  }
  *sched = s;
  hipStream_t st = (hipStream_t)stream;
  return hip_status(
      timed(F_SCHED, st, [&] {
        return launch_build_schedule(expert_ids, topk_weights, s, tables, st);
      }));
}
}  // namespace
}  // namespace moe

extern "C" {

int moe_build_schedule(const int32_t *expert_ids, const float *topk_weights, int64_t T, int32_t k,
                       int32_t E, int32_t layout, int32_t capacity, void *workspace,
                       size_t workspace_bytes, moe_schedule *sched, void *stream) {
  return moe::build_schedule(expert_ids, topk_weights, T, k, E, layout, capacity, workspace,
                             workspace_bytes, sched, stream, false);
}

int moe_build_schedule_noalloc(const int32_t *expert_ids, const float *topk_weights, int64_t T,
                               int32_t k, int32_t E, int32_t layout, int32_t capacity,
                               void *workspace, size_t workspace_bytes, moe_schedule *sched,
                               void *stream) {
  return moe::build_schedule(expert_ids, topk_weights, T, k, E, layout, capacity, workspace,
                             workspace_bytes, sched, stream, true);
}

int grouped_gemm(const void *A, const void *W, const int32_t *offsets, void *C, int64_t M,
                 int64_t K, int64_t N, int32_t E, int32_t dtype, int32_t out_dtype,
                 void *stream) {
  int rc = check_dtype_dims(dtype, K, N);
  if (rc) return rc;
  if (M < 0 || E < 1) return MOE_ERR_SHAPE;
  if (E > kMaxExperts) return MOE_ERR_LIMIT;
  if (dtype == MOE_F32 && out_dtype != MOE_F32) return MOE_ERR_DTYPE;
  if (out_dtype != MOE_F32 && out_dtype != MOE_BF16) return MOE_ERR_DTYPE;
  if (M == 0) return MOE_OK;
  if (!A || !W || !offsets || !C) return MOE_ERR_NULL;
  if (!fits(M, K, dtype) || !fits(N, K, dtype)) return MOE_ERR_LIMIT;  // (C: 64-bit addresses)
  const size_t al = dtype == MOE_BF16 ? 16 : 4;
  if (!aligned(A, al) || !aligned(W, al) || !aligned(offsets, 4) || !aligned(C, esize(out_dtype)))
    return MOE_ERR_ALIGN;
  hipStream_t st = (hipStream_t)stream;
  return hip_status(timed(F_BARE, st, [&] {
    if (dtype == MOE_BF16 && mfma_supported((int)K, (int)N))
      return mfma_grouped_gemm(A, W, offsets, C, (int)M, (int)K, (int)N, E, out_dtype, st);
    return simt_grouped_gemm(A, W, offsets, C, (int)M, (int)K, (int)N, E, dtype, out_dtype, st);
  }));
}

int moe_fused_fwd(const void *x, const void *W, const moe_schedule *sched, float *y, int64_t K,
                  int64_t N, int32_t dtype, void *stream) {
  int rc = check_sched(sched);
  if (rc) return rc;
  rc = check_dtype_dims(dtype, K, N);
  if (rc) return rc;
  if (!x || !W || !y) return MOE_ERR_NULL;
  const moe_schedule &s = *sched;
  if (!fits(s.T, K, dtype) || !fits(N, K, dtype)) return MOE_ERR_LIMIT;
  const size_t al = dtype == MOE_BF16 ? 16 : 4;
  if (!aligned(x, al) || !aligned(W, al) || !aligned(y, 4)) return MOE_ERR_ALIGN;
  hipStream_t st = (hipStream_t)stream;
  const bool mfma = dtype == MOE_BF16 && mfma_supported((int)K, (int)N);
  const bool ranked = mfma && use_ranked(s, N, false);
  if (ranked && !fits(s.T, N, MOE_F32)) return MOE_ERR_LIMIT;
  if (!ranked) {
    hipError_t e = timed(F_FILL, st, [&] {
      return launch_fill_zero(y, (size_t)s.T * N * sizeof(float), nullptr, 0, st);
    });
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  return hip_status(timed(F_FWD, st, [&] {
    if (mfma) return mfma_fused_fwd(x, W, s, y, (int)K, (int)N, false, ranked, st);
    return simt_fused_fwd(x, W, s, y, (int)K, (int)N, dtype, st);
  }));
}

int moe_fused_fwd_fp8(const void *x_q, const float *x_scale, const void *W_q,
                      const float *w_scale, const moe_schedule *sched, float *y, int64_t K,
                      int64_t N, void *stream) {
  int rc = check_sched(sched);
  if (rc) return rc;
  if (K < 16 || N < 1 || K % 16 != 0) return MOE_ERR_SHAPE;
  if (K >= kMax32 || N >= kMax32) return MOE_ERR_LIMIT;
  if (!x_q || !x_scale || !W_q || !w_scale || !y) return MOE_ERR_NULL;
  const moe_schedule &s = *sched;
  if ((double)s.T * K >= (double)kMax32 || (double)N * K >= (double)kMax32)
    return MOE_ERR_LIMIT;
  if (!aligned(x_q, 16) || !aligned(W_q, 16) || !aligned(x_scale, 4) || !aligned(w_scale, 4) ||
      !aligned(y, 4))
    return MOE_ERR_ALIGN;
  hipStream_t st = (hipStream_t)stream;
  const bool ranked = use_ranked(s, N, false);
  if (ranked && !fits(s.T, N, MOE_F32)) return MOE_ERR_LIMIT;
  if (!ranked) {
    hipError_t e = timed(F_FILL, st, [&] {
      return launch_fill_zero(y, (size_t)s.T * N * sizeof(float), nullptr, 0, st);
    });
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  return hip_status(timed(F_FWD_FP8, st, [&] {
    return mfma_fused_fwd_fp8(x_q, x_scale, W_q, w_scale, s, y, (int)K, (int)N, ranked, st);
  }));
}

int moe_fused_fwd_mx(const void *x_q, const uint8_t *x_bs, const void *W_q, const uint8_t *w_bs,
                     const moe_schedule *sched, float *y, int64_t K, int64_t N, void *stream) {
  int rc = check_sched(sched);
  if (rc) return rc;
  if (K < 128 || N < 1 || K % 128 != 0) return MOE_ERR_SHAPE;
  if (K >= kMax32 || N >= kMax32) return MOE_ERR_LIMIT;
  if (!x_q || !x_bs || !W_q || !w_bs || !y) return MOE_ERR_NULL;
  const moe_schedule &s = *sched;
  if ((double)s.T * K >= (double)kMax32 || (double)N * K >= (double)kMax32)
    return MOE_ERR_LIMIT;
  if (!aligned(x_q, 16) || !aligned(W_q, 16) || !aligned(x_bs, 4) || !aligned(w_bs, 4) ||
      !aligned(y, 4))
    return MOE_ERR_ALIGN;
  hipStream_t st = (hipStream_t)stream;
  const bool ranked = use_ranked(s, N, false);
  if (ranked && !fits(s.T, N, MOE_F32)) return MOE_ERR_LIMIT;
  if (!ranked) {
    hipError_t e = timed(F_FILL, st, [&] {
      return launch_fill_zero(y, (size_t)s.T * N * sizeof(float), nullptr, 0, st);
    });
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  return hip_status(timed(F_FWD_MX, st, [&] {
    return mfma_fused_fwd_mx(x_q, x_bs, W_q, w_bs, s, y, (int)K, (int)N, ranked, st);
  }));
}

int moe_gated_ffn_fwd(const void *x, const void *W_gu, const void *W_down,
                      const moe_schedule *sched, void *h, void *gu, float *y, int64_t K, int64_t F,
                      int64_t N, int32_t dtype, void *stream) {
  int rc = check_sched(sched);
  if (rc) return rc;
  rc = check_dtype_dims(dtype, K, N);
  if (rc) return rc;
  if (F < 1) return MOE_ERR_SHAPE;
  if (F >= kMax32) return MOE_ERR_LIMIT;
  if (!x || !W_gu || !W_down || !h || !y) return MOE_ERR_NULL;
  const moe_schedule &s = *sched;
  // matrix cores for bf16 with K, F, N multiples of 8; the vector-ALU kernels
  // (64-bit addressing, element alignment) otherwise
  const bool mfma = gated_mfma(dtype, K, F, N);
  if (mfma) {
    if (!fits(s.T, K, dtype) || !fits(2 * F, K, dtype) || !fits(N, F, dtype) ||
        !fits(s.R, F, dtype))
      return MOE_ERR_LIMIT;
    if (gu && !fits(s.R, 2 * F, MOE_F32)) return MOE_ERR_LIMIT;
  }
  const size_t al = mfma ? 16 : esize(dtype);
  if (!aligned(x, al) || !aligned(W_gu, al) || !aligned(W_down, al) || !aligned(h, al) ||
      (gu && !aligned(gu, mfma ? 16 : 4)) || !aligned(y, 4))
    return MOE_ERR_ALIGN;
  hipStream_t st = (hipStream_t)stream;
  hipError_t e = timed(F_GATED_UP, st, [&] {
    return mfma ? mfma_gated_up(x, W_gu, s, h, gu, (int)K, (int)F, st)
                : simt_gated_up(x, W_gu, s, h, (float *)gu, (int)K, (int)F, dtype, st);
  });
  if (e == hipSuccess)
    e = timed(F_FILL, st, [&] {
      return launch_fill_zero(y, (size_t)s.T * N * sizeof(float), nullptr, 0, st);
    });
  if (e == hipSuccess)
    e = timed(F_GATED_DOWN, st, [&] {
      return mfma ? mfma_fused_fwd(h, W_down, s, y, (int)F, (int)N, true, false, st)
                  : simt_gated_down(h, W_down, s, y, (int)F, (int)N, dtype, st);
    });
  return hip_status(e);
}

size_t moe_gated_ffn_bwd_workspace_bytes(const moe_schedule *sched, int64_t F) {
  if (!sched || F < 1 || F >= kMax32) return 0;
  return align256((size_t)sched->R * 2 * (size_t)F * 4);  // dgu [R, 2F], fp32 at most
}

int moe_gated_ffn_bwd(const void *dY, const void *x, const void *W_gu, const void *W_down,
                      const moe_schedule *sched, const void *gu, const void *h, float *dX,
                      void *dW_gu, void *dW_down, float *d_topk, int64_t K, int64_t F, int64_t N,
                      int32_t dtype, void *workspace, size_t workspace_bytes, void *stream) {
  int rc = check_sched(sched);
  if (rc) return rc;
  rc = check_dtype_dims(dtype, K, N);
  if (rc) return rc;
  if (F < 1) return MOE_ERR_SHAPE;
  if (F >= kMax32) return MOE_ERR_LIMIT;
  if (!dY || !x || !W_gu || !W_down || !gu || !h) return MOE_ERR_NULL;
  const moe_schedule &s = *sched;
  const bool need_dgu = dX || dW_gu;
  const bool mfma = gated_mfma(dtype, K, F, N);
  if (mfma && (!fits(s.T, K, dtype) || !fits(s.T, N, dtype) || !fits(2 * F, K, dtype) ||
               !fits(N, F, dtype) || !fits(s.R, 2 * F, MOE_F32)))
    return MOE_ERR_LIMIT;
  const size_t ws_need = moe_gated_ffn_bwd_workspace_bytes(sched, F);
  if (need_dgu && (!workspace || workspace_bytes < ws_need)) return MOE_ERR_WORKSPACE;
  const size_t al = mfma ? 16 : esize(dtype);
  if (!aligned(dY, al) || !aligned(x, al) || !aligned(W_gu, al) || !aligned(W_down, al) ||
      !aligned(gu, mfma ? 16 : 4) || !aligned(h, al) || (dX && !aligned(dX, 4)) ||
      (dW_gu && !aligned(dW_gu, al)) || (dW_down && !aligned(dW_down, al)) ||
      (d_topk && !aligned(d_topk, 4)) || (workspace && !aligned(workspace, 256)))
    return MOE_ERR_ALIGN;
  hipStream_t st = (hipStream_t)stream;
  void *dgu = workspace;
  const size_t dx_bytes = dX ? (size_t)s.T * K * sizeof(float) : 0;
  const size_t dt_bytes = d_topk ? (size_t)s.S * sizeof(float) : 0;
  hipError_t e = hipSuccess;
  if (!mfma) {
    // vector-ALU kernels: zero dX / d_topk, dW_down, dh / dgu / d_topk, dX, dW_gu
    if (dx_bytes || dt_bytes)
      e = timed(F_FILL, st, [&] { return launch_fill_zero(dX, dx_bytes, d_topk, dt_bytes, st); });
    if (e == hipSuccess && dW_down)
      e = timed(F_GB_DWD, st, [&] {
        return simt_bwd_dw_rows(dY, false, h, true, s, dW_down, (int)F, (int)N, dtype, st);
      });
    if (e == hipSuccess && (need_dgu || d_topk))
      e = timed(F_GB_DH, st, [&] {
        return simt_gated_bwd_dh(dY, h, W_down, s, d_topk, (int)F, (int)N, (const float *)gu,
                                 need_dgu ? dgu : nullptr, dtype, st);
      });
    if (e == hipSuccess && dX)
      e = timed(F_GB_DX, st, [&] {
        return simt_gated_bwd_dx(dgu, W_gu, s, dX, (int)K, (int)F, dtype, st);
      });
    if (e == hipSuccess && dW_gu)
      e = timed(F_GB_DWGU, st, [&] {
        return simt_bwd_dw_rows(dgu, true, x, false, s, dW_gu, (int)K, (int)(2 * F), dtype, st);
      });
    return hip_status(e);
  }
  // 1. dW_down = sum (w dY)^T h (zeroes dX and d_topk on the side), or one fill
  if (dW_down)
    e = timed(F_GB_DWD, st, [&] {
      return mfma_bwd_dw_rows(dY, false, h, true, s, dW_down, (int)F, (int)N, true, dX, dx_bytes,
                              d_topk, dt_bytes, st);
    });
  else if (dX || d_topk)
    e = timed(F_FILL, st, [&] { return launch_fill_zero(dX, dx_bytes, d_topk, dt_bytes, st); });
  // 2. G = dY W_down per row; d_topk += <G, h>; dgu from the saved gate / up
  if (e == hipSuccess && (need_dgu || d_topk))
    e = timed(F_GB_DH, st, [&] {
      return mfma_gated_bwd_dh(dY, h, W_down, s, d_topk, (int)F, (int)N, gu,
                               need_dgu ? dgu : nullptr, st);
    });
  // 3. dX[t] += dgu[r] W_gu[e]
  if (e == hipSuccess && dX)
    e = timed(F_GB_DX, st, [&] { return mfma_gated_bwd_dx(dgu, W_gu, s, dX, (int)K, (int)F, st); });
  // 4. dW_gu = sum dgu^T x
  if (e == hipSuccess && dW_gu)
    e = timed(F_GB_DWGU, st, [&] {
      return mfma_bwd_dw_rows(dgu, true, x, false, s, dW_gu, (int)K, (int)(2 * F), false,
                              nullptr, 0, nullptr, 0, st);
    });
  return hip_status(e);
}

size_t moe_fused_bwd_workspace_bytes(const moe_schedule *sched, int64_t K, int64_t N,
                                     int32_t dtype) {
  (void)sched;
  (void)K;
  (void)N;
  (void)dtype;
  return 0;
}

int moe_fused_bwd(const void *dY, const void *x, const void *W, const moe_schedule *sched,
                  float *dX, void *dW, float *d_topk, int64_t K, int64_t N, int32_t dtype,
                  void *workspace, size_t workspace_bytes, void *stream) {
  (void)workspace;
  (void)workspace_bytes;
  int rc = check_sched(sched);
  if (rc) return rc;
  rc = check_dtype_dims(dtype, K, N);
  if (rc) return rc;
  if (!dY || !x) return MOE_ERR_NULL;
  if ((dX || d_topk) && !W) return MOE_ERR_NULL;
  const moe_schedule &s = *sched;
  if (!fits(s.T, K, dtype) || !fits(s.T, N, dtype) || !fits(N, K, dtype)) return MOE_ERR_LIMIT;
  const size_t al = dtype == MOE_BF16 ? 16 : 4;
  if (!aligned(dY, al) || !aligned(x, al) || (W && !aligned(W, al)) || (dX && !aligned(dX, 4)) ||
      (dW && !aligned(dW, dtype == MOE_BF16 ? 16 : 4)) || (d_topk && !aligned(d_topk, 4)))
    return MOE_ERR_ALIGN;
  hipStream_t st = (hipStream_t)stream;
  const bool mfma = dtype == MOE_BF16 && mfma_supported((int)K, (int)N);
  hipError_t e = hipSuccess;
  const size_t dx_bytes = dX ? (size_t)s.T * K * sizeof(float) : 0;
  const size_t dt_bytes = d_topk ? (size_t)s.S * sizeof(float) : 0;
  // With the ranked combine the input-gradient launches store dX (rank 0) and
  // add to it (later ranks), so only d_topk (atomic partial sums over column
  // blocks) needs zeros.  On the matrix-core path the weight gradient runs
  // first and writes those zeros on the side (it reads neither); the kernel
  // boundary orders them before the input-gradient kernel.  Otherwise one fill.
  const bool ranked = mfma && (dX || d_topk) && use_ranked(s, K, true);
  if (ranked && !fits(s.T, K, MOE_F32)) return MOE_ERR_LIMIT;
  const size_t dxz_bytes = ranked ? 0 : dx_bytes;
  const bool dw_first = mfma && dW != nullptr;
  if (dw_first)
    e = timed(F_DW, st, [&] {
      return mfma_bwd_dw(dY, x, s, dW, (int)K, (int)N, dxz_bytes ? dX : nullptr, dxz_bytes,
                         d_topk, dt_bytes, st);
    });
  else if (dxz_bytes || dt_bytes)
    e = timed(F_FILL, st, [&] {
      return launch_fill_zero(dxz_bytes ? dX : nullptr, dxz_bytes, d_topk, dt_bytes, st);
    });
  if (e == hipSuccess && (dX || d_topk))
    e = timed(F_DX, st, [&] {
      return mfma ? mfma_bwd_dx(dY, x, W, s, dX, d_topk, (int)K, (int)N, ranked, st)
                  : simt_bwd_dx(dY, x, W, s, dX, d_topk, (int)K, (int)N, dtype, st);
    });
  if (e == hipSuccess && dW && !dw_first)
    e = timed(F_DW, st, [&] { return simt_bwd_dw(dY, x, s, dW, (int)K, (int)N, dtype, st); });
  return hip_status(e);
}

int moe_tile_map(const moe_schedule *sched, int64_t N, int32_t BM, int32_t BN, int32_t *tile_start,
                 int32_t *total, int32_t *owner, int64_t owner_capacity, void *stream) {
  int rc = check_sched(sched);
  if (rc) return rc;
  if (bm_index(BM) < 0 || BN < 1 || N < 1 || N >= kMax32 || owner_capacity < 0) return MOE_ERR_SHAPE;
  if (!tile_start || !total || (owner_capacity > 0 && !owner)) return MOE_ERR_NULL;
  hipStream_t st = (hipStream_t)stream;
  return hip_status(timed(F_TILEMAP, st, [&] {
    return launch_tile_map(*sched, (int)N, BM, BN, tile_start, total, owner, owner_capacity, st);
  }));
}

int moe_set_tile_rows(int32_t rows) { return set_tile_rows(rows); }

int moe_set_combine(int32_t mode) {
  if (mode != MOE_COMBINE_AUTO && mode != MOE_COMBINE_ATOMIC && mode != MOE_COMBINE_RANKED)
    return MOE_ERR_SHAPE;
  g_combine.store(mode, std::memory_order_relaxed);
  return MOE_OK;
}

int moe_timing_enable(int enable) {
  Timing &t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  if (enable) {
    for (auto &v : t.ev) {
      for (auto &pr : v) {
        (void)hipEventDestroy(pr.first);
        (void)hipEventDestroy(pr.second);
      }
      v.clear();
    }
  }
  t.on = enable != 0;
  return MOE_OK;
}

int moe_timing_read(const char *family, double *total_ms, int64_t *launches) {
  if (!family || !total_ms || !launches) return MOE_ERR_NULL;
  const int f = family_index(family);
  if (f < 0) return MOE_ERR_SHAPE;
  Timing &t = timing();
  std::lock_guard<std::mutex> g(t.mu);
  double sum = 0.0;
  for (auto &pr : t.ev[f]) {
    if (hipEventSynchronize(pr.second) != hipSuccess) return MOE_ERR_HIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, pr.first, pr.second) != hipSuccess) return MOE_ERR_HIP;
    sum += ms;
  }
  *total_ms = sum;
  *launches = (int64_t)t.ev[f].size();
  return MOE_OK;
}

}  // extern "C"
