// Shared device/host helpers of the MoE grouped GEMM library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/moe_vs.h"

#define MOE_DEV __device__ __forceinline__

namespace moe {

typedef uint16_t bf16_t;  // raw bfloat16 bit pattern

constexpr int kWave = 64;            // CDNA wavefront width
constexpr int kMaxExperts = 1024;    // E limit (LDS-resident per-expert tables)
constexpr int kRowPad = 64;          // spare entries after each schedule row array
constexpr int kMaxRankK = 8;         // rank-ordered view: at most this many slots per token
constexpr int kMaxRankKeys = 1024;   // ... and k * E groups
// completion counters of the ranked combine: [kMaxRankK][kRankSyncCols] words,
// then a finished-workgroup count and a count of waits that gave up
constexpr int kRankSyncCols = 64;    // at most 64 output column blocks of 256
constexpr int kRankSyncInts = kMaxRankK * kRankSyncCols + 2;
constexpr int kBmValues[MOE_NUM_BM] = {32, 64, 128, 256};

MOE_DEV float bf16_to_f32(bf16_t v) { return __uint_as_float(((uint32_t)v) << 16); }

// fp32 -> bf16, round to nearest even (inputs are finite).
MOE_DEV bf16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (bf16_t)(u >> 16);
}

MOE_DEV int cdiv(int a, int b) { return (a + b - 1) / b; }

// Index of the bm value in block_start (32 << i).
__host__ __device__ inline int bm_index(int bm) {
  return bm == 32 ? 0 : bm == 64 ? 1 : bm == 128 ? 2 : bm == 256 ? 3 : -1;
}

// Owner of flat tile `tau`: upper bound of tau in starts[0..E) (non-decreasing,
// starts[0] = 0), minus one.  With empty groups several starts are equal; the
// upper bound lands after all of them, on the one group that owns tiles there.
template <typename Idx>
MOE_DEV int upper_bound_minus_one(const Idx *starts, int E, Idx tau) {
  int lo = 0, hi = E;  // first index with starts[i] > tau lies in [lo, hi]
  while (lo < hi) {
    int mid = (lo + hi) >> 1;
    if (starts[mid] <= tau) lo = mid + 1; else hi = mid;
  }
  return lo - 1;
}

// Buffer resource for raw (untyped) buffer loads: an access whose offset is at
// or beyond num_records bytes returns zero instead of touching memory.
MOE_DEV __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t num_records) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)num_records,
                                           0x00020000);
}

// An offset that is always out of range for a buffer of < 2^31 bytes, even after
// adding any in-range byte offset of a row.
constexpr uint32_t kOobOffset = 0x80000000u;

}  // namespace moe

// Internal launchers implemented in the .hip files (C++ linkage, not exported).
namespace moe {
struct LaunchCtx {
  hipStream_t stream;
  int num_cu;
};
int device_cu_count();

// scratch: schedule_scratch_bytes(S, E, k, s.phases > 0) bytes of device
// memory (part of the caller's schedule workspace)
hipError_t launch_build_schedule(const int32_t *ids, const float *w, const moe_schedule &s,
                                 int32_t *scratch, hipStream_t st);
size_t schedule_scratch_bytes(int64_t S, int E, int k, bool ranked);
// the current device's static block tables for the build (address and size);
// shared by every call on that device
hipError_t static_schedule_scratch(int32_t **tables, size_t *bytes);
// whether the schedule also gets the rank-ordered row view (one phase per rank)
bool rank_order_supported(int layout, int k, int E);
hipError_t launch_tile_map(const moe_schedule &s, int N, int BM, int BN, int32_t *tile_start,
                           int32_t *total, int32_t *owner, int64_t owner_cap, hipStream_t st);
// zero [p, p + bytes) and [p2, p2 + bytes2) in one launch (either pointer may be
// NULL); 16-byte stores cover whole multiples of 16 bytes from each start (4-byte
// aligned), byte stores the rest
hipError_t launch_fill_zero(void *p, size_t bytes, void *p2, size_t bytes2, hipStream_t st);

// fp32 / generic SIMT path
hipError_t simt_grouped_gemm(const void *A, const void *W, const int32_t *offsets, void *C,
                             int M, int K, int N, int E, int dtype, int out_dtype,
                             hipStream_t st);
hipError_t simt_fused_fwd(const void *x, const void *W, const moe_schedule &s, float *y, int K,
                          int N, int dtype, hipStream_t st);
hipError_t simt_bwd_dx(const void *dY, const void *x, const void *W, const moe_schedule &s,
                       float *dX, float *d_w, int K, int N, int dtype, hipStream_t st);
hipError_t simt_bwd_dw(const void *dY, const void *x, const moe_schedule &s, void *dW, int K,
                       int N, int dtype, hipStream_t st);
// gated expert FFN on the vector ALUs (fp32, or bf16 with K, F or N not a
// multiple of 8): h [R, F] and dgu [R, 2F] in the input dtype, gu [R, 2F] fp32
hipError_t simt_gated_up(const void *x, const void *W_gu, const moe_schedule &s, void *h,
                         float *gu, int K, int F, int dtype, hipStream_t st);
hipError_t simt_gated_down(const void *h, const void *W_down, const moe_schedule &s, float *y,
                           int F, int N, int dtype, hipStream_t st);
hipError_t simt_gated_bwd_dh(const void *dY, const void *h, const void *W_down,
                             const moe_schedule &s, float *d_w, int F, int N, const float *gu,
                             void *dgu, int dtype, hipStream_t st);
hipError_t simt_gated_bwd_dx(const void *dgu, const void *W_gu, const moe_schedule &s, float *dX,
                             int K, int F, int dtype, hipStream_t st);
// dW[e] = sum over rows of a^T b with a (N columns) and b (K columns) read by
// schedule row (by_row) or gathered by token (dY with the routing weight)
hipError_t simt_bwd_dw_rows(const void *A, bool a_by_row, const void *B, bool b_by_row,
                            const moe_schedule &s, void *dW, int K, int N, int dtype,
                            hipStream_t st);

// bf16 MFMA path
bool mfma_supported(int K, int N);
// process-wide tile height of the routed kernels: 0 (device pick), 128 or 256
int set_tile_rows(int rows);
hipError_t mfma_grouped_gemm(const void *A, const void *W, const int32_t *offsets, void *C,
                             int M, int K, int N, int E, int out_dtype, hipStream_t st);
// a_by_row: the A operand is already in schedule row order ([R, K]) instead of
// being gathered from x [T, K] by token
// ranked: one launch over the schedule's rank-ordered view whose rank-0 tiles
// store and whose later ranks add in rank order (no atomics, y need not be
// zeroed); otherwise one launch adding atomically into a zeroed y
hipError_t mfma_fused_fwd(const void *x, const void *W, const moe_schedule &s, float *y, int K,
                          int N, bool a_by_row, bool ranked, hipStream_t st);
// 8-bit (E4M3) operands: y[t] += w * x_scale[t] * w_scale[e, n] * (xq[t] . Wq[e, n]);
// K a multiple of 16 (16-byte rows)
hipError_t mfma_fused_fwd_fp8(const void *xq, const float *x_scale, const void *Wq,
                              const float *w_scale, const moe_schedule &s, float *y, int K, int N,
                              bool ranked, hipStream_t st);
// 8-bit (E4M3) operands with E8M0 block scales per 32 reduction elements:
// x_bs [T, K/32], w_bs [E, N, K/32]; K a multiple of 128
hipError_t mfma_fused_fwd_mx(const void *xq, const uint8_t *x_bs, const void *Wq,
                             const uint8_t *w_bs, const moe_schedule &s, float *y, int K, int N,
                             bool ranked, hipStream_t st);
// h [R, F] bf16 = silu(x W_gate^T) * (x W_up^T) per schedule row; W_gu [E, 2F, K]
// gu (optional, NULL to skip): [R, 2F] fp32 gate and up values kept for a backward
hipError_t mfma_gated_up(const void *x, const void *W_gu, const moe_schedule &s, void *h, void *gu,
                         int K, int F, hipStream_t st);
// ranked: as for mfma_fused_fwd (dX need not be zeroed; d_w must be)
hipError_t mfma_bwd_dx(const void *dY, const void *x, const void *W, const moe_schedule &s,
                       float *dX, float *d_w, int K, int N, bool ranked, hipStream_t st);
// zero0 / zero1: byte ranges the kernel zeroes on the side (NULL / 0 when unused)
hipError_t mfma_bwd_dw(const void *dY, const void *x, const moe_schedule &s, void *dW, int K,
                       int N, float *zero0, size_t zero0_bytes, float *zero1, size_t zero1_bytes,
                       hipStream_t st);
// dW[e] = sum over rows r of e of (w_r? dY[.])^T x[.], each operand read by token
// or, with *_by_row, by schedule row (an operand already in schedule order)
hipError_t mfma_bwd_dw_rows(const void *dY, bool dy_by_row, const void *x, bool x_by_row,
                            const moe_schedule &s, void *dW, int K, int N, bool weighted,
                            float *zero0, size_t zero0_bytes, float *zero1, size_t zero1_bytes,
                            hipStream_t st);
// gated FFN backward, first step: G = dY W_down (dY by token), d_w += <G, h>
// (h [R, F] by row), dgu [R, 2F] = (dh u silu'(g) | dh silu(g)), dh = w G
hipError_t mfma_gated_bwd_dh(const void *dY, const void *h, const void *W_down,
                             const moe_schedule &s, float *d_w, int F, int N, const void *gu,
                             void *dgu, hipStream_t st);
// gated FFN backward: dX[t] += dgu[r] W_gu[e] (dgu by row, unweighted scatter)
hipError_t mfma_gated_bwd_dx(const void *dgu, const void *W_gu, const moe_schedule &s, float *dX,
                             int K, int F, hipStream_t st);
}  // namespace moe

namespace moe {

// Per-group tables every grouped kernel keeps in LDS: row-block prefix `bs`
// ([E+1]), first row `rstart` and valid rows `rcnt` of each group.
// Filled by all NT threads of the block; ends with a barrier.

// Block-wide exclusive scan of one int per thread; scratch holds NT/64 + 1 ints.
template <int NT>
MOE_DEV int block_scan_excl(int v, int *scratch, int *total) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  int inc = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    int t = __shfl_up(inc, d, kWave);
    if (lane >= d) inc += t;
  }
  if (lane == kWave - 1) scratch[wid] = inc;
  __syncthreads();
  if (threadIdx.x == 0) {
    int run = 0;
    for (int i = 0; i < NW; ++i) {
      int c = scratch[i];
      scratch[i] = run;
      run += c;
    }
    scratch[NW] = run;
  }
  __syncthreads();
  int r = scratch[wid] + inc - v;
  *total = scratch[NW];
  __syncthreads();
  return r;
}

// Tables from END offsets (bare grouped GEMM): m_e = offs[e] - offs[e-1].
template <int NT>
MOE_DEV void group_tables_from_offsets(const int32_t *__restrict__ offsets, int E, int BM, int *bs,
                                       int *rstart, int *rcnt, int *scratch) {
  const int per = (E + NT - 1) / NT;
  const int e0 = threadIdx.x * per;
  int local = 0;
  for (int i = 0; i < per; ++i) {
    const int e = e0 + i;
    if (e < E) {
      const int lo = e == 0 ? 0 : offsets[e - 1];
      const int m = max(0, offsets[e] - lo);
      rstart[e] = lo;
      rcnt[e] = m;
      local += (m + BM - 1) / BM;
    }
  }
  int total;
  int pre = block_scan_excl<NT>(local, scratch, &total);
  for (int i = 0; i < per; ++i) {
    const int e = e0 + i;
    if (e < E) {
      bs[e] = pre;
      pre += (rcnt[e] + BM - 1) / BM;
    }
  }
  if (threadIdx.x == 0) bs[E] = total;
  __syncthreads();
}

// Tables from a routing schedule (either layout).
template <int NT>
MOE_DEV void group_tables_from_schedule(const int32_t *__restrict__ counts,
                                        const int32_t *__restrict__ offsets,
                                        const int32_t *__restrict__ bstart, int E, int layout,
                                        int capacity, int *bs, int *rstart, int *rcnt) {
  // bstart may be a window of a longer prefix (one rank's groups of the
  // rank-ordered view): entries are taken relative to its first
  const int b0 = bstart[0];
  for (int e = threadIdx.x; e <= E; e += NT) {
    bs[e] = bstart[e] - b0;
    if (e < E) {
      const int c = counts[e];
      rcnt[e] = c;
      rstart[e] = layout == MOE_LAYOUT_MASKED ? e * capacity : offsets[e] - c;
    }
  }
  __syncthreads();
}

// Tile tau of a flat space with tiles_n column blocks per row block, walked
// column-block-major inside each group.
struct TileCoord {
  int g;      // owning group
  int mb;     // row block inside the group
  int nb;     // column block
  int row0;   // first row (row space of the schedule / of A)
  int rows;   // valid rows in this tile (<= BM)
};

MOE_DEV TileCoord tile_coord(const int *bs, const int *rstart, const int *rcnt, int E, int tau,
                             int tiles_n, int BM) {
  TileCoord c;
  c.g = upper_bound_minus_one(bs, E, tau / tiles_n);
  const int local = tau - bs[c.g] * tiles_n;
  const int mblocks = bs[c.g + 1] - bs[c.g];
  c.nb = local / mblocks;
  c.mb = local - c.nb * mblocks;
  c.row0 = rstart[c.g] + c.mb * BM;
  c.rows = min(BM, rcnt[c.g] - c.mb * BM);
  // the same for every lane (tau is): keep the coordinates in scalar registers
  c.g = __builtin_amdgcn_readfirstlane(c.g);
  c.mb = __builtin_amdgcn_readfirstlane(c.mb);
  c.nb = __builtin_amdgcn_readfirstlane(c.nb);
  c.row0 = __builtin_amdgcn_readfirstlane(c.row0);
  c.rows = __builtin_amdgcn_readfirstlane(c.rows);
  return c;
}

}  // namespace moe
