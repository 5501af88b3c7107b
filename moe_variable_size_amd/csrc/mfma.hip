// bf16 grouped GEMM kernels on the gfx950 matrix cores (MFMA), fp32 accumulation.
//
// [GG] = "Grouped GEMM for MoE, in depth" (aicassindra.com)
// [CARD] = "grouped-gemm-moe" model card
// [NOTE] = "Grouped GEMM" study notes (scholia-log)
//
// All kernels share one tile core:
//   * a workgroup of 4 waves (WGM x WGN) owns a BM x BN output tile made of
//     32 x 32 blocks, each block one v_mfma_f32_32x32x16_bf16 accumulator (16
//     fp32 per lane); wave (wm, wn) owns row blocks wm, wm + WGM, ... and column
//     blocks wn, wn + WGN, ... (interleaved, so that a wave's LDS addresses differ
//     by constants and fit in instruction offsets);
//   * the reduction advances 64 elements per stage; both operands sit in LDS as
//     [operand row][64 reduction elements] (128 bytes per row), with the eight
//     16-byte chunks of a row XOR-swizzled by the row index so that the 16-byte
//     MFMA operand reads and the 16-byte stores both spread over all banks;
//   * two LDS stages: while the waves multiply stage i, the global loads of stage
//     i+1 are in flight into registers and are stored to the other stage after the
//     multiply ([GG] "Problem descriptors and the tile scheduler": the per-tile K
//     loop; [CARD] "How it works": the next chunk streams while the current one
//     computes);
//   * global loads are raw buffer loads: an out-of-range offset returns zeros, so
//     rows past a group's end, columns past N and reduction chunks past K are
//     masked without branches and without touching memory ([GG] "Problem
//     descriptors and the tile scheduler": ragged rows masked on load and store).
//
// Operands whose reduction index is the contiguous one ("K-major": token rows,
// weight rows in the forward) are stored to LDS as loaded.  Operands whose
// reduction index is strided (the weights in the input gradient, both operands
// of the weight gradient) are loaded as 8 x 8 element blocks and transposed in
// registers before the store.
//
// The persistent grid has one workgroup per compute unit.  Workgroup ids are
// remapped so that the 8 XCDs (each with its own L2) each take one contiguous
// slice of the flat tile space; inside a group tiles are walked
// column-block-major, so the workgroups of one XCD share the same weight column
// blocks ([GG] "Problem descriptors and the tile scheduler", reuse of B_g from
// L2).
#include "common.hpp"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int NT = 256;        // 4 waves
constexpr int BK = 64;         // reduction elements per stage
constexpr int ROWB = BK * 2;   // bytes per LDS operand row

// Byte offset of 16-byte chunk `chunk` (0..7) of LDS operand row `row`.
MOE_DEV int lds_off(int row, int chunk) {
  return row * ROWB + ((chunk ^ ((row ^ (row >> 3)) & 7)) << 4);
}

MOE_DEV u32x4 bload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
}

MOE_DEV void lds_store(char *lds, int off, u32x4 v) { *(u32x4 *)(lds + off) = v; }

// Logical workgroup id: consecutive ids land on one XCD (the hardware deals
// workgroup ids to the 8 XCDs round robin).
MOE_DEV int logical_block() {
  const int G = gridDim.x, b = blockIdx.x;
  return (G & 7) ? b : (b & 7) * (G >> 3) + (b >> 3);
}

// One stage of the tile multiply: 4 steps of 16 reduction elements.  The
// operand fragments of step s+1 are read from LDS while step s multiplies.
// A rows of the wave: a_row0 + mi * a_str + (0..31); B rows: b_row0 + ni * b_str.
// SKIP: row blocks at or past `live_mi` (no valid row) skip their MFMAs.
template <int MI, int NI, bool SKIP>
MOE_DEV void mma_stage(const char *As, const char *Bs, int a_row0, int a_str, int b_row0,
                       int b_str, int lane, int live_mi, f32x16 (&acc)[MI][NI]) {
  bf16x8_t a[2][MI], b[2][NI];
  auto frag = [&](int s, int buf) __attribute__((always_inline)) {
    const int ch = 2 * s + (lane >> 5);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
      a[buf][mi] = *(const bf16x8_t *)(As + lds_off(a_row0 + mi * a_str + (lane & 31), ch));
#pragma unroll
    for (int ni = 0; ni < NI; ++ni)
      b[buf][ni] = *(const bf16x8_t *)(Bs + lds_off(b_row0 + ni * b_str + (lane & 31), ch));
  };
  frag(0, 0);
#pragma unroll
  for (int s = 0; s < BK / 16; ++s) {
    if (s + 1 < BK / 16) frag(s + 1, (s + 1) & 1);
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      if (SKIP && mi >= live_mi) continue;  // wave-uniform
#pragma unroll
      for (int ni = 0; ni < NI; ++ni)
        acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s & 1][mi], b[s & 1][ni],
                                                              acc[mi][ni], 0, 0, 0);
    }
  }
}

// 8 x 8 transpose of bf16 straight into LDS: in[r] holds row r (8 elements,
// element 2d in the low half of dword d); column c (rows 0..7) is stored as one
// 16-byte chunk at LDS operand row row0 + c, chunk `chunk`.
MOE_DEV void transpose8x8_store(const u32x4 (&in)[8], char *lds, int row0, int chunk) {
#pragma unroll
  for (int c = 0; c < 8; ++c) {
    const uint32_t sel = (c & 1) ? 0x07060302u : 0x05040100u;
    u32x4 o;
#pragma unroll
    for (int p = 0; p < 4; ++p)  // low half: row 2p, high half: row 2p+1, column c
      o[p] = __builtin_amdgcn_perm(in[2 * p + 1][c >> 1], in[2 * p][c >> 1], sel);
    lds_store(lds, lds_off(row0 + c, chunk), o);
  }
}

// Row r of a 32x32 MFMA accumulator held in register i of lane `lane`.
MOE_DEV int acc_row(int i, int lane) { return ((i >> 2) << 3) + ((lane >> 5) << 2) + (i & 3); }

// ============================================================================
// Forward-shaped kernel: out[r, n] = sum_k A[src(r), k] * W[g, n, k].
//   FUSED: src(r) = row_to_token[r], y[src(r), n] += row_weight[r] * acc
//          (atomic; rows of both layouts) -- [CARD] gather on load,
//          scatter-combine on store.
//   bare : src(r) = r, C[r, n] = acc (plain store, fp32 or bf16).
// ============================================================================
struct FwdArgs {
  const bf16_t *A;
  const bf16_t *W;
  void *C;
  const int32_t *offsets;
  const int32_t *counts;
  const int32_t *bstart;
  const int32_t *row_to_token;
  const float *row_weight;
  int E, layout, capacity, K, N;
  uint32_t a_bytes;  // bytes of A (x or the bare A)
  int stream_k;      // 1: split the (tile, stage) space evenly over workgroups
  int M;             // bare: rows of A and C (rows at or past M are never touched)
};

template <int BM, int BN, int WGM, int WGN, bool FUSED, typename Tout>
__global__ __launch_bounds__(NT) void mfma_fwd_kernel(FwdArgs p) {
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int MI = WTM / 32, NI = WTN / 32;
  constexpr int CA = BM / 32, CB = BN / 32;  // 16-byte chunks per thread per stage
  static_assert(WGM * WGN == 4, "4 waves");
  extern __shared__ __attribute__((aligned(16))) char lds[];  // 2 stages x (BM + BN) rows
  __shared__ int bs[kMaxExperts + 1], rstart[kMaxExperts], rcnt[kMaxExperts];
  __shared__ __attribute__((aligned(16))) int tok[BM];
  __shared__ __attribute__((aligned(16))) float wgt[BM];
  __shared__ int scratch[NT / kWave + 1];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid / WGN, wn = wid % WGN;
  const int E = p.E, K = p.K, N = p.N;
  if (FUSED)
    group_tables_from_schedule<NT>(p.counts, p.offsets, p.bstart, E, p.layout, p.capacity, bs,
                                   rstart, rcnt);
  else
    group_tables_from_offsets<NT>(p.offsets, E, BM, bs, rstart, rcnt, scratch);

  const int tiles_n = (N + BN - 1) / BN;
  const int KI = (K + BK - 1) / BK;
  const int total = bs[E] * tiles_n;
  const __amdgpu_buffer_rsrc_t rsA = make_rsrc(p.A, p.a_bytes);
  const uint32_t wbytes = (uint32_t)N * K * 2;
  const int ch = tid & 7, rsub = tid >> 3;

  const int G = gridDim.x, Lb = logical_block();
  const bool sk = p.stream_k != 0;
  const int64_t tot_it = (int64_t)total * KI;
  int64_t it = sk ? tot_it * Lb / G : (int64_t)Lb * KI;
  int64_t it_end = sk ? tot_it * (Lb + 1) / G : min(tot_it, it + KI);
  // stream-K: one contiguous slice of the (tile, stage) space per workgroup;
  // otherwise whole tiles Lb, Lb + G, ...
  for (; it < it_end;) {
    const int tau = (int)(it / KI);
    const int kb = (int)(it - (int64_t)tau * KI);
    const int ke = (int)min((int64_t)KI, kb + (it_end - it));
    it += ke - kb;
    if (!sk && it >= it_end) {
      it += (int64_t)(G - 1) * KI;
      it_end = min(tot_it, it + KI);
    }
    const TileCoord c = tile_coord(bs, rstart, rcnt, E, tau, tiles_n, BM);
    if (c.rows <= 0) continue;
    const int n0 = c.nb * BN;
    __syncthreads();  // LDS stages and row tables free
    if (tid < BM) {
      const bool ok = tid < c.rows;
      const int r = c.row0 + tid;
      tok[tid] = ok ? (FUSED ? p.row_to_token[r] : (r < p.M ? r : -1)) : -1;
      wgt[tid] = (FUSED && ok) ? p.row_weight[r] : 0.f;
    }
    __syncthreads();
    const __amdgpu_buffer_rsrc_t rsW = make_rsrc(p.W + (size_t)c.g * N * K, wbytes);
    uint32_t ao[CA], bo[CB];
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int t = tok[rsub + 32 * i];
      ao[i] = t >= 0 ? (uint32_t)t * (uint32_t)K * 2u + ch * 16 : kOobOffset;
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const int n = n0 + rsub + 32 * i;
      bo[i] = n < N ? (uint32_t)n * (uint32_t)K * 2u + ch * 16 : kOobOffset;
    }
    const int live_mi = min(MI, max(0, (c.rows - wm * 32 + 32 * WGM - 1) / (32 * WGM)));
    f32x16 acc[MI][NI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = f32x16{};

    u32x4 ra[CA], rb[CB];
    auto gload = [&](int kt) {
      const bool kin = kt * BK + ch * 8 < K;
      const uint32_t dk = (uint32_t)kt * ROWB;
#pragma unroll
      for (int i = 0; i < CA; ++i) ra[i] = bload(rsA, kin ? ao[i] + dk : kOobOffset);
#pragma unroll
      for (int i = 0; i < CB; ++i) rb[i] = bload(rsW, kin ? bo[i] + dk : kOobOffset);
    };
    auto sstore = [&](int stage) {
      char *As = lds + stage * (BM + BN) * ROWB;
      char *Bs = As + BM * ROWB;
#pragma unroll
      for (int i = 0; i < CA; ++i) lds_store(As, lds_off(rsub + 32 * i, ch), ra[i]);
#pragma unroll
      for (int i = 0; i < CB; ++i) lds_store(Bs, lds_off(rsub + 32 * i, ch), rb[i]);
    };
    gload(kb);
    sstore(0);
    __syncthreads();
    for (int kt = kb; kt < ke; ++kt) {
      const int cur = (kt - kb) & 1;
      const bool more = kt + 1 < ke;
      if (more) gload(kt + 1);
      const char *As = lds + cur * (BM + BN) * ROWB;
      mma_stage<MI, NI, (BM <= 64)>(As, As + BM * ROWB, wm * 32, 32 * WGM, wn * 32, 32 * WGN,
                                    lane, live_mi, acc);
      if (more) sstore(cur ^ 1);
      __syncthreads();
    }
    // epilogue: 4 consecutive accumulator rows share one 16-byte read of the
    // row tables; each row's base address is formed once for all column blocks
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      if (BM <= 64 && mi >= live_mi) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rq = wm * 32 + mi * 32 * WGM + 8 * j + 4 * (lane >> 5);
        const i32x4 t4 = *(const i32x4 *)(tok + rq);
        const f32x4 w4 = *(const f32x4 *)(wgt + rq);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int t = t4[q];
          if (t < 0) continue;
          const size_t rowoff = (size_t)t * N;
#pragma unroll
          for (int ni = 0; ni < NI; ++ni) {
            const int col = n0 + wn * 32 + ni * 32 * WGN + (lane & 31);
            if (col >= N) continue;
            const float v = acc[mi][ni][4 * j + q];
            if (FUSED) {
              unsafeAtomicAdd((float *)p.C + rowoff + col, w4[q] * v);
            } else if (sizeof(Tout) == 4) {
              ((float *)p.C)[rowoff + col] = v;
            } else {
              ((bf16_t *)p.C)[rowoff + col] = f32_to_bf16(v);
            }
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// ============================================================================
// Input gradient (+ routing-weight gradient):
//   G[r, kc] = sum_n dY[tok(r), n] * W[g, n, kc]           (MFMA, fp32 acc)
//   dX[tok(r), kc] += w_r * G[r, kc]                       (atomic)
//   d_w[assign(r)] += sum_{kc in tile} G[r, kc] * x[tok(r), kc]   (atomic)
// [GG] "The backward pass": the forward pattern with the weights transposed;
// [CARD] "How it works": the same gather / scatter-combine as the forward, and
// the routing-weight gradient as the inner product of dY with the unweighted
// product, here taken through the identity <dY W_e, x> = <dY, x W_e^T>.
// ============================================================================
struct DxArgs {
  const bf16_t *dY;
  const bf16_t *x;
  const bf16_t *W;
  float *dX;
  float *d_w;
  const int32_t *offsets;
  const int32_t *counts;
  const int32_t *bstart;
  const int32_t *row_to_assign;
  const int32_t *row_to_token;
  const float *row_weight;
  int E, layout, capacity, K, N;
  uint32_t dy_bytes;
  int stream_k;
};

template <int BM, int BN, int WGM, int WGN>
__global__ __launch_bounds__(NT) void mfma_dx_kernel(DxArgs p) {
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int MI = WTM / 32, NI = WTN / 32;
  constexpr int CA = BM / 32;
  static_assert(BN == 256, "transposing loader covers 256 output columns");
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ int bs[kMaxExperts + 1], rstart[kMaxExperts], rcnt[kMaxExperts];
  __shared__ __attribute__((aligned(16))) int tok[BM];
  __shared__ __attribute__((aligned(16))) float wgt[BM];
  __shared__ __attribute__((aligned(16))) int asg[BM];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid / WGN, wn = wid % WGN;
  const int E = p.E, K = p.K, N = p.N;
  group_tables_from_schedule<NT>(p.counts, p.offsets, p.bstart, E, p.layout, p.capacity, bs,
                                 rstart, rcnt);
  const int tiles_n = (K + BN - 1) / BN;  // output columns run over K
  const int KI = (N + BK - 1) / BK;       // reduction runs over N
  const int total = bs[E] * tiles_n;
  const __amdgpu_buffer_rsrc_t rsA = make_rsrc(p.dY, p.dy_bytes);
  const uint32_t wbytes = (uint32_t)N * K * 2;
  const int ch = tid & 7, rsub = tid >> 3;
  const int cb = tid & 31, nb = tid >> 5;  // transposing loader: 8 cols x 8 rows block

  const int G = gridDim.x, Lb = logical_block();
  const bool sk = p.stream_k != 0;
  const int64_t tot_it = (int64_t)total * KI;
  int64_t it = sk ? tot_it * Lb / G : (int64_t)Lb * KI;
  int64_t it_end = sk ? tot_it * (Lb + 1) / G : min(tot_it, it + KI);
  // stream-K: one contiguous slice of the (tile, stage) space per workgroup;
  // otherwise whole tiles Lb, Lb + G, ...
  for (; it < it_end;) {
    const int tau = (int)(it / KI);
    const int kb = (int)(it - (int64_t)tau * KI);
    const int ke = (int)min((int64_t)KI, kb + (it_end - it));
    it += ke - kb;
    if (!sk && it >= it_end) {
      it += (int64_t)(G - 1) * KI;
      it_end = min(tot_it, it + KI);
    }
    const TileCoord c = tile_coord(bs, rstart, rcnt, E, tau, tiles_n, BM);
    if (c.rows <= 0) continue;
    const int kc0 = c.nb * BN;
    __syncthreads();
    if (tid < BM) {
      const bool ok = tid < c.rows;
      const int r = c.row0 + tid;
      tok[tid] = ok ? p.row_to_token[r] : -1;
      wgt[tid] = ok ? p.row_weight[r] : 0.f;
      asg[tid] = ok ? p.row_to_assign[r] : -1;
    }
    __syncthreads();
    const __amdgpu_buffer_rsrc_t rsW = make_rsrc(p.W + (size_t)c.g * N * K, wbytes);
    uint32_t ao[CA];
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int t = tok[rsub + 32 * i];
      ao[i] = t >= 0 ? (uint32_t)t * (uint32_t)N * 2u + ch * 16 : kOobOffset;
    }
    const int kcol = kc0 + cb * 8;
    const bool col_ok = kcol < K;
    const int live_mi = min(MI, max(0, (c.rows - wm * 32 + 32 * WGM - 1) / (32 * WGM)));
    f32x16 acc[MI][NI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = f32x16{};

    u32x4 ra[CA], rb[8];
    auto gload = [&](int kt) {
      const bool kin = kt * BK + ch * 8 < N;
      const uint32_t dk = (uint32_t)kt * ROWB;
#pragma unroll
      for (int i = 0; i < CA; ++i) ra[i] = bload(rsA, kin ? ao[i] + dk : kOobOffset);
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int n = kt * BK + nb * 8 + j;
        rb[j] = bload(rsW, (col_ok && n < N) ? (uint32_t)n * (uint32_t)K * 2u + (uint32_t)kcol * 2u
                                              : kOobOffset);
      }
    };
    auto sstore = [&](int stage) {
      char *As = lds + stage * (BM + BN) * ROWB;
      char *Bs = As + BM * ROWB;
#pragma unroll
      for (int i = 0; i < CA; ++i) lds_store(As, lds_off(rsub + 32 * i, ch), ra[i]);
      transpose8x8_store(rb, Bs, cb * 8, nb);
    };
    gload(kb);
    sstore(0);
    __syncthreads();
    for (int kt = kb; kt < ke; ++kt) {
      const int cur = (kt - kb) & 1;
      const bool more = kt + 1 < ke;
      if (more) gload(kt + 1);
      const char *As = lds + cur * (BM + BN) * ROWB;
      mma_stage<MI, NI, (BM <= 64)>(As, As + BM * ROWB, wm * 32, 32 * WGM, wn * 32, 32 * WGN,
                                    lane, live_mi, acc);
      if (more) sstore(cur ^ 1);
      __syncthreads();
    }
    // epilogue: weighted atomic scatter of G into dX and, per row, the partial
    // inner product of G with x over this tile's columns into d_w
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
      if (BM <= 64 && mi >= live_mi) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rq = wm * 32 + mi * 32 * WGM + 8 * j + 4 * (lane >> 5);
        const i32x4 t4 = *(const i32x4 *)(tok + rq);
        const f32x4 w4 = *(const f32x4 *)(wgt + rq);
        const i32x4 a4 = *(const i32x4 *)(asg + rq);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int t = t4[q];
          float part = 0.f;
          if (t >= 0) {
            const size_t rowoff = (size_t)t * K;
#pragma unroll
            for (int ni = 0; ni < NI; ++ni) {
              const int col = kc0 + wn * 32 + ni * 32 * WGN + (lane & 31);
              if (col >= K) continue;
              const float g = acc[mi][ni][4 * j + q];
              if (p.dX) unsafeAtomicAdd(p.dX + rowoff + col, w4[q] * g);
              if (p.d_w) part = fmaf(g, bf16_to_f32(p.x[rowoff + col]), part);
            }
          }
          if (p.d_w) {
            // lanes 0-31 hold one row, lanes 32-63 another
#pragma unroll
            for (int d = 16; d >= 1; d >>= 1) part += __shfl_xor(part, d, 32);
            if ((lane & 31) == 0 && t >= 0) unsafeAtomicAdd(p.d_w + a4[q], part);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// ============================================================================
// Weight gradient: dW[e, n, kc] = sum over rows r of e of (w_r dY[tok(r), n]) x[tok(r), kc].
// [GG] "The backward pass": a grouped GEMM whose reduction length (the group's
// rows) varies; every expert's output is written, zeros for an empty one.  Work
// units (expert, 256 x 256 output tile) are taken in descending expert load and
// dealt to workgroups in a snake order, so the longest reductions start first
// and the per-workgroup sums even out ([NOTE] 4.2: hot experts get more work
// units and the persistent workgroups absorb the imbalance).
// The routing weight is applied to dY in fp32 and rounded to bf16 before the
// multiply (one bf16 rounding per product).
// ============================================================================
struct DwArgs {
  const bf16_t *dY;
  const bf16_t *x;
  void *dW;
  const int32_t *offsets;
  const int32_t *counts;
  const int32_t *expert_order;
  const int32_t *row_to_token;
  const float *row_weight;
  int E, layout, capacity, K, N;
  uint32_t dy_bytes, x_bytes;
  int weighted;
};

template <typename Tout>
__global__ __launch_bounds__(NT) void mfma_dw_kernel(DwArgs p) {
  constexpr int BM = 256, BN = 256, WGM = 2, WGN = 2;
  constexpr int WTM = BM / WGM, WTN = BN / WGN;
  constexpr int MI = WTM / 32, NI = WTN / 32;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int wm = wid / WGN, wn = wid % WGN;
  const int K = p.K, N = p.N, E = p.E;
  const int tn = (N + BM - 1) / BM, tk = (K + BN - 1) / BN;
  const int per_e = tn * tk;
  const int units = E * per_e;
  const int G = gridDim.x, L = logical_block();
  const __amdgpu_buffer_rsrc_t rsY = make_rsrc(p.dY, p.dy_bytes);
  const __amdgpu_buffer_rsrc_t rsX = make_rsrc(p.x, p.x_bytes);
  const int cb = tid & 31, rb = tid >> 5;

  for (int round = 0;; ++round) {
    const int base = round * G;
    if (base >= units) break;
    const int u = base + ((round & 1) ? (G - 1 - L) : L);
    if (u >= units) continue;
    const int e = p.expert_order[u / per_e];
    const int t = u - (u / per_e) * per_e;
    const int n0 = (t / tk) * BM, kc0 = (t % tk) * BN;
    const int m = p.counts[e];
    const int r0 = p.layout == MOE_LAYOUT_MASKED ? e * p.capacity : p.offsets[e] - m;
    const int ncol = n0 + cb * 8, kcol = kc0 + cb * 8;
    const bool n_ok = ncol < N, k_ok = kcol < K;
    const int KI = (m + BK - 1) / BK;

    f32x16 acc[MI][NI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = f32x16{};

    u32x4 ra[8], rbx[8];
    float wr[8];
    auto gload = [&](int kt) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int q = kt * BK + rb * 8 + j;
        const bool ok = q < m;
        const int tk_ = ok ? p.row_to_token[r0 + q] : 0;
        wr[j] = ok ? (p.weighted ? p.row_weight[r0 + q] : 1.f) : 0.f;
        ra[j] = bload(rsY, (ok && n_ok) ? (uint32_t)tk_ * (uint32_t)N * 2u + (uint32_t)ncol * 2u
                                        : kOobOffset);
        rbx[j] = bload(rsX, (ok && k_ok) ? (uint32_t)tk_ * (uint32_t)K * 2u + (uint32_t)kcol * 2u
                                         : kOobOffset);
      }
    };
    auto sstore = [&](int stage) {
      char *As = lds + stage * (BM + BN) * ROWB;
      char *Bs = As + BM * ROWB;
      if (p.weighted) {
#pragma unroll
        for (int j = 0; j < 8; ++j)
#pragma unroll
          for (int d = 0; d < 4; ++d) {
            const uint32_t v = ra[j][d];
            const bf16_t lo = f32_to_bf16(wr[j] * __uint_as_float(v << 16));
            const bf16_t hi = f32_to_bf16(wr[j] * __uint_as_float(v & 0xFFFF0000u));
            ra[j][d] = (uint32_t)lo | ((uint32_t)hi << 16);
          }
      }
      transpose8x8_store(ra, As, cb * 8, rb);
      transpose8x8_store(rbx, Bs, cb * 8, rb);
    };
    if (KI > 0) {
      __syncthreads();  // previous unit done with LDS
      gload(0);
      sstore(0);
      __syncthreads();
      for (int kt = 0; kt < KI; ++kt) {
        const int cur = kt & 1;
        const bool more = kt + 1 < KI;
        if (more) gload(kt + 1);
        const char *As = lds + cur * (BM + BN) * ROWB;
        mma_stage<MI, NI, false>(As, As + BM * ROWB, wm * 32, 32 * WGM, wn * 32, 32 * WGN, lane,
                                 MI, acc);
        if (more) sstore(cur ^ 1);
        __syncthreads();
      }
    }
    // store (exact zeros for an empty expert)
    Tout *out = (Tout *)p.dW + (size_t)e * N * K;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const int col = kc0 + wn * 32 + ni * 32 * WGN + (lane & 31);
        if (col >= K) continue;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int n = n0 + wm * 32 + mi * 32 * WGM + acc_row(i, lane);
          if (n >= N) continue;
          if (sizeof(Tout) == 4)
            ((float *)out)[(size_t)n * K + col] = acc[mi][ni][i];
          else
            ((bf16_t *)out)[(size_t)n * K + col] = f32_to_bf16(acc[mi][ni][i]);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// dynamic LDS: the two operand stages (the row tables are static LDS)
template <int BM, int BN>
constexpr size_t gemm_smem() {
  return (size_t)2 * (BM + BN) * ROWB;
}

template <typename K>
hipError_t set_smem(K kernel, size_t bytes) {
  return hipFuncSetAttribute((const void *)kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)bytes);
}

int env_int(const char *name, int dflt) {
  const char *v = getenv(name);
  return v ? atoi(v) : dflt;
}

}  // namespace

bool mfma_supported(int K, int N) { return K % 8 == 0 && N % 8 == 0; }

hipError_t mfma_grouped_gemm(const void *A, const void *W, const int32_t *offsets, void *C, int M,
                             int K, int N, int E, int out_dtype, hipStream_t st) {
  FwdArgs a{(const bf16_t *)A, (const bf16_t *)W, C, offsets, nullptr, nullptr, nullptr, nullptr,
            E, 0, 0, K, N, (uint32_t)((size_t)M * K * 2), 0, M};
  constexpr int BM = 256, BN = 256;
  const size_t smem = gemm_smem<BM, BN>();
  const dim3 grid(device_cu_count()), block(NT);
  if (out_dtype == MOE_F32) {
    auto k = mfma_fwd_kernel<BM, BN, 2, 2, false, float>;
    hipError_t e = set_smem(k, smem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k, grid, block, smem, st, a);
  } else {
    auto k = mfma_fwd_kernel<BM, BN, 2, 2, false, bf16_t>;
    hipError_t e = set_smem(k, smem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k, grid, block, smem, st, a);
  }
  return hipGetLastError();
}

hipError_t mfma_fused_fwd(const void *x, const void *W, const moe_schedule &s, float *y, int K,
                          int N, hipStream_t st) {
  const dim3 grid(device_cu_count()), block(NT);
  FwdArgs a{(const bf16_t *)x, (const bf16_t *)W, y, s.offsets, s.counts, nullptr,
            s.row_to_token, s.row_weight, s.E, s.layout, s.capacity, K, N,
            (uint32_t)((size_t)s.T * K * 2), env_int("MOE_VS_STREAM_K", 1), (int)s.T};
  if (s.layout == MOE_LAYOUT_MASKED && s.capacity <= 64) {
    constexpr int BM = 64, BN = 256;
    a.bstart = s.block_start + bm_index(BM) * (s.E + 1);
    auto k = mfma_fwd_kernel<BM, BN, 1, 4, true, float>;
    const size_t smem = gemm_smem<BM, BN>();
    hipError_t e = set_smem(k, smem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k, grid, block, smem, st, a);
  } else {
    constexpr int BM = 256, BN = 256;
    a.bstart = s.block_start + bm_index(BM) * (s.E + 1);
    auto k = mfma_fwd_kernel<BM, BN, 2, 2, true, float>;
    const size_t smem = gemm_smem<BM, BN>();
    hipError_t e = set_smem(k, smem);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k, grid, block, smem, st, a);
  }
  return hipGetLastError();
}

hipError_t mfma_bwd_dx(const void *dY, const void *x, const void *W, const moe_schedule &s,
                       float *dX, float *d_w, int K, int N, hipStream_t st) {
  constexpr int BM = 256, BN = 256;
  DxArgs a{(const bf16_t *)dY, (const bf16_t *)x, (const bf16_t *)W, dX, d_w, s.offsets,
           s.counts, s.block_start + bm_index(BM) * (s.E + 1), s.row_to_assign, s.row_to_token,
           s.row_weight, s.E, s.layout, s.capacity, K, N, (uint32_t)((size_t)s.T * N * 2),
           env_int("MOE_VS_STREAM_K", 1)};
  auto k = mfma_dx_kernel<BM, BN, 2, 2>;
  const size_t smem = gemm_smem<BM, BN>();
  hipError_t e = set_smem(k, smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k, dim3(device_cu_count()), dim3(NT), smem, st, a);
  return hipGetLastError();
}

hipError_t mfma_bwd_dw(const void *dY, const void *x, const moe_schedule &s, void *dW, int K,
                       int N, hipStream_t st) {
  DwArgs a{(const bf16_t *)dY, (const bf16_t *)x, dW, s.offsets, s.counts, s.expert_order,
           s.row_to_token, s.row_weight, s.E, s.layout, s.capacity, K, N,
           (uint32_t)((size_t)s.T * N * 2), (uint32_t)((size_t)s.T * K * 2), 1};
  auto k = mfma_dw_kernel<bf16_t>;
  const size_t smem = (size_t)2 * 512 * ROWB;
  hipError_t e = set_smem(k, smem);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(k, dim3(device_cu_count()), dim3(NT), smem, st, a);
  return hipGetLastError();
}

}  // namespace moe
