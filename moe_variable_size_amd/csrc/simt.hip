// Exact fp32 (and generic-shape) grouped GEMM kernels on the vector ALUs.
//
// [GG] = "Grouped GEMM for MoE, in depth" (aicassindra.com)
// [CARD] = "grouped-gemm-moe" model card
//
// This is the register-blocked tile loop the card describes for the exact fp32
// path ([CARD] "How it works"): every output element is one fp32 FMA chain over
// the reduction index in ascending order, so the bare and the fused kernels
// produce identical bits for the same row, and the fused fp32 forward equals the
// explicit gather -> grouped GEMM -> scatter path bit for bit when each output
// receives at most two atomic contributions ([CARD] "Correctness").  The same
// kernels, instantiated for bf16 storage, serve shapes the MFMA kernels do not
// take (K or N not a multiple of 8).
//
// Tile: 128 x 128 outputs per 256-thread block, reduction step 8; thread
// (ty, tx) owns rows 8 ty .. 8 ty + 7 and columns 8 tx .. 8 tx + 7 (64
// accumulators; per reduction index two 16-byte LDS reads of each operand feed
// 64 FMAs).  The next step's operands are loaded from memory into registers
// while the current step multiplies.  A persistent grid strides over the flat
// tile space ([GG] "Problem descriptors and the tile scheduler").
#include "common.hpp"

namespace moe {
namespace {

constexpr int BM = 128, BN = 128, BK = 8, NT = 256, TM = 8, TN = 8;
constexpr int LDP = BM + 4;  // LDS row pitch (floats): 16-byte aligned, rows offset by 4 banks

MOE_DEV float ld(const float *p, size_t i) { return p[i]; }
MOE_DEV float ld(const bf16_t *p, size_t i) { return bf16_to_f32(p[i]); }
MOE_DEV void st(float *p, size_t i, float v) { p[i] = v; }
MOE_DEV void st(bf16_t *p, size_t i, float v) { p[i] = f32_to_bf16(v); }

enum Mode { kBare = 0, kFused = 1 };

// acc[i][j] += A[kk][8 ty + i] * B[kk][8 tx + j] over the BK reduction indices
// of one step, each output's FMAs in ascending reduction order.
MOE_DEV void step_fma(const float (*As)[LDP], const float (*Bs)[LDP], int ty, int tx,
                      float (&acc)[TM][TN]) {
  typedef float f4 __attribute__((ext_vector_type(4)));
#pragma unroll
  for (int kk = 0; kk < BK; ++kk) {
    const f4 a0 = *(const f4 *)&As[kk][8 * ty], a1 = *(const f4 *)&As[kk][8 * ty + 4];
    const f4 b0 = *(const f4 *)&Bs[kk][8 * tx], b1 = *(const f4 *)&Bs[kk][8 * tx + 4];
    const float a[TM] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
    const float b[TN] = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
  }
}

// Forward-shaped product: out[r, n] = sum_k A[src(r), k] * W[g, n, k].
//  kBare : src(r) = r, plain store of C[r, n] (row space = A's rows).
//  kFused: src(r) = row_to_token[r]; y[src(r), n] += row_weight[r] * acc.
// Operand loads: thread t brings row t / 2, reduction indices 4 (t % 2) .. +3
// of both the A rows and the W rows of the step.
template <int MODE, typename Tin, typename Tout>
__global__ __launch_bounds__(NT) void simt_fwd_kernel(
    const Tin *__restrict__ A, const Tin *__restrict__ W, Tout *__restrict__ C,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ counts,
    const int32_t *__restrict__ bstart, const int32_t *__restrict__ row_to_token,
    const float *__restrict__ row_weight, int E, int layout, int capacity, int K, int N, int M) {
  __shared__ __attribute__((aligned(16))) float As[BK][LDP];
  __shared__ __attribute__((aligned(16))) float Bs[BK][LDP];
  __shared__ int bs[kMaxExperts + 1], rstart[kMaxExperts], rcnt[kMaxExperts];
  __shared__ int src[BM];
  __shared__ float wrow[BM];
  __shared__ int scratch[NT / kWave + 1];

  if (MODE == kBare)
    group_tables_from_offsets<NT>(offsets, E, BM, bs, rstart, rcnt, scratch);
  else
    group_tables_from_schedule<NT>(counts, offsets, bstart, E, layout, capacity, bs, rstart, rcnt);

  const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
  const int lr = tid / 2, lk = (tid % 2) * 4;  // this thread's load row / reduction offset
  const int tiles_n = (N + BN - 1) / BN;
  const int total = bs[E] * tiles_n;
  for (int tau = blockIdx.x; tau < total; tau += gridDim.x) {
    const TileCoord c = tile_coord(bs, rstart, rcnt, E, tau, tiles_n, BM);
    if (c.rows <= 0) continue;  // masked layout: no valid rows in this block
    const int n0 = c.nb * BN;
    __syncthreads();
    if (tid < BM) {
      const int r = c.row0 + tid;
      const bool ok = tid < c.rows;
      src[tid] = ok ? (MODE == kBare ? (r < M ? r : -1) : row_to_token[r]) : -1;
      wrow[tid] = (ok && MODE != kBare) ? row_weight[r] : 0.f;
    }
    __syncthreads();
    const Tin *Wg = W + (size_t)c.g * N * K;
    const int s_ld = src[lr], n_ld = n0 + lr;
    float ra[4], rb[4];
    auto load = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int kx = k0 + lk + q;
        ra[q] = (s_ld >= 0 && kx < K) ? ld(A, (size_t)s_ld * K + kx) : 0.f;
        rb[q] = (n_ld < N && kx < K) ? ld(Wg, (size_t)n_ld * K + kx) : 0.f;
      }
    };
    float acc[TM][TN] = {};
    load(0);
    for (int k0 = 0; k0 < K; k0 += BK) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        As[lk + q][lr] = ra[q];
        Bs[lk + q][lr] = rb[q];
      }
      __syncthreads();
      if (k0 + BK < K) load(k0 + BK);  // in flight while this step multiplies
      step_fma(As, Bs, ty, tx, acc);
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int rr = 8 * ty + i;
      const int s = src[rr];
      if (s < 0) continue;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int n = n0 + 8 * tx + j;
        if (n >= N) continue;
        if (MODE == kBare)
          st(C, (size_t)s * N + n, acc[i][j]);
        else
          atomicAdd((float *)C + (size_t)s * N + n, wrow[rr] * acc[i][j]);
      }
    }
  }
}

// Input gradient: G[r, kc] = sum_n dY[tok(r), n] * W[g, n, kc];
// dX[tok(r), kc] += w_r * G[r, kc];  d_w[assign(r)] += sum_kc G[r, kc] * x[tok(r), kc].
// Operand loads: the dY rows as the forward's A rows (thread t: row t / 2,
// n 4 (t % 2) .. +3); W rows n0 + t / 32, columns kc0 + 4 (t % 32) .. +3.
template <typename Tin>
__global__ __launch_bounds__(NT) void simt_dx_kernel(
    const Tin *__restrict__ dY, const Tin *__restrict__ x, const Tin *__restrict__ W,
    float *__restrict__ dX, float *__restrict__ d_w, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ counts, const int32_t *__restrict__ bstart,
    const int32_t *__restrict__ row_to_assign, const int32_t *__restrict__ row_to_token,
    const float *__restrict__ row_weight, int E, int layout, int capacity, int K, int N) {
  __shared__ __attribute__((aligned(16))) float As[BK][LDP];
  __shared__ __attribute__((aligned(16))) float Bs[BK][LDP];
  __shared__ int bs[kMaxExperts + 1], rstart[kMaxExperts], rcnt[kMaxExperts];
  __shared__ int src[BM], asg[BM];
  __shared__ float wrow[BM];

  group_tables_from_schedule<NT>(counts, offsets, bstart, E, layout, capacity, bs, rstart, rcnt);
  const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
  const int lr = tid / 2, ln = (tid % 2) * 4;   // dY rows
  const int wr = tid / 32, wc = (tid % 32) * 4;  // W rows (reduction) and columns
  const int tiles_n = (K + BN - 1) / BN;  // output columns are the K dimension
  const int total = bs[E] * tiles_n;
  for (int tau = blockIdx.x; tau < total; tau += gridDim.x) {
    const TileCoord c = tile_coord(bs, rstart, rcnt, E, tau, tiles_n, BM);
    if (c.rows <= 0) continue;
    const int kc0 = c.nb * BN;
    __syncthreads();
    if (tid < BM) {
      const int r = c.row0 + tid;
      const bool ok = tid < c.rows;
      src[tid] = ok ? row_to_token[r] : -1;
      asg[tid] = ok ? row_to_assign[r] : -1;
      wrow[tid] = ok ? row_weight[r] : 0.f;
    }
    __syncthreads();
    const Tin *Wg = W + (size_t)c.g * N * K;
    const int s_ld = src[lr];
    float ra[4], rb[4];
    auto load = [&](int n0) __attribute__((always_inline)) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int nx = n0 + ln + q;
        ra[q] = (s_ld >= 0 && nx < N) ? ld(dY, (size_t)s_ld * N + nx) : 0.f;
        const int kx = kc0 + wc + q, nw = n0 + wr;
        rb[q] = (nw < N && kx < K) ? ld(Wg, (size_t)nw * K + kx) : 0.f;
      }
    };
    float acc[TM][TN] = {};
    load(0);
    for (int n0 = 0; n0 < N; n0 += BK) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        As[ln + q][lr] = ra[q];
        Bs[wr][wc + q] = rb[q];
      }
      __syncthreads();
      if (n0 + BK < N) load(n0 + BK);
      step_fma(As, Bs, ty, tx, acc);
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int rr = 8 * ty + i;
      const int s = src[rr];
      float part = 0.f;
      if (s >= 0) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int kc = kc0 + 8 * tx + j;
          if (kc >= K) continue;
          if (dX) atomicAdd(dX + (size_t)s * K + kc, wrow[rr] * acc[i][j]);
          if (d_w) part = fmaf(acc[i][j], ld(x, (size_t)s * K + kc), part);
        }
      }
      if (d_w) {
        // the 16 threads with the same ty are 16 consecutive lanes of one wave
#pragma unroll
        for (int d = 8; d >= 1; d >>= 1) part += __shfl_xor(part, d, 16);
        if (tx == 0 && s >= 0) atomicAdd(d_w + asg[rr], part);
      }
    }
  }
}

// Weight gradient: dW[e, n, kc] = sum over rows r of e of w_r dY[tok(r), n] x[tok(r), kc].
// Work units are (expert, output tile) taken in descending expert load and dealt
// to blocks in a snake order so that long reductions are spread out; every unit
// of an empty expert stores zeros.  Operand loads: reduction row t / 32 of the
// step, columns 4 (t % 32) .. +3 of both the weighted dY row and the x row.
template <typename Tin, typename Tout>
__global__ __launch_bounds__(NT) void simt_dw_kernel(
    const Tin *__restrict__ dY, const Tin *__restrict__ x, Tout *__restrict__ dW,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ counts,
    const int32_t *__restrict__ expert_order, const int32_t *__restrict__ row_to_token,
    const float *__restrict__ row_weight, int E, int layout, int capacity, int K, int N) {
  __shared__ __attribute__((aligned(16))) float As[BK][LDP];
  __shared__ __attribute__((aligned(16))) float Bs[BK][LDP];
  const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
  const int lq = tid / 32, lc = (tid % 32) * 4;
  const int tn = (N + BM - 1) / BM, tk = (K + BN - 1) / BN;
  const int per_e = tn * tk;
  const int units = E * per_e;
  const int G = gridDim.x;
  for (int round = 0;; ++round) {
    const int base = round * G;
    if (base >= units) break;
    const int u = base + ((round & 1) ? (G - 1 - (int)blockIdx.x) : (int)blockIdx.x);
    if (u >= units) continue;
    const int e = expert_order[u / per_e];
    const int t = u % per_e;
    const int n0 = (t / tk) * BM, kc0 = (t % tk) * BN;
    const int m = counts[e];
    const int r0 = layout == MOE_LAYOUT_MASKED ? e * capacity : offsets[e] - m;
    float ra[4], rb[4];
    auto load = [&](int q0) __attribute__((always_inline)) {
      const bool ok = q0 + lq < m;
      const int s = ok ? row_to_token[r0 + q0 + lq] : -1;
      const float wv = ok ? row_weight[r0 + q0 + lq] : 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + lc + q, kc = kc0 + lc + q;
        ra[q] = (s >= 0 && n < N) ? wv * ld(dY, (size_t)s * N + n) : 0.f;
        rb[q] = (s >= 0 && kc < K) ? ld(x, (size_t)s * K + kc) : 0.f;
      }
    };
    float acc[TM][TN] = {};
    if (m > 0) load(0);
    for (int q0 = 0; q0 < m; q0 += BK) {
      __syncthreads();  // the previous step (or unit) is done with the LDS
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        As[lq][lc + q] = ra[q];
        Bs[lq][lc + q] = rb[q];
      }
      __syncthreads();
      if (q0 + BK < m) load(q0 + BK);
      step_fma(As, Bs, ty, tx, acc);
    }
    Tout *out = dW + (size_t)e * N * K;
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const int n = n0 + 8 * ty + i;
      if (n >= N) continue;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const int kc = kc0 + 8 * tx + j;
        if (kc < K) st(out, (size_t)n * K + kc, acc[i][j]);
      }
    }
  }
}

int simt_grid(int num_cu) { return num_cu * 4; }

}  // namespace

hipError_t simt_grouped_gemm(const void *A, const void *W, const int32_t *offsets, void *C, int M,
                             int K, int N, int E, int dtype, int out_dtype, hipStream_t st) {
  const dim3 grid(simt_grid(device_cu_count())), block(NT);
  if (dtype == MOE_F32) {
    hipLaunchKernelGGL((simt_fwd_kernel<kBare, float, float>), grid, block, 0, st,
                       (const float *)A, (const float *)W, (float *)C, offsets, nullptr, nullptr,
                       nullptr, nullptr, E, 0, 0, K, N, M);
  } else if (out_dtype == MOE_F32) {
    hipLaunchKernelGGL((simt_fwd_kernel<kBare, bf16_t, float>), grid, block, 0, st,
                       (const bf16_t *)A, (const bf16_t *)W, (float *)C, offsets, nullptr,
                       nullptr, nullptr, nullptr, E, 0, 0, K, N, M);
  } else {
    hipLaunchKernelGGL((simt_fwd_kernel<kBare, bf16_t, bf16_t>), grid, block, 0, st,
                       (const bf16_t *)A, (const bf16_t *)W, (bf16_t *)C, offsets, nullptr,
                       nullptr, nullptr, nullptr, E, 0, 0, K, N, M);
  }
  return hipGetLastError();
}

hipError_t simt_fused_fwd(const void *x, const void *W, const moe_schedule &s, float *y, int K,
                          int N, int dtype, hipStream_t st) {
  const dim3 grid(simt_grid(device_cu_count())), block(NT);
  const int32_t *bst = s.block_start + bm_index(BM) * (s.E + 1);
  if (dtype == MOE_F32)
    hipLaunchKernelGGL((simt_fwd_kernel<kFused, float, float>), grid, block, 0, st,
                       (const float *)x, (const float *)W, y, s.offsets, s.counts, bst,
                       s.row_to_token, s.row_weight, s.E, s.layout, s.capacity, K, N, (int)s.T);
  else
    hipLaunchKernelGGL((simt_fwd_kernel<kFused, bf16_t, float>), grid, block, 0, st,
                       (const bf16_t *)x, (const bf16_t *)W, y, s.offsets, s.counts, bst,
                       s.row_to_token, s.row_weight, s.E, s.layout, s.capacity, K, N, (int)s.T);
  return hipGetLastError();
}

hipError_t simt_bwd_dx(const void *dY, const void *x, const void *W, const moe_schedule &s,
                       float *dX, float *d_w, int K, int N, int dtype, hipStream_t st) {
  const dim3 grid(simt_grid(device_cu_count())), block(NT);
  const int32_t *bst = s.block_start + bm_index(BM) * (s.E + 1);
  if (dtype == MOE_F32)
    hipLaunchKernelGGL((simt_dx_kernel<float>), grid, block, 0, st, (const float *)dY,
                       (const float *)x, (const float *)W, dX, d_w, s.offsets, s.counts, bst,
                       s.row_to_assign, s.row_to_token, s.row_weight, s.E, s.layout, s.capacity,
                       K, N);
  else
    hipLaunchKernelGGL((simt_dx_kernel<bf16_t>), grid, block, 0, st, (const bf16_t *)dY,
                       (const bf16_t *)x, (const bf16_t *)W, dX, d_w, s.offsets, s.counts, bst,
                       s.row_to_assign, s.row_to_token, s.row_weight, s.E, s.layout, s.capacity,
                       K, N);
  return hipGetLastError();
}

hipError_t simt_bwd_dw(const void *dY, const void *x, const moe_schedule &s, void *dW, int K,
                       int N, int dtype, hipStream_t st) {
  const dim3 grid(simt_grid(device_cu_count())), block(NT);
  if (dtype == MOE_F32)
    hipLaunchKernelGGL((simt_dw_kernel<float, float>), grid, block, 0, st, (const float *)dY,
                       (const float *)x, (float *)dW, s.offsets, s.counts, s.expert_order,
                       s.row_to_token, s.row_weight, s.E, s.layout, s.capacity, K, N);
  else
    hipLaunchKernelGGL((simt_dw_kernel<bf16_t, bf16_t>), grid, block, 0, st,
                       (const bf16_t *)dY, (const bf16_t *)x, (bf16_t *)dW, s.offsets, s.counts,
                       s.expert_order, s.row_to_token, s.row_weight, s.E, s.layout, s.capacity,
                       K, N);
  return hipGetLastError();
}

}  // namespace moe
