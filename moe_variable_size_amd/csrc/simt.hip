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
// Tile: 64 x 64 outputs per 256-thread block, reduction step 16; thread
// (ty, tx) owns rows ty + 16 i and columns tx + 16 j (i, j < 4).  A persistent
// grid strides over the flat tile space ([GG] "Problem descriptors and the tile
// scheduler").
#include "common.hpp"

namespace moe {
namespace {

constexpr int BM = 64, BN = 64, BK = 16, NT = 256;

MOE_DEV float ld(const float *p, size_t i) { return p[i]; }
MOE_DEV float ld(const bf16_t *p, size_t i) { return bf16_to_f32(p[i]); }
MOE_DEV void st(float *p, size_t i, float v) { p[i] = v; }
MOE_DEV void st(bf16_t *p, size_t i, float v) { p[i] = f32_to_bf16(v); }

enum Mode { kBare = 0, kFused = 1 };

// Forward-shaped product: out[r, n] = sum_k A[src(r), k] * W[g, n, k].
//  kBare : src(r) = r, plain store of C[r, n] (row space = A's rows).
//  kFused: src(r) = row_to_token[r]; y[src(r), n] += row_weight[r] * acc.
template <int MODE, typename Tin, typename Tout>
__global__ __launch_bounds__(NT) void simt_fwd_kernel(
    const Tin *__restrict__ A, const Tin *__restrict__ W, Tout *__restrict__ C,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ counts,
    const int32_t *__restrict__ bstart, const int32_t *__restrict__ row_to_token,
    const float *__restrict__ row_weight, int E, int layout, int capacity, int K, int N, int M) {
  __shared__ float As[BK][BM + 4];
  __shared__ float Bs[BK][BN + 4];
  __shared__ int bs[kMaxExperts + 1], rstart[kMaxExperts], rcnt[kMaxExperts];
  __shared__ int src[BM];
  __shared__ float wrow[BM];
  __shared__ int scratch[NT / kWave + 1];

  if (MODE == kBare)
    group_tables_from_offsets<NT>(offsets, E, BM, bs, rstart, rcnt, scratch);
  else
    group_tables_from_schedule<NT>(counts, offsets, bstart, E, layout, capacity, bs, rstart, rcnt);

  const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
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
    float acc[4][4] = {};
    for (int k0 = 0; k0 < K; k0 += BK) {
      {  // A: row tid/4, k (tid%4)*4 .. +3
        const int rr = tid / 4, kk = (tid % 4) * 4;
        const int s = src[rr];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int kx = k0 + kk + q;
          As[kk + q][rr] = (s >= 0 && kx < K) ? ld(A, (size_t)s * K + kx) : 0.f;
        }
        const int nn = n0 + rr;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int kx = k0 + kk + q;
          Bs[kk + q][rr] = (nn < N && kx < K) ? ld(Wg, (size_t)nn * K + kx) : 0.f;
        }
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < BK; ++kk) {
        float a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = As[kk][ty + 16 * i];
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx + 16 * j];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
      }
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = ty + 16 * i;
      const int s = src[rr];
      if (s < 0) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = n0 + tx + 16 * j;
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
template <typename Tin>
__global__ __launch_bounds__(NT) void simt_dx_kernel(
    const Tin *__restrict__ dY, const Tin *__restrict__ x, const Tin *__restrict__ W,
    float *__restrict__ dX, float *__restrict__ d_w, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ counts, const int32_t *__restrict__ bstart,
    const int32_t *__restrict__ row_to_assign, const int32_t *__restrict__ row_to_token,
    const float *__restrict__ row_weight, int E, int layout, int capacity, int K, int N) {
  __shared__ float As[BK][BM + 4];
  __shared__ float Bs[BK][BN + 4];
  __shared__ int bs[kMaxExperts + 1], rstart[kMaxExperts], rcnt[kMaxExperts];
  __shared__ int src[BM], asg[BM];
  __shared__ float wrow[BM];

  group_tables_from_schedule<NT>(counts, offsets, bstart, E, layout, capacity, bs, rstart, rcnt);
  const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
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
    float acc[4][4] = {};
    for (int n0 = 0; n0 < N; n0 += BK) {
      {  // A: dY row tid/4, n (tid%4)*4..+3
        const int rr = tid / 4, nn = (tid % 4) * 4;
        const int s = src[rr];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int nx = n0 + nn + q;
          As[nn + q][rr] = (s >= 0 && nx < N) ? ld(dY, (size_t)s * N + nx) : 0.f;
        }
      }
      {  // B: W row n0 + tid/16, columns kc0 + (tid%16)*4 .. +3
        const int nr = tid / 16, kk = (tid % 16) * 4;
        const int nx = n0 + nr;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int kx = kc0 + kk + q;
          Bs[nr][kk + q] = (nx < N && kx < K) ? ld(Wg, (size_t)nx * K + kx) : 0.f;
        }
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < BK; ++kk) {
        float a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = As[kk][ty + 16 * i];
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx + 16 * j];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
      }
      __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rr = ty + 16 * i;
      const int s = src[rr];
      float part = 0.f;
      if (s >= 0) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int kc = kc0 + tx + 16 * j;
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
// of an empty expert stores zeros.
template <typename Tin, typename Tout>
__global__ __launch_bounds__(NT) void simt_dw_kernel(
    const Tin *__restrict__ dY, const Tin *__restrict__ x, Tout *__restrict__ dW,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ counts,
    const int32_t *__restrict__ expert_order, const int32_t *__restrict__ row_to_token,
    const float *__restrict__ row_weight, int E, int layout, int capacity, int K, int N) {
  __shared__ float As[BK][BM + 4];
  __shared__ float Bs[BK][BN + 4];
  __shared__ int src[BK];
  __shared__ float wrow[BK];
  const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
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
    float acc[4][4] = {};
    for (int q0 = 0; q0 < m; q0 += BK) {
      __syncthreads();
      if (tid < BK) {
        const bool ok = q0 + tid < m;
        src[tid] = ok ? row_to_token[r0 + q0 + tid] : -1;
        wrow[tid] = ok ? row_weight[r0 + q0 + tid] : 0.f;
      }
      __syncthreads();
      {
        const int rr = tid / 16, cc = (tid % 16) * 4;
        const int s = src[rr];
        const float wv = wrow[rr];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n0 + cc + q, kc = kc0 + cc + q;
          As[rr][cc + q] = (s >= 0 && n < N) ? wv * ld(dY, (size_t)s * N + n) : 0.f;
          Bs[rr][cc + q] = (s >= 0 && kc < K) ? ld(x, (size_t)s * K + kc) : 0.f;
        }
      }
      __syncthreads();
#pragma unroll
      for (int kk = 0; kk < BK; ++kk) {
        float a[4], b[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] = As[kk][ty + 16 * i];
#pragma unroll
        for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx + 16 * j];
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
      }
    }
    Tout *out = dW + (size_t)e * N * K;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = n0 + ty + 16 * i;
      if (n >= N) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kc = kc0 + tx + 16 * j;
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
