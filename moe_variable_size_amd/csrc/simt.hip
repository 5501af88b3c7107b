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
// elements i .. i+3 (i a multiple of 4, the row 4-element aligned), or zeros
MOE_DEV void ld4(const float *p, size_t i, bool ok, float (&v)[4]) {
  typedef float f4 __attribute__((ext_vector_type(4)));
  const f4 a = ok ? *(const f4 *)(p + i) : f4{0.f, 0.f, 0.f, 0.f};
  v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
}
MOE_DEV void ld4(const bf16_t *p, size_t i, bool ok, float (&v)[4]) {
  typedef uint32_t u2 __attribute__((ext_vector_type(2)));
  const u2 a = ok ? *(const u2 *)(p + i) : u2{0u, 0u};
  v[0] = __uint_as_float(a[0] << 16); v[1] = __uint_as_float(a[0] & 0xffff0000u);
  v[2] = __uint_as_float(a[1] << 16); v[3] = __uint_as_float(a[1] & 0xffff0000u);
}
MOE_DEV void st(bf16_t *p, size_t i, float v) { p[i] = f32_to_bf16(v); }

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

// Forward-shaped products: out[r, n] = sum_k A[src(r), k] * B[n, k] with B the
// group's weight rows.
//  kBare   : src(r) = r, plain store of C[r, n] (row space = A's rows).
//  kFused  : src(r) = row_to_token[r]; y[src(r), n] += row_weight[r] * acc.
//  kGatedUp: src(r) = row_to_token[r]; a tile's 128 columns are 64 gate /
//            up pairs: column c is W_gu row f (c % 8 < 4, gate) or F + f (up)
//            with f = f0 + 4 (c / 8) + c % 4, so a thread holds the gate and
//            up values of 4 f for its 8 rows and stores h[r, f] = silu(g) u
//            (and g, u into gu[r, f], gu[r, F + f] when gu is given).  N = F.
//  kRowsOut: src(r) = r over the schedule's rows (A = h, one row per
//            assignment); y[row_to_token[r], n] += row_weight[r] * acc.
enum Mode { kBare = 0, kFused = 1, kGatedUp = 2, kRowsOut = 3 };

MOE_DEV float silu(float g) { return g / (1.f + __expf(-g)); }

// Operand loads: thread t brings row t / 2, reduction indices 4 (t % 2) .. +3
// of both the A rows and the W rows of the step.
template <int MODE, typename Tin, typename Tout>
__global__ __launch_bounds__(NT) void simt_fwd_kernel(
    const Tin *__restrict__ A, const Tin *__restrict__ W, Tout *__restrict__ C,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ counts,
    const int32_t *__restrict__ bstart, const int32_t *__restrict__ row_to_token,
    const float *__restrict__ row_weight, int E, int layout, int capacity, int K, int N, int M,
    float *__restrict__ gu) {
  constexpr bool GATED = MODE == kGatedUp;
  constexpr int TILE_N = GATED ? BN / 2 : BN;  // output columns (f) per tile
  __shared__ __attribute__((aligned(16))) float As[BK][LDP];
  __shared__ __attribute__((aligned(16))) float Bs[BK][LDP];
  __shared__ int bs[kMaxExperts + 1], rstart[kMaxExperts], rcnt[kMaxExperts];
  __shared__ int src[BM], dst[BM];
  __shared__ float wrow[BM];
  __shared__ int scratch[NT / kWave + 1];

  if (MODE == kBare)
    group_tables_from_offsets<NT>(offsets, E, BM, bs, rstart, rcnt, scratch);
  else
    group_tables_from_schedule<NT>(counts, offsets, bstart, E, layout, capacity, bs, rstart, rcnt);

  const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
  const int lr = tid / 2, lk = (tid % 2) * 4;  // this thread's load row / reduction offset
  const int tiles_n = (N + TILE_N - 1) / TILE_N;
  const int total = bs[E] * tiles_n;
  for (int tau = blockIdx.x; tau < total; tau += gridDim.x) {
    const TileCoord c = tile_coord(bs, rstart, rcnt, E, tau, tiles_n, BM);
    if (c.rows <= 0) continue;  // masked layout: no valid rows in this block
    const int n0 = c.nb * TILE_N;
    __syncthreads();
    if (tid < BM) {
      const int r = c.row0 + tid;
      const bool ok = tid < c.rows;
      int sa = -1, so = -1;
      if (ok) {
        if (MODE == kBare) {
          sa = r < M ? r : -1;
          so = sa;
        } else if (MODE == kRowsOut) {
          sa = r;
          so = row_to_token[r];
        } else {
          sa = row_to_token[r];
          so = GATED ? r : sa;
        }
      }
      src[tid] = sa;
      dst[tid] = so;
      wrow[tid] = (ok && MODE != kBare && !GATED) ? row_weight[r] : 0.f;
    }
    __syncthreads();
    const Tin *Wg = W + (size_t)c.g * (GATED ? 2 * (size_t)N : (size_t)N) * K;
    // 4 consecutive reduction elements per operand row in one load when every
    // row starts on a 4-element boundary
    const bool vec4 = K % 4 == 0 && (uintptr_t)A % (4 * sizeof(Tin)) == 0 &&
                      (uintptr_t)W % (4 * sizeof(Tin)) == 0;
    const int s_ld = src[lr];
    // the weight row this thread loads for tile column lr, or -1
    int w_ld;
    if constexpr (GATED) {
      const int f = n0 + 4 * (lr / 8) + (lr % 4);
      w_ld = f < N ? ((lr % 8) < 4 ? f : N + f) : -1;
    } else {
      w_ld = n0 + lr < N ? n0 + lr : -1;
    }
    float ra[4], rb[4];
    auto load = [&](int k0) __attribute__((always_inline)) {
      if (vec4) {  // one 4-element load per operand (K % 4 == 0: in range or not as a whole)
        const int kx = k0 + lk;
        ld4(A, (size_t)s_ld * K + kx, s_ld >= 0 && kx < K, ra);
        ld4(Wg, (size_t)w_ld * K + kx, w_ld >= 0 && kx < K, rb);
        return;
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int kx = k0 + lk + q;
        ra[q] = (s_ld >= 0 && kx < K) ? ld(A, (size_t)s_ld * K + kx) : 0.f;
        rb[q] = (w_ld >= 0 && kx < K) ? ld(Wg, (size_t)w_ld * K + kx) : 0.f;
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
      const int s = dst[rr];
      if (s < 0) continue;
      if constexpr (GATED) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int f = n0 + 4 * tx + j;
          if (f >= N) continue;
          const float g = acc[i][j], u = acc[i][j + 4];
          st(C, (size_t)s * N + f, silu(g) * u);
          if (gu) {
            gu[(size_t)s * 2 * N + f] = g;
            gu[(size_t)s * 2 * N + N + f] = u;
          }
        }
      } else {
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
}

// Input-gradient-shaped products: G[r, kc] = sum_n A[src(r), n] * W[g, n, kc]
// (the weight read transposed).
//  kDx     : A = dY, src(r) = row_to_token[r]; dX[tok(r), kc] += w_r G[r, kc];
//            d_w[assign(r)] += sum_kc G[r, kc] * x[tok(r), kc].
//  kGatedDh: A = dY, src(r) = row_to_token[r], W = W_down (kc runs over F):
//            dh = w_r G; d_w[assign(r)] += sum_f G[r, f] h[r, f]; from the
//            saved g = gu[r, f], u = gu[r, F + f]:
//            dgu[r, f] = dh u s (1 + g (1 - s)), dgu[r, F + f] = dh g s,
//            s = 1 / (1 + exp(-g)).
//  kGatedDx: A = dgu, src(r) = r (the schedule's rows), W = W_gu (n runs
//            over 2F); dX[tok(r), kc] += G[r, kc] (the weight is in dgu).
// Operand loads: the A rows as the forward's (thread t: row t / 2, n 4 (t % 2)
// .. +3); W rows n0 + t / 32, columns kc0 + 4 (t % 32) .. +3.
enum DxMode { kDx = 0, kGatedDh = 1, kGatedDx = 2 };
template <int MODE, typename Tin>
__global__ __launch_bounds__(NT) void simt_dx_kernel(
    const Tin *__restrict__ dY, const Tin *__restrict__ x, const Tin *__restrict__ W,
    float *__restrict__ dX, float *__restrict__ d_w, const int32_t *__restrict__ offsets,
    const int32_t *__restrict__ counts, const int32_t *__restrict__ bstart,
    const int32_t *__restrict__ row_to_assign, const int32_t *__restrict__ row_to_token,
    const float *__restrict__ row_weight, int E, int layout, int capacity, int K, int N,
    const float *__restrict__ gu, Tin *__restrict__ dgu) {
  __shared__ __attribute__((aligned(16))) float As[BK][LDP];
  __shared__ __attribute__((aligned(16))) float Bs[BK][LDP];
  __shared__ int bs[kMaxExperts + 1], rstart[kMaxExperts], rcnt[kMaxExperts];
  __shared__ int src[BM], tokr[BM], asg[BM];
  __shared__ float wrow[BM];

  group_tables_from_schedule<NT>(counts, offsets, bstart, E, layout, capacity, bs, rstart, rcnt);
  const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
  const int lr = tid / 2, ln = (tid % 2) * 4;   // A rows
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
      const int t = ok ? row_to_token[r] : -1;
      src[tid] = ok ? (MODE == kGatedDx ? r : t) : -1;
      tokr[tid] = MODE == kGatedDh ? (ok ? r : -1) : t;  // the row the epilogue addresses
      asg[tid] = ok ? row_to_assign[r] : -1;
      wrow[tid] = ok ? row_weight[r] : 0.f;
    }
    __syncthreads();
    const Tin *Wg = W + (size_t)c.g * N * K;
    const int s_ld = src[lr];
    // 4-element loads where every row starts on a 4-element boundary
    const bool va = N % 4 == 0 && (uintptr_t)dY % (4 * sizeof(Tin)) == 0;
    const bool vb = K % 4 == 0 && (uintptr_t)W % (4 * sizeof(Tin)) == 0;
    float ra[4], rb[4];
    auto load = [&](int n0) __attribute__((always_inline)) {
      const int nw = n0 + wr;
      if (va) {
        ld4(dY, (size_t)s_ld * N + n0 + ln, s_ld >= 0 && n0 + ln < N, ra);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int nx = n0 + ln + q;
          ra[q] = (s_ld >= 0 && nx < N) ? ld(dY, (size_t)s_ld * N + nx) : 0.f;
        }
      }
      if (vb) {
        ld4(Wg, (size_t)nw * K + kc0 + wc, nw < N && kc0 + wc < K, rb);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int kx = kc0 + wc + q;
          rb[q] = (nw < N && kx < K) ? ld(Wg, (size_t)nw * K + kx) : 0.f;
        }
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
      const int s = tokr[rr];
      float part = 0.f;
      if (s >= 0) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          const int kc = kc0 + 8 * tx + j;
          if (kc >= K) continue;
          const float g = acc[i][j];
          if (MODE == kDx) {
            if (dX) atomicAdd(dX + (size_t)s * K + kc, wrow[rr] * g);
            if (d_w) part = fmaf(g, ld(x, (size_t)s * K + kc), part);
          } else if (MODE == kGatedDx) {
            atomicAdd(dX + (size_t)s * K + kc, g);
          } else {  // kGatedDh: s is the schedule row, K is F
            if (d_w) part = fmaf(g, ld(x, (size_t)s * K + kc), part);
            if (dgu) {
              const float dh = wrow[rr] * g;
              const float gv = gu[(size_t)s * 2 * K + kc], uv = gu[(size_t)s * 2 * K + K + kc];
              const float sg = 1.f / (1.f + __expf(-gv));
              st(dgu, (size_t)s * 2 * K + kc, dh * uv * sg * (1.f + gv * (1.f - sg)));
              st(dgu, (size_t)s * 2 * K + K + kc, dh * gv * sg);
            }
          }
        }
      }
      if (MODE != kGatedDx && d_w) {
        // the 16 threads with the same ty are 16 consecutive lanes of one wave
#pragma unroll
        for (int d = 8; d >= 1; d >>= 1) part += __shfl_xor(part, d, 16);
        if (tx == 0 && s >= 0) atomicAdd(d_w + asg[rr], part);
      }
    }
  }
}

// Weight gradient: dW[e, n, kc] = sum over rows r of e of a(r, n) b(r, kc) with
// a(r, n) = w_r dY[tok(r), n] (or A[r, n], unweighted, with A_ROWS) and
// b(r, kc) = x[tok(r), kc] (or B[r, kc] with B_ROWS).  Work units are (expert,
// output tile) taken in descending expert load and dealt to blocks in a snake
// order so that long reductions are spread out; every unit of an empty expert
// stores zeros.  Operand loads: reduction row t / 32 of the step, columns
// 4 (t % 32) .. +3 of both rows.
template <typename Tin, typename Tout, bool A_ROWS = false, bool B_ROWS = false>
__global__ __launch_bounds__(NT) void simt_dw_kernel(
    const Tin *__restrict__ dY, const Tin *__restrict__ x, Tout *__restrict__ dW,
    const int32_t *__restrict__ offsets, const int32_t *__restrict__ counts,
    const int32_t *__restrict__ expert_order, const int32_t *__restrict__ row_to_token,
    const float *__restrict__ row_weight, int E, int layout, int capacity, int K, int N) {
  __shared__ __attribute__((aligned(16))) float As[BK][LDP];
  __shared__ __attribute__((aligned(16))) float Bs[BK][LDP];
  const int tid = threadIdx.x, ty = tid / 16, tx = tid % 16;
  const int lq = tid / 32, lc = (tid % 32) * 4;
  // 4-element loads where every row starts on a 4-element boundary
  const bool va = N % 4 == 0 && (uintptr_t)dY % (4 * sizeof(Tin)) == 0;
  const bool vb = K % 4 == 0 && (uintptr_t)x % (4 * sizeof(Tin)) == 0;
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
      const int r = r0 + q0 + lq;
      const int tok = ok ? row_to_token[r] : -1;
      const int sa = A_ROWS ? (ok ? r : -1) : tok, sb = B_ROWS ? (ok ? r : -1) : tok;
      const float wv = A_ROWS ? 1.f : (ok ? row_weight[r] : 0.f);
      if (va) {
        ld4(dY, (size_t)sa * N + n0 + lc, sa >= 0 && n0 + lc < N, ra);
#pragma unroll
        for (int q = 0; q < 4; ++q) ra[q] *= wv;
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = n0 + lc + q;
          ra[q] = (sa >= 0 && n < N) ? wv * ld(dY, (size_t)sa * N + n) : 0.f;
        }
      }
      if (vb) {
        ld4(x, (size_t)sb * K + kc0 + lc, sb >= 0 && kc0 + lc < K, rb);
      } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int kc = kc0 + lc + q;
          rb[q] = (sb >= 0 && kc < K) ? ld(x, (size_t)sb * K + kc) : 0.f;
        }
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

template <typename T>
const int32_t *bst128(const T &s) { return s.block_start + bm_index(BM) * (s.E + 1); }

}  // namespace

hipError_t simt_grouped_gemm(const void *A, const void *W, const int32_t *offsets, void *C, int M,
                             int K, int N, int E, int dtype, int out_dtype, hipStream_t st) {
  const dim3 grid(simt_grid(device_cu_count())), block(NT);
  if (dtype == MOE_F32) {
    hipLaunchKernelGGL((simt_fwd_kernel<kBare, float, float>), grid, block, 0, st,
                       (const float *)A, (const float *)W, (float *)C, offsets, nullptr, nullptr,
                       nullptr, nullptr, E, 0, 0, K, N, M, nullptr);
  } else if (out_dtype == MOE_F32) {
    hipLaunchKernelGGL((simt_fwd_kernel<kBare, bf16_t, float>), grid, block, 0, st,
                       (const bf16_t *)A, (const bf16_t *)W, (float *)C, offsets, nullptr,
                       nullptr, nullptr, nullptr, E, 0, 0, K, N, M, nullptr);
  } else {
    hipLaunchKernelGGL((simt_fwd_kernel<kBare, bf16_t, bf16_t>), grid, block, 0, st,
                       (const bf16_t *)A, (const bf16_t *)W, (bf16_t *)C, offsets, nullptr,
                       nullptr, nullptr, nullptr, E, 0, 0, K, N, M, nullptr);
  }
  return hipGetLastError();
}

namespace {
template <int MODE, typename Tin>
hipError_t launch_fwd(const void *A, const void *W, const moe_schedule &s, void *C, int K, int N,
                      float *gu, hipStream_t st) {
  const dim3 grid(simt_grid(device_cu_count())), block(NT);
  using Tout = std::conditional_t<MODE == kGatedUp, Tin, float>;
  hipLaunchKernelGGL((simt_fwd_kernel<MODE, Tin, Tout>), grid, block, 0, st, (const Tin *)A,
                     (const Tin *)W, (Tout *)C, s.offsets, s.counts, bst128(s), s.row_to_token,
                     s.row_weight, s.E, s.layout, s.capacity, K, N, (int)s.T, gu);
  return hipGetLastError();
}

template <int MODE, typename Tin>
hipError_t launch_dx(const void *A, const void *x, const void *W, const moe_schedule &s,
                     float *dX, float *d_w, int K, int N, const float *gu, void *dgu,
                     hipStream_t st) {
  const dim3 grid(simt_grid(device_cu_count())), block(NT);
  hipLaunchKernelGGL((simt_dx_kernel<MODE, Tin>), grid, block, 0, st, (const Tin *)A,
                     (const Tin *)x, (const Tin *)W, dX, d_w, s.offsets, s.counts, bst128(s),
                     s.row_to_assign, s.row_to_token, s.row_weight, s.E, s.layout, s.capacity, K,
                     N, gu, (Tin *)dgu);
  return hipGetLastError();
}

template <typename Tin, bool A_ROWS, bool B_ROWS>
hipError_t launch_dw(const void *A, const void *B, const moe_schedule &s, void *dW, int K, int N,
                     hipStream_t st) {
  const dim3 grid(simt_grid(device_cu_count())), block(NT);
  hipLaunchKernelGGL((simt_dw_kernel<Tin, Tin, A_ROWS, B_ROWS>), grid, block, 0, st,
                     (const Tin *)A, (const Tin *)B, (Tin *)dW, s.offsets, s.counts,
                     s.expert_order, s.row_to_token, s.row_weight, s.E, s.layout, s.capacity, K,
                     N);
  return hipGetLastError();
}
}  // namespace

hipError_t simt_fused_fwd(const void *x, const void *W, const moe_schedule &s, float *y, int K,
                          int N, int dtype, hipStream_t st) {
  return dtype == MOE_F32 ? launch_fwd<kFused, float>(x, W, s, y, K, N, nullptr, st)
                          : launch_fwd<kFused, bf16_t>(x, W, s, y, K, N, nullptr, st);
}

hipError_t simt_bwd_dx(const void *dY, const void *x, const void *W, const moe_schedule &s,
                       float *dX, float *d_w, int K, int N, int dtype, hipStream_t st) {
  return dtype == MOE_F32
             ? launch_dx<kDx, float>(dY, x, W, s, dX, d_w, K, N, nullptr, nullptr, st)
             : launch_dx<kDx, bf16_t>(dY, x, W, s, dX, d_w, K, N, nullptr, nullptr, st);
}

hipError_t simt_bwd_dw(const void *dY, const void *x, const moe_schedule &s, void *dW, int K,
                       int N, int dtype, hipStream_t st) {
  return dtype == MOE_F32 ? launch_dw<float, false, false>(dY, x, s, dW, K, N, st)
                          : launch_dw<bf16_t, false, false>(dY, x, s, dW, K, N, st);
}

hipError_t simt_gated_up(const void *x, const void *W_gu, const moe_schedule &s, void *h,
                         float *gu, int K, int F, int dtype, hipStream_t st) {
  return dtype == MOE_F32 ? launch_fwd<kGatedUp, float>(x, W_gu, s, h, K, F, gu, st)
                          : launch_fwd<kGatedUp, bf16_t>(x, W_gu, s, h, K, F, gu, st);
}

hipError_t simt_gated_down(const void *h, const void *W_down, const moe_schedule &s, float *y,
                           int F, int N, int dtype, hipStream_t st) {
  return dtype == MOE_F32 ? launch_fwd<kRowsOut, float>(h, W_down, s, y, F, N, nullptr, st)
                          : launch_fwd<kRowsOut, bf16_t>(h, W_down, s, y, F, N, nullptr, st);
}

hipError_t simt_gated_bwd_dh(const void *dY, const void *h, const void *W_down,
                             const moe_schedule &s, float *d_w, int F, int N, const float *gu,
                             void *dgu, int dtype, hipStream_t st) {
  return dtype == MOE_F32
             ? launch_dx<kGatedDh, float>(dY, h, W_down, s, nullptr, d_w, F, N, gu, dgu, st)
             : launch_dx<kGatedDh, bf16_t>(dY, h, W_down, s, nullptr, d_w, F, N, gu, dgu, st);
}

hipError_t simt_gated_bwd_dx(const void *dgu, const void *W_gu, const moe_schedule &s, float *dX,
                             int K, int F, int dtype, hipStream_t st) {
  return dtype == MOE_F32
             ? launch_dx<kGatedDx, float>(dgu, nullptr, W_gu, s, dX, nullptr, K, 2 * F, nullptr,
                                          nullptr, st)
             : launch_dx<kGatedDx, bf16_t>(dgu, nullptr, W_gu, s, dX, nullptr, K, 2 * F,
                                           nullptr, nullptr, st);
}

hipError_t simt_bwd_dw_rows(const void *A, bool a_by_row, const void *B, bool b_by_row,
                            const moe_schedule &s, void *dW, int K, int N, int dtype,
                            hipStream_t st) {
  if (a_by_row && b_by_row) return hipErrorInvalidValue;
  if (dtype == MOE_F32) {
    if (a_by_row) return launch_dw<float, true, false>(A, B, s, dW, K, N, st);
    if (b_by_row) return launch_dw<float, false, true>(A, B, s, dW, K, N, st);
    return launch_dw<float, false, false>(A, B, s, dW, K, N, st);
  }
  if (a_by_row) return launch_dw<bf16_t, true, false>(A, B, s, dW, K, N, st);
  if (b_by_row) return launch_dw<bf16_t, false, true>(A, B, s, dW, K, N, st);
  return launch_dw<bf16_t, false, false>(A, B, s, dW, K, N, st);
}

}  // namespace moe
