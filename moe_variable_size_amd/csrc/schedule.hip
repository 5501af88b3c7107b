// Device-side routing schedule builder.
//
// [GG] = "Grouped GEMM for MoE, in depth" (aicassindra.com)
// [CARD] = "grouped-gemm-moe" model card
// [NOTE] = "Grouped GEMM" study notes (scholia-log)
//
// One workgroup of 1024 threads does the whole build in three phases, with no
// host readback ([GG] "Problem descriptors and the tile scheduler": group sizes
// stay on the device; "Failure modes": no host sync):
//   1. histogram: every wave owns a contiguous range of assignments and counts
//      its ids per expert (bincount, [GG] "Data layout, offsets and alignment");
//   2. scans: per-expert counts, int32 END offsets (inclusive prefix), the
//      row-block prefix for each tile height (tile counts and their exclusive
//      prefix, [GG] "Problem descriptors and the tile scheduler"), each wave's
//      first rank inside each expert, and the experts ordered by load;
//   3. a stable counting sort: every wave walks its range again in order and
//      places each assignment at (expert base + wave base + rank among equal ids
//      earlier in the same 64-wide chunk), giving row -> assignment, row ->
//      token and the per-row routing weight ([CARD] "How it works"; [NOTE] 4.1).
// Equal ids inside a chunk are matched with one ballot per id bit, so ranks
// never depend on the order in which hardware executes atomics: the result is
// deterministic and equals a stable argsort by expert.
#include "common.hpp"

namespace moe {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;

MOE_DEV uint64_t ballot(bool p) { return __ballot(p); }

// Exclusive prefix sum over the block of one int per thread (1024 threads).
// `scratch` holds kWaves ints.  Returns the prefix; *total gets the sum.
MOE_DEV int block_exclusive_scan(int v, int *scratch, int *total) {
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
  if (wid == 0) {
    int w = lane < kWaves ? scratch[lane] : 0;
    int winc = w;
#pragma unroll
    for (int d = 1; d < kWaves; d <<= 1) {
      int t = __shfl_up(winc, d, kWave);
      if (lane >= d) winc += t;
    }
    if (lane < kWaves) scratch[lane] = winc - w;        // exclusive wave base
    if (lane == kWaves - 1) scratch[kWaves] = winc;     // grand total
  }
  __syncthreads();
  int r = scratch[wid] + inc - v;
  *total = scratch[kWaves];
  __syncthreads();  // scratch is reused by the next call
  return r;
}

// Lanes of this wave holding the same valid id as the calling lane.
MOE_DEV uint64_t peers(int id, bool valid, int nbits) {
  uint64_t m = ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    bool bit = (id >> b) & 1;
    uint64_t bb = ballot(valid && bit);
    m &= bit ? bb : ~bb;
  }
  return m;
}

__global__ __launch_bounds__(kThreads) void build_schedule_kernel(
    const int32_t *__restrict__ ids, const float *__restrict__ w, int S, int k, int E,
    int layout, int capacity, int R, int32_t *__restrict__ counts, int32_t *__restrict__ offsets,
    int32_t *__restrict__ block_start, int32_t *__restrict__ expert_order,
    int32_t *__restrict__ row_to_assign, int32_t *__restrict__ row_to_token,
    float *__restrict__ row_weight, int32_t *__restrict__ status) {
  extern __shared__ int smem[];
  int *hist = smem;                      // [kWaves][E]: per-wave counts, then rank bases
  int *rowbase = hist + kWaves * E;      // [E]: first row of each expert
  int *cnt = rowbase + E;                // [E]: valid rows per expert
  int *scratch = cnt + E;                // [kWaves + 1]
  int *tally = scratch + kWaves + 1;     // [2]: invalid ids, dropped assignments

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = tid / kWave;
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));

  for (int i = tid; i < kWaves * E; i += kThreads) hist[i] = 0;
  if (tid < 2) tally[tid] = 0;
  __syncthreads();

  int nbits = 1;
  while ((1 << nbits) < E) ++nbits;
  const int per = (((S + kWaves - 1) / kWaves) + kWave - 1) / kWave * kWave;
  const int s_begin = min(S, wid * per);
  const int s_end = min(S, s_begin + per);

  // ---- phase 1: per-wave histogram ------------------------------------------
  int invalid = 0;
  for (int base = s_begin; base < s_end; base += kWave) {
    const int s = base + lane;
    const bool in = s < s_end;
    const int id = in ? ids[s] : -1;
    const bool valid = in && id >= 0 && id < E;
    invalid += (in && !valid) ? 1 : 0;
    const uint64_t m = peers(id, valid, nbits);
    if (valid && (m & below) == 0) hist[wid * E + id] += __popcll(m);
  }
  if (invalid) atomicAdd(&tally[0], invalid);
  __syncthreads();

  // ---- phase 2: counts, offsets, tile prefixes, rank bases -------------------
  const int e = tid;
  int m_e = 0;
  if (e < E) {
    int run = 0;
    for (int v = 0; v < kWaves; ++v) {  // per-wave exclusive rank base
      int c = hist[v * E + e];
      hist[v * E + e] = run;
      run += c;
    }
    m_e = run;
  }
  const bool masked = layout == MOE_LAYOUT_MASKED;
  const int valid_rows = (e < E) ? (masked ? min(m_e, capacity) : m_e) : 0;
  if (masked && e < E && m_e > capacity) atomicAdd(&tally[1], m_e - capacity);
  int total;
  const int start = block_exclusive_scan(valid_rows, scratch, &total);
  if (e < E) {
    counts[e] = valid_rows;
    offsets[e] = start + valid_rows;
    rowbase[e] = masked ? e * capacity : start;
    cnt[e] = valid_rows;
  }
#pragma unroll
  for (int i = 0; i < MOE_NUM_BM; ++i) {
    const int bm = 32 << i;
    const int nblk = (e < E) ? (masked ? (capacity + bm - 1) / bm : (valid_rows + bm - 1) / bm) : 0;
    int tot;
    const int pre = block_exclusive_scan(nblk, scratch, &tot);
    if (e < E) block_start[i * (E + 1) + e] = pre;
    if (tid == 0) block_start[i * (E + 1) + E] = tot;
  }
  __syncthreads();  // cnt[] complete

  // experts by descending row count, ties by id
  if (e < E) {
    int rank = 0;
    for (int o = 0; o < E; ++o) {
      const int c = cnt[o];
      rank += (c > valid_rows || (c == valid_rows && o < e)) ? 1 : 0;
    }
    expert_order[rank] = e;
  }

  // empty rows: past the last valid row (contiguous) or past each expert's
  // valid prefix (masked); disjoint from the rows phase 3 writes.
  if (!masked) {
    for (int r = total + tid; r < R; r += kThreads) {
      row_to_assign[r] = -1;
      row_to_token[r] = -1;
      row_weight[r] = 0.f;
    }
  } else {
    for (int r = tid; r < R; r += kThreads) {
      const int ex = r / capacity;
      if (r - ex * capacity >= cnt[ex]) {
        row_to_assign[r] = -1;
        row_to_token[r] = -1;
        row_weight[r] = 0.f;
      }
    }
  }

  // ---- phase 3: stable placement -------------------------------------------
  for (int base = s_begin; base < s_end; base += kWave) {
    const int s = base + lane;
    const bool in = s < s_end;
    const int id = in ? ids[s] : -1;
    const bool valid = in && id >= 0 && id < E;
    const uint64_t m = peers(id, valid, nbits);
    int rank = 0;
    if (valid) rank = hist[wid * E + id] + __popcll(m & below);
    if (valid && (m & below) == 0) hist[wid * E + id] += __popcll(m);
    if (valid && (!masked || rank < capacity)) {
      const int r = rowbase[id] + rank;
      row_to_assign[r] = s;
      row_to_token[r] = s / k;
      row_weight[r] = w ? w[s] : 1.f;
    }
  }
  __syncthreads();
  if (tid == 0) {
    status[0] = tally[0];
    status[1] = tally[1];
  }
}

// Owner of every tile of the flat space (export for tests / inspection).
__global__ void tile_map_kernel(const int32_t *__restrict__ bstart, int E, int tiles_n,
                                int32_t *__restrict__ tile_start, int32_t *__restrict__ total,
                                int32_t *__restrict__ owner, int64_t owner_cap) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int tot = bstart[E] * tiles_n;
  if (i == 0) *total = tot;
  if (i < E) tile_start[i] = bstart[i] * tiles_n;
  if (i < owner_cap && i < tot) {
    // tile tau lies in group g iff bstart[g]*tn <= tau < bstart[g+1]*tn, i.e.
    // bstart[g] <= floor(tau / tn): the upper bound of the row-block index.
    owner[i] = upper_bound_minus_one(bstart, E, (int32_t)(i / tiles_n));
  }
}

__global__ void fill_zero_kernel(uint4 *__restrict__ p, size_t n16, uint8_t *__restrict__ tail,
                                 int ntail) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    p[i] = make_uint4(0, 0, 0, 0);
  if (blockIdx.x == 0 && (int)threadIdx.x < ntail) tail[threadIdx.x] = 0;
}

}  // namespace

size_t schedule_smem_bytes(int E) { return sizeof(int) * ((size_t)kWaves * E + 2 * E + kWaves + 3); }

hipError_t launch_build_schedule(const int32_t *ids, const float *w, const moe_schedule &s,
                                 hipStream_t st) {
  const size_t smem = schedule_smem_bytes(s.E);
  if (smem > 65536) {
    hipError_t e = hipFuncSetAttribute((const void *)build_schedule_kernel,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(build_schedule_kernel, dim3(1), dim3(kThreads), smem, st, ids, w, (int)s.S,
                     s.k, s.E, s.layout, s.capacity, (int)s.R, s.counts, s.offsets,
                     s.block_start, s.expert_order, s.row_to_assign, s.row_to_token,
                     s.row_weight, s.status);
  return hipGetLastError();
}

hipError_t launch_tile_map(const moe_schedule &s, int N, int BM, int BN, int32_t *tile_start,
                           int32_t *total, int32_t *owner, int64_t owner_cap, hipStream_t st) {
  const int tn = (N + BN - 1) / BN;
  const int bi = bm_index(BM);
  int64_t n = owner_cap > s.E ? owner_cap : s.E;
  if (n < 1) n = 1;
  const int blocks = (int)((n + 255) / 256);
  hipLaunchKernelGGL(tile_map_kernel, dim3(blocks), dim3(256), 0, st,
                     s.block_start + bi * (s.E + 1), s.E, tn, tile_start, total, owner, owner_cap);
  return hipGetLastError();
}

hipError_t launch_fill_zero(void *p, size_t bytes, hipStream_t st) {
  if (bytes == 0) return hipSuccess;
  const size_t n16 = bytes / 16;
  const int ntail = (int)(bytes - n16 * 16);
  int blocks = (int)((n16 + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks), dim3(256), 0, st, (uint4 *)p, n16,
                     (uint8_t *)p + n16 * 16, ntail);
  return hipGetLastError();
}

}  // namespace moe
