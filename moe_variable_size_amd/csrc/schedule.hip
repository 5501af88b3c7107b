// Device-side routing schedule builder.
//
// [GG] = "Grouped GEMM for MoE, in depth" (aicassindra.com)
// [CARD] = "grouped-gemm-moe" model card
// [NOTE] = "Grouped GEMM" study notes (scholia-log)
//
// Two launches, no host readback ([GG] "Problem descriptors and the tile
// scheduler": group sizes stay on the device; "Failure modes": no host sync).
// The assignments s = 0 .. S-1 are cut into nblk blocks of B consecutive ids.
//   1. hist  (nblk workgroups): per-block count of each expert id
//      (bincount, [GG] "Data layout, offsets and alignment") and of ids
//      outside [0, E);
//   2. place (nblk workgroups): every workgroup sums the block x expert table
//      itself: its own block's base inside each expert (the counts of the
//      blocks before it) and each expert's total, whose exclusive prefix gives
//      the expert's first row.  Four workgroups also write, one job each, the
//      per-expert counts with the int32 END offsets (inclusive prefix) and the
//      status; the row-block prefix for each tile height (tile counts and their
//      exclusive prefix, [GG] "Problem descriptors and the tile scheduler");
//      the experts ordered by load; the rows no assignment fills.  Then a
//      stable counting sort inside
//      each block: every wave counts its range per expert, takes its base from
//      the block base and the waves before it, then walks its range in order
//      and places each assignment at (base + rank among equal ids earlier in
//      the same 64-wide chunk), giving row -> assignment, row -> token and the
//      per-row routing weight ([CARD] "How it works"; [NOTE] 4.1).
// Equal ids inside a chunk are matched with one ballot per id bit, so ranks do
// not depend on the order in which hardware executes atomics: the result is
// deterministic and equals a stable argsort by expert.
#include <string.h>

#include <mutex>

#include "common.hpp"

namespace moe {

namespace {

constexpr int kBlkThreads = 256;  // hist / place workgroups: 4 waves
constexpr int kBlkWaves = kBlkThreads / kWave;
constexpr int kTableInts = 16384;  // bound on the block x expert table

MOE_DEV uint64_t ballot(bool p) { return __ballot(p); }

// Exclusive prefix sum over the workgroup's kBlkThreads threads, one int each.
// `scratch` holds kBlkWaves + 1 ints.  Returns the prefix; *total gets the sum.
MOE_DEV int block_exclusive_scan(int v, int *scratch, int *total) {
  constexpr int kWaves = kBlkWaves;
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

struct BlockRange {
  int begin, end;  // this wave's assignments [begin, end)
};
// Wave w of block b owns a contiguous quarter of the block's B ids (B % 256 == 0).
MOE_DEV BlockRange wave_range(int b, int B, int S, int w) {
  const int q = B / kBlkWaves;
  const int s0 = min(S, b * B + w * q);
  return BlockRange{s0, min(S, s0 + q)};
}

// One counting sort of the assignments by a key, with everything it writes.
//   by_rank 0: key = the expert id (the canonical schedule);
//   by_rank 1: key = p * E + e, p = the assignment's rank among the valid
//              assignments of its token (0 for the first valid slot, ...):
//              rows ordered by (rank, expert, s).  A token with no valid
//              assignment gets one row of key 0 (rank 0, expert 0) with weight
//              0 and assignment -1, placed at its last slot's s, so that every
//              token has exactly one rank-0 row.
struct SortJob {
  int nkeys;        // E, or k * E
  int by_rank;
  int32_t *table;   // [nblk][nkeys] per-block counts
  int32_t *inv;     // [nblk] excluded assignments per block (by_rank 0), else NULL
  int32_t *counts, *offsets;  // [nkeys]
  int32_t *block_start;       // [MOE_NUM_BM][nkeys + 1]
  int32_t *expert_order;      // [nkeys] (by_rank 0), else NULL
  int32_t *row_to_assign, *row_to_token;
  float *row_weight;
  int32_t *status;            // (by_rank 0), else NULL
  int32_t *sync;              // (by_rank 1) ranked-combine counters, zeroed here
  int32_t *queue;             // (by_rank 0) the weight gradient's work-queue counters, zeroed here
};
struct SortJobs {
  SortJob j[2];
};

// Key of assignment s (id = ids[s]) for a sort, or -1 when s is in no group.
MOE_DEV int sort_key(const SortJob &job, const int32_t *__restrict__ ids, int s, int id, int k,
                     int E) {
  const bool valid = id >= 0 && id < E;
  if (!job.by_rank) return valid ? id : -1;
  const int t = s / k, j = s - t * k;
  int before = 0, others = 0;
  for (int jj = 0; jj < k; ++jj) {
    if (jj == j) continue;
    const int o = ids[t * k + jj];
    const int v = (o >= 0 && o < E) ? 1 : 0;
    before += jj < j ? v : 0;
    others += v;
  }
  if (valid) return before * E + id;
  return (j == k - 1 && others == 0) ? 0 : -1;
}

// ---- 1. per-block histogram ---------------------------------------------------
// Workgroup (job, b) counts the keys of block b's assignments for sort `job`.
__global__ __launch_bounds__(kBlkThreads) void sched_hist_kernel(
    const int32_t *__restrict__ ids, int S, int k, int E, int B, int nblk, SortJobs jobs) {
  extern __shared__ int hist[];  // [nkeys + 1]
  const int tid = threadIdx.x;
  const int jb = blockIdx.x / nblk, b = blockIdx.x - jb * nblk;
  const SortJob &job = jobs.j[jb];
  const int nk = job.nkeys;
  for (int e = tid; e <= nk; e += kBlkThreads) hist[e] = 0;
  __syncthreads();
  int invalid = 0;
  const int s0 = b * B, s1 = min(S, s0 + B);
  for (int s = s0 + tid; s < s1; s += kBlkThreads) {
    const int id = ids[s];
    const int key = sort_key(job, ids, s, id, k, E);
    if (key >= 0)
      atomicAdd(&hist[key], 1);
    if (id < 0 || id >= E) ++invalid;
  }
  for (int d = kWave / 2; d >= 1; d >>= 1) invalid += __shfl_xor(invalid, d, kWave);
  __syncthreads();
  if ((tid & (kWave - 1)) == 0 && invalid) atomicAdd(&hist[nk], invalid);  // hist has nk+1 ints
  __syncthreads();
  for (int e = tid; e < nk; e += kBlkThreads) job.table[(size_t)b * nk + e] = hist[e];
  if (tid == 0 && job.inv) job.inv[b] = hist[nk];
}

// Exclusive prefix over keys of val[0 .. n-1] (LDS) into out[] (LDS), each
// thread summing a run of consecutive keys; returns the total.
MOE_DEV int scan_experts(const int *val, int *out, int n, int *scratch) {
  const int chunk = (n + kBlkThreads - 1) / kBlkThreads;
  const int e0 = min(n, (int)threadIdx.x * chunk), e1 = min(n, e0 + chunk);
  int sum = 0;
  for (int e = e0; e < e1; ++e) sum += val[e];
  int total;
  int pre = block_exclusive_scan(sum, scratch, &total);
  for (int e = e0; e < e1; ++e) {
    out[e] = pre;
    pre += val[e];
  }
  __syncthreads();
  return total;
}

// ---- 2. bases, per-key outputs, stable placement ------------------------------
// Workgroup (job, b): block b's placement for sort `job`.
__global__ __launch_bounds__(kBlkThreads) void sched_place_kernel(
    const int32_t *__restrict__ ids, const float *__restrict__ w, int S, int k, int E, int B,
    int nblk, int layout, int capacity, int R, SortJobs jobs) {
  extern __shared__ int smem[];
  const int jb = blockIdx.x / nblk, b = blockIdx.x - jb * nblk;
  const SortJob &job = jobs.j[jb];
  const int nk = job.nkeys;
  int *hist = smem;                      // [kBlkWaves][nk]: per-wave counts, then running bases
  int *base = hist + kBlkWaves * nk;     // [nk] this block's base inside each key
  int *cnt = base + nk;                  // [nk] rows per key
  int *rowbase = cnt + nk;               // [nk] first row of each key
  int *tmp = rowbase + nk;               // [2][nk] tile counts and their prefix
  int *scratch = tmp + 2 * nk;           // [kBlkWaves + 1]
  int *tally = scratch + kBlkWaves + 1;  // [2] invalid ids, assignments over capacity
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
  const bool masked = !job.by_rank && layout == MOE_LAYOUT_MASKED;
  // this wave's first kBatch x 64 ids and weights, loaded before anything
  // else so their latency overlaps the table sums (with B <= 1024 that is the
  // wave's whole range)
  constexpr int kBatch = 4;
  const BlockRange rg = wave_range(b, B, S, wid);
  int idv0[kBatch];
  float wv0[kBatch];
#pragma unroll
  for (int u = 0; u < kBatch; ++u) {
    const int s = rg.begin + u * kWave + lane;
    idv0[u] = s < rg.end ? ids[s] : -1;
    wv0[u] = (s < rg.end && w) ? w[s] : 1.f;
  }
  const bool one_batch = rg.end - rg.begin <= kBatch * kWave;  // wave-uniform
  for (int i = tid; i < kBlkWaves * nk; i += kBlkThreads) hist[i] = 0;
  if (tid < 2) tally[tid] = 0;
  __syncthreads();
  // the table's column sums: this block's base and each key's total
  for (int e = tid; e < nk; e += kBlkThreads) {
    int before = 0, m_e = 0;
    for (int b0 = 0; b0 < nblk; b0 += 8) {
      int c[8];
#pragma unroll
      for (int u = 0; u < 8; ++u)  // eight loads in flight, then the sums
        c[u] = b0 + u < nblk ? job.table[(size_t)(b0 + u) * nk + e] : 0;
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        before += b0 + u < b ? c[u] : 0;
        m_e += c[u];
      }
    }
    base[e] = before;
    cnt[e] = masked ? min(m_e, capacity) : m_e;
    if (b == 0 && masked && m_e > capacity) atomicAdd(&tally[1], m_e - capacity);
  }
  __syncthreads();
  // packed prefix of the counts: END offsets in both layouts, first rows in the
  // contiguous one (the masked layout starts expert e at e * capacity)
  const int total = scan_experts(cnt, rowbase, nk, scratch);
  for (int e = tid; e < nk; e += kBlkThreads) {
    if (b == 0) {
      job.counts[e] = cnt[e];
      job.offsets[e] = rowbase[e] + cnt[e];
    }
    if (masked) rowbase[e] = e * capacity;
  }
  // the per-key outputs, one job per workgroup (workgroup j % nblk takes
  // job j), each on the counts every workgroup has summed
  if (b == 1 % nblk) {
#pragma unroll
    for (int i = 0; i < MOE_NUM_BM; ++i) {
      const int bm = 32 << i;
      for (int e = tid; e < nk; e += kBlkThreads)
        tmp[e] = masked ? (capacity + bm - 1) / bm : (cnt[e] + bm - 1) / bm;
      __syncthreads();
      const int tot = scan_experts(tmp, tmp + nk, nk, scratch);
      for (int e = tid; e < nk; e += kBlkThreads) job.block_start[i * (nk + 1) + e] = tmp[nk + e];
      if (tid == 0) job.block_start[i * (nk + 1) + nk] = tot;
      __syncthreads();
    }
  }
  if (b == 2 % nblk && job.expert_order) {
    // experts by descending row count, ties by id
    for (int e = tid; e < nk; e += kBlkThreads) {
      const int c = cnt[e];
      int rank = 0;
      for (int o = 0; o < nk; ++o) {
        const int co = cnt[o];
        rank += (co > c || (co == c && o < e)) ? 1 : 0;
      }
      job.expert_order[rank] = e;
    }
  }
  if (b == 2 % nblk && job.sync) {
    for (int i = tid; i < kRankSyncInts; i += kBlkThreads) job.sync[i] = 0;
  }
  if (b == 2 % nblk && job.queue && tid < 2) job.queue[tid] = 0;
  if (b == 3 % nblk) {
    // rows no assignment fills: past the last filled row (contiguous) or past
    // each expert's valid prefix (masked)
    if (!masked) {
      for (int r = total + tid; r < R; r += kBlkThreads) {
        job.row_to_assign[r] = -1;
        job.row_to_token[r] = -1;
        job.row_weight[r] = 0.f;
      }
    } else {
      for (int r = tid; r < R; r += kBlkThreads) {
        const int ex = r / capacity;
        if (r - ex * capacity >= cnt[ex]) {
          job.row_to_assign[r] = -1;
          job.row_to_token[r] = -1;
          job.row_weight[r] = 0.f;
        }
      }
    }
  }
  if (b == 0 && job.status) {
    int inv = 0;
    for (int i = tid; i < nblk; i += kBlkThreads) inv += job.inv[i];
    if (inv) atomicAdd(&tally[0], inv);
    __syncthreads();
    if (tid == 0) {
      job.status[0] = tally[0];
      job.status[1] = tally[1];
    }
  }
  // keys of this wave's assignments (the preloaded batch)
  int kv0[kBatch];
#pragma unroll
  for (int u = 0; u < kBatch; ++u) {
    const int s = rg.begin + u * kWave + lane;
    kv0[u] = s < rg.end ? sort_key(job, ids, s, idv0[u], k, E) : -1;
  }
  if (one_batch) {
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
      if (kv0[u] >= 0) atomicAdd(&hist[wid * nk + kv0[u]], 1);
  } else {
    for (int s = rg.begin + lane; s < rg.end; s += kWave) {
      const int key = sort_key(job, ids, s, ids[s], k, E);
      if (key >= 0) atomicAdd(&hist[wid * nk + key], 1);
    }
  }
  __syncthreads();
  // per-wave base = rank base of this block inside the key + earlier waves
  for (int e = tid; e < nk; e += kBlkThreads) {
    int run = base[e];
    for (int v = 0; v < kBlkWaves; ++v) {
      const int c = hist[v * nk + e];
      hist[v * nk + e] = run;
      run += c;
    }
  }
  __syncthreads();

  int nbits = 1;
  while ((1 << nbits) < nk) ++nbits;
  for (int b0 = rg.begin; b0 < rg.end; b0 += kBatch * kWave) {
    int kv[kBatch];
    float wv[kBatch];
    if (b0 == rg.begin) {  // wave-uniform: the preloaded batch
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        kv[u] = kv0[u];
        wv[u] = wv0[u];
      }
    } else {
      int idv[kBatch];
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {  // all loads of the batch before any use
        const int s = b0 + u * kWave + lane;
        idv[u] = s < rg.end ? ids[s] : -1;
        wv[u] = (s < rg.end && w) ? w[s] : 1.f;
      }
#pragma unroll
      for (int u = 0; u < kBatch; ++u) {
        const int s = b0 + u * kWave + lane;
        kv[u] = s < rg.end ? sort_key(job, ids, s, idv[u], k, E) : -1;
      }
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      if (b0 + u * kWave >= rg.end) break;  // wave-uniform
      const int s = b0 + u * kWave + lane;
      const int key = kv[u];
      const bool valid = s < rg.end && key >= 0;
      const uint64_t m = peers(key, valid, nbits);
      int rank = 0;
      if (valid) rank = hist[wid * nk + key] + __popcll(m & below);
      if (valid && (m & below) == 0) hist[wid * nk + key] += __popcll(m);
      if (valid && (!masked || rank < capacity)) {
        const int r = rowbase[key] + rank;
        // a token's row with no valid assignment (rank order only): weight 0
        const int id = ids[s];
        const bool real = id >= 0 && id < E;
        job.row_to_assign[r] = real ? s : -1;
        job.row_to_token[r] = s / k;
        job.row_weight[r] = real ? wv[u] : 0.f;
      }
    }
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

// Zero up to two byte ranges in one launch: 16-byte stores over the aligned part
// of each, then the bytes of each tail.  Plain stores rather than nontemporal
// ones: 134 MB took 22 instead of 29 us, and the zeros the next kernel's
// atomics update partly stay in the caches.
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
struct FillRange {
  u32x4_t *p;
  size_t n16;
  uint8_t *tail;
  int ntail;
};
__global__ void fill_zero_kernel(FillRange a, FillRange b) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  const u32x4_t z = {0u, 0u, 0u, 0u};
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < a.n16 + b.n16; i += stride) {
    if (i < a.n16)
      a.p[i] = z;
    else
      b.p[i - a.n16] = z;
  }
  if (blockIdx.x == 0 && (int)threadIdx.x < a.ntail) a.tail[threadIdx.x] = 0;
  if (blockIdx.x == 0 && (int)threadIdx.x < b.ntail) b.tail[threadIdx.x] = 0;
}

}  // namespace

// Block size of the build: a power of two of at least 256 ids.  Small builds
// take about 16 blocks (more workgroups share the placement; measured on
// MI355X: S = 1024 in 13.6 us against 20.7 with one 1024-id block, S = 8192
// 14.2 against 14.9), larger ones blocks of 1024 (smaller blocks were slower
// there: S = 32768 20.5 against 17.2 us); and large enough that the block x
// key table of the larger sort fits the scan's LDS.
int schedule_block(int64_t S, int nkeys) {
  int64_t B = 256;
  while (B < 1024 && (S + B - 1) / B > 16) B *= 2;
  while (((S + B - 1) / B) * nkeys > kTableInts) B *= 2;
  return (int)B;
}
int schedule_blocks(int64_t S, int nkeys) {
  const int B = schedule_block(S, nkeys);
  return (int)((S + B - 1) / B);
}

bool rank_order_supported(int layout, int k, int E) {
  return layout == MOE_LAYOUT_CONTIGUOUS && k <= kMaxRankK && k * E <= kMaxRankKeys;
}

hipError_t launch_build_schedule(const int32_t *ids, const float *w, const moe_schedule &s,
                                 int32_t *scratch, hipStream_t st) {
  const int S = (int)s.S, E = s.E, k = s.k;
  const bool ranked = s.phases > 0;
  const int nk1 = ranked ? k * E : 0;
  const int nkmax = nk1 > E ? nk1 : E;
  const int B = schedule_block(S, nkmax), nblk = schedule_blocks(S, nkmax);
  SortJobs jobs;
  memset(&jobs, 0, sizeof(jobs));
  SortJob &c = jobs.j[0];
  c.nkeys = E;
  c.by_rank = 0;
  c.table = scratch;                         // [nblk * E]
  c.inv = c.table + (size_t)nblk * E;        // [nblk]
  c.counts = s.counts;
  c.offsets = s.offsets;
  c.block_start = s.block_start;
  c.expert_order = s.expert_order;
  c.row_to_assign = s.row_to_assign;
  c.row_to_token = s.row_to_token;
  c.row_weight = s.row_weight;
  c.status = s.status;
  c.queue = s.dw_queue;
  if (ranked) {
    SortJob &p = jobs.j[1];
    p.nkeys = nk1;
    p.by_rank = 1;
    p.table = c.inv + nblk;                  // [nblk * k * E]
    p.counts = s.phase_counts;
    p.offsets = s.phase_offsets;
    p.block_start = s.phase_block_start;
    p.row_to_assign = s.phase_row_to_assign;
    p.row_to_token = s.phase_row_to_token;
    p.row_weight = s.phase_row_weight;
    p.sync = s.phase_sync;
  }
  const int grid = nblk * (ranked ? 2 : 1);
  hipLaunchKernelGGL(sched_hist_kernel, dim3(grid), dim3(kBlkThreads), sizeof(int) * (nkmax + 1),
                     st, ids, S, k, E, B, nblk, jobs);
  const size_t place_smem = sizeof(int) * ((size_t)(kBlkWaves + 5) * nkmax + kBlkWaves + 1 + 2);
  hipLaunchKernelGGL(sched_place_kernel, dim3(grid), dim3(kBlkThreads), place_smem, st, ids, w, S,
                     k, E, B, nblk, s.layout, s.capacity, (int)s.R, jobs);
  return hipGetLastError();
}

// Block tables of the build for callers that cannot allocate device memory:
// one array per device, as large as any build needs (each of the two sort jobs
// keeps at most kTableInts block x key counts, and one word per block), held
// until the process ends.  Its device address is taken once per device with
// hipGetSymbolAddress (in host code the name stands for a host-side shadow).
constexpr size_t kStaticTableInts = 3 * (size_t)kTableInts;
static __device__ __align__(256) int32_t sched_scratch[kStaticTableInts];

hipError_t static_schedule_scratch(int32_t **tables, size_t *bytes) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static int32_t *addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(sched_scratch));
    if (e != hipSuccess) return e;
    addr[dev] = (int32_t *)p;
  }
  *tables = addr[dev];
  *bytes = sizeof(int32_t) * kStaticTableInts;
  return hipSuccess;
}

size_t schedule_scratch_bytes(int64_t S, int E, int k, bool ranked) {
  const int nk1 = ranked ? k * E : 0;
  const int nkmax = nk1 > E ? nk1 : E;
  const int nblk = schedule_blocks(S, nkmax);
  return sizeof(int32_t) * ((size_t)nblk * (E + nk1) + nblk);
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

hipError_t launch_fill_zero(void *p, size_t bytes, void *p2, size_t bytes2, hipStream_t st) {
  if (!p) bytes = 0;
  if (!p2) bytes2 = 0;
  if (bytes + bytes2 == 0) return hipSuccess;
  auto range = [](void *q, size_t n) {
    const size_t n16 = n / 16;
    return FillRange{(u32x4_t *)q, n16, (uint8_t *)q + n16 * 16, (int)(n - n16 * 16)};
  };
  const FillRange a = range(p, bytes), b = range(p2, bytes2);
  int blocks = (int)((a.n16 + b.n16 + 255) / 256);
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(fill_zero_kernel, dim3(blocks), dim3(256), 0, st, a, b);
  return hipGetLastError();
}

}  // namespace moe
