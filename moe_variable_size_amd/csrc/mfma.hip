// bf16 grouped GEMM kernels on the gfx950 matrix cores (MFMA), fp32 accumulation.
//
// [GG] = "Grouped GEMM for MoE, in depth" (aicassindra.com)
// [CARD] = "grouped-gemm-moe" model card
// [NOTE] = "Grouped GEMM" study notes (scholia-log)
//
// All kernels share one tile core (tile_multiply).
//  * A persistent workgroup per compute unit owns a 256 x 256 fp32 output tile
//    made of 32 x 32 blocks, each one v_mfma_f32_32x32x16_bf16 accumulator
//    (16 fp32 per lane).  Wave grids: forward 8 waves, 2 x 4 (128 x 64 per
//    wave, two waves per SIMD); input gradient 4 waves, 2 x 2 (128 x 128 per
//    wave, one per SIMD: its routing-weight epilogue needs the registers);
//    weight gradient 8 waves, 4 x 2.  Wave (wm, wn) owns row blocks wm,
//    wm + WGM, ... and column blocks wn, wn + WGN, ...
//  * The reduction advances 64 elements (128 bytes of a bf16 row) per stage.
//    An operand tile sits in LDS in one of two layouts:
//      K-major : [tile row][64 reduction elements], 128 B per row -- token rows
//                and weight rows whose reduction index is contiguous in memory
//                (both operands of the forward, dY in the input gradient);
//      MN-major: [64 reduction rows][256 tile columns], 512 B per row --
//                operands whose reduction index is strided in memory (the
//                weights in the input gradient, both weight-gradient operands).
//    16-byte chunks are XOR-swizzled by the row so that the operand reads and
//    the DMA writes are free of bank conflicts.
//  * Tiles are loaded by direct global->LDS DMA (buffer_load ... lds, 16 bytes
//    per lane, any global address per lane): gathered token rows land in LDS
//    without passing through registers ([CARD] "How it works": rows gathered
//    on load).  A per-lane offset past the buffer returns zeros, which masks
//    rows past a group's end and columns past N ([GG] "Problem descriptors and
//    the tile scheduler").  Every stage but the last of a reduction range keeps
//    fixed per-lane offsets and passes the stage's advance as the scalar
//    offset (outside the range check, so only stages wholly inside every row
//    take it); the last stage is checked per lane.
//  * MFMA operands come from K-major tiles with one 16-byte read per lane and
//    from MN-major tiles with two ds_read_b64_tr_b16 (transposing reads).
//  * Two LDS stages of 64 KB (A then B).  A stage is four 16-deep MFMA steps
//    (two 64-deep steps for 8-bit operands); each step's MFMAs have the next
//    step's fragment reads placed between them; one vector-memory wait and one
//    barrier per stage, then the last step issues the DMA of the stage two
//    ahead into the buffer just released.  The DMA is issued from inline
//    assembly with explicit wait accounting, so the compiler's conservative
//    waits on LDS DMA do not serialise the pipeline.  The masked decode's
//    64-row tiles take a streaming loop instead (tile_multiply_deep: compact
//    stages, several in flight).
//  * Workgroup ids are remapped so that each of the 8 XCDs (one L2 each) takes
//    a contiguous slice of the flat tile space; inside a group tiles are
//    walked column-block-major ([GG] "Problem descriptors and the tile
//    scheduler": consecutive tiles share a weight column block in L2).  Whole
//    tiles go out in rounds of one tile per workgroup; the tiles of a last
//    partial round are cut into 8, 4 or 2 sub-tiles, each run before its
//    workgroup's whole tiles.  Forward tiles that end past a group's rows or
//    past N leave out the MFMAs of their dead 32-row and 32-column blocks.
//  * Outputs of the routed forward and of the input gradient are combined by
//    fp32 atomic adds (the default), or by plain stores and read-add-stores in
//    rank order over the schedule's rank-ordered view (COMBINE_RANKED).  The
//    weight gradient stores bf16 tiles through LDS.
#include "common.hpp"

#include <atomic>
#include <type_traits>
#include <utility>

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

#define LDS_AS __attribute__((address_space(3)))

constexpr int NT = 256;        // 4 waves
constexpr int BK = 64;         // reduction elements per stage
constexpr int KS = BK / 16;    // 16-deep MFMA steps per stage
constexpr int KROW = BK * 2;   // bytes per K-major LDS row (one 128-byte line)
constexpr int MNROW = 256 * 2; // bytes per MN-major LDS row (256 columns)
constexpr int NSTAGE = 2;      // LDS stages
constexpr int OPND = 256 * KROW;                  // 32 KB: one 256 x 64 operand tile
constexpr int STAGE = 2 * OPND;                   // A then B
constexpr int TOKSLOTS = 4;                       // token ring slots (weight gradient)
static_assert(OPND == BK * MNROW, "K-major and MN-major operand tiles have one size");

// ---- LDS layouts --------------------------------------------------------------
// The LDS serves 256 bytes per clock (64 banks x 4 B), i.e. sixteen 16-byte
// lane accesses.  The swizzles make 16 consecutive lanes of an operand read hit
// 16 different 16-byte bank groups.
// K-major: chunk c (0..7) of row r at r*128 + ((c ^ ((r >> 1) & 7)) << 4): of the
// 16 rows read together, two share each 256-byte line of banks, and within the
// pair the chunks differ, so the 16 lanes hit 16 different bank groups.
MOE_DEV int kmaj_off(int row, int chunk) { return row * KROW + ((chunk ^ ((row >> 1) & 7)) << 4); }
// MN-major: chunk c (0..31) of reduction row r at r*512 + ((c ^ ((r & 3) << 2)) << 4):
// a transposing read touches 4 rows x 2 chunks per 16 lanes (4 chunks per 32).
MOE_DEV int mnmaj_off(int row, int chunk) { return row * MNROW + ((chunk ^ ((row & 3) << 2)) << 4); }

// ---- DMA and waits ---------------------------------------------------------------
// 16 (dma16) or 4 (dma4) bytes per lane from global (rsrc + voff) to LDS byte
// address lds + size * lane.  `lds` is taken from the first lane.  Nothing else
// in these kernels uses m0, so setting it here disturbs no compiler-held value.
MOE_DEV void dma16(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t lds) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(m0v), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}
// dma16 / dma16_so (below) as non-temporal loads: for operands read once and
// streamed past (the masked decode's expert weights), so their lines do not
// push out of L2 the ones every tile reads again (token rows, scale words);
// measured on the masked decode, E = 64, K = 7168, N = 2048: bf16 318 -> 282
// us, E4M3 165 -> 142, block-scaled 177 -> 147.
MOE_DEV void dma16_nt(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t lds) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen nt lds"
               :
               : "s"(m0v), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}
MOE_DEV void dma16_so_nt(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen nt lds"
               :
               : "s"(m0v), "v"(voff), "s"(rsrc), "s"(soff)
               : "memory", "m0");
}
// As dma16, with a wave-uniform byte offset `soff` added to the address (the
// per-stage advance of a tile whose per-lane offsets stay fixed).  The
// buffer's range check looks at voff (and an immediate offset) only; soff is
// added after it, so a lane whose voff passes the check is not stopped at the
// buffer's end.  Callers therefore use it only for stages that lie wholly
// inside every row (each stage of a reduction range but the last, which takes
// per-lane checked offsets), where voff + soff + 16 stays inside the lane's
// row; a lane masked with voff = kOobOffset stays out of range whatever soff
// is (buffers are smaller than 2^31 bytes).
MOE_DEV void dma16_so(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds"
               :
               : "s"(m0v), "v"(voff), "s"(rsrc), "s"(soff)
               : "memory", "m0");
}
MOE_DEV void dma4(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t lds) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(m0v), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}
// As dma4, with the wave-uniform byte offset `soff` added (cf. dma16_so).
MOE_DEV void dma4_so(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t soff, uint32_t lds) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :
               : "s"(m0v), "v"(voff), "s"(rsrc), "s"(soff)
               : "memory", "m0");
}
template <int N>
MOE_DEV void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// wait until at most `stages` stages of D operations each are outstanding
template <int D>
MOE_DEV void wait_stages(int stages) {
  if (stages >= 3)
    wait_vmcnt<3 * D>();
  else if (stages >= 2)
    wait_vmcnt<2 * D>();
  else if (stages == 1)
    wait_vmcnt<D>();
  else
    wait_vmcnt<0>();
}
MOE_DEV void wait_lgkm0() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
MOE_DEV void barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __syncthreads();
  __builtin_amdgcn_sched_barrier(0);
}

// Data-parallel-primitive moves inside rows of 16 lanes (gfx9 DPP controls).
template <int CTRL>
MOE_DEV float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF,
                                                            0xF, false));
}
// Sum of v over each 32-lane half of the wave, by DPP adds instead of LDS
// permutes: quad_perm [1,0,3,2] and [2,3,0,1] (quads), row_half_mirror (8
// lanes), row_mirror (16 lanes), then row_bcast15 into rows 1 and 3 only.
// The half's sum is valid in lanes 16..31 (first half) and 48..63 (second).
MOE_DEV float half_wave_sum(float v) {
  v += dpp_mov<0xB1>(v);
  v += dpp_mov<0x4E>(v);
  v += dpp_mov<0x141>(v);
  v += dpp_mov<0x140>(v);
  v += __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x142, 0xA, 0xF, false));
  return v;
}

// f(integral_constant<int, 0>) ... f(integral_constant<int, N-1>) in sequence:
// a loop that is unrolled whatever its body's size, so that register arrays
// indexed by its counter stay in registers
template <class F, int... I>
MOE_DEV void unroll_seq(F &&f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>()), ...);
}
template <int N, class F>
MOE_DEV void unroll(F &&f) {
  unroll_seq(f, std::make_integer_sequence<int, N>());
}

// Buffer resource built from wave-uniform values (scalar registers), as the
// DMA instructions require.
MOE_DEV __amdgpu_buffer_rsrc_t uniform_rsrc(const void *p, uint32_t num_records) {
  const uint64_t a = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  const void *q = (const void *)(uintptr_t)(((uint64_t)hi << 32) | lo);
  return make_rsrc(q, __builtin_amdgcn_readfirstlane(num_records));
}

MOE_DEV uint32_t lds_addr(const void *p) {
  return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(const LDS_AS void *)p);
}

// Logical workgroup id: consecutive ids land on one XCD (the hardware deals
// workgroup ids to the 8 XCDs round robin).
MOE_DEV int logical_block() {
  const int G = gridDim.x, b = blockIdx.x;
  return (G & 7) ? b : (b & 7) * (G >> 3) + (b >> 3);
}

// Work split of `total` tiles over G workgroups.  Whole tiles go out in
// rounds of G (workgroup Lb takes tiles Lb, Lb + G, ...).  The tiles of the
// last partial round are cut into S sub-tiles each (S = 8, 4 or 2 with rows
// and columns split, at most one sub-tile per workgroup; S = 1 when even the
// 2-way split leaves more pieces than workgroups), so no workgroup idles for a
// whole tile time and every output element is still produced by exactly one
// workgroup.  A workgroup runs its sub-tile BEFORE its whole tiles, so the
// sub-tile's scatter drains while the whole tiles multiply (run after them, it
// would wait behind the whole tiles' atomics, which retire in order).
struct WorkSplit {
  int G, Lb;
  int next_tile, full, pieces, S;
  bool piece_done;
  int s, nS;  // sub-tile of the current piece (0 of 1 for a whole tile)
  enum { WHOLE = 0, SUBTILE_TAIL = 1 };
  bool pieces_last;  // the piece after the whole tiles (tiles in increasing order)
  MOE_DEV void init(int total, int G_, int Lb_, int mode, int max_split = 8,
                    bool pieces_last_ = false) {
    G = G_;
    Lb = Lb_;
    pieces_last = pieces_last_;
    s = 0;
    nS = 1;
    full = (total / G) * G;
    const int rem = total - full;
    S = 1;
    if (mode == SUBTILE_TAIL && rem > 0)
      S = (max_split >= 8 && rem * 8 <= G) ? 8
          : (max_split >= 4 && rem * 4 <= G) ? 4
          : (max_split >= 2 && rem * 2 <= G) ? 2 : 1;
    pieces = rem * S;
    next_tile = Lb;
    piece_done = false;
  }
  // next piece (tile tau; sub-tile s of nS); false when done
  MOE_DEV bool next(int &tau) {
    // a workgroup's piece of the last round comes first: its few atomics
    // drain while the whole tiles multiply, instead of queueing behind them
    // (with pieces_last, after them: tiles then run in increasing index order)
    if (!piece_done && Lb < pieces && (!pieces_last || next_tile >= full)) {
      piece_done = true;
      tau = full + Lb / S;
      s = Lb % S;
      nS = S;
      return true;
    }
    if (!pieces_last) piece_done = true;
    if (next_tile < full) {
      tau = next_tile;
      next_tile += G;
      s = 0;
      nS = 1;
      return true;
    }
    return false;
  }
};

// Sub-tile s of nS (2: 128 x 256, 4: 128 x 128, 8: 64 x 128) of a 256 x 256 tile.
struct SubTile {
  int r0, c0, rows, cols;  // offsets inside the tile and extents
};
MOE_DEV SubTile sub_tile(int s, int nS) {
  if (nS == 2) return SubTile{s * 128, 0, 128, 256};
  const int rows = nS == 8 ? 64 : 128, cols = 128;
  return SubTile{(s >> 1) * rows, (s & 1) * cols, rows, cols};
}

// Rows per tile of a launch over a routing schedule, picked on the device from
// the row-block totals the schedule already holds (no read-back): 256-row
// tiles unless 128-row tiles (computed with the 128 x 256 shape) are estimated
// to finish sooner ([GG] "Worked example: tile counts under skew": small tiles
// waste fewer rows but reuse each loaded weight tile half as often).  The
// estimate is rounds of tiles over the G workgroups (at least one) times the
// time of one tile, a 128 x 256 tile counted at 0.75 of a 256 x 256 one: whole
// rounds of 128 x 256 tiles took 0.64 of the time on MI355X, and at estimates
// closer than 0.75 the 256-row tiles still won (their last round splits
// better).  Every workgroup reads the same totals and takes the same decision.
// forced = 128 or 256 overrides the estimate.
// bstart_all: the prefixes of the launch's E groups for each tile height,
// `stride` ints apart (a window of the rank-ordered view's longer prefixes is
// read relative to its first entry).
MOE_DEV int pick_tile_rows(const int32_t *bstart_all, int stride, int E, int tiles_n, int G,
                           int forced) {
  if (forced == 128 || forced == 256) return forced;
  const int32_t *b256 = bstart_all + bm_index(256) * stride;
  const int32_t *b128 = bstart_all + bm_index(128) * stride;
  const float r256 = (float)(b256[E] - b256[0]) * tiles_n / G;
  const float r128 = (float)(b128[E] - b128[0]) * tiles_n / G;
  return __builtin_amdgcn_readfirstlane(0.75f * fmaxf(r128, 1.f) < fmaxf(r256, 1.f) ? 128 : 256);
}

// Sub-tile s of nS (2: 128 x 128, 4: 64 x 128) of a 128 x 256 tile.
MOE_DEV SubTile sub_tile128(int s, int nS) {
  if (nS == 2) return SubTile{0, s * 128, 128, 128};
  return SubTile{(s >> 1) * 64, (s & 1) * 128, 64, 128};
}

// ---- MFMA operand fragments ----------------------------------------------------
// Lane l of a 32x32x16 MFMA holds, for operand row/column (l & 31), the 8
// reduction elements 8*(l >> 5) .. +7 of the 16-element step.

// K-major: one 16-byte read.
MOE_DEV bf16x8_t frag_kmaj(const char *tile, int row, int step, int lane) {
  return *(const bf16x8_t *)(tile + kmaj_off(row, 2 * step + (lane >> 5)));
}

// 8-bit operands: a step is 64 reduction elements (64 bytes of the row, 16-byte
// chunks 4 step + 0..3).  The matrix core takes bytes 0-15 of both lane halves
// as its first 32-element block (scaled by the half-0 lane's block scale) and
// bytes 16-31 as its second (half-1 lane's scale) -- measured with one-hot
// operands on gfx950.  So lane half h loads chunk h (elements 16h .. 16h+15)
// into bytes 0-15 and chunk 2 + h (32 + 16h ..) into bytes 16-31: the first
// block is elements 0-31 of the step, the second 32-63, as the block scales
// count them.  A and B fragments use the same pattern.
MOE_DEV i32x8 frag_kmaj8(const char *tile, int row, int step, int lane) {
  const int c = 4 * step + (lane >> 5);
  const i32x4 lo = *(const i32x4 *)(tile + kmaj_off(row, c));
  const i32x4 hi = *(const i32x4 *)(tile + kmaj_off(row, c + 2));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// 32 x 32 x 64 product of E4M3 operands (format code 0 for A and B), fp32
// accumulation; the block scales of the instruction are left at 2^0 (E8M0 127).
MOE_DEV f32x16 mfma_f8(const i32x8 &a, const i32x8 &b, const f32x16 &c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0x7f7f7f7f, 0,
                                                         0x7f7f7f7f);
}

// MN-major: two transposing reads.  In each 16-lane group, lane j supplies the
// address of 4 consecutive columns of reduction row (j >> 2) and receives the
// 4 rows of column (j & 15) of the 4 x 16 block.
MOE_DEV bf16x8_t frag_mnmaj(const char *tile, int col0, int step, int lane) {
  const int j = lane & 15;
  const int col = col0 + ((lane >> 4) & 1) * 16 + 4 * (j & 3);
  const int r = step * 16 + 8 * (lane >> 5) + (j >> 2);
  const int inchunk = (col & 7) * 2;
  LDS_AS i16x4 *p0 = (LDS_AS i16x4 *)(LDS_AS char *)(tile + mnmaj_off(r, col >> 3) + inchunk);
  LDS_AS i16x4 *p1 = (LDS_AS i16x4 *)(LDS_AS char *)(tile + mnmaj_off(r + 4, col >> 3) + inchunk);
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p0);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(p1);
  const i16x8 v = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  return __builtin_bit_cast(bf16x8_t, v);
}

// Multiply the 8 elements of a fragment by 8 fp32 factors, rounding to bf16.
MOE_DEV bf16x8_t scale_frag(bf16x8_t f, const float (&w)[8]) {
  bf16x8_t o;
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = (__bf16)((float)f[i] * w[i]);
  return o;
}

// Row r of a 32x32 MFMA accumulator held in register i of lane `lane`.
MOE_DEV int acc_row(int i, int lane) { return ((i >> 2) << 3) + ((lane >> 5) << 2) + (i & 3); }

// ---- the pipelined tile multiply --------------------------------------------
// Op supplies:
//   static constexpr bool A_KMAJ, B_KMAJ  operand layouts
//   static constexpr bool A_SCALED        A fragments are multiplied by per-
//       reduction-row factors read with row_scale(buf, step, lane, w)
//   static constexpr bool PREFETCH        prefetch(kt) must run (LDS reads)
//       before the parts of stage kt are issued
//   static constexpr int DMA_PER_STAGE    DMA instructions per thread per stage
//   static constexpr bool CHECKED_TAIL    only the last stage of a range needs
//       bounds checks (its whole stages take the cheaper unchecked DMA)
//   template <bool SKIP, bool CHECKED> void issue_part(int kt, int buf, int j)
//       j-th DMA instruction of stage kt (SKIP: may be left out for dead rows;
//       CHECKED: the stage may reach past the reduction length, so each lane's
//       chunk is bounds-checked; otherwise the stage lies wholly inside it)
// Buffer b: A at lds + b * STAGE, B at + OPND.
//
// A stage holds 64 reduction elements = four 16-deep MFMA steps; operand
// fragments alternate between register slots 0 and 1 (step s uses slot s & 1).
//   steps 0..2: the MFMAs of the step, with the reads of the next step of the
//               same stage placed between them;
//   then:       wait for the next stage's DMA and this wave's reads; barrier
//               (every wave is done with this stage's buffer);
//   step 3:     the MFMAs, with the DMA of stage +2 into the freed buffer and
//               the reads of the next stage's step 0 placed between them.
// So a stage's DMA has one whole stage of MFMAs to land, and the MFMA pipe is
// idle only across the barrier.  The order inside a step is pinned with
// scheduling fences.
#define MOE_FENCE() __builtin_amdgcn_sched_barrier(0)
// SKIP: wave-uniform live_mi / live_ni bound the row / column blocks this wave
// multiplies, and the Op may leave out DMA instructions of dead rows.
// DSKIP: the Op leaves out DMA instructions whose rows are all dead.
template <int MI, int NI, int WGM, int WGN, bool SKIP, class Op, bool DSKIP = SKIP,
          bool NTW = false>
MOE_DEV void tile_multiply(Op &op, char *lds, int kb, int ke, int wm, int wn, int lane,
                           int live_mi, int live_ni, f32x16 (&acc)[MI][NI]) {
  constexpr int D = Op::DMA_PER_STAGE;
  constexpr bool F8 = Op::F8;                           // 8-bit operands, 64-deep steps
  constexpr int KSt = F8 ? 2 : KS;                      // steps per stage
  constexpr int NM = MI * NI;                           // MFMAs per step
  constexpr int NR = MI + NI + (Op::A_SCALED ? 1 : 0);  // read items per step
  constexpr int NS = Op::A_SCALED ? MI : 0;             // scale items per step
  constexpr int NP = Op::PREFETCH ? 1 : 0;
  constexpr int SLOTS = NM - NS;                        // MFMA slots for reads / DMA
  static_assert(SLOTS > 0, "tile too small");
  static_assert((KSt == 4 || KSt == 2) && NSTAGE == 2, "pipeline written for 2 or 4 steps x 2 stages");
  static_assert(!F8 || (Op::A_KMAJ && Op::B_KMAJ && !Op::A_SCALED), "8-bit operands are K-major");
  using frag_t = std::conditional_t<F8, i32x8, bf16x8_t>;
  frag_t fa[2][MI], fb[2][NI];
  float sc[2][8];
  constexpr bool MXS = Op::MX;  // block scales ride with each fragment
  uint32_t fsa[2][MXS ? MI : 1], fsb[2][MXS ? NI : 1];

  // read item f, in order of first use by the next step's MFMAs (mi outer,
  // ni inner): [scale factors], A0, B0 .. B(NI-1), A1 .. A(MI-1)
  auto read_item = [&](int buf, int step, int slot, int f) __attribute__((always_inline)) {
    const char *As = lds + buf * STAGE;
    const char *Bs = As + OPND;
    if (Op::A_SCALED && f == 0) {
      op.row_scale(buf, step, lane, sc[slot]);
      return;
    }
    const int g = f - (Op::A_SCALED ? 1 : 0);
    if constexpr (F8) {
      if (g == 0 || g > NI) {
        const int mi = g == 0 ? 0 : g - NI;
        const int row = wm * 32 + mi * 32 * WGM + (lane & 31);
        fa[slot][mi] = frag_kmaj8(As, row, step, lane);
        if constexpr (MXS) fsa[slot][mi] = op.scale_of(buf, false, row, step, lane);
      } else {
        const int ni = g - 1;
        const int row = wn * 32 + ni * 32 * WGN + (lane & 31);
        fb[slot][ni] = frag_kmaj8(Bs, row, step, lane);
        if constexpr (MXS) fsb[slot][ni] = op.scale_of(buf, true, row, step, lane);
      }
      return;
    } else {
      if (g == 0 || g > NI) {
        const int mi = g == 0 ? 0 : g - NI;
        if (Op::A_KMAJ)
          fa[slot][mi] = frag_kmaj(As, wm * 32 + mi * 32 * WGM + (lane & 31), step, lane);
        else
          fa[slot][mi] = frag_mnmaj(As, wm * 32 + mi * 32 * WGM, step, lane);
      } else {
        const int ni = g - 1;
        if (Op::B_KMAJ)
          fb[slot][ni] = frag_kmaj(Bs, wn * 32 + ni * 32 * WGN + (lane & 31), step, lane);
        else
          fb[slot][ni] = frag_mnmaj(Bs, wn * 32 + ni * 32 * WGN, step, lane);
      }
    }
  };
  auto mfma = [&](int slot, int i) __attribute__((always_inline)) {
    const int mi = i / NI, ni = i % NI;
    if (SKIP && (mi >= live_mi || ni >= live_ni)) return;  // wave-uniform
    if constexpr (MXS)
      acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          fa[slot][mi], fb[slot][ni], acc[mi][ni], 0, 0, 0, fsa[slot][mi], 0, fsb[slot][ni]);
    else if constexpr (F8)
      acc[mi][ni] = mfma_f8(fa[slot][mi], fb[slot][ni], acc[mi][ni]);
    else
      acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[slot][mi], fb[slot][ni],
                                                            acc[mi][ni], 0, 0, 0);
  };
  // step `step` (< KS-1) of the stage in `buf`: MFMAs on slot step&1, reads of
  // step+1 into the other slot; with PF, the prefetch for stage pf
  auto step_inner = [&](int buf, int step, int pf, auto PF) __attribute__((always_inline)) {
    const int slot = step & 1, nslot = slot ^ 1;
    constexpr int NIT = NR + NP;
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      mfma(slot, i);
      MOE_FENCE();
      // reads spread evenly over the step (bunching them saturates the LDS),
      // in first-use order so each has >= 10 MFMAs to land; then the prefetch
#pragma unroll
      for (int j = 0; j < NIT; ++j) {
        if (j * SLOTS / NIT != i) continue;
        if (j < NR)
          read_item(buf, step + 1, nslot, j);
        else if (decltype(PF)::value)
          op.prefetch(pf);
      }
      if constexpr (NS > 0) {
        if (i >= NM - NS)
          fa[nslot][i - (NM - NS)] = scale_frag(fa[nslot][i - (NM - NS)], sc[nslot]);
      }
      MOE_FENCE();
    }
  };
  // last step of the stage in `buf` (slot 1): reads of step 0 of `nbuf` into
  // slot 0; with DMA, stage `dma` is issued into `buf`
  auto step_last = [&](int buf, int nbuf, int dma, auto DMA, auto CHK) __attribute__((always_inline)) {
    constexpr int DD = decltype(DMA)::value ? D : 0;
#pragma unroll
    for (int i = 0; i < NM; ++i) {
      mfma(1, i);
      MOE_FENCE();
      // reads and DMA parts each spread evenly over the step
#pragma unroll
      for (int j = 0; j < NR; ++j)
        if (j * SLOTS / NR == i) read_item(nbuf, 0, 0, j);
#pragma unroll
      for (int j = 0; j < DD; ++j)
        if (j * SLOTS / DD == i) op.template issue_part<DSKIP, decltype(CHK)::value, NTW>(dma, buf, j);
      if constexpr (NS > 0) {
        if (i >= NM - NS) fa[0][i - (NM - NS)] = scale_frag(fa[0][i - (NM - NS)], sc[0]);
      }
      MOE_FENCE();
    }
  };
  auto sync = [&]() __attribute__((always_inline)) {
    wait_lgkm0();
    MOE_FENCE();
    __builtin_amdgcn_s_barrier();
    MOE_FENCE();
  };
  auto issue_stage = [&](int kt, int buf) __attribute__((always_inline)) {
    if (Op::PREFETCH) op.prefetch(kt);
#pragma unroll
    for (int j = 0; j < D; ++j) op.template issue_part<DSKIP, true, NTW>(kt, buf, j);
  };

  // prologue: the first two stages in flight; wait for the first
  const int n = ke - kb;
  issue_stage(kb, 0);
  if (n > 1) {
    issue_stage(kb + 1, 1);
    if (DSKIP)
      wait_vmcnt<0>();  // the instruction count of a stage varies
    else
      wait_vmcnt<D>();
  } else {
    wait_vmcnt<0>();
  }
  sync();
#pragma unroll
  for (int j = 0; j < NR; ++j) read_item(0, 0, 0, j);
  if constexpr (NS > 0) {
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) fa[0][mi] = scale_frag(fa[0][mi], sc[0]);
  }
  MOE_FENCE();

  int kt = kb;
  // stages whose buffer is refilled with stage kt + 2; every stage but the
  // last one of the range lies wholly inside the reduction (an Op whose DMA
  // does not depend on that issues every stage the same way)
  constexpr int PEEL = Op::CHECKED_TAIL ? 1 : 0;
  // steps 1 .. KSt-2 of a stage (no prefetch, no DMA)
  auto middle_steps = [&](int buf) __attribute__((always_inline)) {
#pragma unroll
    for (int st = 1; st < KSt - 1; ++st) step_inner(buf, st, 0, std::false_type());
  };
  for (; kt + 2 + PEEL < ke; ++kt) {
    const int buf = (kt - kb) & 1;
    step_inner(buf, 0, kt + 2, std::integral_constant<bool, Op::PREFETCH>());
    middle_steps(buf);
    wait_vmcnt<0>();  // stage kt+1 landed
    sync();
    step_last(buf, buf ^ 1, kt + 2, std::true_type(), std::false_type());
  }
  // the last stage of the range is issued with bounds checks
  if (PEEL && kt + 2 < ke) {
    const int buf = (kt - kb) & 1;
    step_inner(buf, 0, kt + 2, std::integral_constant<bool, Op::PREFETCH>());
    middle_steps(buf);
    wait_vmcnt<0>();
    sync();
    step_last(buf, buf ^ 1, kt + 2, std::true_type(), std::true_type());
    ++kt;
  }
  // the stage before the last: nothing more to issue
  if (kt + 1 < ke) {
    const int buf = (kt - kb) & 1;
    step_inner(buf, 0, 0, std::false_type());
    middle_steps(buf);
    wait_vmcnt<0>();
    sync();
    step_last(buf, buf ^ 1, 0, std::false_type(), std::false_type());
    ++kt;
  }
  // final stage
  {
    const int buf = (kt - kb) & 1;
    step_inner(buf, 0, 0, std::false_type());
    middle_steps(buf);
#pragma unroll
    for (int i = 0; i < NM; ++i) mfma(1, i);
    MOE_FENCE();
  }
}

// K-major DMA of a tile of R rows x 64 reduction elements (128 bytes per row) by
// NW waves: one instruction fills 8 rows (1 KB of LDS).  Thread (wave w, lane
// p), instruction i loads row (w * R/(8 NW) + i) * 8 + p/8, physical chunk p % 8.
template <int R, int NW = 4>
struct KmajDma {
  static constexpr int PER_WAVE = R / (8 * NW);
  uint32_t base[PER_WAVE];  // per-lane global byte offset of the row chunk, stage 0
  int chunk[PER_WAVE];      // logical chunk (reduction elements 8*chunk .. +7)
  int live_rows;            // rows at or past this are never read (wave-uniform)
  MOE_DEV void setup(int wid, int lane, const int *rowoff /* byte offset of tile row or -1 */,
                     int live = R) {
    live_rows = live;
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) {
      const int row = (wid * PER_WAVE + i) * 8 + (lane >> 3);
      const int c = (lane & 7) ^ ((row >> 1) & 7);
      chunk[i] = c;
      const int ro = rowoff[row];
      base[i] = ro >= 0 ? (uint32_t)ro + (uint32_t)c * 16u : kOobOffset;
    }
  }
  // instruction i of stage kt (SKIP: left out when all its rows are dead; the
  // LDS rows then keep stale values, which only reach dead accumulator rows).
  // CHECKED: chunks at or past the reduction length `kred` read zeros;
  // otherwise the whole stage lies inside every row.  NTL: non-temporal loads.
  template <bool SKIP, bool CHECKED, bool NTL = false>
  MOE_DEV void issue_one(__amdgpu_buffer_rsrc_t rs, int kt, int kred, uint32_t lds_tile, int wid,
                         int i) {
    if (SKIP && (wid * PER_WAVE + i) * 8 >= live_rows) return;
    const uint32_t lds = lds_tile + (uint32_t)((wid * PER_WAVE + i) * 1024);
    if (CHECKED) {
      const bool in = kt * BK + chunk[i] * 8 < kred;
      if (NTL) dma16_nt(rs, in ? base[i] + (uint32_t)kt * KROW : kOobOffset, lds);
      else dma16(rs, in ? base[i] + (uint32_t)kt * KROW : kOobOffset, lds);
    } else {
      if (NTL) dma16_so_nt(rs, base[i], (uint32_t)kt * KROW, lds);
      else dma16_so(rs, base[i], (uint32_t)kt * KROW, lds);
    }
  }
};

// MN-major DMA of a 64 x 256 tile (512 bytes per reduction row) by NW waves: one
// instruction fills 2 rows.  Thread (wave w, lane p), instruction i loads
// reduction row 2 * (w * 32/NW + i) + p/32, physical chunk p % 32.
template <int NW>
struct MnmajMapT {
  static constexpr int PER_WAVE = 32 / NW;
  MOE_DEV static int row_of(int wid, int i, int lane) { return 2 * (wid * PER_WAVE + i) + (lane >> 5); }
  MOE_DEV static int chunk_of(int wid, int i, int lane) {
    return (lane & 31) ^ ((row_of(wid, i, lane) & 3) << 2);
  }
  MOE_DEV static uint32_t lds_of(int wid, int i) { return (uint32_t)((wid * PER_WAVE + i) * 1024); }
};
using MnmajMap = MnmajMapT<4>;

// ---- deep pipeline for streaming tiles ----------------------------------------
// A 64-row masked-decode tile streams its weights through HBM and does few
// MFMAs per stage: its speed is the number of bytes in flight.  It keeps
// NSTAGES stages in flight in a compact LDS layout (stage s at s * STAGE_BYTES,
// B at + A_BYTES) and runs a plain loop per stage: wait for the stage, barrier,
// refill the buffer just released with the stage NSTAGES-1 ahead, multiply.
// (Sub-tiles of a last partial round gain nothing from it: their time per
// stage is the barrier and the read -> MFMA chain, not the DMA.)

// wait until at most n vector-memory operations are outstanding (n >= 16: all)
MOE_DEV void wait_vmcnt_upto(int n) {
  switch (n) {
#define MOE_W(c) \
  case c:        \
    wait_vmcnt<c>(); \
    break;
    MOE_W(1) MOE_W(2) MOE_W(3) MOE_W(4) MOE_W(5) MOE_W(6) MOE_W(7) MOE_W(8)
    MOE_W(9) MOE_W(10) MOE_W(11) MOE_W(12) MOE_W(13) MOE_W(14) MOE_W(15)
#undef MOE_W
    default:
      wait_vmcnt<0>();
  }
}

// Op supplies STAGE_BYTES, A_BYTES, NSTAGES, DMA_PER_STAGE and
// issue_part<SKIP, CHECKED>(kt, buf, j) with SKIP always on; `parts` is the
// number of DMA instructions this wave issues per stage (fixed for the tile,
// as the rows it skips are).  Only the range's last stage is bounds-checked.
template <int MI, int NI, int WGM, int WGN, class Op>
MOE_DEV void tile_multiply_deep(Op &op, char *lds, int kb, int ke, int wm, int wn, int lane,
                                int live_mi, f32x16 (&acc)[MI][NI]) {
  constexpr int NS = Op::NSTAGES, D = Op::DMA_PER_STAGE;
  auto issue = [&](int kt) __attribute__((always_inline)) {
    const int buf = (kt - kb) % NS;
    if (kt == ke - 1) {
#pragma unroll
      for (int j = 0; j < D; ++j) op.template issue_part<true, true>(kt, buf, j);
    } else {
#pragma unroll
      for (int j = 0; j < D; ++j) op.template issue_part<true, false>(kt, buf, j);
    }
  };
  const int pro = min(NS - 1, ke - kb);
  for (int s = 0; s < pro; ++s) issue(kb + s);
  for (int kt = kb; kt < ke; ++kt) {
    const int buf = (kt - kb) % NS;
    // stages issued after kt: kt+1 .. min(kt+NS-2, ke-1)
    int after = 0;
    for (int s2 = kt + 1; s2 <= min(kt + NS - 2, ke - 1); ++s2) after += op.parts_at(s2);
    wait_vmcnt_upto(after);
    wait_lgkm0();
    barrier();  // stage kt in LDS for every wave; the buffer of stage kt-1 is free
    if (kt + NS - 1 < ke) issue(kt + NS - 1);
    const char *As = lds + buf * Op::STAGE_BYTES;
    const char *Bs = As + Op::A_BYTES;
    constexpr bool F8 = Op::F8;
#pragma unroll
    for (int step = 0; step < (F8 ? 2 : KS); ++step) {
      using frag_t = std::conditional_t<F8, i32x8, bf16x8_t>;
      frag_t fa[MI], fb[NI];
      uint32_t sa[Op::MX ? MI : 1], sb[Op::MX ? NI : 1];
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        const int row = wm * 32 + mi * 32 * WGM + (lane & 31);
        if constexpr (F8)
          fa[mi] = frag_kmaj8(As, row, step, lane);
        else
          fa[mi] = frag_kmaj(As, row, step, lane);
        if constexpr (Op::MX) sa[mi] = op.scale_of(kt, false, row, step, lane);
      }
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const int row = wn * 32 + ni * 32 * WGN + (lane & 31);
        if constexpr (F8)
          fb[ni] = frag_kmaj8(Bs, row, step, lane);
        else
          fb[ni] = frag_kmaj(Bs, row, step, lane);
        if constexpr (Op::MX) sb[ni] = op.scale_of(kt, true, row, step, lane);
      }
#pragma unroll
      for (int mi = 0; mi < MI; ++mi) {
        if (mi >= live_mi) continue;  // wave-uniform
#pragma unroll
        for (int ni = 0; ni < NI; ++ni) {
          if constexpr (Op::MX)
            acc[mi][ni] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                fa[mi], fb[ni], acc[mi][ni], 0, 0, 0, sa[mi], 0, sb[ni]);
          else if constexpr (F8)
            acc[mi][ni] = mfma_f8(fa[mi], fb[ni], acc[mi][ni]);
          else
            acc[mi][ni] =
                __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[mi], fb[ni], acc[mi][ni], 0, 0, 0);
        }
      }
    }
  }
}

// ============================================================================
// Forward-shaped kernel: out[r, n] = sum_k A[src(r), k] * W[g, n, k].
//   FUSED: src(r) = row_to_token[r], y[src(r), n] += row_weight[r] * acc
//          (atomic; both layouts) -- [CARD] gather on load, scatter-combine on
//          store, so neither [S, K] nor [S, N] is stored.
//   bare : src(r) = r, C[r, n] = acc (plain store, fp32 or bf16).
// ============================================================================
struct FwdArgs {
  const bf16_t *A;
  const bf16_t *W;
  void *C;
  const int32_t *offsets;
  const int32_t *counts;
  const int32_t *bstart;  // routed: the schedule's row-block prefixes [MOE_NUM_BM][E+1]
  const int32_t *row_to_token;
  const float *row_weight;
  int E, layout, capacity, K, N;
  uint32_t a_bytes;  // bytes of A (x or the bare A)
  int M;             // bare: rows of A and C (rows at or past M are never touched)
  int tile_rows;     // routed, BM = 256: 0 = picked on the device, 128 / 256 = forced
  int bstride;       // routed: ints between the row-block prefixes of two tile heights
  int combine;       // routed scatter: COMBINE_ATOMIC or COMBINE_RANKED
  int nranks;        // COMBINE_RANKED: ranks of the view (the launch has nranks * E groups)
  int32_t *sync;     // COMBINE_RANKED: completion counters
  const float *x_scale;  // 8-bit operands: per-token scale [T]
  const float *w_scale;  // 8-bit operands: per-expert output-channel scale [E, N]
  float *gu_out;         // gated: [R, 2F] gate and up values (fp32) kept for a backward, or NULL
  const uint8_t *x_bs;   // 8-bit with block scales: E8M0 codes [T, K/32]
  const uint8_t *w_bs;   // 8-bit with block scales: E8M0 codes [E, N, K/32]
};

// What a forward-shaped kernel writes:
//   FWD_BARE    C[r, n] = acc (fp32 or bf16 store; rows grouped by end offsets)
//   FWD_SCATTER y[token(r), n] += w_r * acc (atomic; routing schedule), A row of
//               schedule row r gathered from token(r)
//   FWD_GATED   h[r, f] = silu(acc_gate) * acc_up in bf16 (routing schedule): the
//               B tile holds 128 gate rows f0.. and the 128 up rows F + f0.. of a
//               doubled [2F, K] weight, so each wave's column block ni < NI/2 and
//               block ni + NI/2 hold the gate and the up value of the same f
//   FWD_SCATTER_ROWS  as FWD_SCATTER with A already in schedule row order (A row
//               r is row r: the gated FFN's intermediate), nothing gathered
enum { FWD_BARE = 0, FWD_SCATTER = 1, FWD_GATED = 2, FWD_SCATTER_ROWS = 3 };

// How a scattering kernel combines its results into the output rows:
//   COMBINE_ATOMIC  atomic adds into a zeroed output (canonical schedule);
//   COMBINE_RANKED  one launch over the k*E groups of the rank-ordered view,
//                   tiles in rank order: rank 0 stores, a tile of rank p > 0
//                   waits until every rank p-1 tile of its column block has
//                   stored, then reads, adds and stores (each rank holds a
//                   token at most once, so no element has two writers at once).
enum { COMBINE_ATOMIC = 0, COMBINE_RANKED = 1 };

// ---- rank-ordered combine: completion counters --------------------------------
// sync (the schedule's phase_sync words): [kMaxRankK][kSyncCols] completed work
// per (rank, column block) in eighths of a tile, then the number of finished
// workgroups of the launch, then the number of waits that gave up.  Zero
// before a launch; the launch's last workgroup zeroes the counters again.
constexpr int kSyncCols = kRankSyncCols;
constexpr int kSyncFin = kMaxRankK * kSyncCols;
constexpr int kSyncFlag = kSyncFin + 1;
static_assert(kSyncFlag + 1 == kRankSyncInts, "counter layout");
// a wait gives up (and counts itself in the flag word) after this many sleeps
// of ~256 clocks, ~0.5 s: every workgroup is resident (one per compute unit),
// so a wait that long means the launch did not get the whole device
constexpr int kSpinLimit = 1 << 21;

// Stores and loads that other XCDs see within the launch: device scope, which
// on gfx950 writes through / reads past the XCD's own L2.
MOE_DEV void store_coherent(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// As dma16, device-scope (coherent) read.
MOE_DEV void dma16_coherent(__amdgpu_buffer_rsrc_t rsrc, uint32_t voff, uint32_t lds) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen sc1 lds"
               :
               : "s"(m0v), "v"(voff), "s"(rsrc)
               : "memory", "m0");
}
// Whole workgroup: wait until *ctr >= need (thread 0 polls, then a barrier).
MOE_DEV void wait_count(int32_t *sync, int idx, int need) {
  if (threadIdx.x == 0) {
    int spins = 0;
    while (__hip_atomic_load(sync + idx, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < need) {
      __builtin_amdgcn_s_sleep(4);
      if (++spins > kSpinLimit) {
        __hip_atomic_fetch_add(sync + kSyncFlag, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        break;
      }
    }
  }
  __syncthreads();
}
// Whole workgroup, after its coherent stores of a tile: every wave waits for
// them to complete, then thread 0 adds `amount` to the tile's counter.
MOE_DEV void count_done(int32_t *sync, int idx, int amount) {
  wait_vmcnt<0>();
  __syncthreads();
  if (threadIdx.x == 0)
    __hip_atomic_fetch_add(sync + idx, amount, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Whole workgroup, at the end of a ranked launch: the last workgroup to get
// here (every other one is past all its waits) zeroes the counters.
MOE_DEV void finish_ranked(int32_t *sync, int nranks) {
  __syncthreads();
  __shared__ int last;
  if (threadIdx.x == 0)
    last = __hip_atomic_fetch_add(sync + kSyncFin, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
           (int)gridDim.x - 1;
  __syncthreads();
  if (last) {
    for (int i = threadIdx.x; i < nranks * kSyncCols; i += blockDim.x)
      __hip_atomic_store(sync + i, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (threadIdx.x == 0) __hip_atomic_store(sync + kSyncFin, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// F8: 8-bit operands (a stage is 128 reduction elements; K below is the
// reduction length in 2-byte units, i.e. row bytes / 2, for the bounds checks).
// MX: 8-bit operands with a power-of-two (E8M0) scale per 32 reduction
// elements of every A and B row, applied by the matrix cores.
template <int BM, int BN, int NW, bool F8_ = false, bool MX_ = false>
struct FwdOp {
  static constexpr bool A_KMAJ = true, B_KMAJ = true, A_SCALED = false, PREFETCH = false;
  static constexpr bool F8 = F8_, MX = MX_;
  static constexpr bool CHECKED_TAIL = true;
  static constexpr int DA = BM / (8 * NW), DB = BN / (8 * NW);
  // MX: the block scales of a stage, one 4-byte word (4 blocks of 32) per A
  // row and per B row, after the stages in LDS (A rows, then B rows)
  static constexpr int SCG = (BM + BN) / 64;           // 64-row scale groups per stage
  static constexpr int DS = MX ? (SCG + NW - 1) / NW : 0;  // scale loads per wave (at most)
  static_assert(!MX || BM % 64 == 0, "whole scale groups");
  static constexpr int SC_STAGE = (BM + BN) * 4;
  static constexpr int SC_OFF = NSTAGE * STAGE;
  static constexpr int DMA_PER_STAGE = DA + DB + DS;
  KmajDma<BM, NW> da;
  KmajDma<BN, NW> db;
  __amdgpu_buffer_rsrc_t rsA, rsW, rsAS, rsWS;
  uint32_t lds0;
  const char *ldsp;
  uint32_t soff[DS > 0 ? DS : 1];  // MX: per-lane byte offset of the row's scales, or OOB
  int K, wid;
  // NTW: the tile's weight block is read by no other tile (non-temporal loads)
  template <bool SKIP, bool CHECKED, bool NTW = false>
  MOE_DEV void issue_part(int kt, int buf, int j) {
    const uint32_t t = lds0 + (uint32_t)buf * STAGE;
    if (j < DA) {
      da.template issue_one<SKIP, CHECKED>(rsA, kt, K, t, wid, j);
    } else if (j < DA + DB) {
      db.template issue_one<SKIP, CHECKED, NTW>(rsW, kt, K, t + OPND, wid, j - DA);
    } else if constexpr (MX) {
      // 64-row group of A rows, then B rows, dealt to the waves round robin
      const int i = j - DA - DB, grp = wid + i * NW;
      if (grp < SCG)
        dma4_so(grp < BM / 64 ? rsAS : rsWS, soff[i], (uint32_t)kt * 4u,
                lds0 + (uint32_t)(SC_OFF + buf * SC_STAGE + grp * 256));
    }
  }
  // E8M0 scale of row `row` (A or B) for step `step`: the lane in half h
  // supplies block 2 step + h of the stage (elements 32h .. 32h+31 of the
  // step, spread over both halves' fragments), in byte 0
  MOE_DEV uint32_t scale_of(int buf, bool b_side, int row, int step, int lane) const {
    const uint32_t w = *(const uint32_t *)(ldsp + SC_OFF + buf * SC_STAGE + (b_side ? BM * 4 : 0) +
                                           row * 4);
    return (w >> (8 * (2 * step + (lane >> 5)))) & 0xffu;
  }
  MOE_DEV void prefetch(int) {}
  MOE_DEV void row_scale(int, int, int, float (&)[8]) {}
};

// A (BM rows) and B (BN rows) K-major for the deep pipeline of small tiles.
template <int BM, int BN, int NW, bool F8_ = false, bool MX_ = false>
struct FwdDeepOp {
  static constexpr bool F8 = F8_, MX = MX_;  // as FwdOp
  static constexpr int DA = BM / (8 * NW), DB = BN / (8 * NW);
  static_assert(DA >= 1 && DB >= 1, "at least one DMA row group per wave");
  // MX: each stage needs one 4-byte scale word per A row and per B row.  They
  // sit in a ring of two slots after the stages, a slot holding the words of
  // four consecutive stages: with K a multiple of 512 (sc16) every row's four
  // words are one 16-byte load issued with the first stage of the four (slot
  // layout [row][4 words]); otherwise each stage loads its 4-byte words (slot
  // layout [stage of the four][row]).  The (BM + BN) / 64 groups of 64 rows are
  // dealt to the waves round robin, so a wave issues DSMAX or fewer scale loads
  // (measured for the masked decode, E = 64, K = 7168, N = 2048: one 4-byte
  // load per row and stage cost 22 us of its 186, the scales' lines being
  // requested as often as the operand rows themselves)
  static constexpr int SCG = MX ? (BM + BN) / 64 : 0;
  static constexpr int DSMAX = (SCG + NW - 1) / NW;
  static_assert(!MX || (BM + BN) % 64 == 0, "whole scale groups");
  static constexpr int DMA_PER_STAGE = DA + DB + DSMAX;
  static constexpr int A_BYTES = BM * KROW, STAGE_BYTES = (BM + BN) * KROW;
  static constexpr int NSTAGES = NSTAGE * STAGE / STAGE_BYTES > 6 ? 6 : NSTAGE * STAGE / STAGE_BYTES;
  static_assert(NSTAGES >= 2, "two stages at least");
  static constexpr int RSLOT = MX ? (BM + BN) * 16 : 0;  // one slot of the scale ring
  static constexpr int RING_OFF = NSTAGES * STAGE_BYTES;
  static constexpr size_t LDS_BYTES = (size_t)RING_OFF + 2 * RSLOT;
  KmajDma<BM, NW> da;
  KmajDma<BN, NW> db;
  __amdgpu_buffer_rsrc_t rsA, rsW, rsAS, rsWS;
  uint32_t lds0;
  const char *ldsp;
  uint32_t soff[DSMAX > 0 ? DSMAX : 1];  // MX: per-lane byte offset of the row's scales, or OOB
  int K, wid;
  bool sc16 = false;                     // MX: four stages' scale words per 16-byte load
  int pbase = 0, pscale = 0;             // DMA instructions of this wave per stage (count_parts)
  template <bool SKIP, bool CHECKED, bool NTW = false>
  MOE_DEV void issue_part(int kt, int buf, int j) {
    const uint32_t t = lds0 + (uint32_t)(buf * STAGE_BYTES);
    if (j < DA) {
      da.template issue_one<SKIP, CHECKED>(rsA, kt, K, t, wid, j);
    } else if (j < DA + DB) {
      // (the weights stream past once: non-temporal)
      db.template issue_one<SKIP, CHECKED, true>(rsW, kt, K, t + A_BYTES, wid, j - DA);
    } else if constexpr (MX) {
      const int i = j - DA - DB, grp = wid + i * NW;
      const uint32_t slot = lds0 + (uint32_t)(RING_OFF + ((kt >> 2) & 1) * RSLOT);
      if (grp < SCG) {
        const __amdgpu_buffer_rsrc_t rs = grp < BM / 64 ? rsAS : rsWS;
        if (sc16) {
          if ((kt & 3) == 0)
            dma16_so(rs, soff[i], (uint32_t)(kt >> 2) * 16u, slot + (uint32_t)(grp * 1024));
        } else {
          dma4_so(rs, soff[i], (uint32_t)kt * 4u,
                  slot + (uint32_t)((kt & 3) * (BM + BN) * 4 + grp * 256));
        }
      }
    }
  }
  // DMA instructions this wave issues for a stage (the others cover dead rows;
  // with sc16 the scale loads come with every fourth stage only)
  MOE_DEV void count_parts() {
    pbase = 0;
    pscale = 0;
#pragma unroll
    for (int i = 0; i < DA; ++i) pbase += (wid * DA + i) * 8 < da.live_rows ? 1 : 0;
#pragma unroll
    for (int i = 0; i < DB; ++i) pbase += (wid * DB + i) * 8 < db.live_rows ? 1 : 0;
#pragma unroll
    for (int i = 0; i < DSMAX; ++i) pscale += wid + i * NW < SCG ? 1 : 0;
  }
  MOE_DEV int parts_at(int kt) const {
    return pbase + ((!sc16 || (kt & 3) == 0) ? pscale : 0);
  }
  // as FwdOp::scale_of, for stage kt (its words in the ring)
  MOE_DEV uint32_t scale_of(int kt, bool b_side, int row, int step, int lane) const {
    const int rr = (b_side ? BM : 0) + row;
    const char *slot = ldsp + RING_OFF + ((kt >> 2) & 1) * RSLOT;
    const uint32_t w = *(const uint32_t *)(slot + (sc16 ? rr * 16 + (kt & 3) * 4
                                                        : (kt & 3) * (BM + BN) * 4 + rr * 4));
    return (w >> (8 * (2 * step + (lane >> 5)))) & 0xffu;
  }
};

template <int BM, int BN, int WGM, int WGN, int MODE, typename Tout, bool F8 = false,
          bool MX = false, int COMB = COMBINE_ATOMIC>
__global__ __launch_bounds__(WGM * WGN * 64) void mfma_fwd_kernel(FwdArgs p) {
  constexpr bool FUSED = MODE != FWD_BARE;       // rows come from a routing schedule
  constexpr bool GATED = MODE == FWD_GATED;
  constexpr bool A_BY_ROW = MODE == FWD_SCATTER_ROWS;
  constexpr int BNO = GATED ? BN / 2 : BN;        // output columns per tile
  constexpr int MI = BM / WGM / 32, NI = BN / WGN / 32;
  static_assert(!GATED || NI % 2 == 0, "gate and up blocks pair up inside a wave");
  static_assert(!F8 || MODE == FWD_SCATTER, "8-bit operands: the routed scatter forward");
  static_assert(!MX || F8, "block scales: 8-bit operands");
  constexpr int NW = WGM * WGN, NTH = NW * 64;
  static_assert(NW == 4 || NW == 8, "4 or 8 waves");
  constexpr int ESZ = F8 ? 1 : 2;                 // bytes per operand element
  extern __shared__ __attribute__((aligned(16))) char lds[];  // NSTAGE x (A, B)
  __shared__ int bs[kMaxExperts + 1], rstart[kMaxExperts], rcnt[kMaxExperts];
  __shared__ __attribute__((aligned(16))) int tok[BM];
  __shared__ __attribute__((aligned(16))) float wgt[BM];
  __shared__ int rowoff_a[BM], rowoff_b[BN];
  __shared__ float cscale[F8 ? BN : 1];           // 8-bit: the tile's output-channel scales
  __shared__ int scratch[NTH / kWave + 1];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = wid / WGN, wn = wid % WGN;
  const int E = p.E, K = p.K, N = p.N;
  const int tiles_n = (N + BNO - 1) / BNO;
  const int KI = (K * ESZ + KROW - 1) / KROW;     // stages of 128 bytes per row
  // rows per tile of this launch (uniform over the grid): BM, or with routed
  // 256-row kernels possibly 128 (the 128 x 256 shape).  8-bit operands with 8
  // waves always take 128-row tiles: a 256 x 256 accumulator with
  // double-buffered 32-byte fragments does not fit the registers of 8 waves
  // per compute unit (4 waves, one per SIMD, have twice the registers).
  constexpr bool F8_HALF = F8 && NW == 8;
  // COMBINE_RANKED: the launch's groups are the nranks * E (rank, expert)
  // groups of the rank-ordered view, group g using expert g % E's weights
  constexpr bool RK = COMB == COMBINE_RANKED;
  const int GE = RK ? p.nranks * E : E;
  const int BMr = (FUSED && BM == 256)
                      ? (F8_HALF ? 128
                                 : pick_tile_rows(p.bstart, p.bstride, GE, tiles_n, gridDim.x,
                                                  p.tile_rows))
                      : BM;
  if (FUSED)
    group_tables_from_schedule<NTH>(p.counts, p.offsets, p.bstart + bm_index(BMr) * p.bstride, GE,
                                    p.layout, p.capacity, bs, rstart, rcnt);
  else
    group_tables_from_offsets<NTH>(p.offsets, E, BM, bs, rstart, rcnt, scratch);
  const int total = bs[GE] * tiles_n;
  FwdOp<BM, BN, NW, F8, MX> op;
  op.rsA = uniform_rsrc(p.A, p.a_bytes);
  op.lds0 = lds_addr(lds);
  op.ldsp = lds;
  const uint32_t kblk = (uint32_t)K / 32;  // MX: scale bytes per row
  if constexpr (MX) op.rsAS = uniform_rsrc(p.x_bs, (uint32_t)p.M * kblk);
  op.K = K * ESZ / 2;  // reduction length in 2-byte units (the bounds checks' unit)
  op.wid = wid;
  const int wrows = GATED ? 2 * N : N;  // rows of one expert's weight
  const uint32_t rowbytes = (uint32_t)K * ESZ;
  const uint32_t wbytes = (uint32_t)wrows * rowbytes;

  const int Lb = logical_block();
  WorkSplit ws;
  // gated tiles split along rows only (a column split would part gate from up);
  // 128-row tiles split at most 4 ways (64 x 128)
  // (ranked: tiles in increasing order, so a workgroup finishes its rank p
  // work before it waits in a rank p+1 tile)
  ws.init(total, gridDim.x, Lb, BM == 256 ? WorkSplit::SUBTILE_TAIL : WorkSplit::WHOLE,
          GATED ? (BMr == BM ? 2 : 1) : (BMr == BM ? 8 : 4), RK);
  int tau;
  const int kb = 0, ke = KI;
  while (ws.next(tau)) {
    TileCoord c = tile_coord(bs, rstart, rcnt, GE, tau, tiles_n, BMr);
    const int ge = RK ? c.g % E : c.g;   // the expert whose weights the tile uses
    const int rank = RK ? c.g / E : 0;
    int n0 = c.nb * BNO, ncols = min(BNO, N - n0);
    if (ws.nS > 1) {  // a sub-tile of a tile of the last round
      const SubTile st = BMr == 128 ? sub_tile128(ws.s, ws.nS) : sub_tile(ws.s, ws.nS);
      c.row0 += st.r0;
      c.rows = min(st.rows, c.rows - st.r0);
      if (!GATED) {
        n0 += st.c0;
        ncols = min(st.cols, N - n0);
      }
    }
    if (c.rows <= 0 || ncols <= 0) {
      // an empty piece still counts as done for the ranks after it
      if constexpr (RK) count_done(p.sync, rank * kSyncCols + c.nb, 8 / ws.nS);
      continue;
    }
    __syncthreads();  // LDS stages and row tables free
    if (tid < BM) {
      const bool ok = tid < c.rows;
      const int r = c.row0 + tid;
      const int t = ok ? (FUSED ? p.row_to_token[r] : (r < p.M ? r : -1)) : -1;
      tok[tid] = t;
      // 8-bit: the token's scale rides on its routing weight
      wgt[tid] = (FUSED && ok) ? p.row_weight[r] * (F8 && !MX && t >= 0 ? p.x_scale[t] : 1.f) : 0.f;
      rowoff_a[tid] = t >= 0 ? (A_BY_ROW ? r : t) * (int)rowbytes : -1;
    }
    for (int j = tid; j < BN; j += NTH) {
      const int jj = GATED ? j % BNO : j;  // gated: gate rows, then the up rows
      rowoff_b[j] = jj < ncols ? (n0 + jj + (GATED && j >= BNO ? N : 0)) * (int)rowbytes : -1;
      if (F8 && !MX) cscale[j] = jj < ncols ? p.w_scale[(size_t)ge * N + n0 + jj] : 0.f;
    }
    __syncthreads();
    op.rsW = uniform_rsrc((const char *)p.W + (size_t)ge * wrows * rowbytes, wbytes);
    // a whole tile of a group with a single row block is the only reader of
    // its weight block in this launch: those weights stream past with
    // non-temporal loads and leave L2 to the token rows the group's other
    // column blocks read again (gated FFN, T = 8192, K = 4096, F = 2048,
    // N = 4096, 64 experts of 256 rows: up-projection 627 -> 588 us, down
    // projection 460 -> 433; the hint on every weight load instead slows the
    // forward of groups of several row blocks, whose tiles share each weight
    // block: T = 4096, K = N = 2048, E = 8 top-2 forward 103 -> 106, Zipf-routed
    // T = 8192, K = 4096, N = 1408, E = 64 top-4 forward 436 -> 468).  Only the
    // gated FFN's two kernels carry the second tile body for it: in the routed
    // forward it cost about 1 % from the larger code alone (the same two
    // shapes: 106.0 -> 106.9 us, 439 -> 443), and in the input gradient more
    // (the Zipf-routed dX 688 -> 698)
    constexpr bool NT_OK = GATED || MODE == FWD_SCATTER_ROWS;
    const bool ntw = NT_OK && !RK && ws.nS == 1 && bs[c.g + 1] - bs[c.g] <= 1;
    if constexpr (MX) {
      // per-lane offsets of the scale rows: group grp of 64 rows (A rows, then
      // B rows), lane = row inside the group; dead rows read out of range
      op.rsWS = uniform_rsrc(p.w_bs + (size_t)ge * N * kblk, (uint32_t)N * kblk);
#pragma unroll
      for (int i = 0; i < op.DS; ++i) {
        const int grp = wid + i * NW;
        const int ra = grp * 64 + lane;  // tile row (A) or column (B)
        uint32_t o = kOobOffset;
        if (grp < BM / 64) {
          const int t = tok[ra];
          if (t >= 0) o = (uint32_t)t * kblk;
        } else if (grp < op.SCG) {
          const int jb = ra - BM;
          if (jb < ncols) o = (uint32_t)(n0 + jb) * kblk;
        }
        op.soff[i] = o;
      }
    }
    const bool part = BM <= 64 || ws.nS > 1 || BMr < BM ||
                      (!GATED && (ncols < BNO || c.rows < BMr));  // rows / columns partly dead
    // (gated: the live B rows are two runs, not a prefix; nothing is skipped)
    const int live_b = GATED ? BN : ncols;
    op.da.setup(wid, lane, rowoff_a, part ? c.rows : BM);
    op.db.setup(wid, lane, rowoff_b, part ? live_b : BN);
    // The tile body, instantiated per accumulator shape: MIc x NIc blocks per
    // wave (a whole tile, or a 128 x 128 / 64 x 128 sub-tile), each with its own
    // accumulators.  SKM: MFMAs of row blocks past the last live row and of
    // column blocks past the last live column are left out (wave-uniform:
    // masked decode, and whole tiles that end past a group's rows or past N,
    // e.g. the last 256-column block of N = 1408); DSK: DMA of dead rows is left out;
    // DEEP: the streaming pipeline with more stages in flight (masked decode).
    auto tile_nt = [&](auto MIc_, auto NIc_, auto SKM_, auto DSK_, auto DEEP_, auto NTW_)
                       __attribute__((always_inline)) {
      constexpr bool NTW = decltype(NTW_)::value;
      constexpr int MIc = decltype(MIc_)::value, NIc = decltype(NIc_)::value;
      constexpr bool SKM = decltype(SKM_)::value, DSK = decltype(DSK_)::value;
      const int live_mi =
          SKM ? min(MIc, max(0, (c.rows - wm * 32 + 32 * WGM - 1) / (32 * WGM))) : MIc;
      const int live_ni =
          SKM ? min(NIc, max(0, (ncols - wn * 32 + 32 * WGN - 1) / (32 * WGN))) : NIc;
      f32x16 acc[MIc][NIc];
#pragma unroll
      for (int mi = 0; mi < MIc; ++mi)
#pragma unroll
        for (int ni = 0; ni < NIc; ++ni) acc[mi][ni] = f32x16{};
      if constexpr (decltype(DEEP_)::value) {
        constexpr int BMs = MIc * 32 * WGM, BNs = NIc * 32 * WGN;  // rows of A and of B
        FwdDeepOp<BMs, BNs, NW, F8, MX> dop;
        dop.rsA = op.rsA;
        dop.rsW = op.rsW;
        dop.lds0 = op.lds0;
        dop.ldsp = lds;
        dop.K = K * ESZ / 2;
        dop.wid = wid;
        dop.da.setup(wid, lane, rowoff_a, c.rows);
        dop.db.setup(wid, lane, rowoff_b, GATED ? BNs : ncols);
        if constexpr (MX) {
          dop.rsAS = op.rsAS;
          dop.rsWS = op.rsWS;
          dop.sc16 = K % 512 == 0;
#pragma unroll
          for (int i = 0; i < dop.DSMAX; ++i) {
            const int grp = wid + i * NW, ra = grp * 64 + lane;
            uint32_t o = kOobOffset;
            if (grp < BMs / 64) {
              const int t = tok[ra];
              if (t >= 0) o = (uint32_t)t * kblk;
            } else if (grp < dop.SCG) {
              const int jb = ra - BMs;
              if (jb < ncols) o = (uint32_t)(n0 + jb) * kblk;
            }
            dop.soff[i] = o;
          }
        }
        dop.count_parts();
        tile_multiply_deep<MIc, NIc, WGM, WGN>(dop, lds, kb, ke, wm, wn, lane, live_mi, acc);
      } else {
        tile_multiply<MIc, NIc, WGM, WGN, SKM, FwdOp<BM, BN, NW, F8, MX>, DSK, NTW>(
            op, lds, kb, ke, wm, wn, lane, live_mi, live_ni, acc);
      }

      // epilogue: 4 consecutive accumulator rows share one 16-byte read of the
      // row tables; each row's base address is formed once for all column blocks
      if constexpr (GATED) {
        // h[r, f] = silu(g) * u, silu(g) = g / (1 + e^-g), stored bf16 at the
        // tile's schedule row r for live rows and f < F
        constexpr int NH = NIc / 2;
        bf16_t *const hb = (bf16_t *)p.C;
        float *const gub = p.gu_out;
        const int cl0 = wn * 32 + (lane & 31);
#pragma unroll
        for (int mi = 0; mi < MIc; ++mi) {
          if (mi >= live_mi) continue;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int rq = wm * 32 + mi * 32 * WGM + 8 * j + 4 * (lane >> 5);
            const i32x4 t4 = *(const i32x4 *)(tok + rq);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              if (t4[q] < 0) continue;
              bf16_t *const hrow = hb + (size_t)(c.row0 + rq + q) * N + n0;
#pragma unroll
              for (int ni = 0; ni < NH; ++ni) {
                const int cl = cl0 + ni * 32 * WGN;
                if (cl >= ncols) continue;
                const float g = acc[mi][ni][4 * j + q], u = acc[mi][ni + NH][4 * j + q];
                hrow[cl] = f32_to_bf16(g / (1.f + __expf(-g)) * u);
                if (gub) {
                  // kept for the backward only: nontemporal, so the lines do
                  // not take L2 from the weight rows (623 against 643 us for
                  // T = 8192, K = 4096, F = 2048, E = 64 top-2)
                  float *const gr = gub + (size_t)(c.row0 + rq + q) * (2 * N) + n0 + cl;
                  __builtin_nontemporal_store(g, gr);
                  __builtin_nontemporal_store(u, gr + N);
                }
              }
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
        return;
      }
      if (FUSED) {
        // weighted scatter-combine on y with 64-bit byte offsets from its
        // base; only live rows and columns are touched (the column test is
        // left out when every column of the accumulator is live).
        //   COMBINE_ATOMIC: atomic adds (any number of rows per token);
        //   COMBINE_RANKED: the tile's rank holds each token at most once, so
        //   no other workgroup writes its elements now: rank 0 stores w * acc;
        //   rank p > 0 waits for rank p-1 of this column block, then stores
        //   the old value plus w * acc (device-coherent stores and reads).
        char *const yb = (char *)p.C;
        const bool all_cols = ncols >= NIc * 32 * WGN;  // wave-uniform
        uint32_t cb[NIc];
#pragma unroll
        for (int ni = 0; ni < NIc; ++ni)
          cb[ni] = (uint32_t)(n0 + wn * 32 + ni * 32 * WGN + (lane & 31)) * 4u;
        const int cl0 = wn * 32 + (lane & 31);
        float cs[NIc];  // 8-bit: output-channel scale of each column block
#pragma unroll
        for (int ni = 0; ni < NIc; ++ni) cs[ni] = F8 && !MX ? cscale[cl0 + ni * 32 * WGN] : 1.f;
        // one row band (64 rows: 32 per row of waves) of the scatter; ranked:
        // oldb holds the band's old values in LDS (1 KB per tile row), or is
        // NULL for rank 0
        auto band = [&](int mi, const char *oldb) __attribute__((always_inline)) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int rq = wm * 32 + mi * 32 * WGM + 8 * j + 4 * (lane >> 5);
            const i32x4 t4 = *(const i32x4 *)(tok + rq);
            const f32x4 w4 = *(const f32x4 *)(wgt + rq);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              if (t4[q] < 0) continue;
              const size_t ro = (size_t)t4[q] * (size_t)N * 4u;  // y may pass 2^32 bytes
#pragma unroll
              for (int ni = 0; ni < NIc; ++ni) {
                const int cl = cl0 + ni * 32 * WGN;
                if (!all_cols && cl >= ncols) continue;
                const float v = F8 && !MX ? w4[q] * cs[ni] * acc[mi][ni][4 * j + q]
                                          : w4[q] * acc[mi][ni][4 * j + q];
                float *const dst = (float *)(yb + ro + cb[ni]);
                if constexpr (!RK) {
                  unsafeAtomicAdd(dst, v);
                } else {
                  const int rb = rq + q - mi * 32 * WGM;  // row inside the band
                  const float o = oldb ? *(const float *)(oldb + rb * 1024 + cl * 4) : 0.f;
                  store_coherent(dst, __fadd_rn(o, v));
                }
              }
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        };
        if constexpr (!RK || !(BM == 256 && WGM == 2)) {  // (ranked launches use 256-row tiles)
          unroll<MIc>([&](auto mi_) __attribute__((always_inline)) {
            if (decltype(mi_)::value < live_mi) band(decltype(mi_)::value, nullptr);
          });
          return;
        } else {
          // rank p > 0: wait for rank p-1 of this column block (in eighths of
          // a tile: its row blocks x 8), then its values of two bands at a
          // time (128 tile rows x 256 columns, 128 KB) go by coherent
          // global -> LDS DMA into the idle stages, one row (1 KB, 16 bytes
          // per lane) per instruction; dead rows and columns read out of range
          if (rank > 0)
            wait_count(p.sync, (rank - 1) * kSyncCols + c.nb, 8 * (bs[rank * E] - bs[(rank - 1) * E]));
          const __amdgpu_buffer_rsrc_t rsY =
              uniform_rsrc(p.C, (uint32_t)((size_t)p.M * (size_t)N * 4u));
          const uint32_t l0 = lds_addr(lds);
          constexpr int RPW = 128 / NW;  // rows per wave per half
          const bool cok = lane * 4 < ncols;
          unroll<(MIc + 1) / 2>([&](auto h_) __attribute__((always_inline)) {
            constexpr int h = decltype(h_)::value;
            if (rank > 0) {
              barrier();  // every wave done with the LDS (stages or previous half)
#pragma unroll
              for (int i = 0; i < RPW; ++i) {
                const int row = h * 128 + wid * RPW + i;
                const int t = tok[row];
                const uint32_t off =
                    (t >= 0 && cok) ? ((uint32_t)t * (uint32_t)N + (uint32_t)(n0 + lane * 4)) * 4u
                                    : kOobOffset;
                dma16_coherent(rsY, off, l0 + (uint32_t)((wid * RPW + i) * 1024));
              }
              wait_vmcnt<0>();
              barrier();
            }
            unroll<2>([&](auto m_) __attribute__((always_inline)) {
              constexpr int m = decltype(m_)::value;
              if (2 * h + m < MIc && 2 * h + m < live_mi)
                band(2 * h + m, rank > 0 ? lds + m * 64 * 1024 : nullptr);
            });
          });
          count_done(p.sync, rank * kSyncCols + c.nb, 8 / ws.nS);
          return;
        }
      }
#pragma unroll
      for (int mi = 0; mi < MIc; ++mi) {
        if (mi >= live_mi) continue;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int rq = wm * 32 + mi * 32 * WGM + 8 * j + 4 * (lane >> 5);
          const i32x4 t4 = *(const i32x4 *)(tok + rq);
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int t = t4[q];
            if (t < 0) continue;
            const size_t rowo = (size_t)t * N;
#pragma unroll
            for (int ni = 0; ni < NIc; ++ni) {
              const int cl = wn * 32 + ni * 32 * WGN + (lane & 31);
              if (cl >= ncols) continue;
              const int col = n0 + cl;
              const float v = acc[mi][ni][4 * j + q];
              if (sizeof(Tout) == 4) {
                ((float *)p.C)[rowo + col] = v;
              } else {
                ((__bf16 *)p.C)[rowo + col] = (__bf16)v;
              }
            }
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // (whole tiles of single-row-block groups take tile_nt with NTW set)
    auto tile = [&](auto MIc_, auto NIc_, auto SKM_, auto DSK_, auto DEEP_)
                    __attribute__((always_inline)) {
      tile_nt(MIc_, NIc_, SKM_, DSK_, DEEP_, std::false_type());
    };
    using std::integral_constant;
    using std::false_type;
    using std::true_type;
    const int nsub = ws.nS;  // row / column pieces of a tail tile
    if constexpr (BM <= 64) {
      tile(integral_constant<int, MI>(), integral_constant<int, NI>(), true_type(), true_type(),
           true_type());
    } else {
      // sub-tiles 64 x 128 (8 per tile) and 128 x 128 (4 per tile)
      constexpr int R8 = 64 / (32 * WGM), R4 = 128 / (32 * WGM), C = 128 / (32 * WGN);
      if constexpr (GATED) {  // whole tiles and 128 x 256 halves only
        if (nsub == 2 || BMr == 128)
          tile(integral_constant<int, R4>(), integral_constant<int, NI>(), false_type(),
               true_type(), false_type());
        else if (ntw)
          tile_nt(integral_constant<int, MI>(), integral_constant<int, NI>(), false_type(),
                  false_type(), false_type(), true_type());
        else
          tile(integral_constant<int, MI>(), integral_constant<int, NI>(), false_type(),
               false_type(), false_type());
      } else if (BMr == 128) {  // 128 x 256 tiles, split 2 (128 x 128) or 4 (64 x 128)
        if (nsub == 4)
          tile(integral_constant<int, R8>(), integral_constant<int, C>(), false_type(),
               true_type(), false_type());
        else if (nsub == 2)
          tile(integral_constant<int, R4>(), integral_constant<int, C>(), false_type(),
               true_type(), false_type());
        else
          tile(integral_constant<int, R4>(), integral_constant<int, NI>(), false_type(),
               true_type(), false_type());
      } else if constexpr (!F8_HALF) {
        if (nsub == 8)
          tile(integral_constant<int, R8>(), integral_constant<int, C>(), false_type(),
               true_type(), false_type());
        else if (nsub == 4)
          tile(integral_constant<int, R4>(), integral_constant<int, C>(), false_type(),
               true_type(), false_type());
        else if (nsub == 2)
          tile(integral_constant<int, R4>(), integral_constant<int, NI>(), false_type(),
               true_type(), false_type());
        else if (ncols < BNO || c.rows < BMr) {
          if constexpr (NT_OK) {
            if (ntw) {
              tile_nt(integral_constant<int, MI>(), integral_constant<int, NI>(), true_type(),
                      true_type(), false_type(), true_type());
              continue;
            }
          }
          tile(integral_constant<int, MI>(), integral_constant<int, NI>(), true_type(),
               true_type(), false_type());
        } else {
          if constexpr (NT_OK) {
            if (ntw) {
              tile_nt(integral_constant<int, MI>(), integral_constant<int, NI>(), false_type(),
                      false_type(), false_type(), true_type());
              continue;
            }
          }
          tile(integral_constant<int, MI>(), integral_constant<int, NI>(), false_type(),
               false_type(), false_type());
        }
      }
    }
  }
  if constexpr (RK) finish_ranked(p.sync, p.nranks);
}

// ============================================================================
// Input gradient (+ routing-weight gradient):
//   G[r, kc] = sum_n dY[tok(r), n] * W[g, n, kc]           (MFMA, fp32 acc)
//   dX[tok(r), kc] += w_r * G[r, kc]                       (atomic)
//   d_w[assign(r)] += sum_{kc in tile} G[r, kc] * x[tok(r), kc]   (atomic)
// [GG] "The backward pass": the forward pattern with the weights read
// transposed (here an MN-major weight tile read with transposing LDS reads);
// [CARD] "How it works": the same gather / scatter-combine as the forward, and
// the routing-weight gradient as the inner product of dY with the unweighted
// product, taken through the identity <dY W_e, x> = <dY, x W_e^T>.
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
  uint32_t dy_bytes, x_bytes;
  int tile_rows;   // 0 = picked on the device, 128 / 256 = forced
  int bstride;     // ints between the row-block prefixes of two tile heights
  int combine;     // dX scatter: COMBINE_ATOMIC or COMBINE_RANKED
  uint32_t dx_bytes;  // bytes of dX (COMBINE_RANKED reads it back)
  int nranks;         // COMBINE_RANKED: ranks of the view
  int32_t *sync;      // COMBINE_RANKED: completion counters
  // gated FFN backward (GB kernels): x is h [R, K] read by schedule row, gu the
  // saved gate/up values [R, 2K] (fp32), dgu the output [R, 2K] (bf16; K here is F)
  const float *gu;
  bf16_t *dgu;
};

template <int NW>
struct DxOp {
  using Map = MnmajMapT<NW>;
  static constexpr bool A_KMAJ = true, B_KMAJ = false, A_SCALED = false, PREFETCH = false;
  static constexpr bool CHECKED_TAIL = true, F8 = false, MX = false;
  static constexpr int DA = 256 / (8 * NW), PW = Map::PER_WAVE;
  static constexpr int DMA_PER_STAGE = DA + PW;
  KmajDma<256, NW> da;
  uint32_t bcol[PW];  // per instruction: byte offset (kc0 + 8 * chunk) * 2, or OOB
  uint32_t bvo[PW];   // the same plus the lane's reduction row inside a stage, or OOB
  __amdgpu_buffer_rsrc_t rsA, rsW;
  uint32_t lds0, rowbytes_w;
  int N, wid, lane;
  // columns kc0 .. kend-1 of W are loaded, the rest read as zeros
  MOE_DEV void setup_b(int kc0, int kend) {
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      const int col = kc0 + 8 * Map::chunk_of(wid, i, lane);
      bcol[i] = col < kend ? (uint32_t)col * 2u : kOobOffset;
      bvo[i] = col < kend ? (uint32_t)Map::row_of(wid, i, lane) * rowbytes_w + (uint32_t)col * 2u
                          : kOobOffset;
    }
  }
  template <bool SKIP, bool CHECKED, bool NTW = false>
  MOE_DEV void issue_part(int kt, int buf, int j) {
    const uint32_t t = lds0 + (uint32_t)buf * STAGE;
    if (j < DA) {
      da.template issue_one<SKIP, CHECKED>(rsA, kt, N, t, wid, j);
    } else {
      const int i = j - DA;
      if (CHECKED) {
        const int n = kt * BK + Map::row_of(wid, i, lane);
        const uint32_t off = (n < N && bcol[i] != kOobOffset)
                                 ? (uint32_t)n * rowbytes_w + bcol[i]
                                 : kOobOffset;
        dma16(rsW, off, t + OPND + Map::lds_of(wid, i));
      } else {
        dma16_so(rsW, bvo[i], (uint32_t)(kt * BK) * rowbytes_w, t + OPND + Map::lds_of(wid, i));
      }
    }
  }
  MOE_DEV void prefetch(int) {}
  MOE_DEV void row_scale(int, int, int, float (&)[8]) {}
};

// NW waves in a 2 x NW/2 grid.  GB (gated FFN backward): the output columns
// run over F; instead of scattering w * G into dX, each element makes
// dh = w * G, reads the saved gate g and up u of its row, and stores
// dg = dh * u * silu'(g) and du = dh * silu(g) into dgu; the routing-weight
// gradient takes h (read by schedule row) where the plain kernel takes x.
// ROWS: A (dY's place) is already in schedule row order and carries the routing
// weight (the gated FFN's dgu): read by row, scattered unweighted.
template <int NW, bool GB = false, bool ROWS = false, int COMB = COMBINE_ATOMIC>
__global__ __launch_bounds__(NW * 64) void mfma_dx_kernel(DxArgs p) {
  constexpr int BM = 256, BN = 256, WGM = 2, WGN = NW / 2, NTH = NW * 64;
  constexpr int MI = BM / WGM / 32, NI = BN / WGN / 32;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  __shared__ int bs[kMaxExperts + 1], rstart[kMaxExperts], rcnt[kMaxExperts];
  __shared__ int scratch[NTH / kWave + 1];
  __shared__ __attribute__((aligned(16))) int tok[BM];
  __shared__ __attribute__((aligned(16))) float wgt[BM];
  __shared__ __attribute__((aligned(16))) int asg[BM];
  __shared__ int rowoff_a[BM];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = wid / WGN, wn = wid % WGN;
  const int E = p.E, K = p.K, N = p.N;
  const int tiles_n = (K + BN - 1) / BN;  // output columns run over K
  const int KI = (N + BK - 1) / BK;       // reduction runs over N
  // COMBINE_RANKED: the nranks * E groups of the rank-ordered view (group g
  // uses expert g % E's weights)
  constexpr bool RK = COMB == COMBINE_RANKED;
  const int GE = RK ? p.nranks * E : E;
  const int BMr = pick_tile_rows(p.bstart, p.bstride, GE, tiles_n, gridDim.x, p.tile_rows);
  group_tables_from_schedule<NTH>(p.counts, p.offsets, p.bstart + bm_index(BMr) * p.bstride, GE,
                                  p.layout, p.capacity, bs, rstart, rcnt);
  const int total = bs[GE] * tiles_n;
  DxOp<NW> op;
  op.rsA = uniform_rsrc(p.dY, p.dy_bytes);
  op.lds0 = lds_addr(lds);
  op.rowbytes_w = (uint32_t)K * 2u;
  op.N = N;
  op.wid = wid;
  op.lane = lane;
  const uint32_t wbytes = (uint32_t)N * K * 2;
  const __amdgpu_buffer_rsrc_t rsX = uniform_rsrc(p.x, p.x_bytes);

  const int Lb = logical_block();
  WorkSplit ws;
  // 128-row tiles split at most 4 ways (64 x 128)
  ws.init(total, gridDim.x, Lb, WorkSplit::SUBTILE_TAIL, BMr == BM ? 8 : 4, RK);
  int tau;
  const int kb = 0, ke = KI;
  while (ws.next(tau)) {
    TileCoord c = tile_coord(bs, rstart, rcnt, GE, tau, tiles_n, BMr);
    const int ge = RK ? c.g % E : c.g;   // the expert whose weights the tile uses
    const int rank = RK ? c.g / E : 0;
    int kc0 = c.nb * BN, ncols = min(BN, K - kc0);
    if (ws.nS > 1) {  // a sub-tile of a tile of the last round
      const SubTile st = BMr == 128 ? sub_tile128(ws.s, ws.nS) : sub_tile(ws.s, ws.nS);
      c.row0 += st.r0;
      c.rows = min(st.rows, c.rows - st.r0);
      kc0 += st.c0;
      ncols = min(st.cols, K - kc0);
    }
    if (c.rows <= 0 || ncols <= 0) {
      // an empty piece still counts as done for the ranks after it
      if constexpr (RK) {
        if (p.dX) count_done(p.sync, rank * kSyncCols + c.nb, 8 / ws.nS);
      }
      continue;
    }
    __syncthreads();
    if (tid < BM) {
      const bool ok = tid < c.rows;
      const int r = c.row0 + tid;
      const int t = ok ? p.row_to_token[r] : -1;
      tok[tid] = t;
      wgt[tid] = ok ? (ROWS ? 1.f : p.row_weight[r]) : 0.f;
      asg[tid] = ok ? p.row_to_assign[r] : -1;
      rowoff_a[tid] = t >= 0 ? (ROWS ? r : t) * N * 2 : -1;
    }
    __syncthreads();
    op.rsW = uniform_rsrc(p.W + (size_t)ge * N * K, wbytes);
    const bool part = ws.nS > 1 || BMr < BM;  // rows / columns partly dead
    op.da.setup(wid, lane, rowoff_a, part ? c.rows : BM);
    op.setup_b(kc0, kc0 + ncols);
    // The tile body, instantiated per accumulator shape: MIc x NIc blocks per
    // wave (a whole tile, or a 128 x 128 / 64 x 128 sub-tile), each with its own
    // accumulators; DSK: DMA of dead rows is left out.
    auto tile = [&](auto MIc_, auto NIc_, auto DSK_) __attribute__((always_inline)) {
      constexpr int MIc = decltype(MIc_)::value, NIc = decltype(NIc_)::value;
      constexpr bool DSK = decltype(DSK_)::value;
      f32x16 acc[MIc][NIc];
#pragma unroll
      for (int mi = 0; mi < MIc; ++mi)
#pragma unroll
        for (int ni = 0; ni < NIc; ++ni) acc[mi][ni] = f32x16{};
      tile_multiply<MIc, NIc, WGM, WGN, false, DxOp<NW>, DSK>(op, lds, kb, ke, wm, wn, lane, MIc,
                                                              NIc, acc);

      // COMBINE_RANKED works band by band (64 tile rows): the x rows of the
      // band (for the routing-weight gradient) and, for rank p > 0 once rank
      // p-1 of this column block is done, the dX values the earlier ranks left
      // go into the idle LDS stages first (coherent reads), then the band is
      // stored (device-coherent stores).  The atomic combine loads the x tile
      // of all rows at once.
      constexpr bool CAN_ADD = !GB && !ROWS;
      constexpr bool add = CAN_ADD && RK;
      // x[tok(r), kc0 .. kc0+255] for the routing-weight gradient: four
      // 64-column K-major sub-tiles into the (now idle) LDS stages
      if (p.d_w && !add) {
        barrier();
        const uint32_t l0 = lds_addr(lds);
        constexpr int XPW = 32 / NW;  // instructions per wave per 64-column sub-tile
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
          for (int i = 0; i < XPW; ++i) {
            const int row = (wid * XPW + i) * 8 + (lane >> 3);
            const int cch = (lane & 7) ^ ((row >> 1) & 7);
            const int t = GB ? (tok[row] >= 0 ? c.row0 + row : -1) : tok[row];
            const int col = kc0 + q * 64 + cch * 8;
            const uint32_t off =
                (t >= 0 && col < K) ? (uint32_t)t * (uint32_t)K * 2u + (uint32_t)col * 2u : kOobOffset;
            dma16(rsX, off, l0 + (uint32_t)(q * OPND + (wid * XPW + i) * 1024));
          }
        }
        wait_vmcnt<0>();
        barrier();
      }
      // epilogue: weighted atomic scatter of G into dX and, per row, the partial
      // inner product of G with x over this tile's columns into d_w.  Register
      // 4j+q of accumulator (mi, ni) holds row rq + q, column cl(ni) of G, with
      // rq = wm*32 + mi*64 + 8j + 4*(lane/32); one transposing read of the K-major
      // x tile gives each lane exactly x at rows rq .. rq+3 of its column.
      const bool has_dw = p.d_w != nullptr, has_dx = p.dX != nullptr;
      // dX scatter: atomics with 64-bit byte offsets from the base of dX, on
      // live rows and columns only
      char *const xb = (char *)p.dX;
      // GB: gate / up and dgu addressed by 32-bit byte offsets from the tile's
      // first row
      const uint32_t grows = GB ? (uint32_t)c.rows * (uint32_t)K : 0u;
      const __amdgpu_buffer_rsrc_t rsG =
          uniform_rsrc(GB ? p.gu + (size_t)c.row0 * 2 * K : nullptr, grows * 8u);
      const __amdgpu_buffer_rsrc_t rsD =
          uniform_rsrc(GB ? p.dgu + (size_t)c.row0 * 2 * K : nullptr, grows * 4u);
      const uint32_t gcol = (uint32_t)(kc0 + wn * 32 + (lane & 31));
      uint32_t cb[NIc];
#pragma unroll
      for (int ni = 0; ni < NIc; ++ni)
        cb[ni] = (uint32_t)(kc0 + wn * 32 + ni * 32 * WGN + (lane & 31)) * 4u;
      // LDS of a band (ranked): x sub-tiles of 64 rows (8 KB each) from
      // offset 0, the old dX rows (1 KB each) from XB_OLD
      constexpr int XB_SUB = 64 * KROW, XB_OLD = 4 * XB_SUB;
      const __amdgpu_buffer_rsrc_t rsO =
          uniform_rsrc(CAN_ADD ? (const void *)p.dX : nullptr, CAN_ADD && p.dX ? p.dx_bytes : 0u);
      // mi and j unrolled by construction: with the gated arithmetic the body
      // is past the compiler's unrolling limit, and a rolled loop would index
      // the accumulators at run time, which moves them to scratch memory
      if constexpr (add) {
        if (rank > 0 && has_dx)
          wait_count(p.sync, (rank - 1) * kSyncCols + c.nb, 8 * (bs[rank * E] - bs[(rank - 1) * E]));
      }
      unroll<MIc>([&](auto mi_) __attribute__((always_inline)) {
        constexpr int mi = decltype(mi_)::value;
        if constexpr (add) {
          // the band's rows mi*64 .. mi*64+63: x chunks (two 8-row groups per
          // wave and sub-tile) and old dX rows (16 per wave), dead rows and
          // columns out of range
          barrier();
          const uint32_t l0 = lds_addr(lds);
          constexpr int RG = 64 / (8 * NW), RO = 64 / NW;
          if (has_dw) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
#pragma unroll
              for (int i = 0; i < RG; ++i) {
                const int rl = (wid * RG + i) * 8 + (lane >> 3);  // row inside the band
                const int row = mi * 64 + rl;
                const int cch = (lane & 7) ^ ((row >> 1) & 7);
                const int t = tok[row];
                const int col = kc0 + q * 64 + cch * 8;
                const uint32_t off = (t >= 0 && col < K)
                                         ? (uint32_t)t * (uint32_t)K * 2u + (uint32_t)col * 2u
                                         : kOobOffset;
                dma16(rsX, off, l0 + (uint32_t)(q * XB_SUB + (wid * RG + i) * 1024));
              }
            }
          }
          // (rank 0 reads nothing: its offsets are all out of range, so the
          // band's old values are zeros and one code path serves every rank)
          if (has_dx) {
            const bool cok = lane * 4 < ncols && rank > 0;
#pragma unroll
            for (int i = 0; i < RO; ++i) {
              const int rl = wid * RO + i;
              const int t = tok[mi * 64 + rl];
              const uint32_t off =
                  (t >= 0 && cok) ? ((uint32_t)t * (uint32_t)K + (uint32_t)(kc0 + lane * 4)) * 4u
                                  : kOobOffset;
              dma16_coherent(rsO, off, l0 + (uint32_t)(XB_OLD + rl * 1024));
            }
          }
          wait_vmcnt<0>();
          barrier();
        }
        unroll<4>([&](auto j_) __attribute__((always_inline)) {
          constexpr int j = decltype(j_)::value;
          const int rq = wm * 32 + mi * 32 * WGM + 8 * j + 4 * (lane >> 5);
          const i32x4 t4 = *(const i32x4 *)(tok + rq);
          const f32x4 w4 = *(const f32x4 *)(wgt + rq);
          const i32x4 a4 = *(const i32x4 *)(asg + rq);
          i16x4 xq[NIc];
          if (has_dw) {
            const int jl = lane & 15;
            const int row = rq + (jl >> 2);
#pragma unroll
            for (int ni = 0; ni < NIc; ++ni) {
              const int cs = wn * 32 + ni * 32 * WGN + 16 * ((lane >> 4) & 1) + 4 * (jl & 3);
              // (a band's sub-tiles hold 64 rows; the swizzle of row - mi*64
              // equals that of row)
              const char *a = add ? lds + (cs >> 6) * XB_SUB + kmaj_off(row - mi * 64, (cs >> 3) & 7) +
                                        (cs & 7) * 2
                                  : lds + (cs >> 6) * OPND + kmaj_off(row, (cs >> 3) & 7) + (cs & 7) * 2;
              xq[ni] = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                  (LDS_AS i16x4 *)(LDS_AS char *)a);
            }
          }
          float dwp[4] = {0.f, 0.f, 0.f, 0.f};
          size_t ro[4];  // dX may pass 2^32 bytes
#pragma unroll
          for (int q = 0; q < 4; ++q) ro[q] = (size_t)t4[q] * (size_t)K * 4u;
          // GB: the saved gate / up values of this lane's 4 rows x NIc columns,
          // all loads issued together; per row one gate and one up offset (both
          // range-checked: a dead row reads zero, a dead column a neighbour or
          // zero, and neither is used), the column blocks in the immediate
          float gvs[GB ? NIc : 1][4], uvs[GB ? NIc : 1][4];
          uint32_t go[4], gd[4];
          if constexpr (GB) {
            if (p.dgu) {
#pragma unroll
              for (int q = 0; q < 4; ++q) {
                const uint32_t r = (uint32_t)(rq + q) * (uint32_t)K * 2u + gcol;
                go[q] = t4[q] >= 0 ? r * 4u : kOobOffset;
                gd[q] = r * 2u;
              }
#pragma unroll
              for (int ni = 0; ni < NIc; ++ni) {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                  gvs[ni][q] = __builtin_bit_cast(
                      float, __builtin_amdgcn_raw_buffer_load_b32(rsG, go[q] + ni * 128 * WGN, 0, 0));
                  uvs[ni][q] = __builtin_bit_cast(
                      float, __builtin_amdgcn_raw_buffer_load_b32(
                                 rsG, go[q] + (uint32_t)K * 4u + ni * 128 * WGN, 0, 0));
                }
              }
            }
          }
#pragma unroll
          for (int ni = 0; ni < NIc; ++ni) {
            const int cl = wn * 32 + ni * 32 * WGN + (lane & 31);  // column inside the tile
            const bool cok = cl < ncols;
#pragma unroll
            for (int q = 0; q < 4; ++q) {
              const float g = cok ? acc[mi][ni][4 * j + q] : 0.f;  // dead columns may hold stale values
              if constexpr (GB) {
                if (p.dgu && t4[q] >= 0 && cok) {
                  const uint32_t so = gd[q] + ni * 64 * WGN;
                  const float gv = gvs[ni][q], uv = uvs[ni][q];
                  const float sg = 1.f / (1.f + __expf(-gv));
                  const float dh = w4[q] * g;
                  __builtin_amdgcn_raw_buffer_store_b16(
                      f32_to_bf16(dh * uv * sg * (1.f + gv * (1.f - sg))), rsD, so, 0, 0);
                  __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(dh * gv * sg), rsD, so, K * 2, 0);
                }
              } else if (has_dx && t4[q] >= 0 && cok) {
                float *const dst = (float *)(xb + ro[q] + cb[ni]);
                const float v = w4[q] * g;
                if constexpr (!add) {
                  unsafeAtomicAdd(dst, v);
                } else {
                  const float o = *(const float *)(lds + XB_OLD + (rq + q - mi * 64) * 1024 + cl * 4);
                  store_coherent(dst, __fadd_rn(o, v));
                }
              }
              if (has_dw) {
                const float xv = __builtin_bit_cast(float, (uint32_t)(uint16_t)xq[ni][q] << 16);
                dwp[q] = fmaf(g, xv, dwp[q]);  // masked rows / columns hold zeros
              }
            }
          }
          if (has_dw) {
            // sum each row over the 32 lanes of its half-wave (the sums land
            // in lanes 16..31 and 48..63)
#pragma unroll
            for (int q = 0; q < 4; ++q) dwp[q] = half_wave_sum(dwp[q]);
            if ((lane & 31) == 16) {
#pragma unroll
              for (int q = 0; q < 4; ++q)
                if (a4[q] >= 0) unsafeAtomicAdd(p.d_w + a4[q], dwp[q]);
            }
          }
        });
        __builtin_amdgcn_sched_barrier(0);
      });
      if constexpr (add) {
        if (has_dx) count_done(p.sync, rank * kSyncCols + c.nb, 8 / ws.nS);
      }
    };
    using std::integral_constant;
    // sub-tiles 64 x 128 (8 per tile) and 128 x 128 (4 per tile)
    const int nsub = ws.nS;
    constexpr int R8 = 64 / (32 * WGM), R4 = 128 / (32 * WGM), C = 128 / (32 * WGN);
    if (BMr == 128) {  // 128 x 256 tiles, split 2 (128 x 128) or 4 (64 x 128)
      if (nsub == 4)
        tile(integral_constant<int, R8>(), integral_constant<int, C>(), std::true_type());
      else if (nsub == 2)
        tile(integral_constant<int, R4>(), integral_constant<int, C>(), std::true_type());
      else
        tile(integral_constant<int, R4>(), integral_constant<int, NI>(), std::true_type());
    } else if (nsub == 8)
      tile(integral_constant<int, R8>(), integral_constant<int, C>(), std::true_type());
    else if (nsub == 4)
      tile(integral_constant<int, R4>(), integral_constant<int, C>(), std::true_type());
    else if (nsub == 2)
      tile(integral_constant<int, R4>(), integral_constant<int, NI>(), std::true_type());
    else
      tile(integral_constant<int, MI>(), integral_constant<int, NI>(), std::false_type());
  }
  if constexpr (RK) finish_ranked(p.sync, p.nranks);
}

// ============================================================================
// Weight gradient: dW[e, n, kc] = sum over rows r of e of (w_r dY[tok(r), n]) x[tok(r), kc].
// [GG] "The backward pass": a grouped GEMM whose reduction length (the group's
// rows) varies; every expert's output is written, zeros for an empty one.  Work
// units (expert, 256 x 256 output tile) are ordered by descending expert load
// and each workgroup takes the next one from a counter in the schedule as soon
// as it is free, so the longest reductions start first and the short ones fill
// in behind them ([NOTE] 4.2: hot experts get more work units and the
// persistent workgroups absorb the imbalance; [GG] "The backward pass": the
// hot expert's long reductions form the tail).  The last workgroup to finish
// resets the counter.
// Both operands are MN-major tiles of 32 gathered token rows, loaded by DMA.
// With routing weights (SC), a stage's weights are DMA'd next to it and each dY
// fragment is multiplied by its rows' weights in fp32 and rounded to bf16
// before the MFMA (one bf16 rounding per product); a schedule built without
// weights (all 1) takes the instantiation without that vector-ALU work.  The tokens that address a stage's rows are
// themselves DMA'd into a small LDS ring four stages ahead, so issuing a stage
// never waits on a global load outside the DMA accounting.
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
  uint32_t dy_bytes, x_bytes, rw_bytes;
  int32_t *queue;  // [2]: next unit, finished workgroups (zero at launch; left zero)
  // zeroed by the kernel on the side (the accumulation targets of the input
  // gradient kernel that runs after it): byte ranges, NULL / 0 when unused
  float *zero0;
  size_t zero0_bytes;
  float *zero1;
  size_t zero1_bytes;
};

// Zero [p, p + bytes) with this workgroup's share of 16-byte nontemporal
// stores (workgroup Lb of G takes chunks Lb*NTH + tid, stepping G*NTH) and the
// trailing bytes from workgroup 0.  p is 4-byte aligned (dword stores).
template <int NTH>
MOE_DEV void zero_share(float *p, size_t bytes, int Lb, int G) {
  if (!p || bytes == 0) return;
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  const size_t n16 = bytes / 16;
  const u32x4_t z = {0u, 0u, 0u, 0u};
  u32x4_t *q = (u32x4_t *)p;
  for (size_t i = (size_t)Lb * NTH + threadIdx.x; i < n16; i += (size_t)G * NTH)
    __builtin_nontemporal_store(z, q + i);
  const size_t tail = bytes - n16 * 16;  // multiple of 4
  if (Lb == 0 && threadIdx.x < tail / 4) p[n16 * 4 + threadIdx.x] = 0.f;
}

// RM: operands read by schedule row instead of by token (an operand already in
// schedule order): 0 none, DW_X_ROWS x, DW_DY_ROWS dY
enum { DW_GATHER = 0, DW_X_ROWS = 1, DW_DY_ROWS = 2 };
template <int NW, int RM = DW_GATHER, bool SC = true>
struct DwOp {
  using Map = MnmajMapT<NW>;
  static constexpr int PW = Map::PER_WAVE;  // dY (and x) instructions per wave per stage
  static constexpr bool A_KMAJ = false, B_KMAJ = false, A_SCALED = SC, PREFETCH = true;
  static constexpr bool CHECKED_TAIL = false;  // offsets are data dependent every stage
  static constexpr bool F8 = false, MX = false;
  // per stage: PW dY + PW x instructions, the stage's routing weights (SC),
  // the tokens of the stage two ahead
  static constexpr int DMA_PER_STAGE = 2 * PW + (SC ? 1 : 0) + 1;
  // LDS after the stages: per stage one 64-float weight strip per wave, then a
  // ring of TOKSLOTS slots holding one 64-token copy per wave
  static constexpr int WSTRIPS = NSTAGE * STAGE;
  static constexpr int WB = NW * 256;
  static constexpr int TOKS = WSTRIPS + NSTAGE * WB;
  static constexpr int TSLOT = NW * 256;
  static constexpr size_t LDS_BYTES = (size_t)TOKS + TOKSLOTS * TSLOT;
  // and last the indices of the units the workgroup holds (from the work queue)
  static constexpr size_t LDS_TOTAL = LDS_BYTES + 16;  // two int slots, padded
  __amdgpu_buffer_rsrc_t rsY, rsX, rsW, rsT;
  uint32_t lds0;
  const char *lds;
  int r0, m, wid, lane, K, N;
  // the next kernel's zero range, cleared on the side: one 16-byte chunk per
  // lane with each stage's token load (this lane's next chunk zi, step zstep)
  typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
  u32x4_t *zp;
  size_t zn16, zi, zstep;
  MOE_DEV void zero_chunk() {
    if (zi < zn16) {
      __builtin_nontemporal_store(u32x4_t{0u, 0u, 0u, 0u}, zp + zi);
      zi += zstep;
    }
  }
  uint32_t ncol[PW], kcol[PW];  // byte offsets of this lane's column chunk (dY / x), or OOB
  i32x4 tq[PW / 2];             // tokens of this wave's 2*PW rows of the stage being issued

  MOE_DEV void setup(int n0, int kc0) {
#pragma unroll
    for (int i = 0; i < PW; ++i) {
      const int ch = Map::chunk_of(wid, i, lane);
      ncol[i] = n0 + 8 * ch < N ? (uint32_t)(n0 + 8 * ch) * 2u : kOobOffset;
      kcol[i] = kc0 + 8 * ch < K ? (uint32_t)(kc0 + 8 * ch) * 2u : kOobOffset;
    }
  }
  MOE_DEV int ring_off(int kt) const { return TOKS + (kt & (TOKSLOTS - 1)) * TSLOT + wid * 256; }
  // Tokens of stages kt0 .. kt0+n-1 into the ring, synchronously (no DMA in flight).
  MOE_DEV void fill_ring(const int32_t *r2t, int kt0, int n) {
    for (int s = 0; s < n; ++s) {
      const int q = (kt0 + s) * BK + lane;
      *(int *)(lds + ring_off(kt0 + s) + lane * 4) = q < m ? r2t[r0 + q] : -1;
    }
  }
  // tokens of this wave's rows 2*PW*wid .. +2*PW-1 of stage kt (ring copy of this wave)
  MOE_DEV void prefetch(int kt) {
#pragma unroll
    for (int i = 0; i < PW / 2; ++i)
      tq[i] = *(const i32x4 *)(lds + ring_off(kt) + wid * (8 * PW) + 16 * i);
  }
  template <bool SKIP, bool CHECKED, bool NTW = false>
  MOE_DEV void issue_part(int kt, int buf, int j) {
    const uint32_t t = lds0 + (uint32_t)buf * STAGE;
    if (j < 2 * PW) {
      const int i = j % PW;
      const int rl = 2 * i + (lane >> 5);  // row within the wave's 2*PW
      const int q = kt * BK + 2 * PW * wid + rl;
      const int te = tq[i >> 1][(2 * i) & 3], to = tq[i >> 1][(2 * i + 1) & 3];
      int tok = (lane >> 5) ? to : te;
      if (q >= m) tok = -1;
      if (j < PW) {
        const int ry = RM == DW_DY_ROWS ? r0 + q : tok;  // row of dY (valid when tok >= 0)
        const uint32_t offy = (tok >= 0 && ncol[i] != kOobOffset)
                                  ? (uint32_t)ry * (uint32_t)N * 2u + ncol[i]
                                  : kOobOffset;
        dma16(rsY, offy, t + Map::lds_of(wid, i));
      } else {
        const int rx = RM == DW_X_ROWS ? r0 + q : tok;
        const uint32_t offx = (tok >= 0 && kcol[i] != kOobOffset)
                                  ? (uint32_t)rx * (uint32_t)K * 2u + kcol[i]
                                  : kOobOffset;
        dma16(rsX, offx, t + OPND + Map::lds_of(wid, i));
      }
    } else if (SC && j == 2 * PW) {
      // routing weights of the stage's 64 rows into this wave's strip
      const int qw = kt * BK + lane;
      const uint32_t offw = qw < m ? (uint32_t)(r0 + qw) * 4u : kOobOffset;
      dma4(rsW, offw, lds0 + (uint32_t)(WSTRIPS + buf * WB + wid * 256));
    } else {
      // tokens of stage kt + 2 into the ring (read by its prefetch after this
      // stage has been waited for)
      const int qt = (kt + 2) * BK + lane;
      const uint32_t offt = qt < m ? (uint32_t)(r0 + qt) * 4u : kOobOffset;
      dma4(rsT, offt, lds0 + (uint32_t)ring_off(kt + 2));
      // at most one more vector-memory operation per stage: the waits of the
      // pipeline stay valid (they drain, or leave at most one stage's count)
      zero_chunk();
    }
  }
  // routing weights of the 8 reduction rows this lane holds in step `step`
  MOE_DEV void row_scale(int buf, int step, int ln, float (&w)[8]) {
    const float *src = (const float *)(lds + WSTRIPS + buf * WB + wid * 256) + step * 16 +
                       8 * (ln >> 5);
    const f32x4 a = *(const f32x4 *)src, b = *(const f32x4 *)(src + 4);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      w[i] = a[i];
      w[4 + i] = b[i];
    }
  }
};

// NW waves: 4 (2 x 2 grid, 128 x 128 per wave) or 8 (4 x 2, 64 x 128 per wave:
// two waves per SIMD, half the LDS reads per wave per MFMA step)
// DYN: units from the work queue (chosen by the host when there are more than
// two rounds of units), else the static deal.
template <typename Tout, int NW, int RM = DW_GATHER, bool SC = true, bool DYN = true>
__global__ __launch_bounds__(NW * 64) void mfma_dw_kernel(DwArgs p) {
  constexpr int BM = 256, BN = 256, WGM = NW == 8 ? 4 : 2, WGN = 2;
  constexpr int MI = BM / WGM / 32, NI = BN / WGN / 32;
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int wm = wid / WGN, wn = wid % WGN;
  const int K = p.K, N = p.N, E = p.E;
  const int tn = (N + BM - 1) / BM, tk = (K + BN - 1) / BN;
  const int per_e = tn * tk;
  const int units = E * per_e;
  const int G = gridDim.x, L = logical_block();
  // the next kernel's accumulation targets: the small one now, the large one
  // (dX) a chunk per stage on the side and the rest at the end
  zero_share<NW * 64>(p.zero1, p.zero1_bytes, L, G);
  DwOp<NW, RM, SC> op;
  op.zp = (typename DwOp<NW, RM, SC>::u32x4_t *)p.zero0;
  op.zn16 = p.zero0 ? p.zero0_bytes / 16 : 0;
  op.zi = (size_t)L * (NW * 64) + tid;
  op.zstep = (size_t)G * (NW * 64);
  op.rsY = uniform_rsrc(p.dY, p.dy_bytes);
  op.rsX = uniform_rsrc(p.x, p.x_bytes);
  op.rsW = uniform_rsrc(p.row_weight, p.rw_bytes);
  op.rsT = uniform_rsrc(p.row_to_token, p.rw_bytes);
  op.lds0 = lds_addr(lds);
  op.lds = lds;
  op.wid = wid;
  op.lane = lane;
  op.K = K;
  op.N = N;

  // Units are ordered heaviest experts first.  With more than two rounds of
  // them they come from the queue: a workgroup claims its next unit while the
  // current one runs, so the claim's latency hides behind it, and the claimed
  // index passes to all waves through an LDS slot (two slots: the unit being
  // worked on and the one claimed).  With at most two rounds the queue has
  // nothing to rebalance and its claims only cost: round r deals unit
  // r G + L (r even) or r G + G - 1 - L (r odd) to logical workgroup L.
  constexpr bool dyn = DYN;
  int *const slot = (int *)(lds + DwOp<NW, RM, SC>::LDS_BYTES);
  if constexpr (dyn) {
    if (tid == 0) slot[0] = __hip_atomic_fetch_add(p.queue, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
  }
  for (int it = 0;; ++it) {
    int u;
    if constexpr (dyn) {
      u = slot[it & 1];
      if ((unsigned)u >= (unsigned)units) break;  // (a counter not from a build stops too)
    } else {
      if (it * G >= units) break;
      u = it * G + ((it & 1) ? G - 1 - L : L);
      if (u >= units) continue;
    }
    const int e = p.expert_order[u / per_e];
    const int t = u - (u / per_e) * per_e;
    const int n0 = (t / tk) * BM, kc0 = (t % tk) * BN;
    const int m = p.counts[e];
    op.r0 = p.layout == MOE_LAYOUT_MASKED ? e * p.capacity : p.offsets[e] - m;
    op.m = m;
    op.setup(n0, kc0);
    const int KI = (m + BK - 1) / BK;
    // the claim, issued after this unit's own loads of the schedule (memory
    // operations complete in order: issued before them, it would hold them up)
    int claim = 0;
    if (dyn && tid == 0)
      claim = __hip_atomic_fetch_add(p.queue, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

    f32x16 acc[MI][NI];
#pragma unroll
    for (int mi = 0; mi < MI; ++mi)
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) acc[mi][ni] = f32x16{};
    if (KI > 0) {
      __syncthreads();  // previous unit done with LDS
      op.fill_ring(p.row_to_token, 0, KI < 2 ? KI : 2);
      tile_multiply<MI, NI, WGM, WGN, false>(op, lds, 0, KI, wm, wn, lane, MI, NI, acc);
    }
    // store (exact zeros for an empty expert): the bf16 tile goes through the
    // (now idle) LDS stages, 256 x 256 row-major, and out with 16-byte row-
    // contiguous stores (a 16-byte chunk is 8 columns; K is a multiple of 8).
    // The stores are nontemporal: nothing reads dW soon, and output lines
    // kept in L2 would push out the operand rows the other units re-read
    // (measured: 581 -> 548 us for the Zipf-routed T = 8192, E = 64 top-4 dW,
    // 1117 -> 986 us for the gated FFN's gate/up weight gradient)
    static_assert(sizeof(Tout) == 2, "bf16 weight gradient");
    __syncthreads();  // every wave done reading the last stage
    __bf16 *const stile = (__bf16 *)lds;
#pragma unroll
    for (int mi = 0; mi < MI; ++mi) {
#pragma unroll
      for (int ni = 0; ni < NI; ++ni) {
        const int cl = wn * 32 + ni * 32 * WGN + (lane & 31);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int rl = wm * 32 + mi * 32 * WGM + acc_row(i, lane);
          stile[rl * BN + cl] = (__bf16)acc[mi][ni][i];
        }
      }
    }
    __syncthreads();
    Tout *const out = (Tout *)p.dW + (size_t)e * N * K;
    typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
    for (int c = tid; c < BM * (BN / 8); c += NW * 64) {
      const int rl = c / (BN / 8), cc = (c % (BN / 8)) * 8;
      const int n = n0 + rl, col = kc0 + cc;
      if (n < N && col < K)
        __builtin_nontemporal_store(*(const u32x4_t *)(stile + rl * BN + cc),
                                    (u32x4_t *)(out + (size_t)n * K + col));
    }
    if constexpr (dyn) {
      if (tid == 0) slot[(it + 1) & 1] = claim;
      __syncthreads();  // the claim is visible; slot[it & 1] is free again
    }
  }
  // the last workgroup out resets the queue for the next launch
  if (tid == 0 &&
      __hip_atomic_fetch_add(p.queue + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == G - 1) {
    __hip_atomic_store(p.queue, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(p.queue + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // the part of the zero range the stages did not reach, and its trailing bytes
  while (op.zi < op.zn16) op.zero_chunk();
  if (p.zero0 && L == 0 && tid < (p.zero0_bytes - op.zn16 * 16) / 4)
    p.zero0[op.zn16 * 4 + tid] = 0.f;
}

// dynamic LDS of the forward and input-gradient kernels: NSTAGE stages of
// (A 32 KB, B 32 KB)
constexpr size_t kStageLds = (size_t)NSTAGE * STAGE;

// Raise a kernel's dynamic LDS limit once per device (the attribute persists).
template <auto KERNEL>
hipError_t set_smem(size_t bytes) {
  static int done[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool slot = dev >= 0 && dev < 64;
  if (slot && done[dev]) return hipSuccess;
  e = hipFuncSetAttribute((const void *)KERNEL, hipFuncAttributeMaxDynamicSharedMemorySize,
                          (int)bytes);
  if (e == hipSuccess && slot) done[dev] = 1;
  return e;
}

// Tile height of the routed forward-shaped and input-gradient kernels: 0 =
// picked on the device per launch, 128 / 256 = forced (moe_set_tile_rows).
std::atomic<int> g_tile_rows{0};

}  // namespace

bool mfma_supported(int K, int N) { return K % 8 == 0 && N % 8 == 0; }

namespace {
// Launch a 256 x 256 forward-shaped kernel with 8 waves (2 x 4).
template <int MODE, typename Tout, bool F8, bool MX, int COMB>
hipError_t launch_fwd256_c(const FwdArgs &a, hipStream_t st) {
  const dim3 grid(device_cu_count());
  // block scales: two stages of (256 + 256) 4-byte scale words after the operands
  constexpr size_t lds = kStageLds + (MX ? 2 * (256 + 256) * 4 : 0);
  hipError_t e = set_smem<mfma_fwd_kernel<256, 256, 2, 4, MODE, Tout, F8, MX, COMB>>(lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((mfma_fwd_kernel<256, 256, 2, 4, MODE, Tout, F8, MX, COMB>), grid, dim3(512),
                     lds, st, a);
  return hipGetLastError();
}
// The combine is a kernel template argument (each variant carries only its own
// epilogue); the rank-ordered modes exist for the routed scatter forward.
template <int MODE, typename Tout, bool F8 = false, bool MX = false>
hipError_t launch_fwd256(const FwdArgs &a, hipStream_t st) {
  if constexpr (MODE == FWD_SCATTER) {
    if (a.combine == COMBINE_RANKED)
      return launch_fwd256_c<MODE, Tout, F8, MX, COMBINE_RANKED>(a, st);
  }
  return launch_fwd256_c<MODE, Tout, F8, MX, COMBINE_ATOMIC>(a, st);
}

// Routed forward-shaped launch: masked schedules of capacity <= 64 take 64-row
// tiles (one row block per expert), everything else 256 x 256 tiles.
template <int MODE, bool F8 = false, bool MX = false>
hipError_t launch_routed(FwdArgs &a, const moe_schedule &s, hipStream_t st) {
  if (!a.bstart) {  // the canonical schedule (a rank launch has set its window)
    a.bstart = s.block_start;
    a.bstride = s.E + 1;
  }
  if (s.layout == MOE_LAYOUT_MASKED && s.capacity <= 64) {
    constexpr int BM = 64, BN = 256;
    // (block scales: the scale ring after the stages)
    constexpr size_t ring_lds = FwdDeepOp<BM, BN, 4, F8, MX>::LDS_BYTES;
    constexpr size_t lds = ring_lds > kStageLds ? ring_lds : kStageLds;
    auto k = mfma_fwd_kernel<BM, BN, 1, 4, MODE, float, F8, MX>;
    hipError_t e = set_smem<mfma_fwd_kernel<BM, BN, 1, 4, MODE, float, F8, MX>>(lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k, dim3(device_cu_count()), dim3(256), lds, st, a);
    return hipGetLastError();
  }
  a.tile_rows = g_tile_rows.load(std::memory_order_relaxed);
  return launch_fwd256<MODE, float, F8, MX>(a, st);
}
}  // namespace

hipError_t mfma_grouped_gemm(const void *A, const void *W, const int32_t *offsets, void *C, int M,
                             int K, int N, int E, int out_dtype, hipStream_t st) {
  FwdArgs a{(const bf16_t *)A, (const bf16_t *)W, C, offsets, nullptr, nullptr, nullptr, nullptr,
            E, 0, 0, K, N, (uint32_t)((size_t)M * K * 2), M};
  if (out_dtype == MOE_F32) return launch_fwd256<FWD_BARE, float>(a, st);
  return launch_fwd256<FWD_BARE, bf16_t>(a, st);
}

namespace {
// The launch's groups: the k*E (rank, expert) groups of the rank-ordered view.
template <typename Args>
void use_ranks(Args &a, const moe_schedule &s) {
  a.counts = s.phase_counts;
  a.offsets = s.phase_offsets;
  a.bstart = s.phase_block_start;
  a.bstride = s.k * s.E + 1;
  a.row_to_token = s.phase_row_to_token;
  a.row_weight = s.phase_row_weight;
  a.layout = MOE_LAYOUT_CONTIGUOUS;
  a.capacity = 0;
  a.combine = COMBINE_RANKED;
  a.nranks = s.k;
  a.sync = s.phase_sync;
}

// A routed scatter forward: atomic adds over the canonical schedule, or one
// ranked launch over the rank-ordered view.
template <bool F8, bool MX>
hipError_t launch_scatter(FwdArgs &a, const moe_schedule &s, bool ranked, hipStream_t st) {
  a.combine = COMBINE_ATOMIC;
  if (ranked) use_ranks(a, s);
  return launch_routed<FWD_SCATTER, F8, MX>(a, s, st);
}
}  // namespace

hipError_t mfma_fused_fwd(const void *x, const void *W, const moe_schedule &s, float *y, int K,
                          int N, bool a_by_row, bool ranked, hipStream_t st) {
  const size_t arows = a_by_row ? (size_t)s.R : (size_t)s.T;
  FwdArgs a{(const bf16_t *)x, (const bf16_t *)W, y, s.offsets, s.counts, nullptr,
            s.row_to_token, s.row_weight, s.E, s.layout, s.capacity, K, N,
            (uint32_t)(arows * K * 2), (int)s.T};
  if (a_by_row) return launch_routed<FWD_SCATTER_ROWS>(a, s, st);
  return launch_scatter<false, false>(a, s, ranked, st);
}

hipError_t mfma_fused_fwd_fp8(const void *xq, const float *x_scale, const void *Wq,
                              const float *w_scale, const moe_schedule &s, float *y, int K, int N,
                              bool ranked, hipStream_t st) {
  FwdArgs a{(const bf16_t *)xq, (const bf16_t *)Wq, y, s.offsets, s.counts, nullptr,
            s.row_to_token, s.row_weight, s.E, s.layout, s.capacity, K, N,
            (uint32_t)((size_t)s.T * K), (int)s.T};
  a.x_scale = x_scale;
  a.w_scale = w_scale;
  return launch_scatter<true, false>(a, s, ranked, st);
}

hipError_t mfma_fused_fwd_mx(const void *xq, const uint8_t *x_bs, const void *Wq,
                             const uint8_t *w_bs, const moe_schedule &s, float *y, int K, int N,
                             bool ranked, hipStream_t st) {
  FwdArgs a{(const bf16_t *)xq, (const bf16_t *)Wq, y, s.offsets, s.counts, nullptr,
            s.row_to_token, s.row_weight, s.E, s.layout, s.capacity, K, N,
            (uint32_t)((size_t)s.T * K), (int)s.T};
  a.x_bs = x_bs;
  a.w_bs = w_bs;
  return launch_scatter<true, true>(a, s, ranked, st);
}

hipError_t mfma_gated_up(const void *x, const void *W_gu, const moe_schedule &s, void *h, void *gu,
                         int K, int F, hipStream_t st) {
  FwdArgs a{(const bf16_t *)x, (const bf16_t *)W_gu, h, s.offsets, s.counts, nullptr,
            s.row_to_token, s.row_weight, s.E, s.layout, s.capacity, K, F,
            (uint32_t)((size_t)s.T * K * 2), (int)s.T};
  a.gu_out = (float *)gu;
  return launch_routed<FWD_GATED>(a, s, st);
}

static hipError_t launch_dx(const DxArgs &a, hipStream_t st);

hipError_t mfma_bwd_dx(const void *dY, const void *x, const void *W, const moe_schedule &s,
                       float *dX, float *d_w, int K, int N, bool ranked, hipStream_t st) {
  DxArgs a{(const bf16_t *)dY, (const bf16_t *)x, (const bf16_t *)W, dX, d_w, s.offsets,
           s.counts, s.block_start, s.row_to_assign, s.row_to_token,
           s.row_weight, s.E, s.layout, s.capacity, K, N, (uint32_t)((size_t)s.T * N * 2),
           (uint32_t)((size_t)s.T * K * 2), g_tile_rows.load(std::memory_order_relaxed)};
  a.bstride = s.E + 1;
  a.combine = COMBINE_ATOMIC;
  a.dx_bytes = (uint32_t)((size_t)s.T * K * 4);
  if (ranked) {
    use_ranks(a, s);
    a.row_to_assign = s.phase_row_to_assign;
  }
  return launch_dx(a, st);
}

hipError_t mfma_gated_bwd_dh(const void *dY, const void *h, const void *W_down,
                             const moe_schedule &s, float *d_w, int F, int N, const void *gu,
                             void *dgu, hipStream_t st) {
  DxArgs a{(const bf16_t *)dY, (const bf16_t *)h, (const bf16_t *)W_down, nullptr, d_w, s.offsets,
           s.counts, s.block_start, s.row_to_assign, s.row_to_token,
           s.row_weight, s.E, s.layout, s.capacity, F, N, (uint32_t)((size_t)s.T * N * 2),
           (uint32_t)((size_t)s.R * F * 2), g_tile_rows.load(std::memory_order_relaxed)};
  a.bstride = s.E + 1;
  a.combine = COMBINE_ATOMIC;
  a.gu = (const float *)gu;
  a.dgu = (bf16_t *)dgu;
  const dim3 grid(device_cu_count());
  hipError_t e = set_smem<mfma_dx_kernel<4, true>>(kStageLds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((mfma_dx_kernel<4, true>), grid, dim3(256), kStageLds, st, a);
  return hipGetLastError();
}

hipError_t mfma_gated_bwd_dx(const void *dgu, const void *W_gu, const moe_schedule &s, float *dX,
                             int K, int F, hipStream_t st) {
  DxArgs a{(const bf16_t *)dgu, nullptr, (const bf16_t *)W_gu, dX, nullptr, s.offsets,
           s.counts, s.block_start, s.row_to_assign, s.row_to_token,
           s.row_weight, s.E, s.layout, s.capacity, K, 2 * F,
           (uint32_t)((size_t)s.R * 2 * F * 2), 0u, g_tile_rows.load(std::memory_order_relaxed)};
  a.bstride = s.E + 1;
  a.combine = COMBINE_ATOMIC;
  const dim3 grid(device_cu_count());
  hipError_t e = set_smem<mfma_dx_kernel<4, false, true>>(kStageLds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((mfma_dx_kernel<4, false, true>), grid, dim3(256), kStageLds, st, a);
  return hipGetLastError();
}

template <int COMB>
static hipError_t launch_dx_c(const DxArgs &a, hipStream_t st) {
  const dim3 grid(device_cu_count());
  hipError_t e = set_smem<mfma_dx_kernel<4, false, false, COMB>>(kStageLds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((mfma_dx_kernel<4, false, false, COMB>), grid, dim3(256), kStageLds, st, a);
  return hipGetLastError();
}
static hipError_t launch_dx(const DxArgs &a, hipStream_t st) {
  if (a.combine == COMBINE_RANKED) return launch_dx_c<COMBINE_RANKED>(a, st);
  return launch_dx_c<COMBINE_ATOMIC>(a, st);
}

template <int RM, bool SC, bool DYN>
static hipError_t launch_dw_q(const DwArgs &a, hipStream_t st) {
  constexpr size_t lds = DwOp<8, RM, SC>::LDS_TOTAL;
  hipError_t e = set_smem<mfma_dw_kernel<bf16_t, 8, RM, SC, DYN>>(lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((mfma_dw_kernel<bf16_t, 8, RM, SC, DYN>), dim3(device_cu_count()), dim3(512),
                     lds, st, a);
  return hipGetLastError();
}

// the work queue only with more than two rounds of units (a round: one unit
// per workgroup, one workgroup per compute unit)
template <int RM, bool SC>
static hipError_t launch_dw(const DwArgs &a, hipStream_t st) {
  const long long units =
      (long long)a.E * ((a.N + 255) / 256) * ((a.K + 255) / 256);
  return units > 2LL * device_cu_count() ? launch_dw_q<RM, SC, true>(a, st)
                                         : launch_dw_q<RM, SC, false>(a, st);
}

hipError_t mfma_bwd_dw(const void *dY, const void *x, const moe_schedule &s, void *dW, int K,
                       int N, float *zero0, size_t zero0_bytes, float *zero1, size_t zero1_bytes,
                       hipStream_t st) {
  return mfma_bwd_dw_rows(dY, false, x, false, s, dW, K, N, s.weighted != 0, zero0, zero0_bytes,
                          zero1, zero1_bytes, st);
}

hipError_t mfma_bwd_dw_rows(const void *dY, bool dy_by_row, const void *x, bool x_by_row,
                            const moe_schedule &s, void *dW, int K, int N, bool weighted,
                            float *zero0, size_t zero0_bytes, float *zero1, size_t zero1_bytes,
                            hipStream_t st) {
  DwArgs a{};
  a.dY = (const bf16_t *)dY;
  a.x = (const bf16_t *)x;
  a.dW = dW;
  a.offsets = s.offsets;
  a.counts = s.counts;
  a.expert_order = s.expert_order;
  a.row_to_token = s.row_to_token;
  a.row_weight = s.row_weight;
  a.E = s.E;
  a.layout = s.layout;
  a.capacity = s.capacity;
  a.K = K;
  a.N = N;
  a.dy_bytes = (uint32_t)((size_t)(dy_by_row ? s.R : s.T) * N * 2);
  a.x_bytes = (uint32_t)((size_t)(x_by_row ? s.R : s.T) * K * 2);
  a.rw_bytes = (uint32_t)((size_t)s.R * 4);
  a.queue = s.dw_queue;
  a.zero0 = zero0;
  a.zero0_bytes = zero0_bytes;
  a.zero1 = zero1;
  a.zero1_bytes = zero1_bytes;
  // the instantiations the callers use: gathered operands with or without
  // weights; x by row (the gated dW_down) weighted; dY by row (dW_gu, whose
  // dgu already holds the weight) unweighted
  if (dy_by_row && x_by_row) return hipErrorInvalidValue;
  if (dy_by_row) return weighted ? hipErrorInvalidValue : launch_dw<DW_DY_ROWS, false>(a, st);
  if (x_by_row) return weighted ? launch_dw<DW_X_ROWS, true>(a, st) : hipErrorInvalidValue;
  return weighted ? launch_dw<DW_GATHER, true>(a, st) : launch_dw<DW_GATHER, false>(a, st);
}

}  // namespace moe

namespace moe {
int set_tile_rows(int rows) {
  if (rows != 0 && rows != 128 && rows != 256) return MOE_ERR_SHAPE;
  g_tile_rows.store(rows, std::memory_order_relaxed);
  return MOE_OK;
}
}  // namespace moe
