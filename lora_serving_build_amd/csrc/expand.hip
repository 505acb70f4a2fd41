// Expand / expand_slice on segments (SGMV form):
//   y[t, off_s + c] = (add ? y : 0) + sum_j v_s[t, j] * B_{s,l}[j, c].
//
// Work item = (run of 128-column chunks of one slice, 64-token tile of one
// segment).  The four waves of a workgroup each take 16 tokens of the tile.
// Per item, each wave converts its tokens' fp32 v once into the matrix-core
// operands: v is split into hi = round(v) and lo = round(v - hi) in the data
// type, so v keeps about 16 significant bits.  For r <= 16, lane groups 0 and
// 1 carry hi and groups 2 and 3 carry lo against the same 16 weights, so one
// 16x16x32 op adds B^T (hi + lo).  For larger r, one weight operand covers 32
// ranks and two ops apply it to hi and to lo, which halves the LDS reads.  Per
// chunk, the weight block (128 rows of B_l^T, one contiguous 128 x r run in
// memory) is loaded by the whole workgroup with linear 16-byte loads one
// chunk ahead and staged in LDS (two buffers up to r = 64, so one barrier per
// chunk), so all waves share one copy.
//
// The product is computed transposed, D[c][token]: lane (m, g) of op tile q
// holds columns 16 q + 4 g .. +4 of token m.  One lane-row swap between the
// op tiles 2p and 2p + 1 leaves every lane with 8 consecutive columns of its
// token (row g: columns 32 p + {0, 16, 8, 24}[g] .. +8), so y is read and
// written straight from registers, 16 bytes per lane (16 rows x 64 bytes per
// instruction) -- the bulk of the traffic, with no staging tile.  A chunk's y
// goes out with the next chunk's weights, before the chunk's matrix ops (the
// first chunk's with v, in the item's set-up); y is rounded once, to nearest
// even.  LDS and registers leave room for four workgroups per CU up to
// r = 32, three at r = 64 and two at r = 128 or with 128-token tiles.
//
// In a batch of many adapters the same launch can also take the one-token
// segments, which a 64- or 128-token tile would waste, as per-token work
// items after the tile items (SG > 0, see expand_kernel).
#include "lora_device.h"
#include "lora_kernels.h"
#include "tiles.h"
#include "token_path.h"

namespace lora {

namespace {

constexpr int kExpandThreads = 256;

struct ExpandArgs {
  SegView seg;
  const float* v;
  int64_t ldv;
  int64_t v_slice_stride;
  ExpandSliceDesc slices[kMaxSlices];
  int32_t run_start[kMaxSlices + 1];  // prefix of chunk runs per slice
  int32_t num_slices;
  int32_t cpr;                        // chunks per run (from the tile bound)
  int32_t cpr_fixed;                  // 1: cpr as set, not to be shortened
  int32_t mt_bound;                   // the host's upper bound on the token tiles
  int32_t r;
  uint16_t* y;
  int64_t ldy;
  int32_t add;
  int32_t min_seg_len;  // segments with fewer tokens are left to another kernel
  int32_t short_cb;     // SG > 0: column blocks of each one-token segment's per-token items
  int32_t balanced;     // tile schedule: 0 chosen per call, 1 round-robin items, 2 balanced ranges
  int32_t line_y;       // aligned data: y loaded (1), or loaded and stored (2), in whole lines (staged in LDS)
};

static_assert(kExpandThreads == kBgThreads, "per-token items run the per-token expand's body");

// LDS of the per-token items' staging rows (one per wave), which reuse the
// weight buffers.
constexpr size_t kShortStageBytes = (size_t)(kBgThreads / kWave) * kSoRow * sizeof(float);

template <int NKS>
struct ExpandLds {
  static constexpr int RK = 16 * NKS;            // padded rank
  // 16-bit elements per LDS weight row.  The operand reads of lanes 0-7 and
  // 16-23 (rows 0-7 at two 16-byte columns) are served together, so the row
  // stride in dwords must be an odd multiple of 8 (mod 64 banks): 8 for
  // r <= 16, else RK / 2 + 8.  Measured with SQ_LDS_BANK_CONFLICT on MI355X:
  // 0 % of LDS cycles, against 34-42 % for a stride of RK / 2 + 4.
  static constexpr int BP = (RK / 32) * 32 + 16;
  static constexpr int NB = NKS <= 4 ? 2 : 1;    // weight buffers
  static constexpr size_t weight_bytes = (size_t)NB * kExpandCols * BP * 2;
  // weights (or, with per-token items, at least their staging rows), then
  // the tile table and scan scratch
  static constexpr size_t region(bool with_short) {
    return with_short && weight_bytes < kShortStageBytes ? kShortStageBytes : weight_bytes;
  }
  static size_t bytes(int L, bool with_short) {
    return region(with_short) + 4 * ((size_t)tile_table_ints(L) + 8);
  }
};

// Resident workgroups per CU the registers allow: four up to r = 32, three
// at r = 64 (and at r = 32 with per-token items, whose expand body needs a
// few more registers), two at r = 128 or with 128-token tiles.
constexpr int expand_wgs_per_cu(int nks, int tb, int sg) {
  return (tb == 2 || nks == 8) ? 2 : ((nks == 1 || (nks == 2 && sg == 0)) ? 4 : 3);
}

// Column offset (inside a 32-column pair of op tiles) of the 8 columns a lane
// of lane group g holds after the swap.
__device__ __forceinline__ int pair_col(int g) { return 8 * (((g & 1) << 1) | (g >> 1)); }

// y of a chunk loaded in whole 128-byte lines (aligned data): each load
// instruction covers 8 rows x 128 B, where the op layout above covers 16
// rows x 64 B, so every line is read by one instruction instead of two.
// Measured on MI355X, a tiled read-modify-write of a 57344-column bf16 y
// (8192 rows, 128-row x 1024-column items): 398.5 -> 380.3 us, whether the
// loads or the stores take the whole lines, and the same with the loads
// passed through LDS into the op layout.  Each wave passes one half chunk
// (16 TB rows x 128 B) at a time through its own LDS rows; the stores take
// whole lines too, through the same rows, where that measured faster.  Row pitch 192 B
// with the 16-byte slot XORed by bit 2 of the row: the line writes (rows two
// apart start 8 bank quads apart) and the op-layout reads (16 rows, two slots)
// are both free of bank conflicts.
constexpr int kYsPitch = 192;  // bytes per staged row
__device__ __forceinline__ int ys_off(int row, int slot) { return row * kYsPitch + 16 * (slot ^ ((row >> 2) & 1)); }
// Between one pass's LDS writes and the reads of other lanes' data: a
// wavefront-scope release / acquire keeps the compiler from moving the LDS
// accesses across it (no wait is needed: a wave's LDS operations run in
// order).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}
constexpr size_t y_stage_bytes(int tb) { return (size_t)(kExpandThreads / kWave) * 16 * tb * kYsPitch; }

// NKS = 16-wide steps of r (r <= 16 * NKS).  TB = 16-token blocks per wave
// (tile = 64 TB tokens; two blocks share every weight operand read from LDS
// and halve the weight traffic per token).  VEC: 16-byte aligned rows, r and
// the slice offsets multiples of 8, ldy a multiple of 8.
// DENSE: one adapter (0) for every token, token index = position (the
// single-adapter form): no metadata is read.
// SG > 0 (r = 8 SG, aligned data, with segment metadata): the launch also
// takes the batch's one-token segments, which its tile table skips, as
// per-token work items after the tile items: (segment slot, column block),
// checked 64 at a time (short_item) and expanded with the per-token expand's
// body, staging through this workgroup's weight buffers.  One launch then
// covers both kinds of segment, and the per-token items fill the tail of the
// tile items.
template <int DT, bool VEC, int NKS, int TB, bool DENSE, int SG>
__global__ __launch_bounds__(kExpandThreads, expand_wgs_per_cu(NKS, TB, SG)) void expand_kernel(ExpandArgs a) {
  static_assert(SG == 0 || (VEC && !DENSE), "per-token items need aligned data and segment metadata");
  using Lds = ExpandLds<NKS>;
  constexpr int BP = Lds::BP;
  constexpr int NB = Lds::NB;
  constexpr int TT = kTileTokens * TB;                       // tokens per tile
  constexpr int PPR = Lds::RK / 8;                           // 16-byte pieces per weight row
  constexpr int BL = kExpandCols * PPR / kExpandThreads;     // pieces per thread per chunk
  constexpr int NQ = kExpandCols / 16;                       // 16-column op tiles per chunk
  constexpr int NP = NQ / 2;                                 // op tile pairs
  constexpr bool kPack = NKS >= 2;                           // 32 ranks per weight operand
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* s_b = reinterpret_cast<uint16_t*>(smem);
  // The y staging rows (when the launch takes whole-line y loads) follow the
  // weights, then the tile table.
  const bool line_y = VEC && a.line_y != 0;
  unsigned char* s_ys = smem + Lds::region(SG > 0) + (size_t)(threadIdx.x / kWave) * (16 * TB * kYsPitch);
  int32_t* s_table =
      reinterpret_cast<int32_t*>(smem + Lds::region(SG > 0) + (a.line_y ? y_stage_bytes(TB) : 0));
  int32_t* s_scan = s_table + tile_table_ints(a.seg.L);

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int m = lane & 15;  // token of the ops / weight row inside a 16-row tile
  const int g = lane >> 4;  // lane group
  const int pc = pair_col(g);

  const TileTable table =
      build_tile_table<kExpandThreads, DENSE>(a.seg, TT, a.r, s_table, s_scan, a.min_seg_len);
  const int mtiles = table.tiles;
  const int grid = gridDim.x;
  // Runs of a slice for cpr chunks per run.
  auto slice_runs = [&](int q, int cpr) {
    return ((a.slices[q].n + kExpandCols - 1) / kExpandCols + cpr - 1) / cpr;
  };
  auto all_runs = [&](int cpr) {
    int n = 0;
    for (int q = 0; q < a.num_slices; ++q) n += slice_runs(q, cpr);
    return n;
  };
  // The host sized the runs for its bound on the tiles; when the batch has
  // under half as many (an adapter pool far larger than the segments in
  // use), shorter runs keep two items per workgroup (the same value in every
  // workgroup).
  int cpr = a.cpr;
  int nruns = a.run_start[a.num_slices];
  if (!a.cpr_fixed && 2 * mtiles <= a.mt_bound) {
    while (cpr > 1 && mtiles * nruns < 2 * grid) {
      cpr >>= 1;
      nruns = all_runs(cpr);
    }
  }
  const int n_tile_items = mtiles * nruns;
  const int n_short = SG > 0 ? min(a.seg.L, a.seg.T) * a.short_cb : 0;

  // Tile work, in one of two schedules (the same choice in every
  // workgroup).  Round-robin: item = (run, tile); consecutive items walk the
  // token tiles under one run of columns, so the weight run is reused from
  // the L2 of one XCD.  Balanced: the same order cut into (run, tile, chunk)
  // units, each workgroup taking one contiguous range of U / grid units
  // (neighbouring ranges on one XCD).  Round-robin spends a whole round on a
  // last round that is only partly filled; a balanced range rarely starts or
  // ends on a run boundary, so it pays about one more item set-up (token ids,
  // v and the first y: a few memory trips, about 1.5 chunk times with
  // 128-token tiles).  Balanced is taken when it is estimated 5% faster.
  // Measured on MI355X (us, round-robin -> balanced): 8192 x 16384 over 4 segments of
  // 1952-2288 tokens, r = 16 / 64: 135.5 / 145.2 -> 123.4 / 131.3 (66 tiles,
  // 4.1 rounds); 8192 x 4096, r = 64: 47.6 -> 40.7 (1.03 rounds); but 4
  // aligned segments of 2048 tokens: 133.0 -> 136.1, the 8192-token layer's
  // gate_up call (7.8 rounds): 442.9 -> 461.6, and with 64-token tiles and
  // 2-chunk runs 8192 x 1024 at r = 128 (1.02 rounds): 21.6 -> 24.0.
  // (Balanced ranges count units in 32 bits: beyond that, round-robin.  The
  // forms with 64-token tiles are always round-robin: there a set-up costs
  // about 3 chunk times, so balanced ranges rarely pay, and the code of the
  // other walk cost them 1-7% (rank 128: 21.8 -> 23.5 us on 8192 x 1024).)
  constexpr bool kCanBalance = TB == 2 && NKS <= 4;
  int64_t chunks = 0;
  for (int q = 0; q < a.num_slices; ++q) chunks += (a.slices[q].n + kExpandCols - 1) / kExpandCols;
  const int64_t units = (int64_t)mtiles * chunks;
  bool balanced = kCanBalance && a.balanced == 2 && units < INT32_MAX;
  if (kCanBalance && a.balanced == 0 && n_tile_items > grid && units < INT32_MAX) {
    constexpr float kSetup = 1.5f;
    const float per = (float)units / (float)grid;
    const float rr = ceilf((float)n_tile_items / (float)grid) * ((float)cpr + kSetup);
    const float bal = per + kSetup * (ceilf(per / (float)cpr) + 1.f);
    balanced = bal < 0.95f * rr;
  }
  // Whole-line stores too (the results pass back through the same LDS rows)
  // at r <= 32 and on round-robin walks at r = 33..64: the 8192-token
  // layer's gate_up call 442.7 -> 432.1 us, r <= 32 1-2.5% faster; but
  // balanced ranges at r = 64 measured 1-2% slower (8192 x 16384 / 8192 /
  // 4096: 120.9 / 66.1 / 41.5 -> 122.4 / 67.0 / 42.4 us) and r = 128 2-3%
  // (8192 x 1024: 22.5 -> 23.1).
  const bool line_st = line_y && a.line_y == 2 && (NKS <= 2 || (NKS == 4 && !balanced));
  // The walk's position and end: item and tile-item count (round-robin,
  // which numbers the per-token items after the tile items in one walk, so
  // the workgroups without a last-round tile item take them first), or unit
  // range (balanced).
  int cur, end;
  if (balanced) {
    // A range breaks at run boundaries, so longer runs leave fewer item
    // set-ups per workgroup; but a run longer than one XCD's share of the
    // units (chunks / 8 per tile) splits each run's tiles over two XCDs, and
    // that measured far slower (8192 x 16384 over four segments, r = 64:
    // runs of 4 / 16 / 32 chunks 129.8 / 118.9 / 177.3 us; 8192 x 4096:
    // runs of 4 / 8 40.1 / 51.3).  So the runs double while they fit.
    if (!a.cpr_fixed) {
      while (2 * (int64_t)cpr <= (chunks >> 3)) cpr *= 2;
    }
    const int w = (grid & 7) == 0 ? (blockIdx.x & 7) * (grid >> 3) + (blockIdx.x >> 3) : blockIdx.x;
    cur = (int)(units * w / grid);
    end = (int)(units * (w + 1) / grid);
  } else {
    cur = xcd_first_item(blockIdx.x, grid, n_tile_items + n_short);
    end = n_tile_items;
  }
  for (;;) {
    if (cur >= end) break;
    int q = 0, mt = 0, c_beg = 0, c_end = 0;
    if (balanced) {
      const int u = cur;
      // Slice, run inside the slice (full runs of cpr chunks, then one
      // shorter run), tile, chunk inside the run.
      int base = 0;  // units before slice q (all below 2^31 here)
      int cq = (a.slices[0].n + kExpandCols - 1) / kExpandCols;
      while (q + 1 < a.num_slices && base + mtiles * cq <= u) {
        base += mtiles * cq;
        ++q;
        cq = (a.slices[q].n + kExpandCols - 1) / kExpandCols;
      }
      const int o = u - base;
      const int j = o / (mtiles * cpr);
      const int len = min(cpr, cq - j * cpr);
      const int o2 = o - j * mtiles * cpr;
      mt = o2 / len;
      const int c = o2 - mt * len;
      c_beg = j * cpr + c;
      c_end = c_beg + min(end - u, len - c);
      cur += c_end - c_beg;
    } else {
      const int cr = cur / mtiles;
      mt = cur - cr * mtiles;
      int rs = 0;
      while (q + 1 < a.num_slices && rs + slice_runs(q, cpr) <= cr) {
        rs += slice_runs(q, cpr);
        ++q;
      }
      c_beg = (cr - rs) * cpr;
      c_end = min(c_beg + cpr, (a.slices[q].n + kExpandCols - 1) / kExpandCols);
      cur += grid;
    }
    const int nq = a.slices[q].n;

    int p0 = 0, p_end = 0, l = 0;
    // The adapter's live rank: weight pieces and v groups at or beyond it
    // are zero and are not read (their pieces read the row's first one,
    // which is loaded anyway), and their matrix ops are skipped.
    int rank_l = 0;
    const bool ok = tile_range_lds(table, a.seg.T, a.seg.L, TT, mt, &p0, &p_end, &l, &rank_l);
    const uint16_t* Bl = a.slices[q].B + (int64_t)l * nq * a.r;
    uint16_t* ybase = a.y + a.slices[q].col_off;

    // Weight chunk loader: piece p = tid + 256 i is row p / PPR, columns
    // 8 (p % PPR) .. +8 of the chunk's B_l^T rows.  Rows past the slice read
    // the last row (their outputs are dropped); ranks >= the live rank read
    // zero.
    u32x4 rb[BL];
    auto gload_b = [&](int c) {
#pragma unroll
      for (int i = 0; i < BL; ++i) {
        const int p = tid + kExpandThreads * i;
        const int row = p / PPR;
        const int col = (p - row * PPR) * 8;
        int n = c * kExpandCols + row;
        n = n < nq ? n : nq - 1;
        if constexpr (VEC) {
          // r % 8 == 0: a piece is whole or past r.  The load is unconditional
          // (pieces at or past the live rank read the row's first piece) so
          // the compiler can count loads in flight exactly.
          const int cs = col < rank_l ? col : 0;
          rb[i] = *reinterpret_cast<const u32x4*>(Bl + (int64_t)n * a.r + cs);
        } else {
          rb[i] = load8_16<false>(Bl + (int64_t)n * a.r + col, rank_l - col);
        }
      }
    };
    // Pieces at or past the live rank are zeroed here, when the chunk is
    // written to LDS, not next to their loads: a select next to a load would
    // make the wave wait for it at once.
    auto swrite_b = [&](int buf) {
#pragma unroll
      for (int i = 0; i < BL; ++i) {
        const int p = tid + kExpandThreads * i;
        const int row = p / PPR;
        const int col = (p - row * PPR) * 8;
        u32x4 w = rb[i];
        if (col >= rank_l) w = u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(&s_b[(buf * kExpandCols + row) * BP + col]) = w;
      }
    };
    // Wave w takes tokens [16 TB w, 16 TB (w + 1)) of the tile, block b the
    // 16 tokens from 16 (TB w + b); every lane reads its own token id.  The
    // id loads go out first (unconditionally, at positions clamped into the
    // batch), then the first chunk's weights, which depend only on the
    // adapter: loads complete in issue order, so the wait for the ids does not
    // include the weight block (32 KB per workgroup at r = 128), which stays
    // in flight behind them.
    int traw[TB];
#pragma unroll
    for (int b = 0; b < TB; ++b) {
      int pos = p0 + 16 * (TB * wave + b) + m;
      pos = pos < 0 ? 0 : (pos < a.seg.T ? pos : a.seg.T - 1);
      traw[b] = DENSE ? pos : a.seg.sorted_token[pos];
    }
    // Unconditional (an invalid tile reads adapter 0's clamped rows and drops
    // them): a load on only some paths would make the compiler's wait for
    // the ids include it.
    gload_b(c_beg);
    // Nothing that uses an id may be scheduled above these loads.
    __builtin_amdgcn_sched_barrier(0);

    bool blk_live[TB], tok_ok[TB];
    int tok[TB];
    uint16_t* yrow[TB];
#pragma unroll
    for (int b = 0; b < TB; ++b) {
      const int pos = p0 + 16 * (TB * wave + b) + m;
      blk_live[b] = ok && p0 + 16 * (TB * wave + b) < p_end;
      int t = (ok && pos < p_end) ? traw[b] : -1;
      t = (t >= 0 && t < a.seg.T) ? t : -1;
      tok[b] = t;
      tok_ok[b] = blk_live[b] && t >= 0;
      yrow[b] = ybase + (int64_t)(tok_ok[b] ? t : 0) * a.ldy;
    }
    const bool wave_live = blk_live[0];
    // Whole-line y loads: instruction i covers rows 8 (i / 2) + lane / 8 of
    // the wave's 16 TB rows and the 128-byte half i % 2 of the chunk; a row's
    // token comes from the lane that holds it in the op layout (row 16 b + m
    // of block b is lane m's).
    uint16_t* yline[2 * TB];
    bool rowok[2 * TB];
    if (line_y) {
#pragma unroll
      for (int hh = 0; hh < 2 * TB; ++hh) {
        const int src = (8 * hh + (lane >> 3)) & 15;  // row 8 hh + lane / 8 is in block hh / 2
        const int row = __shfl(tok_ok[hh >> 1] ? tok[hh >> 1] : 0, src, kWave);
        yline[hh] = ybase + (int64_t)row * a.ldy;
        rowok[hh] = line_st && __shfl(tok_ok[hh >> 1] ? 1 : 0, src, kWave) != 0;
      }
    }

    // y of this lane for chunk c: pair p covers columns 32 p + pc .. +8.  The
    // vector path loads unconditionally (rows of inactive lanes point at row
    // 0 and columns are clamped into the slice, n % 8 == 0), so the compiler
    // counts the loads in flight exactly; values that no store uses are
    // simply ignored.
    auto gload_y = [&](int c, u32x4 (*yv)[NP]) {
      if (line_y) {
        // register i = (b, p) with b = i / NP, p = i % NP holds line load i
#pragma unroll
        for (int i = 0; i < TB * NP; ++i) {
          const int col = c * kExpandCols + 64 * (i & 1) + 8 * (lane & 7);
          const int cs = col + 8 <= nq ? col : nq - 8;
          yv[i / NP][i % NP] = *reinterpret_cast<const u32x4*>(yline[i >> 1] + cs);
        }
        return;
      }
#pragma unroll
      for (int b = 0; b < TB; ++b) {
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          yv[b][p] = u32x4{0u, 0u, 0u, 0u};
          if constexpr (VEC) {
            const int col = c * kExpandCols + 32 * p + pc;
            const int cs = col + 8 <= nq ? col : nq - 8;
            yv[b][p] = *reinterpret_cast<const u32x4*>(yrow[b] + cs);
          }
        }
      }
    };
    // v of each block's 16 tokens as hi / lo operands, once per item.  All
    // loads go out before any is used (addresses clamped into the row, ranks
    // >= r replaced by zeros afterwards).  For r <= 16 one operand holds hi
    // (lane groups 0, 1) and lo (groups 2, 3) of the same 16 ranks; for larger
    // r, operand 2 p holds hi and 2 p + 1 lo of ranks 32 p .. +32, so one
    // weight operand read from LDS feeds two products.
    u32x4 bop[TB][NKS];
    // y of the first chunk depends only on the tokens: it goes out right
    // behind v (a scheduling barrier keeps it there), so the wait for v does
    // not hold it back and it is in flight through v's conversion and the
    // first barrier.
    u32x4 yfirst[TB][NP];
    // With 64-token tiles an item is short (a few chunks, often one item per
    // workgroup), so its chain of memory trips sets the time: the second
    // chunk's y goes out with the first's.
    constexpr bool kPeel = TB == 1;
    u32x4 ysecond[TB][NP];
    // Per token: 2^k of the binary16 prescale (1 for bfloat16, whose range is
    // fp32's), applied to the fp32 products before y is added.
    float vscale[TB];
    {
      constexpr int NV = kPack ? NKS / 2 : NKS;  // 8-rank groups per lane
      f32x4 vraw[TB][NV][2];
#pragma unroll
      for (int b = 0; b < TB; ++b) {
        const float* vrow = a.v + (int64_t)(tok_ok[b] ? tok[b] : 0) * a.ldv + (int64_t)q * a.v_slice_stride;
#pragma unroll
        for (int st = 0; st < NV; ++st) {
          const int rk = kPack ? st * 32 + g * 8 : st * 16 + (g & 1) * 8;
          if constexpr (VEC) {
            const int rs = rk + 8 <= a.r ? rk : 0;
            vraw[b][st][0] = *reinterpret_cast<const f32x4*>(vrow + rs);
            vraw[b][st][1] = *reinterpret_cast<const f32x4*>(vrow + rs + 4);
          } else {
            float vv[8];
            load8_f32<false>(vrow + rk, a.r - rk, vv);
            vraw[b][st][0] = f32x4{vv[0], vv[1], vv[2], vv[3]};
            vraw[b][st][1] = f32x4{vv[4], vv[5], vv[6], vv[7]};
          }
        }
      }
      gload_y(c_beg, yfirst);  // unconditional: addresses are clamped, c_beg < c_end
      if constexpr (kPeel) gload_y(c_beg + 1, ysecond);  // clamped too, also past c_end
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int b = 0; b < TB; ++b) {
        float vk[NV][8];
        float vmax = 0.f;
#pragma unroll
        for (int st = 0; st < NV; ++st) {
          const int rk = kPack ? st * 32 + g * 8 : st * 16 + (g & 1) * 8;
          const bool keep = tok_ok[b] && rk < rank_l && (VEC ? rk + 8 <= a.r : true);
          const float vv[8] = {vraw[b][st][0].x, vraw[b][st][0].y, vraw[b][st][0].z, vraw[b][st][0].w,
                               vraw[b][st][1].x, vraw[b][st][1].y, vraw[b][st][1].z, vraw[b][st][1].w};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            vk[st][e] = keep ? vv[e] : 0.f;
            vmax = fmaxf(vmax, fabsf(vk[st][e]));
          }
        }
        // The four lane groups of row position m together hold every rank of
        // token m (groups 2 and 3 repeat 0 and 1 for r <= 16).
        float down = 1.f;
        vscale[b] = 1.f;
        if constexpr (DT == 0) f16_prescale(max_over_lane_groups(vmax), &down, &vscale[b]);
#pragma unroll
        for (int st = 0; st < NV; ++st) {
          uint32_t h4[4], l4[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float f0 = vk[st][2 * e] * down, f1 = vk[st][2 * e + 1] * down;
            const uint32_t hi = cvt_pack2<DT>(f0, f1);
            float h0, h1;
            unpack2<DT>(hi, &h0, &h1);
            const float l0 = __builtin_isfinite(h0) ? f0 - h0 : 0.f;
            const float l1 = __builtin_isfinite(h1) ? f1 - h1 : 0.f;
            h4[e] = hi;
            l4[e] = cvt_pack2<DT>(l0, l1);
          }
          if constexpr (kPack) {
            bop[b][2 * st] = u32x4{h4[0], h4[1], h4[2], h4[3]};
            bop[b][2 * st + 1] = u32x4{l4[0], l4[1], l4[2], l4[3]};
          } else {
            bop[b][st] = g < 2 ? u32x4{h4[0], h4[1], h4[2], h4[3]} : u32x4{l4[0], l4[1], l4[2], l4[3]};
          }
        }
      }
    }

    if (ok && c_beg < c_end) swrite_b(0);
    __syncthreads();
    // One chunk: the next chunk's weights and this chunk's y go out first,
    // the products run from LDS while they are in flight, then one wait and
    // the y update.  The latency of y is covered by the other workgroups on
    // the CU (up to four), not by a longer prefetch: a longer prefetch would
    // not survive the compiler's conservative load counting across the loop.
    // src (a constant at every call): 0 the set-up's first y, 1 its second,
    // 2 loaded here.
    auto chunk = [&](int c, int src) {
      const int buf = NB == 2 ? ((c - c_beg) & 1) : 0;
      const bool has_next = c + 1 < c_end;
      if (has_next) gload_b(c + 1);
      u32x4 ycur[TB][NP];
      if (src == 0) {
#pragma unroll
        for (int b = 0; b < TB; ++b)
#pragma unroll
          for (int p = 0; p < NP; ++p) ycur[b][p] = yfirst[b][p];
      } else if (src == 1) {
#pragma unroll
        for (int b = 0; b < TB; ++b)
#pragma unroll
          for (int p = 0; p < NP; ++p) ycur[b][p] = ysecond[b][p];
      } else {
        gload_y(c, ycur);
      }
      // Nothing below may be scheduled between these loads.
      __builtin_amdgcn_sched_barrier(0);
      if (wave_live) {
        const uint16_t* sb = s_b + buf * kExpandCols * BP;
        // Two halves of 64 columns keep fewer accumulators live at a time.
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          f32x4 acc[TB][NQ / 2];
#pragma unroll
          for (int b = 0; b < TB; ++b)
#pragma unroll
            for (int qq = 0; qq < NQ / 2; ++qq) acc[b][qq] = f32x4{0.f, 0.f, 0.f, 0.f};
          if constexpr (kPack) {
#pragma unroll
            for (int st = 0; st < NKS / 2; ++st) {
              if (32 * st >= rank_l) continue;  // ranks past the live rank are zero
#pragma unroll
              for (int qq = 0; qq < NQ / 2; ++qq) {
                const int row = (h * (NQ / 2) + qq) * 16 + m;
                const u32x4 aop = *reinterpret_cast<const u32x4*>(&sb[row * BP + st * 32 + g * 8]);
#pragma unroll
                for (int b = 0; b < TB; ++b) {
                  acc[b][qq] = mfma16x16x32<DT>(aop, bop[b][2 * st], acc[b][qq]);
                  acc[b][qq] = mfma16x16x32<DT>(aop, bop[b][2 * st + 1], acc[b][qq]);
                }
              }
            }
          } else {
#pragma unroll
            for (int qq = 0; qq < NQ / 2; ++qq) {
              const int row = (h * (NQ / 2) + qq) * 16 + m;
              const u32x4 aop = *reinterpret_cast<const u32x4*>(&sb[row * BP + (g & 1) * 8]);
#pragma unroll
              for (int b = 0; b < TB; ++b) acc[b][qq] = mfma16x16x32<DT>(aop, bop[b][0], acc[b][qq]);
            }
          }
          // This half's y in the op layout: straight from the registers, or
          // (whole-line loads) the half's lines through the wave's LDS rows.
          u32x4 yh[TB][NP / 2];
          if (line_y) {
#pragma unroll
            for (int hh = 0; hh < 2 * TB; ++hh) {
              const int i = 2 * hh + h;
              *reinterpret_cast<u32x4*>(s_ys + ys_off(8 * hh + (lane >> 3), lane & 7)) = ycur[i / NP][i % NP];
            }
            wave_lds_sync();
#pragma unroll
            for (int b = 0; b < TB; ++b)
#pragma unroll
              for (int pp = 0; pp < NP / 2; ++pp)
                yh[b][pp] = *reinterpret_cast<const u32x4*>(s_ys + ys_off(16 * b + m, 4 * pp + (pc >> 3)));
            wave_lds_sync();
          } else {
#pragma unroll
            for (int b = 0; b < TB; ++b)
#pragma unroll
              for (int pp = 0; pp < NP / 2; ++pp) yh[b][pp] = ycur[b][h * (NP / 2) + pp];
          }
#pragma unroll
          for (int b = 0; b < TB; ++b) {
            if (!tok_ok[b]) continue;
#pragma unroll
            for (int pp = 0; pp < NP / 2; ++pp) {
              const int p = h * (NP / 2) + pp;
              float out[8];
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                const auto sw = __builtin_amdgcn_permlane16_swap(__float_as_uint(acc[b][2 * pp][e]),
                                                                 __float_as_uint(acc[b][2 * pp + 1][e]), false, false);
                out[e] = __uint_as_float(sw[0]);
                out[4 + e] = __uint_as_float(sw[1]);
              }
              if constexpr (DT == 0) {
#pragma unroll
                for (int e = 0; e < 8; ++e) out[e] *= vscale[b];
              }
              const int col = c * kExpandCols + 32 * p + pc;
              const int cvalid = nq - col;
              if (cvalid <= 0) continue;
              uint16_t* yp = yrow[b] + col;
              if constexpr (VEC) {  // n % 8 == 0: the lane's 8 columns are all in the slice
                if (a.add) {
                  const uint32_t d[4] = {yh[b][pp].x, yh[b][pp].y, yh[b][pp].z, yh[b][pp].w};
#pragma unroll
                  for (int e = 0; e < 4; ++e) {
                    float y0, y1;
                    unpack2<DT>(d[e], &y0, &y1);
                    out[2 * e] += y0;
                    out[2 * e + 1] += y1;
                  }
                }
                const u32x4 res = u32x4{cvt_pack2<DT>(out[0], out[1]), cvt_pack2<DT>(out[2], out[3]),
                                        cvt_pack2<DT>(out[4], out[5]), cvt_pack2<DT>(out[6], out[7])};
                if (line_st)  // back to the slot its y came from; stored in whole lines below
                  *reinterpret_cast<u32x4*>(s_ys + ys_off(16 * b + m, 4 * pp + (pc >> 3))) = res;
                else
                  *reinterpret_cast<u32x4*>(yp) = res;
              } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                  if (e < cvalid) {
                    float o = out[e];
                    if (a.add) o += to_f32<DT>(yp[e]);
                    yp[e] = (uint16_t)(cvt_pack2<DT>(o, 0.f) & 0xffffu);
                  }
                }
              }
            }
          }
          if (line_st) {
            // The half's results in whole lines: every row with a token and
            // every column inside the slice (n % 8 == 0).
            wave_lds_sync();
#pragma unroll
            for (int hh = 0; hh < 2 * TB; ++hh) {
              const u32x4 res = *reinterpret_cast<const u32x4*>(s_ys + ys_off(8 * hh + (lane >> 3), lane & 7));
              const int col = c * kExpandCols + 64 * h + 8 * (lane & 7);
              if (rowok[hh] && col < nq) *reinterpret_cast<u32x4*>(yline[hh] + col) = res;
            }
            wave_lds_sync();
          }
        }
      }
      if constexpr (NB == 2) {
        // The other buffer was last read in the previous chunk, which every
        // wave finished before the barrier that ended it.
        if (has_next) swrite_b(buf ^ 1);
        __syncthreads();
      } else {
        __syncthreads();  // every wave is done with this chunk's weights
        if (has_next) swrite_b(0);
        __syncthreads();
      }
    };
    if (c_beg < c_end) chunk(c_beg, 0);
    if constexpr (kPeel) {
      if (c_beg + 1 < c_end) chunk(c_beg + 1, 1);
      for (int c = c_beg + 2; c < c_end; ++c) chunk(c, 2);
    } else {
      for (int c = c_beg + 1; c < c_end; ++c) chunk(c, 2);
    }
  }

  if constexpr (SG > 0) {
    // Per-token items: each takes its slot's segment if it holds one token.
    // Round-robin goes on with the walk above; balanced ranges start a
    // grid-stride walk of their own.  Every chunk above ended with a
    // barrier, so the staging rows (the weight buffers) are free.
    ShortBatch sb;
    int n_seen = 0;
    for (int it = balanced ? xcd_first_item(blockIdx.x, grid, n_short) : cur - n_tile_items; it < n_short;
         it += grid) {
      int t = 0, l = -1;
      if (short_item(a.seg, 1, a.short_cb, n_short, it, n_seen++, sb, &t, &l)) {
        const int k = it / a.short_cb;
        expand_token_aligned<DT, SG, 1>(
            a, t, it - k * a.short_cb, a.short_cb,
            [&](int qs) { return a.v + (int64_t)t * a.ldv + (int64_t)qs * a.v_slice_stride; },
            [&]() { return l; }, reinterpret_cast<float*>(smem) + wave * kSoRow);
      }
      __syncthreads();  // the staging rows are reused by the next item
    }
  }
}

}  // namespace

namespace {

// The tile expand with per-token items for r = 8, 16, 32, 64 (aligned, with
// metadata).
template <int DT, int TB>
void launch_with_short(int r, int64_t grid, size_t lds, hipStream_t s, const ExpandArgs& a) {
  switch (r) {
    case 8: hipLaunchKernelGGL((expand_kernel<DT, true, 1, TB, false, 1>), dim3(grid), dim3(kExpandThreads), lds, s, a); break;
    case 16: hipLaunchKernelGGL((expand_kernel<DT, true, 1, TB, false, 2>), dim3(grid), dim3(kExpandThreads), lds, s, a); break;
    case 32: hipLaunchKernelGGL((expand_kernel<DT, true, 2, TB, false, 4>), dim3(grid), dim3(kExpandThreads), lds, s, a); break;
    default: hipLaunchKernelGGL((expand_kernel<DT, true, 4, TB, false, 8>), dim3(grid), dim3(kExpandThreads), lds, s, a); break;
  }
}

}  // namespace

hipError_t launch_expand(const SegView& seg, const float* v, int64_t ldv, int64_t v_slice_stride,
                         const ExpandSliceDesc* slices, int32_t num_slices, int32_t r,
                         uint16_t* y, int64_t ldy, int add, int dtype, bool vec, hipStream_t s,
                         int min_seg_len, bool short_items) {
  ExpandArgs a{};
  a.min_seg_len = min_seg_len > 1 ? min_seg_len : 1;
  // Per-token items for the one-token segments: aligned data, segment
  // metadata and r = 8 SG only (the caller checks).
  const int sg = short_items ? r / 8 : 0;
  a.seg = seg;
  a.v = v;
  a.ldv = ldv;
  a.v_slice_stride = v_slice_stride;
  a.num_slices = num_slices;
  a.r = r;
  a.y = y;
  a.ldy = ldy;
  a.add = add;
  const int nks = r <= 16 ? 1 : r <= 32 ? 2 : r <= 64 ? 4 : 8;
  int64_t chunks = 0;
  for (int q = 0; q < num_slices; ++q) chunks += (slices[q].n + kExpandCols - 1) / kExpandCols;
  // 128-token tiles (two 16-token blocks per wave) halve the weight reads per
  // y byte and double each wave's y loads in flight, but give fewer, larger
  // items (two workgroups per CU instead of three or four).  Measured on
  // MI355X, each call alone with inputs in HBM (64-token tiles against
  // 128-token tiles with runs of 4 chunks):
  //   8192 x 16384, r = 16 / 32 / 64:   119.7 / 121.3 / 138.8 us -> 115.3 / 118.5 / 123.1
  //   8192 x 4096,  r = 16 / 64:         32.6 / 40.7 us -> 33.0 / 36.0
  //   8192-token layer, qkv slices:      95.5 us -> 92.1
  //   2048 x 16384 / 2048 x 4096, r = 64: 40.5 / 13.2 us -> 41.7 / 19.1
  //   2048 x 128256 (logits), r = 16:   266 us -> 228
  // so they are taken from 64 tiles of 128 tokens and 2048 tile-chunks up,
  // or from 16384 tile-chunks up, for r <= 64 (r = 128 keeps 64-token tiles
  // for its registers).
  const int64_t mt128 = max_token_tiles(seg.T, seg.L, 2 * kTileTokens);
  int tb = (nks <= 4 && ((mt128 >= 64 && mt128 * chunks >= 2048) || mt128 * chunks >= 16384)) ? 2 : 1;
  if (tuning().expand_tb == 1 || tuning().expand_tb == 2) tb = tuning().expand_tb;
  if (nks == 8) tb = 1;
  const int64_t tt = (int64_t)kTileTokens * tb;
  const int64_t mt_max = max_token_tiles(seg.T, seg.L, tt);
  // Chunks per run: long runs amortise an item's set-up (its token list, v
  // and the first y and weights, about two memory trips) and keep each y row
  // streaming, but leave a few items per resident workgroup.  64-token
  // tiles: 2 to 8 chunks, about 4096 items -- measured best on the 2048-token
  // and mixed-rank workloads (a run of one chunk spends about two thirds of
  // its time in the set-up).  128-token tiles: 4 chunks, 8 from 32768
  // tile-chunks up (the 8192-token layer's gate_up call: 445.6 us at 8, 450.7
  // at 4).  Runs of 3 or 6 chunks, which leave ragged runs at the slice ends,
  // measured 7-30% slower than 2, 4 or 8 on every shape above.
  int64_t cpr;
  if (tb == 2) {
    cpr = mt_max * chunks >= 32768 ? 8 : 4;
  } else {
    const int64_t want = mt_max * chunks / 4096;
    cpr = want >= 8 ? 8 : (want >= 4 ? 4 : 2);
  }
  a.balanced = tuning().expand_balance == 1 || tuning().expand_balance == 2 ? tuning().expand_balance : 0;
  a.cpr_fixed = 0;
  if (tuning().expand_cpr >= 1) {
    cpr = tuning().expand_cpr;
    a.cpr_fixed = 1;
  }
  a.cpr = (int32_t)cpr;
  a.mt_bound = (int32_t)mt_max;
  int32_t runs = 0;
  for (int q = 0; q < num_slices; ++q) {
    a.slices[q] = slices[q];
    a.run_start[q] = runs;
    const int64_t cq = (slices[q].n + kExpandCols - 1) / kExpandCols;
    runs += (int32_t)((cq + cpr - 1) / cpr);
  }
  a.run_start[num_slices] = runs;
  int64_t items = mt_max * runs;
  if (sg > 0) {
    // Column blocks of a one-token segment's items: one round of 512 columns
    // of the widest slice per wave, as in the per-token expand.
    int64_t rounds = 1;
    for (int q = 0; q < num_slices; ++q) {
      const int64_t rq = (slices[q].n + kRoundCols - 1) / kRoundCols;
      rounds = rq > rounds ? rq : rounds;
    }
    const int64_t nw = kBgThreads / kWave;
    a.short_cb = (int32_t)((rounds + nw - 1) / nw);
    items += (int64_t)(seg.L < seg.T ? seg.L : seg.T) * a.short_cb;
  }
  const bool ws = sg > 0;
  size_t lds = nks == 1 ? ExpandLds<1>::bytes(seg.L, ws)
               : nks == 2 ? ExpandLds<2>::bytes(seg.L, ws)
               : nks == 4 ? ExpandLds<4>::bytes(seg.L, ws) : ExpandLds<8>::bytes(seg.L, ws);
  // Persistent workgroups: as many as fit on the 256 CUs (LDS and register
  // bound), at most four per CU.
  const int64_t reg_cu = expand_wgs_per_cu(nks, tb, sg);
  auto fit_cu = [&](size_t bytes) {
    const int64_t n = (int64_t)(160 * 1024 / bytes);
    return n < 1 ? 1 : (n > reg_cu ? reg_cu : n);
  };
  int64_t per_cu = fit_cu(lds);
  // Whole-line y loads on aligned data, when their LDS
  // rows keep as many workgroups per CU (a large adapter pool's table may
  // not leave room).
  a.line_y = 0;
  if (vec && tuning().expand_line_y != 2 && fit_cu(lds + y_stage_bytes(tb)) >= per_cu) {
    a.line_y = tuning().expand_line_y == 1 ? 1 : 2;
    lds += y_stage_bytes(tb);
  }
  if (tuning().expand_wgs_per_cu >= 1 && tuning().expand_wgs_per_cu < per_cu) per_cu = tuning().expand_wgs_per_cu;
  int64_t grid = items < 256 * per_cu ? items : 256 * per_cu;
  grid = (grid + 7) / 8 * 8;
  if (grid < 8) grid = 8;
  if (sg > 0) {
    if (dtype == 0) {
      if (tb == 2) launch_with_short<0, 2>(r, grid, lds, s, a);
      else launch_with_short<0, 1>(r, grid, lds, s, a);
    } else {
      if (tb == 2) launch_with_short<1, 2>(r, grid, lds, s, a);
      else launch_with_short<1, 1>(r, grid, lds, s, a);
    }
    return hipGetLastError();
  }
#define LORA_EXPAND_LAUNCH(DT_, VEC_, TB_, DN_)                                                      \
  switch (nks) {                                                                                    \
    case 1: hipLaunchKernelGGL((expand_kernel<DT_, VEC_, 1, TB_, DN_, 0>), dim3(grid), dim3(kExpandThreads), lds, s, a); break; \
    case 2: hipLaunchKernelGGL((expand_kernel<DT_, VEC_, 2, TB_, DN_, 0>), dim3(grid), dim3(kExpandThreads), lds, s, a); break; \
    case 4: hipLaunchKernelGGL((expand_kernel<DT_, VEC_, 4, TB_, DN_, 0>), dim3(grid), dim3(kExpandThreads), lds, s, a); break; \
    default: hipLaunchKernelGGL((expand_kernel<DT_, VEC_, 8, 1, DN_, 0>), dim3(grid), dim3(kExpandThreads), lds, s, a); break; \
  }
#define LORA_EXPAND_TYPED(DN_)                                                                       \
  if (tb == 2) {                                                                                    \
    if (dtype == 0) {                                                                               \
      if (vec) { LORA_EXPAND_LAUNCH(0, true, 2, DN_) } else { LORA_EXPAND_LAUNCH(0, false, 2, DN_) } \
    } else {                                                                                        \
      if (vec) { LORA_EXPAND_LAUNCH(1, true, 2, DN_) } else { LORA_EXPAND_LAUNCH(1, false, 2, DN_) } \
    }                                                                                               \
  } else {                                                                                          \
    if (dtype == 0) {                                                                               \
      if (vec) { LORA_EXPAND_LAUNCH(0, true, 1, DN_) } else { LORA_EXPAND_LAUNCH(0, false, 1, DN_) } \
    } else {                                                                                        \
      if (vec) { LORA_EXPAND_LAUNCH(1, true, 1, DN_) } else { LORA_EXPAND_LAUNCH(1, false, 1, DN_) } \
    }                                                                                               \
  }
  if (seg.dense) {
    LORA_EXPAND_TYPED(true)
  } else {
    LORA_EXPAND_TYPED(false)
  }
#undef LORA_EXPAND_TYPED
#undef LORA_EXPAND_LAUNCH
  return hipGetLastError();
}

}  // namespace lora
