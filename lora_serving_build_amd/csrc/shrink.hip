// Shrink on segments (SGMV form): v[t, j] = sum_h x[t, h] * A_l[h, j].
//
// One workgroup of four waves owns a 64-token tile of one segment and a range
// of H (the whole of H unless the batch has too few tiles to fill the GPU).
// Wave w multiplies tokens 16w..16w+15 against all of r with 16x16x32 ops,
// accumulating the transposed product D[j][token] in fp32, so each lane ends
// with four consecutive j of one token.  H is walked in blocks of 128:
//  - x is private to a wave, so each lane loads its own operand straight into
//    registers (token m of the wave, 8 consecutive h per 32-wide k step: one
//    load instruction covers 16 rows x 64 contiguous bytes), one block ahead,
//    in two register sets that the loop alternates (no copy waits for a load);
//  - A_l is shared by the four waves: its block (r rows x 256 B, 16 lanes per
//    row) is loaded cooperatively one block ahead and written to a
//    double-buffered LDS tile (row pitch 288 B, see kSkPitch), so A_l is read
//    from L2 once per 64 tokens.
// At r = 33..64 from 4096 tokens and H = 2048 (TB = 2), tiles hold 128
// tokens: wave w takes tokens 32w..32w+31 as two blocks of 16, and each A
// operand read from LDS feeds both blocks' ops (half the A reads per x byte;
// three workgroups per CU for the registers).
// Loads are unconditional (addresses clamped into the chunk): values past the
// end of the chunk are zeroed where they are used, so the compiler can count
// the loads in flight exactly.  LDS holds only A and the tile table, which
// leaves room for four workgroups per CU.
//
// When H is split across workgroups (ks chunks), each chunk writes its fp32
// partial rows to the workspace (indexed by sorted position) and a second
// small kernel adds the ks partials in chunk order and writes v: the kernel
// boundary orders the two, and the sum order is fixed.
//
// The host picks ks from an upper bound on the tiles (T / 64 plus one partial
// tile per adapter), since it never sees the segments.  When the adapter pool
// is much larger than the number of segments in use, that bound is loose and
// the split leaves most of the GPU idle; every workgroup then recomputes ks
// from the true tile count (the same value in all of them), up to the number
// of chunks the workspace holds, and workgroup 0 leaves it in the workspace
// header for the reduce kernel.  With 128-token tiles the kernel always
// chooses ks itself, from the true tile count, by the CUs' share of the work
// (split_by_cu).
#include "lora_device.h"
#include "lora_kernels.h"
#include "tiles.h"

namespace lora {

namespace {

constexpr int kShrinkThreads = 256;
constexpr int kSkTile = 64;              // tokens per tile (4 waves x 16)
constexpr int kSkKB = kShrinkKStep;      // H elements per block
// Resident workgroups per CU the registers allow, by rank tiles (NJT) and
// 16-token blocks per wave (TB).
constexpr int shrink_wgs_per_cu(int njt, int tb) {
  return tb == 1 ? (njt <= 4 ? 4 : 2) : (njt <= 2 ? 4 : njt <= 4 ? 3 : 2);
}
// 16-bit elements per LDS row of A.  A 16-byte LDS read is served for 16
// lanes at a time, lanes 0-7 with 16-23 (and so on); here those are rows 0-7
// of the operand at two 16-byte columns.  A row stride that is an odd
// multiple of 8 dwords (mod 64 banks) puts those 16 pieces on distinct banks:
// 72 dwords.  Measured with SQ_LDS_BANK_CONFLICT on MI355X: 0 % of LDS cycles,
// against 34-39 % for a 68-dword stride.
constexpr int kSkPitch = kSkKB + 16;
constexpr int kSkChunks = kSkKB / 8;     // 16-byte pieces per row and block

struct ShrinkArgs {
  SegView seg;
  const uint16_t* x;
  int64_t ldx;
  const uint16_t* A;
  int32_t H;
  int32_t r;
  float* v;
  int64_t ldv;
  float* partial;  // [ks_cap][T][rp] when ks_cap > 1
  int32_t* ks_out; // workspace header: the ks used (when ks_cap > 1)
  int32_t ks;      // chunks chosen on the host
  int32_t ks_cap;  // chunks the workspace holds (ks when the choice is fixed)
  int32_t resident;  // workgroups resident at once
  int32_t kchunk;  // H elements per workgroup chunk (multiple of kSkKB)
  int32_t rp;      // padded rank of the partial rows (16 * NJT)
  int32_t min_seg_len;  // segments with fewer tokens are left to another kernel
  int32_t fixed;   // 1: the split is as set (an override), not re-planned
};

// H split for 128-token tiles.  The CUs stream their items concurrently, so
// a CU's time is about its share of the work: ceil(items / 256) items times
// the blocks of one plus about two blocks' worth per item (its set-up and its
// partial rows, as many bytes as one block of x).  Measured on MI355X, 8192 x
// 16384 at r = 64, one adapter: 4 chunks 62.3 us, 8 chunks 63.6, 5 chunks
// 83.8; over four segments of 1952-2288 tokens: 11 chunks 73.6, 4 chunks
// 97.6; 8192 x 4096: 3 chunks 28.3, 7 chunks 32.5; the 8192-token layer (71
// tiles): 3 chunks 48.2, 7 chunks 50.6.  Splits that give a CU more items
// than it holds workgroups run far slower (their items wait for a second
// round) and are not taken, except one chunk.  Among the rest, the least
// time, ties to fewer chunks.
// (32-bit divisions, two per candidate: in the kernel every workgroup runs
// this before its first item, and 64-bit divisions are long sequences there.)
__host__ __device__ inline int split_by_cu(int tiles, int H, int ks_max, int per_cu, int* chunk_out) {
  int best = 1;
  int64_t best_cost = -1;
  int best_chunk = (((H - 1) >> 7) + 1) << 7;
  for (int k = 1; k <= ks_max; ++k) {
    const int ch = ((((H - 1) / k) >> 7) + 1) << 7;  // ceil(H / k) rounded up to a block
    if ((H - 1) / ch + 1 != k) continue;               // this chunk size makes fewer chunks: counted there
    const int64_t per = ((int64_t)tiles * k + 255) >> 8;
    if (per > per_cu && k > 1) continue;
    const int64_t cost = per * ((ch >> 7) + 2);
    if (best_cost < 0 || cost < best_cost) {
      best_cost = cost;
      best = k;
      best_chunk = ch;
    }
  }
  *chunk_out = best_chunk;
  return best;
}

template <int NJT>
struct ShrinkLds {
  static constexpr size_t a_bytes = (size_t)2 * 16 * NJT * kSkPitch * 2;
  // A blocks, then the tile table and scan scratch
  static size_t bytes(int L) { return a_bytes + 4 * ((size_t)tile_table_ints(L) + 8); }
};

// Stores four consecutive j values of one row (j0 = first), clipped at r.
template <bool VEC>
__device__ __forceinline__ void store4(float* p, int j0, int r, f32x4 val) {
  if (VEC && j0 + 4 <= r) {
    *reinterpret_cast<f32x4*>(p) = val;
    return;
  }
  if (j0 + 0 < r) p[0] = val.x;
  if (j0 + 1 < r) p[1] = val.y;
  if (j0 + 2 < r) p[2] = val.z;
  if (j0 + 3 < r) p[3] = val.w;
}

// NJT = 16-row tiles of r (r <= 16 * NJT).  VEC: 16-byte aligned rows with H
// and ldx multiples of 8 (otherwise element-wise loads).
// DENSE: one adapter (0) for every token, token index = position (the
// single-adapter form): no metadata is read.
template <int DT, bool VEC, int NJT, bool DENSE, int TB>
__global__ __launch_bounds__(kShrinkThreads, shrink_wgs_per_cu(NJT, TB)) void shrink_kernel(ShrinkArgs a) {
  constexpr int RP = 16 * NJT;
  constexpr int TT = kSkTile * TB;  // tokens per tile
  constexpr int AL = RP * kSkChunks / kShrinkThreads;  // A pieces per thread per block (NJT)
  constexpr int KS = kSkKB / 32;                        // 32-wide k steps per block
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* s_a = reinterpret_cast<uint16_t*>(smem);    // [2][RP * kSkPitch]
  int32_t* s_table = reinterpret_cast<int32_t*>(smem + ShrinkLds<NJT>::a_bytes);
  int32_t* s_scan = s_table + tile_table_ints(a.seg.L);

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int m = lane & 15;  // token column of D / row of A inside a 16-row tile
  const int g = lane >> 4;  // lane group: which 8 of the 32 elements of an op
  // Cooperative A layout: piece c = tid + 256 i, row c / 16, 16-byte column c % 16.
  const int lrow = tid >> 4;
  const int lcol = (tid & 15) * 8;

  const TileTable table =
      build_tile_table<kShrinkThreads, DENSE>(a.seg, TT, a.r, s_table, s_scan, a.min_seg_len);
  const int tiles = table.tiles;
  int ks = a.ks, kchunk = a.kchunk;
  if constexpr (TB == 2) {
    // The split from the true tile count, by the CUs' share of the blocks
    // (the same in every workgroup; within what the workspace holds).
    if (!a.fixed && a.ks_cap > 1 && tiles > 0) {
      ks = split_by_cu(tiles, a.H, a.ks_cap, a.resident >> 8, &kchunk);
    }
  } else if (a.ks_cap > ks && tiles > 0 && 2 * tiles * ks <= a.resident) {
    // Under half the resident workgroups busy: the host's bound was loose.
    int k = (a.resident + tiles - 1) / tiles;
    if (tiles * k - a.resident > a.resident / 50) k = a.resident / tiles;
    k = k < ks ? ks : (k > a.ks_cap ? a.ks_cap : k);
    kchunk = ((a.H + k - 1) / k + kSkKB - 1) / kSkKB * kSkKB;
    ks = (a.H + kchunk - 1) / kchunk;
  }
  if (a.ks_out && blockIdx.x == 0 && tid == 0) *a.ks_out = ks;
  const int n_items = tiles * ks;
  const int grid = gridDim.x;

  for (int item = xcd_first_item(blockIdx.x, grid, n_items); item < n_items; item += grid) {
    // Consecutive items share the chunk of H and walk the tiles of a segment,
    // so neighbouring workgroups of an XCD read the same A_l block.
    const int ksi = item / tiles;
    const int tile = item - ksi * tiles;
    int p0 = 0, p_end = 0, l = 0;
    int rank_l = 0;
    const bool ok = tile_range_lds(table, a.seg.T, a.seg.L, TT, tile, &p0, &p_end, &l, &rank_l);
    const int kbeg = ksi * kchunk;
    const int kend = min(a.H, kbeg + kchunk);
    // Wave w takes tokens [16 TB w, 16 TB (w + 1)) of the tile, block b the
    // 16 from 16 (TB w + b).
    int pos[TB], t[TB];
    bool tok_ok[TB], blk_live[TB];
#pragma unroll
    for (int b = 0; b < TB; ++b) {
      pos[b] = p0 + 16 * (TB * wave + b) + m;
      int tb = (ok && pos[b] < p_end) ? (DENSE ? pos[b] : a.seg.sorted_token[pos[b]]) : -1;
      t[b] = (tb >= 0 && tb < a.seg.T) ? tb : -1;
      tok_ok[b] = t[b] >= 0;
      blk_live[b] = ok && p0 + 16 * (TB * wave + b) < p_end;
    }
    const bool wave_live = blk_live[0];
    // A missing token reads row 0 (its output column is dropped).  Rows
    // at or beyond the adapter's live rank (and the padding of r to 16 NJT)
    // read row 0 -- lines this block loads anyway, so they cost no HBM
    // traffic -- and are zeroed when written to LDS.  (Their matrix ops still
    // run on the zeros: skipping them cost 7% on full-rank batches.)
    const uint16_t* xrow[TB];
#pragma unroll
    for (int b = 0; b < TB; ++b) xrow[b] = a.x + (int64_t)(tok_ok[b] ? t[b] : 0) * a.ldx;
    const uint16_t* Al = a.A + (int64_t)l * a.r * a.H;
    const uint16_t* asrc[AL];
#pragma unroll
    for (int i = 0; i < AL; ++i) {
      const int j = lrow + 16 * i;
      asrc[i] = Al + (int64_t)(j < rank_l ? j : 0) * a.H;
    }

    u32x4 ra[AL];
    auto gload_a = [&](int kb) {
      const int off = kb + lcol;
#pragma unroll
      for (int i = 0; i < AL; ++i) {
        if constexpr (VEC) {
          const int oc = off < kend ? off : kend - 8;  // kend is a multiple of 8 here
          ra[i] = *reinterpret_cast<const u32x4*>(asrc[i] + oc);
        } else {
          ra[i] = ok ? load8_16<false>(asrc[i] + off, kend - off) : u32x4{0u, 0u, 0u, 0u};
        }
      }
    };
    // Zeroes the pieces past the chunk when the block goes to LDS.
    auto swrite_a = [&](int buf, int kb) {
      const int off = kb + lcol;
#pragma unroll
      for (int i = 0; i < AL; ++i) {
        u32x4 w = ra[i];
        if (!(ok && off < kend) || lrow + 16 * i >= rank_l) w = u32x4{0u, 0u, 0u, 0u};
        *reinterpret_cast<u32x4*>(&s_a[(buf * RP + lrow + 16 * i) * kSkPitch + lcol]) = w;
      }
    };
    auto gload_x = [&](int kb, u32x4 (*xr)[KS]) {
#pragma unroll
      for (int b = 0; b < TB; ++b) {
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
          const int off = kb + 32 * kk + 8 * g;
          if constexpr (VEC) {
            const int oc = off < kend ? off : kend - 8;
            xr[b][kk] = *reinterpret_cast<const u32x4*>(xrow[b] + oc);
          } else {
            xr[b][kk] = tok_ok[b] ? load8_16<false>(xrow[b] + off, kend - off) : u32x4{0u, 0u, 0u, 0u};
          }
        }
      }
    };

    f32x4 acc[TB][NJT];
#pragma unroll
    for (int b = 0; b < TB; ++b)
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt) acc[b][jt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int nblk = kend > kbeg ? (kend - kbeg + kSkKB - 1) / kSkKB : 0;
    // The blocks of the chunk are walked in a rotated order that starts at
    // block (tile mod nblk).  The concurrent items otherwise read x at the
    // same few offsets inside their rows, and when the row pitch is a
    // multiple of the HBM interleave those offsets fall on the same few
    // channels: measured on MI355X (8192 tokens x 8192, r = 64), chunks that
    // start at multiples of 4 KB in the 16 KB rows (4 or 8 chunks) ran
    // 15-20% slower than 3, 5 or 7 chunks.  Block s of the walk is block
    // (s + rot) mod nblk; positions past the walk map to kend (clamped loads
    // whose data is dropped).
    const int rot = nblk > 0 ? tile % nblk : 0;
    auto kb_of = [&](int step) {
      if (step >= nblk) return kend;
      const int blk = step + rot < nblk ? step + rot : step + rot - nblk;
      return kbeg + blk * kSkKB;
    };

    // One block: the next block's A and x go out first, then the ops of this
    // one from LDS (A) and registers (x).
    auto block = [&](int b, u32x4 (*xcur)[KS], u32x4 (*xnext)[KS]) {
      const int buf = b & 1;
      const int kb = kb_of(b);
      const bool has_next = b + 1 < nblk;
      // Issued on every block (the last one reads clamped addresses and drops
      // the data): a load that only some paths issue would make the compiler
      // assume none and wait for everything before the ops below.
      gload_a(kb_of(b + 1));
      gload_x(kb_of(b + 1), xnext);
      __builtin_amdgcn_sched_barrier(0);
      if (wave_live) {
        const uint16_t* as = &s_a[(buf * RP + m) * kSkPitch + 8 * g];
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) {
          // Elements past the chunk (last block only) are zero.
          const bool in = kb + 32 * kk + 8 * g < kend;
#pragma unroll
          for (int jt = 0; jt < NJT; ++jt) {
            // One A operand from LDS feeds the ops of all TB token blocks.
            const u32x4 aop = *reinterpret_cast<const u32x4*>(as + jt * 16 * kSkPitch + 32 * kk);
#pragma unroll
            for (int bb = 0; bb < TB; ++bb) {
              const u32x4 xop = in ? xcur[bb][kk] : u32x4{0u, 0u, 0u, 0u};
              acc[bb][jt] = mfma16x16x32<DT>(aop, xop, acc[bb][jt]);
            }
          }
        }
      }
      if (has_next) swrite_a(buf ^ 1, kb_of(b + 1));
      __syncthreads();
    };

    u32x4 xa[TB][KS], xb[TB][KS];
    if (nblk > 0) {
      gload_a(kb_of(0));
      gload_x(kb_of(0), xa);
      swrite_a(0, kb_of(0));
    }
    __syncthreads();
    for (int b = 0; b < nblk; b += 2) {
      block(b, xa, xb);
      if (b + 1 < nblk) block(b + 1, xb, xa);
    }

    // Lane (m, g) holds D[j = 16 jt + 4 g + e][token 16 (TB wave + b) + m].
#pragma unroll
    for (int bb = 0; bb < TB; ++bb) {
      if (!(blk_live[bb] && tok_ok[bb])) continue;
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt) {
        const int j0 = jt * 16 + 4 * g;
        if (ks == 1) {
          store4<VEC>(a.v + (int64_t)t[bb] * a.ldv + j0, j0, a.r, acc[bb][jt]);
        } else {
          float* part = a.partial + ((int64_t)ksi * a.seg.T + pos[bb]) * a.rp + j0;
          *reinterpret_cast<f32x4*>(part) = acc[bb][jt];
        }
      }
    }
  }
}

// 16-token groups with the H split inside the workgroup (r <= 32).  Item =
// one 16-token tile of a segment; its eight waves take the 256-element blocks
// of H in turn (wave w: blocks w, w + 8, ...), each streaming its blocks of x
// and of the adapter's A rows straight into matrix-op operands (no wave
// shares a weight block, so nothing is staged in LDS), one block ahead.  The
// eight partial sums meet in LDS and are added in wave order, so v is written
// in the same launch: no partial rows, no workspace, no reduce launch.  For
// mid-size batches, where the tile kernel's H split pays a second launch and a
// chain of memory trips per item.
constexpr int kGrpThreads = 512;
constexpr int kGrpWaves = kGrpThreads / kWave;
constexpr int kGrpKB = 256;  // H elements per wave block

template <int NJT>
struct GroupLds {
  static constexpr size_t red_bytes = (size_t)kGrpWaves * NJT * kWave * 16;
  // the partial sums, then the tile table and the scan's scratch (one int per
  // wave and the total)
  static size_t bytes(int L) { return red_bytes + 4 * ((size_t)tile_table_ints(L) + kGrpWaves + 1); }
};

template <int DT, bool VEC, int NJT, bool DENSE>
__global__ __launch_bounds__(kGrpThreads) void shrink_group_kernel(ShrinkArgs a) {
  constexpr int KS = kGrpKB / 32;  // 32-wide k steps per block
  extern __shared__ __align__(16) unsigned char smem[];
  f32x4* s_red = reinterpret_cast<f32x4*>(smem);  // [wave][NJT][lane]
  int32_t* s_table = reinterpret_cast<int32_t*>(smem + GroupLds<NJT>::red_bytes);
  int32_t* s_scan = s_table + tile_table_ints(a.seg.L);

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int m = lane & 15;  // token of the tile / row of A inside a 16-row tile
  const int g = lane >> 4;  // which 8 of the 32 elements of an op

  const TileTable table =
      build_tile_table<kGrpThreads, DENSE>(a.seg, 16, a.r, s_table, s_scan, a.min_seg_len);
  const int tiles = table.tiles;
  const int grid = gridDim.x;
  const int nb = (a.H + kGrpKB - 1) / kGrpKB;
  const int nbw = wave < nb ? (nb - 1 - wave) / kGrpWaves + 1 : 0;  // blocks of this wave

  for (int item = xcd_first_item(blockIdx.x, grid, tiles); item < tiles; item += grid) {
    int p0 = 0, p_end = 0, l = 0, rank_l = 0;
    const bool ok = tile_range_lds(table, a.seg.T, a.seg.L, 16, item, &p0, &p_end, &l, &rank_l);
    const int pos = p0 + m;
    int t = (ok && pos < p_end) ? (DENSE ? pos : a.seg.sorted_token[pos]) : -1;
    t = (t >= 0 && t < a.seg.T) ? t : -1;
    const bool tok_ok = t >= 0;
    // A missing token reads row 0 and a rank row at or past the live rank
    // reads the adapter's row 0; their outputs are dropped or zeroed below.
    const uint16_t* xrow = a.x + (int64_t)(tok_ok ? t : 0) * a.ldx;
    const uint16_t* Al = a.A + (int64_t)(ok ? l : 0) * a.r * a.H;
    const uint16_t* arow[NJT];
    bool row_ok[NJT];
#pragma unroll
    for (int jt = 0; jt < NJT; ++jt) {
      const int j = 16 * jt + m;
      row_ok[jt] = ok && j < rank_l;
      arow[jt] = Al + (int64_t)(row_ok[jt] ? j : 0) * a.H;
    }
    // Block i of this wave (i may be past its last block: the prefetch after
    // the last one reads clamped addresses and is dropped).
    auto gload = [&](int i, u32x4* xr, u32x4 (*ar)[KS]) {
      const int kb = (wave + kGrpWaves * i) * kGrpKB;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        const int off = kb + 32 * kk + 8 * g;
        if constexpr (VEC) {
          const int oc = off < a.H ? off : a.H - 8;  // H is a multiple of 8 here
          xr[kk] = *reinterpret_cast<const u32x4*>(xrow + oc);
#pragma unroll
          for (int jt = 0; jt < NJT; ++jt) ar[jt][kk] = *reinterpret_cast<const u32x4*>(arow[jt] + oc);
        } else {
          xr[kk] = tok_ok ? load8_16<false>(xrow + off, a.H - off) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
          for (int jt = 0; jt < NJT; ++jt)
            ar[jt][kk] = row_ok[jt] ? load8_16<false>(arow[jt] + off, a.H - off) : u32x4{0u, 0u, 0u, 0u};
        }
      }
    };
    f32x4 acc[NJT];
#pragma unroll
    for (int jt = 0; jt < NJT; ++jt) acc[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](int i, const u32x4* xr, const u32x4 (*ar)[KS]) {
      const int kb = (wave + kGrpWaves * i) * kGrpKB;
#pragma unroll
      for (int kk = 0; kk < KS; ++kk) {
        // Elements past H (the last block) are zero.
        const bool in = kb + 32 * kk + 8 * g < a.H;
        const u32x4 xop = in ? xr[kk] : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int jt = 0; jt < NJT; ++jt) acc[jt] = mfma16x16x32<DT>(ar[jt][kk], xop, acc[jt]);
      }
    };
    if (nbw > 0) {
      u32x4 x0[KS], x1[KS], a0[NJT][KS], a1[NJT][KS];
      gload(0, x0, a0);
      for (int i = 0; i < nbw; i += 2) {
        gload(i + 1, x1, a1);
        compute(i, x0, a0);
        if (i + 1 < nbw) {
          gload(i + 2, x0, a0);
          compute(i + 1, x1, a1);
        }
      }
    }
    // Lane (m, g) holds D[j = 16 jt + 4 g + e][token m] of this wave's blocks.
#pragma unroll
    for (int jt = 0; jt < NJT; ++jt) s_red[(wave * NJT + jt) * kWave + lane] = acc[jt];
    __syncthreads();
    if (wave < NJT && tok_ok) {
      const int jt = wave;
      f32x4 sum = s_red[jt * kWave + lane];
#pragma unroll
      for (int w = 1; w < kGrpWaves; ++w) {
        const f32x4 o = s_red[(w * NJT + jt) * kWave + lane];
        sum.x += o.x;
        sum.y += o.y;
        sum.z += o.z;
        sum.w += o.w;
      }
      const int j0 = 16 * jt + 4 * g;
      if (j0 + 0 >= rank_l) sum.x = 0.f;
      if (j0 + 1 >= rank_l) sum.y = 0.f;
      if (j0 + 2 >= rank_l) sum.z = 0.f;
      if (j0 + 3 >= rank_l) sum.w = 0.f;
      store4<VEC>(a.v + (int64_t)t * a.ldv + j0, j0, a.r, sum);
    }
    __syncthreads();  // the partial sums' rows are reused by the next item
  }
}

// v[t, :r] = sum over the ks chunks of the partial rows, in chunk order (ks
// as the shrink kernel left it in the workspace header, or ks_fixed when the
// kernel cannot have changed the host's split: then the partial rows' loads
// need not wait for the header; nothing to do when the shrink kernel wrote v
// itself).
// Every load of a row -- the active count, its token, eight partial rows at a
// time -- goes out before any of them is checked, so a reduction of up to
// eight chunks is one memory trip; positions past the active tokens (whose
// partial rows were never written) and ranks past r are dropped at the store.
template <bool VEC>
__global__ __launch_bounds__(256) void shrink_reduce_kernel(SegView seg, const float* partial,
                                                            const int32_t* ks_in, int32_t ks_fixed,
                                                            int32_t ks_cap, int32_t rp, int32_t r, float* v,
                                                            int64_t ldv) {
  int ks = ks_fixed > 0 ? ks_fixed : *ks_in;
  ks = ks > ks_cap ? ks_cap : ks;
  if (ks <= 1) return;
  const int per_row = rp / 4;
  const int64_t n = (int64_t)seg.T * per_row;
  for (int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; o < n;
       o += (int64_t)gridDim.x * blockDim.x) {
    const int p = (int)(o / per_row);
    const int j0 = (int)(o - (int64_t)p * per_row) * 4;
    int ta = seg.dense ? seg.T : seg.counts[1];
    const int t = seg.dense ? p : seg.sorted_token[p];
    f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int q0 = 0; q0 < ks; q0 += 8) {
      f32x4 part[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int q = q0 + u < ks ? q0 + u : ks - 1;
        part[u] = *reinterpret_cast<const f32x4*>(partial + ((int64_t)q * seg.T + p) * rp + j0);
      }
#pragma unroll
      for (int u = 0; u < 8; ++u)
        if (q0 + u < ks) sum += part[u];
    }
    ta = ta < 0 ? 0 : (ta > seg.T ? seg.T : ta);
    if (p < ta && j0 < r && t >= 0 && t < seg.T) store4<VEC>(v + (int64_t)t * ldv + j0, j0, r, sum);
  }
}

size_t shrink_lds_bytes(int njt, int L) {
  return njt == 1 ? ShrinkLds<1>::bytes(L)
         : njt == 2 ? ShrinkLds<2>::bytes(L)
         : njt == 4 ? ShrinkLds<4>::bytes(L) : ShrinkLds<8>::bytes(L);
}

template <int DT, bool VEC, bool DENSE>
hipError_t launch_typed(const ShrinkArgs& args, int njt, int tb, int grid, hipStream_t s) {
  const size_t lds = shrink_lds_bytes(njt, args.seg.L);
  switch (njt) {
    case 1:
      hipLaunchKernelGGL((shrink_kernel<DT, VEC, 1, DENSE, 1>), dim3(grid), dim3(kShrinkThreads), lds, s, args);
      break;
    case 2:
      hipLaunchKernelGGL((shrink_kernel<DT, VEC, 2, DENSE, 1>), dim3(grid), dim3(kShrinkThreads), lds, s, args);
      break;
    case 4:
      if (tb == 2)
        hipLaunchKernelGGL((shrink_kernel<DT, VEC, 4, DENSE, 2>), dim3(grid), dim3(kShrinkThreads), lds, s, args);
      else
        hipLaunchKernelGGL((shrink_kernel<DT, VEC, 4, DENSE, 1>), dim3(grid), dim3(kShrinkThreads), lds, s, args);
      break;
    default:
      hipLaunchKernelGGL((shrink_kernel<DT, VEC, 8, DENSE, 1>), dim3(grid), dim3(kShrinkThreads), lds, s, args);
      break;
  }
  return hipGetLastError();
}

size_t group_lds_bytes(int njt, int L) { return njt == 1 ? GroupLds<1>::bytes(L) : GroupLds<2>::bytes(L); }

template <int DT, bool VEC, bool DENSE>
hipError_t launch_group_typed(const ShrinkArgs& args, int njt, int grid, hipStream_t s) {
  const size_t lds = group_lds_bytes(njt, args.seg.L);
  if (njt == 1)
    hipLaunchKernelGGL((shrink_group_kernel<DT, VEC, 1, DENSE>), dim3(grid), dim3(kGrpThreads), lds, s, args);
  else
    hipLaunchKernelGGL((shrink_group_kernel<DT, VEC, 2, DENSE>), dim3(grid), dim3(kGrpThreads), lds, s, args);
  return hipGetLastError();
}

template <int DT, bool VEC>
hipError_t launch_group(const ShrinkArgs& args, int njt, int grid, hipStream_t s) {
  return args.seg.dense ? launch_group_typed<DT, VEC, true>(args, njt, grid, s)
                        : launch_group_typed<DT, VEC, false>(args, njt, grid, s);
}

template <int DT, bool VEC>
hipError_t launch_dense(const ShrinkArgs& args, int njt, int tb, int grid, hipStream_t s) {
  return args.seg.dense ? launch_typed<DT, VEC, true>(args, njt, tb, grid, s)
                        : launch_typed<DT, VEC, false>(args, njt, tb, grid, s);
}

}  // namespace

ShrinkPlan plan_shrink(int32_t T, int32_t L, int32_t H, int32_t r, size_t ws_limit) {
  ShrinkPlan p{};
  const int njt0 = (r + 15) / 16;
  p.jtw = njt0 <= 1 ? 1 : njt0 <= 2 ? 2 : njt0 <= 4 ? 4 : 8;  // rank tiles (template)
  p.rp = 16 * p.jtw;
  // 16-token blocks per wave: two at r = 33..64 from 4096 tokens and H =
  // 2048 up (tiles of 128 tokens, each A operand read from LDS feeding two
  // matrix ops: half the A traffic and LDS reads per x byte).  Measured on
  // MI355X, each call alone (64-token tiles -> 128-token tiles at their best
  // split): the 8192-token layer 50.5 -> 48.2 us, 8192 x 16384 one adapter
  // 74.9 -> 62.3, over four segments 81.8 -> 73.6, 8192 x 4096 32.7 -> 28.3;
  // but 512 x 4096 12.4 -> 14.6 (fewer, longer items) and 8192 x 1024
  // 17.0 -> 17.7 (two chunks at most).
  // 16-token groups with the H split inside the workgroup (shrink_group_kernel)
  // at r <= 32, when the groups fit one round of workgroups (one per CU) and
  // each moves at most 128 KB of x and A (H (16 + r) <= 65536 elements).  A
  // CU sustains only so many lines in flight, so a group's bytes set its
  // time; past that size the tile kernel's H split over every CU wins.
  // Measured on MI355X (fp16, 4 adapters, each call alone, tiles -> groups):
  // r = 16, H = 1024: 1024 tokens 10.5 -> 6.3 us, 2048 11.1 -> 6.6; H = 2048:
  // 1024 tokens 11.1 -> 8.6, 2048 11.5 -> 9.0; r = 32, H = 1024: 2048 tokens
  // 11.4 -> 7.8; but r = 32, H = 2048: 4096 tokens 13.6 -> 17.5, and the
  // 2048-token prefill at H = 4096, r = 16: 13.0 -> 16.3.
  {
    const int64_t g_tiles = max_token_tiles(T, L, 16);
    const bool fit = p.jtw <= 2 && group_lds_bytes(p.jtw, L) <= 64 * 1024 && g_tiles < INT32_MAX;
    const bool want = tuning().shrink_group == 1 ||
                      (tuning().shrink_group == 0 && g_tiles <= 256 && (int64_t)H * (16 + r) <= 65536);
    if (fit && want) {
      p.group = 1;
      p.tb = 1;
      p.ksplit = 1;
      p.ks_cap = 1;
      p.kchunk = (int32_t)H;
      p.max_tiles = (int32_t)g_tiles;
      p.resident = 256;  // one eight-wave workgroup per CU
      p.partial_bytes = 0;
      int64_t grid = g_tiles < 256 ? g_tiles : 256;
      grid = (grid + 7) / 8 * 8;
      p.grid = (int32_t)(grid < 8 ? 8 : grid);
      return p;
    }
  }
  p.tb = (p.jtw == 4 && ((tuning().shrink_tb == 0 && T >= 4096 && H >= 2048) || tuning().shrink_tb == 2)) ? 2 : 1;
  const int64_t tt = (int64_t)kSkTile * p.tb;
  const int64_t tiles = max_token_tiles(T, L, tt);
  p.max_tiles = (int32_t)tiles;
  // Persistent workgroups: as many as are resident at once (LDS and register
  // bound: four per CU up to r = 64 with 64-token tiles, three with 128-token
  // tiles, two at r = 128).
  int64_t per_cu = (int64_t)(160 * 1024 / shrink_lds_bytes(p.jtw, L));
  const int64_t reg_cu = shrink_wgs_per_cu(p.jtw, p.tb);
  per_cu = per_cu < 1 ? 1 : (per_cu > reg_cu ? reg_cu : per_cu);
  const int64_t resident = 256 * per_cu;
  p.resident = (int32_t)resident;
  // Split H across workgroups so that the items fill one round of resident
  // workgroups, with at least four blocks per chunk: the extra partial-row
  // traffic costs less than idle CUs.  Rounding the chunk count up leaves
  // some items for a second round.  A few of them cost little, but more
  // than 2% of a round leave most CUs idle while they run, and then the
  // count is rounded down.  Measured on MI355X (upper-bound tile counts):
  //   8192-token layer, 192 tiles: 6 chunks 56.5 us, 5 chunks 52.5 us;
  //   8192 x 4096 at r = 128, 132 tiles (512 resident): 4 -> 46 us, 3 -> 40 us;
  //   16384 x 4096 at r = 16, 260 tiles: 4 -> 37.8 us, 3 -> 40.5 us.
  // The kernel applies the same rule to the true tile count (see the kernel).
  int64_t ks_max = H / (4 * kSkKB);
  if (ks_max < 1) ks_max = 1;
  auto split_for = [&](int64_t n) {
    int64_t ks = 1;
    if (n > 0 && n < resident) {
      ks = (resident + n - 1) / n;
      if (n * ks - resident > resident / 50) ks = resident / n;
    }
    ks = ks > ks_max ? ks_max : (ks < 1 ? 1 : ks);
    const int64_t chunk = ((H + ks - 1) / ks + kSkKB - 1) / kSkKB * kSkKB;
    return (H + chunk - 1) / chunk;
  };
  int64_t ks = split_for(tiles);
  // With 64-token tiles the kernel may raise the split up to what the fewest
  // tiles T tokens can make (all of them in whole tiles) would take: about
  // one round of resident workgroups' partial rows, whatever T.
  int64_t ks_cap = split_for(T > 0 ? ((int64_t)T + tt - 1) / tt : 0);
  const int64_t row_bytes = (int64_t)T * p.rp * 4;
  if (p.tb == 2) {
    // By the CUs' share of the blocks (see split_by_cu); every split it can
    // take has tiles * ks <= per_cu * 256, so the fewest tiles bound it.  A
    // caller's workspace limit bounds it too.
    int64_t lim = ks_max;
    if (row_bytes > 0 && ws_limit > kShrinkWsHeader) {
      const int64_t fit = (int64_t)((ws_limit - kShrinkWsHeader) / (size_t)row_bytes);
      lim = fit < lim ? (fit < 1 ? 1 : fit) : lim;
    }
    int ch = 0;
    ks = split_by_cu((int)(tiles < INT32_MAX ? tiles : INT32_MAX), H, (int)lim, (int)per_cu, &ch);
    const int64_t n_min = T > 0 ? ((int64_t)T + tt - 1) / tt : 1;
    ks_cap = per_cu * 256 / n_min;
    ks_cap = ks_cap > lim ? lim : (ks_cap < 1 ? 1 : ks_cap);
    if (ks_cap < ks) ks_cap = ks;
  }
  p.fixed = 0;
  if (tuning().shrink_ksplit > 0) {
    p.fixed = 1;
    const int64_t want = tuning().shrink_ksplit;
    const int64_t chunk = ((H + want - 1) / want + kSkKB - 1) / kSkKB * kSkKB;
    ks = (H + chunk - 1) / chunk;
    ks_cap = ks;  // a fixed split, as set
  }
  if (ks_cap > ks && row_bytes > 0 && ws_limit > kShrinkWsHeader) {
    const int64_t fit = (int64_t)((ws_limit - kShrinkWsHeader) / (size_t)row_bytes);
    if (ks_cap > fit) ks_cap = fit;
  }
  if (ks_cap < ks) ks_cap = ks;
  p.ksplit = (int32_t)ks;
  p.ks_cap = (int32_t)ks_cap;
  p.kchunk = (int32_t)(((H + ks - 1) / ks + kSkKB - 1) / kSkKB * kSkKB);
  p.partial_bytes = ks_cap > 1 ? kShrinkWsHeader + (size_t)(ks_cap * row_bytes) : 0;
  // Every resident workgroup is launched when the kernel may change the split.
  const int64_t items = (ks_cap > ks || (p.tb == 2 && !p.fixed && ks_cap > 1)) ? resident : tiles * ks;
  int64_t grid = items < resident ? items : resident;
  grid = (grid + 7) / 8 * 8;
  if (grid < 8) grid = 8;
  p.grid = (int32_t)grid;
  return p;
}

hipError_t launch_shrink(const SegView& seg, const uint16_t* x, int64_t ldx, const uint16_t* A,
                         int32_t H, int32_t r, float* v, int64_t ldv, void* workspace,
                         const ShrinkPlan& plan, int dtype, bool vec, hipStream_t s, int min_seg_len) {
  ShrinkArgs a{};
  a.min_seg_len = min_seg_len > 1 ? min_seg_len : 1;
  a.seg = seg;
  a.x = x;
  a.ldx = ldx;
  a.A = A;
  a.H = H;
  a.r = r;
  a.v = v;
  a.ldv = ldv;
  const bool split = plan.ks_cap > 1;
  a.partial = split ? reinterpret_cast<float*>(static_cast<char*>(workspace) + kShrinkWsHeader) : nullptr;
  a.ks_out = split ? static_cast<int32_t*>(workspace) : nullptr;
  a.ks = plan.ksplit;
  a.ks_cap = plan.ks_cap;
  a.resident = plan.resident;
  a.kchunk = plan.kchunk;
  a.rp = plan.rp;
  a.fixed = plan.fixed;
  if (plan.group) {
    a.partial = nullptr;
    a.ks_out = nullptr;
    if (dtype == 0)
      return vec ? launch_group<0, true>(a, plan.jtw, plan.grid, s) : launch_group<0, false>(a, plan.jtw, plan.grid, s);
    return vec ? launch_group<1, true>(a, plan.jtw, plan.grid, s) : launch_group<1, false>(a, plan.jtw, plan.grid, s);
  }
  hipError_t e;
  if (dtype == 0)
    e = vec ? launch_dense<0, true>(a, plan.jtw, plan.tb, plan.grid, s)
            : launch_dense<0, false>(a, plan.jtw, plan.tb, plan.grid, s);
  else
    e = vec ? launch_dense<1, true>(a, plan.jtw, plan.tb, plan.grid, s)
            : launch_dense<1, false>(a, plan.jtw, plan.tb, plan.grid, s);
  if (e != hipSuccess || !split) return e;
  int64_t blocks = ((int64_t)seg.T * (plan.rp / 4) + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  if (blocks < 1) blocks = 1;
  // The split is known here only when the kernel cannot change it: with
  // 64-token tiles when the workspace holds no more chunks than the host's
  // split, with 128-token tiles (re-planned from the true tile count in
  // every call) only when an override fixes it or nothing is split.
  const bool kernel_may_change = plan.tb == 2 ? (!plan.fixed && plan.ks_cap > 1) : plan.ks_cap > plan.ksplit;
  const int32_t ks_fixed = kernel_may_change ? 0 : plan.ksplit;
  if (vec)
    hipLaunchKernelGGL((shrink_reduce_kernel<true>), dim3((unsigned)blocks), dim3(256), 0, s, seg,
                       a.partial, a.ks_out, ks_fixed, plan.ks_cap, plan.rp, r, v, ldv);
  else
    hipLaunchKernelGGL((shrink_reduce_kernel<false>), dim3((unsigned)blocks), dim3(256), 0, s, seg,
                       a.partial, a.ks_out, ks_fixed, plan.ks_cap, plan.rp, r, v, ldv);
  return hipGetLastError();
}

}  // namespace lora
