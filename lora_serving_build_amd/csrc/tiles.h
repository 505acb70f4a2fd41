// Token tiles over segments, shared by the segment (SGMV) kernels.
//
// A segment of len tokens is cut into ceil(len / tile_tokens) token tiles.
// Each workgroup copies the segment metadata into an LDS table, rebuilds the
// prefix of tile counts over the S segments there (S <= L <= 2048: a few KB
// read from L2) and maps a tile index to its segment with a binary search.
// The host never learns S or the segment lengths, so launch geometry stays
// independent of the data.
#pragma once

#include "lora_device.h"
#include "lora_kernels.h"

namespace lora {

// Segment that owns token tile `tile` (tile < tile_start[S]).
__device__ __forceinline__ int tile_segment(const int32_t* tile_start, int S, int tile) {
  int lo = 0, hi = S - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (tile_start[mid] <= tile)
      lo = mid;
    else
      hi = mid - 1;
  }
  return lo;
}

// LDS copy of everything a tile lookup needs, so that mapping a work item to
// its tokens costs no global round trip: tile_start[0..S], seg_start[0..S],
// seg_lora[0..S) and the live ranks (r when the metadata gives none).  Each
// array has room for L + 1 ints.  The ranks are per adapter (rank[0..L)) for
// pools of up to kEagerTable adapters, where every array is copied whole in
// one round of loads; for larger pools only the S segments in use are
// copied, and the ranks are per segment (rank[0..S)).
struct TileTable {
  int32_t* tile_start;
  int32_t* seg_start;
  int32_t* seg_lora;
  int32_t* rank;
  int S;
  int tiles;
  bool rank_by_seg;
};

// Pools up to this many adapters copy their whole metadata at once.
constexpr int kEagerTable = 256;

// Tiles of tile_tokens tokens that T tokens over at most L segments can make:
// one partial tile per segment at most.
__host__ __device__ inline int64_t max_token_tiles(int64_t T, int64_t L, int64_t tile_tokens) {
  return T > 0 ? (T + tile_tokens - 1) / tile_tokens + (L < T ? L : T) : 0;
}

// LDS ints a TileTable of L adapters occupies.
__host__ __device__ constexpr int64_t tile_table_ints(int64_t L) { return 4 * (L + 1); }

// Fills a TileTable from the metadata (S clamped to [0, L]).  DENSE: the
// single-adapter form, one segment of all T tokens on adapter 0 at its full
// rank, written without reading any metadata.
// Every thread of the block must call it.
template <int NT, bool DENSE = false>
__device__ TileTable build_tile_table(const SegView& seg, int tile_tokens, int r, int32_t* lds,
                                      int32_t* scratch, int min_len = 1) {
  TileTable tt;
  tt.tile_start = lds;
  tt.seg_start = lds + seg.L + 1;
  tt.seg_lora = lds + 2 * (seg.L + 1);
  tt.rank = lds + 3 * (seg.L + 1);
  tt.rank_by_seg = false;
  if constexpr (DENSE) {
    const int tiles = seg.T > 0 ? (seg.T + tile_tokens - 1) / tile_tokens : 0;
    if (threadIdx.x == 0) {
      tt.tile_start[0] = 0;
      tt.tile_start[1] = tiles;
      tt.seg_start[0] = 0;
      tt.seg_start[1] = seg.T;
      tt.seg_lora[0] = 0;
      tt.rank[0] = r;
    }
    __syncthreads();
    tt.S = 1;
    tt.tiles = tiles;
    return tt;
  }
  auto clamp_rank = [&](int k) { return k < 0 ? 0 : (k > r ? r : k); };
  int S = seg.counts[0];
  if (seg.L <= kEagerTable) {
    // All L + 1 entries are copied (they exist whatever S is), so these loads
    // go out together with the load of S instead of one round trip after it.
    for (int s = threadIdx.x; s <= seg.L; s += NT) tt.seg_start[s] = seg.seg_start[s];
    for (int s = threadIdx.x; s < seg.L; s += NT) tt.seg_lora[s] = seg.seg_lora[s];
    for (int s = threadIdx.x; s < seg.L; s += NT) tt.rank[s] = clamp_rank(seg.lora_rank ? seg.lora_rank[s] : r);
    S = S < 0 ? 0 : (S > seg.L ? seg.L : S);
  } else {
    // A large pool, most of it usually idle: the first NE segments go out with
    // the load of S, the rest (if S is larger) one round trip later, and each
    // segment's rank is looked up from its adapter.
    // (NE <= kEagerTable < L: indices up to NE exist.)
    constexpr int NE = NT < kEagerTable ? NT : kEagerTable;
    if (threadIdx.x < NE) {
      tt.seg_start[threadIdx.x] = seg.seg_start[threadIdx.x];
      tt.seg_lora[threadIdx.x] = seg.seg_lora[threadIdx.x];
    }
    if (threadIdx.x == NE - 1) tt.seg_start[NE] = seg.seg_start[NE];
    S = S < 0 ? 0 : (S > seg.L ? seg.L : S);
    for (int s = NE + 1 + threadIdx.x; s <= S; s += NT) tt.seg_start[s] = seg.seg_start[s];
    for (int s = NE + threadIdx.x; s < S; s += NT) tt.seg_lora[s] = seg.seg_lora[s];
    if (seg.lora_rank) {
      __syncthreads();
      for (int s = threadIdx.x; s < S; s += NT) {
        const int l = tt.seg_lora[s];
        tt.rank[s] = (l >= 0 && l < seg.L) ? clamp_rank(seg.lora_rank[l]) : 0;
      }
    } else {
      for (int s = threadIdx.x; s < S; s += NT) tt.rank[s] = r;
    }
    tt.rank_by_seg = true;
  }
  __syncthreads();
  const int per = (S + NT - 1) / NT;
  const int lo = min((int)threadIdx.x * per, S);
  const int hi = min(lo + per, S);
  // Segments shorter than min_len get no tiles (another kernel takes them).
  auto seg_tiles = [&](int s) {
    const int len = tt.seg_start[s + 1] - tt.seg_start[s];
    return (len > 0 && len >= min_len) ? (len + tile_tokens - 1) / tile_tokens : 0;
  };
  int mine = 0;
  for (int s = lo; s < hi; ++s) mine += seg_tiles(s);
  int total;
  int run = block_exclusive_sum<NT>(mine, scratch, &total);
  for (int s = lo; s < hi; ++s) {
    tt.tile_start[s] = run;
    run += seg_tiles(s);
  }
  if (threadIdx.x == 0) tt.tile_start[S] = total;
  __syncthreads();
  tt.S = S;
  // Metadata that breaks its invariants (the caller may fill it) can claim
  // more tiles than T tokens make; the walk never goes past what a valid
  // batch can hold, so such a call costs no more than a valid one.  Tiles
  // past the claimed segments' tokens are refused by tile_range_lds.
  const int64_t cap = max_token_tiles(seg.T, seg.L, tile_tokens);
  tt.tiles = total < 0 ? 0 : (total > cap ? (int)cap : total);
  return tt;
}

// tile_range on a TileTable (LDS only), with the live rank of the tile's
// adapter.
__device__ __forceinline__ bool tile_range_lds(const TileTable& tt, int T, int L, int tile_tokens,
                                               int tile, int* p0, int* p_end, int* lora_id, int* rank) {
  const int s = tile_segment(tt.tile_start, tt.S, tile);
  const int start = tt.seg_start[s];
  const int end = tt.seg_start[s + 1];
  const int b = start + (tile - tt.tile_start[s]) * tile_tokens;
  const int e = min(b + tile_tokens, end);
  const int l = tt.seg_lora[s];
  if (b < 0 || e > T || b >= e || l < 0 || l >= L) return false;
  *p0 = b;
  *p_end = e;
  *lora_id = l;
  *rank = tt.rank[tt.rank_by_seg ? s : l];
  return true;
}

}  // namespace lora
