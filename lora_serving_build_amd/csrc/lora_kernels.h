// Launchers of the gfx950 kernels, called by the C-ABI layer (lora_api.hip)
// after it has validated every argument.  They return the hipError_t of the
// launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lora {

constexpr int kMaxSlices = 8;
constexpr int kMaxRank = 128;
constexpr int kMaxLoras = 2048;

// Token tile of the expand kernel: 4 waves x 16 tokens.
constexpr int kTileTokens = 64;
// Largest token tile of the shrink kernel (4 token groups of 16).
constexpr int kMaxShrinkTile = 64;
// Columns per expand work item (per wave: 16 tokens x 128 columns).
constexpr int kExpandCols = 128;
// H elements one shrink K-step covers (4 lane groups x 32 elements).
constexpr int kShrinkKStep = 128;

// Launch-plan overrides for tests and measurement, read from the
// environment once when the library is loaded (and again on
// lora_reload_tuning): LORA_SHRINK_KSPLIT, LORA_EXPAND_TB, LORA_EXPAND_CPR,
// LORA_EXPAND_WGS_PER_CU, LORA_EXPAND_BALANCE (1 round-robin items, 2 balanced
// ranges), LORA_SHRINK_TB (2: 128-token shrink tiles at r = 33..64),
// LORA_SHRINK_GROUP (1: 16-token groups with the H split inside the
// workgroup at r <= 32, 2: never), LORA_EXPAND_LINE_Y (whole-line y in the
// tile expand; 1: loads only, 2: neither), LORA_BGMV_SHRINK_RT, LORA_BGMV_RPI,
// LORA_BGMV_CB.  0 = not set: the launchers' own choice.
struct Tuning {
  int shrink_ksplit;
  int expand_tb;
  int expand_cpr;
  int bgmv_shrink_rt;
  int bgmv_rpi;
  int bgmv_cb;
  int expand_wgs_per_cu;
  int expand_balance;
  int shrink_tb;
  int shrink_group;
  int expand_line_y;
};
const Tuning& tuning();
void reload_tuning();

struct SegView {
  const int32_t* token_lora;
  const int32_t* sorted_token;
  const int32_t* seg_lora;
  const int32_t* seg_start;
  const int32_t* counts;
  const int32_t* lora_rank;  // [L] live rank per adapter, or nullptr
  int32_t T;
  int32_t L;
  // 1: the single-adapter form -- every token uses adapter 0 and token index
  // = position; no metadata pointer is read (they may be null).
  int32_t dense;
};

hipError_t launch_build_segments(const int32_t* token_lora, int32_t T, int32_t L,
                                 int32_t* sorted_token, int32_t* seg_lora,
                                 int32_t* seg_start, int32_t* counts, hipStream_t s);

struct ShrinkPlan {
  int32_t jtw;          // 16-row tiles of r per wave (1, 2, 4 or 8)
  int32_t tb;           // 16-token blocks per wave (tiles of 64 tb tokens)
  int32_t group;        // 1: 16-token groups, H split inside the workgroup (no workspace)
  int32_t fixed;        // 1: the split is set by an override (the kernel keeps it)
  int32_t rp;           // rank padded to the rank groups
  int32_t ksplit;       // number of H chunks split across workgroups (from the tile bound)
  int32_t ks_cap;       // most chunks the kernel may choose from the true tile count
  int32_t kchunk;       // H elements per chunk (multiple of kShrinkKStep)
  int32_t max_tiles;    // upper bound on token tiles
  int32_t resident;     // workgroups resident at once
  int32_t grid;         // persistent workgroups
  size_t partial_bytes; // workspace: header + ks_cap chunks of partial rows (ks_cap > 1)
};

// Bytes at the start of the shrink workspace that hold the split the kernel
// chose (the partial rows follow, 16-byte aligned).
constexpr size_t kShrinkWsHeader = 256;

// ws_limit: the workspace available (0 = as much as the plan asks for); a
// smaller one lowers ks_cap, never below ksplit.
ShrinkPlan plan_shrink(int32_t T, int32_t L, int32_t H, int32_t r, size_t ws_limit = 0);

// min_seg_len: segments with fewer tokens are left to another kernel.
hipError_t launch_shrink(const SegView& seg, const uint16_t* x, int64_t ldx, const uint16_t* A,
                         int32_t H, int32_t r, float* v, int64_t ldv, void* workspace,
                         const ShrinkPlan& plan, int dtype, bool vec, hipStream_t s,
                         int min_seg_len = 1);

struct ExpandSliceDesc {
  const uint16_t* B;
  int32_t n;
  int64_t col_off;
};

// Per-token (BGMV) kernels for decode-shaped batches.  The shrink takes any
// r <= 128; the expand takes r <= 64, and r = 128 on aligned data.
constexpr int kBgmvMaxRank = 64;
inline bool bgmv_supports(bool expand, int32_t r, bool vec) {
  return expand ? (r <= kBgmvMaxRank || (r == 128 && vec)) : r <= kMaxRank;
}

// Ranks per workgroup of the per-token shrink (4, 8 or 16) for T tokens at
// rank r over rows of H: the largest that still gives 256 workgroups (512
// for H >= 12288), 4 if none does.
int bgmv_shrink_ranks(int64_t T, int32_t r, int32_t H);

// short_max as for launch_bgmv_expand.
hipError_t launch_bgmv_shrink(const SegView& seg, const uint16_t* x, int64_t ldx, const uint16_t* A,
                              int32_t H, int32_t r, float* v, int64_t ldv, int dtype, bool vec,
                              hipStream_t s, int short_max = 0);

// short_max = 0: every token; k >= 1: only the tokens of segments of at most
// k tokens (found from the segment metadata).
hipError_t launch_bgmv_expand(const SegView& seg, const float* v, int64_t ldv, int64_t v_slice_stride,
                              const ExpandSliceDesc* slices, int32_t num_slices, int32_t r,
                              uint16_t* y, int64_t ldy, int add, int dtype, bool vec, hipStream_t s,
                              int short_max = 0);

// Shrink then expand_slice of each token in one launch (decode batches): r is
// 8, 16, 32 or 64 and every row and size is 16-byte aligned; the slices share
// v, which is written as by the shrink.
hipError_t launch_fused_decode(const SegView& seg, const uint16_t* x, int64_t ldx, const uint16_t* A,
                               int32_t H, int32_t r, float* v, int64_t ldv, const ExpandSliceDesc* slices,
                               int32_t num_slices, uint16_t* y, int64_t ldy, int add, int dtype,
                               hipStream_t s);

// min_seg_len: segments with fewer tokens are left to another kernel.
// short_items (vec, segment metadata, r = 8, 16, 32 or 64, with min_seg_len
// 2): the same launch takes the one-token segments as per-token items.
hipError_t launch_expand(const SegView& seg, const float* v, int64_t ldv, int64_t v_slice_stride,
                         const ExpandSliceDesc* slices, int32_t num_slices, int32_t r,
                         uint16_t* y, int64_t ldy, int add, int dtype, bool vec, hipStream_t s,
                         int min_seg_len = 1, bool short_items = false);

}  // namespace lora
