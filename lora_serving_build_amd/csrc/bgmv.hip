// Per-token (BGMV) shrink and expand, for decode-shaped batches.
//
// The punica issue describes BGMV as each input using its own model, with the
// speed-up coming from spreading many small products over many compute units.
// Here a workgroup takes one token (with a small batch, one block of its ranks
// or of its output columns) at a time, in token order.  Over a whole batch
// these kernels read only token_lora: for a small batch, the sorted metadata
// would add dependent round trips before the first weight load, and every
// adapter of the batch fits in L2 anyway.  (A compile-time variant takes only
// the one-token segments of a mixed batch, from the metadata.)  Rows that do
// not depend on the adapter (x, y, v) are loaded before the adapter id is
// needed.  The whole H-sum of a token stays inside its workgroup, so no
// partial sums leave it.  The pieces the tile expand shares live in
// token_path.h.
//
// shrink: a workgroup takes one token and a block of up to 16 ranks; lane i
//   owns elements 8 (i + 256 k) .. +8 of H (each wave instruction reads 1 KB
//   of one row); v_dot2 (two 16-bit products into fp32) accumulates
//   x . A_l[j] for each j; a transposing wave reduction and an LDS step across
//   the four waves add them up.
// expand: the token's v is split into hi + lo 16-bit parts; each output
//   column is the balanced pairwise sum of per-8-rank group dot products (see
//   group_dot), rounded once when added to y.  The aligned kernel for
//   r = 8, 16, 32, 64, 128 reads the weight block front to back, 1 KB per wave
//   instruction; the general kernel covers every other shape with the same
//   arithmetic.
#include <algorithm>

#include "lora_device.h"
#include "lora_kernels.h"
#include "token_path.h"

namespace lora {

namespace {

struct BgShrinkArgs {
  SegView seg;
  const uint16_t* x;
  int64_t ldx;
  const uint16_t* A;
  int32_t H;
  int32_t r;
  float* v;
  int64_t ldv;
  int32_t jb;  // rank blocks per token
  // 0: every token, by token index; k >= 1: only the tokens of segments of
  // at most k tokens, from the segment metadata (as in BgExpandArgs).
  int32_t short_max;
};

struct BgExpandArgs {
  SegView seg;
  const float* v;
  int64_t ldv;
  int64_t v_slice_stride;
  ExpandSliceDesc slices[kMaxSlices];
  int32_t num_slices;
  int32_t r;
  uint16_t* y;
  int64_t ldy;
  int32_t add;
  int32_t cb;  // column blocks per token (aligned kernel)
  // 0: every token of the batch, by token index.  k >= 1: only the tokens of
  // segments of at most k tokens (the decode requests of a mixed batch),
  // found from the segment metadata; the tile kernel takes the others.
  int32_t short_max;
};

// x . A_l[j0 + j] for j < RT over this thread's pieces of an aligned row:
// lane i owns elements 8 (i + 256 k) .. +8 of H (each wave instruction reads
// 1 KB of one row); UNR blocks of 2048 elements are in flight per trip, more
// when RT is small.  The x row does not depend on the adapter: its loads go
// out before adapter() (a uniform id, -1 for none) is waited for.  Rows
// j0 + j >= r read row 0; their sums are never stored.  Returns the adapter.
template <int DT, int RT, class Adapter>
__device__ __forceinline__ int token_rank_dots(const uint16_t* xrow, const uint16_t* A, int H, int r, int j0,
                                               Adapter adapter, float (&acc)[RT]) {
  constexpr int BLK = kBgThreads * 8;
  constexpr int UNR = RT <= 4 ? 8 : RT <= 8 ? 4 : 2;  // blocks per trip (register bound)
  int l = 0;
  for (int h0 = threadIdx.x * 8; h0 < H; h0 += UNR * BLK) {
    u32x4 xv[UNR];
#pragma unroll
    for (int u = 0; u < UNR; ++u)
      xv[u] = h0 + u * BLK < H ? *reinterpret_cast<const u32x4*>(xrow + h0 + u * BLK) : u32x4{0u, 0u, 0u, 0u};
    l = adapter();
    if (l < 0) return l;
    const uint16_t* Al = A + (int64_t)l * r * H;
#pragma unroll
    for (int j = 0; j < RT; ++j) {
      const uint16_t* arow = Al + (int64_t)(j0 + j < r ? j0 + j : 0) * H;
      float s = acc[j];
#pragma unroll
      for (int u = 0; u < UNR; ++u) {
        const u32x4 av = h0 + u * BLK < H ? *reinterpret_cast<const u32x4*>(arow + h0 + u * BLK)
                                          : u32x4{0u, 0u, 0u, 0u};
        s = dot2<DT>(xv[u].x, av.x, s);
        s = dot2<DT>(xv[u].y, av.y, s);
        s = dot2<DT>(xv[u].z, av.z, s);
        s = dot2<DT>(xv[u].w, av.w, s);
      }
      acc[j] = s;
    }
  }
  if (H > 0) l = adapter();
  return l;
}

// Workgroup total of each of RT per-thread partial sums: a transposing wave
// reduction leaves lane i with its wave's total of rank i >> (6 - log2 RT),
// one lane of each group parks it in s_red, and thread j < RT returns rank
// j's sum over the waves (others return 0).  The caller syncs before s_red
// is written again.
template <int RT>
__device__ __forceinline__ float block_rank_sum(float (&acc)[RT], float (*s_red)[RT]) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  wave_transpose_sum<RT>(acc);
  constexpr int kShift = 6 - log2_of<RT>();
  if ((lane & ((1 << kShift) - 1)) == 0) s_red[wave][lane >> kShift] = acc[0];
  __syncthreads();
  float s = 0.f;
  if ((int)threadIdx.x < RT) {
#pragma unroll
    for (int w = 0; w < kBgThreads / kWave; ++w) s += s_red[w][threadIdx.x];
  }
  return s;
}

// Work item = (token, block of RT ranks): a small batch is spread over
// T ceil(r / RT) workgroups, each of which reads the token's x row (again, from
// L2, for every block after the first) and RT rows of A (token_rank_dots).
// SH: the short segments' tokens only (a compile-time variant, so the
// every-token kernels carry none of its code).
template <int DT, bool VEC, int RT, bool SH>
__global__ __launch_bounds__(kBgThreads) void bgmv_shrink_kernel(BgShrinkArgs a) {
  __shared__ float s_red[kBgThreads / kWave][RT];
  const int tid = threadIdx.x;
  const int items = bg_items(a.seg, SH ? a.short_max : 0) * a.jb;
  ShortBatch sb;
  int n = 0;
  for (int it = blockIdx.x; it < items; it += gridDim.x, ++n) {
    const int k = it / a.jb;
    const int j0 = (it - k * a.jb) * RT;
    // With every token, the adapter id is loaded (scalar) while x is in
    // flight; a short-segment token has its adapter from the segment.
    int t = k, l_short = -1;
    if constexpr (SH) {
      if (!short_item(a.seg, a.short_max, a.jb, items, it, n, sb, &t, &l_short)) continue;
    }
    auto adapter = [&]() { return SH ? l_short : token_adapter(a.seg, t); };
    const uint16_t* xrow = a.x + (int64_t)t * a.ldx;
    float acc[RT];
#pragma unroll
    for (int j = 0; j < RT; ++j) acc[j] = 0.f;
    int l = 0;
    if constexpr (VEC) {
      l = token_rank_dots<DT, RT>(xrow, a.A, a.H, a.r, j0, adapter, acc);
    } else {
      l = adapter();
      if (l >= 0) {
        const uint16_t* Al = a.A + (int64_t)l * a.r * a.H;
        for (int h = tid; h < a.H; h += kBgThreads) {
          const float xf = to_f32<DT>(xrow[h]);
#pragma unroll
          for (int j = 0; j < RT; ++j)
            if (j0 + j < a.r) acc[j] += xf * to_f32<DT>(Al[(int64_t)(j0 + j) * a.H + h]);
        }
      }
    }
    if (l < 0) continue;  // uniform: no adapter, v row left as it is
    const float s = block_rank_sum<RT>(acc, s_red);
    if (tid < RT && j0 + tid < a.r) a.v[(int64_t)t * a.ldv + j0 + tid] = s;
    __syncthreads();
  }
}

// Output columns c0..c0+7 of one slice for one token: returns them in out[].
// NG = rank groups of 8 (r <= 8 NG, a power of two).
template <int DT, bool VEC, int NG>
__device__ __forceinline__ void bg_expand_cols(const uint16_t* Bl, int nq, int r, int c0,
                                               const uint32_t* vhi, const uint32_t* vlo,
                                               float out[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int c = c0 + e < nq ? c0 + e : nq - 1;  // past the slice: dropped by the caller
    const uint16_t* brow = Bl + (int64_t)c * r;
    float p[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      u32x4 b;
      if constexpr (VEC) {
        b = load8_16<true>(brow + 8 * g, r - 8 * g);  // r % 8 == 0: whole group or zeros
      } else {
        uint32_t d[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int k = 8 * g + 2 * i;
          d[i] = pack2(k < r ? (uint32_t)brow[k] : 0u, k + 1 < r ? (uint32_t)brow[k + 1] : 0u);
        }
        b = u32x4{d[0], d[1], d[2], d[3]};
      }
      p[g] = group_dot<DT>(vhi + 4 * g, vlo + 4 * g, b);
    }
#pragma unroll
    for (int m = 1; m < NG; m *= 2)
#pragma unroll
      for (int g = 0; g < NG; g += 2 * m) p[g] = p[g] + p[g + m];
    out[e] = p[0];
  }
}

// General per-token expand: any r <= RT, any alignment.  Lane i owns 8
// consecutive output columns and reads their weight rows itself.  SH as for
// the shrink.
template <int DT, bool VEC, int RT, bool SH>
__global__ __launch_bounds__(kBgThreads) void bgmv_expand_kernel(BgExpandArgs a) {
  constexpr int BLK = kBgThreads * 8;
  constexpr int UNR = RT <= 16 ? 2 : 1;  // column blocks per trip (register bound)
  const int tid = threadIdx.x;
  const int ntok = bg_items(a.seg, SH ? a.short_max : 0);
  ShortBatch sb;
  int n = 0;
  for (int k = blockIdx.x; k < ntok; k += gridDim.x, ++n) {
    int t = k, l = -1;
    if constexpr (SH) {
      if (!short_item(a.seg, a.short_max, 1, ntok, k, n, sb, &t, &l)) continue;
    } else {
      l = token_adapter(a.seg, t);
    }
    if (l < 0) continue;  // uniform: the row of y stays as it is
    for (int q = 0; q < a.num_slices; ++q) {
      const float* vrow = a.v + (int64_t)t * a.ldv + (int64_t)q * a.v_slice_stride;
      const int nq = a.slices[q].n;
      const uint16_t* Bl = a.slices[q].B + (int64_t)l * nq * a.r;
      uint16_t* yrow = a.y + (int64_t)t * a.ldy + a.slices[q].col_off;
      // hi / lo 16-bit pairs of v (ranks >= r are zero), after the binary16
      // prescale of the token's v (f16_prescale; none for bfloat16).
      float vv[RT];
      float vmax = 0.f;
#pragma unroll
      for (int k = 0; k < RT; ++k) {
        vv[k] = k < a.r ? vrow[k] : 0.f;
        vmax = fmaxf(vmax, fabsf(vv[k]));
      }
      float down = 1.f, up = 1.f;
      if constexpr (DT == 0) f16_prescale(vmax, &down, &up);
      uint32_t vhi[RT / 2], vlo[RT / 2];
#pragma unroll
      for (int k = 0; k < RT / 2; ++k) split_hilo<DT>(vv[2 * k] * down, vv[2 * k + 1] * down, &vhi[k], &vlo[k]);
      // Up to two column blocks per trip; their y loads are issued first.
      for (int c0 = tid * 8; c0 < nq; c0 += UNR * BLK) {
        u32x4 yv[UNR];
#pragma unroll
        for (int u = 0; u < UNR; ++u) {
          const int cu = c0 + u * BLK;
          yv[u] = (VEC && a.add && cu + 8 <= nq) ? *reinterpret_cast<const u32x4*>(yrow + cu)
                                                 : u32x4{0u, 0u, 0u, 0u};
        }
        float out[UNR][8];
#pragma unroll
        for (int u = 0; u < UNR; ++u)
          if (c0 + u * BLK < nq) {
            bg_expand_cols<DT, VEC, RT / 8>(Bl, nq, a.r, c0 + u * BLK, vhi, vlo, out[u]);
            if constexpr (DT == 0) {
#pragma unroll
              for (int e = 0; e < 8; ++e) out[u][e] *= up;
            }
          }
#pragma unroll
        for (int u = 0; u < UNR; ++u)
          if (c0 + u * BLK < nq) bg_store_cols<DT, VEC>(yrow, nq, c0 + u * BLK, a.add, yv[u], out[u]);
      }
    }
  }
}

// Per-token expand for r = 8 G (G = 1, 2, 4, 8, 16) on aligned data
// (expand_token_aligned: weight blocks read front to back, 1 KB per wave
// instruction; columns summed over the G lanes of a group with DPP, the same
// balanced tree as the general kernel).  A token's columns are spread over cb
// workgroups (work item = (token, column block)), so a small batch still
// fills the chip: in every slice, block b takes the rounds whose index
// divided by 4 RPI is b modulo cb.
template <int DT, int G, int RPI, bool SH>
__global__ __launch_bounds__(kBgThreads) void bgmv_expand_fast_kernel(BgExpandArgs a) {
  constexpr int NW = kBgThreads / kWave;
  __shared__ __align__(16) float s_out[NW][RPI * kSoRow];
  float* so = s_out[threadIdx.x / kWave];
  const int items = bg_items(a.seg, SH ? a.short_max : 0) * a.cb;
  ShortBatch sb;
  int n = 0;
  for (int it = blockIdx.x; it < items; it += gridDim.x, ++n) {
    const int k = it / a.cb;
    const int cb = it - k * a.cb;
    // With every token, the adapter id is loaded (scalar) while y and v are
    // in flight; short-segment tokens have theirs from the segment.
    int t = k, l_short = -1;
    if constexpr (SH) {
      if (!short_item(a.seg, a.short_max, a.cb, items, it, n, sb, &t, &l_short)) continue;
    }
    expand_token_aligned<DT, G, RPI>(
        a, t, cb, a.cb, [&](int q) { return a.v + (int64_t)t * a.ldv + (int64_t)q * a.v_slice_stride; },
        [&]() { return SH ? l_short : token_adapter(a.seg, t); }, so);
  }
}

struct FusedArgs {
  BgExpandArgs ex;  // the expand's view (its v is not read: v comes from LDS)
  const uint16_t* x;
  int64_t ldx;
  const uint16_t* A;
  int32_t H;
  float* v;         // [T][ex.ldv], written by the first column block of each token
};

// Shrink then expand of one token in one workgroup, for decode batches: the
// launch and the round trip of v between two kernels are what a decode
// step's shrink and expand mostly cost.  The workgroup sums x . A_l for all
// r = 8 G ranks (token_rank_dots in blocks of up to 16 ranks, then across
// the waves into LDS), the first column block writes v out, and the expand
// of its column block (expand_token_aligned) reads v from LDS.  A token's
// columns are spread over cb workgroups as in the aligned per-token expand;
// each of them computes the token's v again (x and A_l come from L2 after
// the first), so no workgroup waits for another.
template <int DT, int G, int RPI>
__global__ __launch_bounds__(kBgThreads) void fused_decode_kernel(FusedArgs f) {
  constexpr int R = 8 * G;
  constexpr int RT = R < 16 ? R : 16;
  constexpr int NW = kBgThreads / kWave;
  __shared__ float s_red[NW][RT];
  __shared__ __align__(16) float s_v[R];
  __shared__ __align__(16) float s_out[NW][RPI * kSoRow];
  float* so = s_out[threadIdx.x / kWave];
  const BgExpandArgs& a = f.ex;
  const int items = a.seg.T * a.cb;
  for (int it = blockIdx.x; it < items; it += gridDim.x) {
    const int t = it / a.cb;
    const int cb = it - t * a.cb;
    const uint16_t* xrow = f.x + (int64_t)t * f.ldx;
    auto adapter = [&]() { return token_adapter(a.seg, t); };
    int l = -1;
    for (int j0 = 0; j0 < R; j0 += RT) {
      float acc[RT];
#pragma unroll
      for (int j = 0; j < RT; ++j) acc[j] = 0.f;
      l = token_rank_dots<DT, RT>(xrow, f.A, f.H, R, j0, adapter, acc);
      if (l < 0) break;  // uniform
      const float s = block_rank_sum<RT>(acc, s_red);
      if ((int)threadIdx.x < RT) s_v[j0 + threadIdx.x] = s;
      __syncthreads();
    }
    if (l < 0) continue;  // no adapter: the v and y rows stay as they are
    if (cb == 0 && (int)threadIdx.x < R) f.v[(int64_t)t * a.ldv + threadIdx.x] = s_v[threadIdx.x];
    expand_token_aligned<DT, G, RPI>(a, t, cb, a.cb, [&](int) { return static_cast<const float*>(s_v); },
                                     [&]() { return l; }, so);
    __syncthreads();  // s_v and s_red are rewritten by the next item
  }
}

int bg_grid(int32_t T) {
  int64_t g = T < 2048 ? T : 2048;
  return g < 1 ? 1 : (int)g;
}

}  // namespace

int bgmv_shrink_ranks(int64_t T, int32_t r, int32_t H) {
  // Measured on MI355X (4 adapters, H = 1024 .. 16384, inputs in HBM): the
  // best choice is the largest block that still gives 256 workgroups --
  // fewer ranks per workgroup re-read x from L2 more often for no gain in
  // parallelism -- except on rows of 12288 elements and more, where a
  // workgroup's row takes several latency-bound trips and 512 workgroups (two
  // per CU) pay: 256 tokens x 16384 at r = 16 went from 13.0 to 11.6 us.
  const int64_t want = H >= 12288 ? 512 : 256;
  int rt = 16;
  while (rt > 4 && (rt / 2 >= r || T * ((r + rt - 1) / rt) < want)) rt /= 2;
  const int f = tuning().bgmv_shrink_rt;
  if (f == 4 || f == 8 || f == 16) rt = f;
  return rt;
}

hipError_t launch_bgmv_shrink(const SegView& seg, const uint16_t* x, int64_t ldx, const uint16_t* A,
                              int32_t H, int32_t r, float* v, int64_t ldv, int dtype, bool vec,
                              hipStream_t s, int short_max) {
  BgShrinkArgs a{seg, x, ldx, A, H, r, v, ldv, 1, short_max > 0 ? short_max : 0};
  // Items walked: every token, or short_max per segment slot.
  const int64_t T_walk = a.short_max > 0 ? (int64_t)std::min(seg.L, seg.T) * a.short_max : seg.T;
  const int64_t T = T_walk > 0 ? T_walk : 1;
  const int rt = bgmv_shrink_ranks(T, r, H);
  a.jb = (r + rt - 1) / rt;
  int64_t grid = T * a.jb;
  if (grid > 8192) grid = 8192;
  // Taking short segments only, most slots may be empty (a batch without
  // decode requests has none): one round of resident workgroups (two per CU
  // at these register counts) walks them, so an empty pass costs little.
  if (a.short_max > 0 && grid > 512) grid = 512;
  const bool sh = a.short_max > 0;
#define LORA_BG_SHRINK(DT_, VEC_, SH_)                                                                \
  if (rt == 16)                                                                                      \
    hipLaunchKernelGGL((bgmv_shrink_kernel<DT_, VEC_, 16, SH_>), dim3(grid), dim3(kBgThreads), 0, s, a); \
  else if (rt == 8)                                                                                  \
    hipLaunchKernelGGL((bgmv_shrink_kernel<DT_, VEC_, 8, SH_>), dim3(grid), dim3(kBgThreads), 0, s, a); \
  else                                                                                               \
    hipLaunchKernelGGL((bgmv_shrink_kernel<DT_, VEC_, 4, SH_>), dim3(grid), dim3(kBgThreads), 0, s, a);
#define LORA_BG_SHRINK_SH(DT_, VEC_) \
  if (sh) { LORA_BG_SHRINK(DT_, VEC_, true) } else { LORA_BG_SHRINK(DT_, VEC_, false) }
  if (dtype == 0) {
    if (vec) { LORA_BG_SHRINK_SH(0, true) } else { LORA_BG_SHRINK_SH(0, false) }
  } else {
    if (vec) { LORA_BG_SHRINK_SH(1, true) } else { LORA_BG_SHRINK_SH(1, false) }
  }
#undef LORA_BG_SHRINK_SH
#undef LORA_BG_SHRINK
  return hipGetLastError();
}

hipError_t launch_bgmv_expand(const SegView& seg, const float* v, int64_t ldv, int64_t v_slice_stride,
                              const ExpandSliceDesc* slices, int32_t num_slices, int32_t r,
                              uint16_t* y, int64_t ldy, int add, int dtype, bool vec, hipStream_t s,
                              int short_max) {
  BgExpandArgs a{};
  a.short_max = short_max > 0 ? short_max : 0;
  // Items walked: every token, or short_max per segment slot.
  const int64_t T_walk = a.short_max > 0 ? (int64_t)std::min(seg.L, seg.T) * a.short_max : seg.T;
  a.seg = seg;
  a.v = v;
  a.ldv = ldv;
  a.v_slice_stride = v_slice_stride;
  for (int q = 0; q < num_slices; ++q) a.slices[q] = slices[q];
  a.num_slices = num_slices;
  a.r = r;
  a.y = y;
  a.ldy = ldy;
  a.add = add;
  if (vec && (r == 8 || r == 16 || r == 32 || r == 64 || r == 128)) {
    // Rounds of 512 columns in the widest slice, and workgroups per token
    // that give each wave RPI rounds of it.  One round per wave (twice the
    // workgroups of two) measured faster on 16- and 256-token batches; two
    // rounds stay selectable for r <= 16.
    constexpr int nw = kBgThreads / kWave;
    int64_t rounds = 1;
    for (int q = 0; q < num_slices; ++q) {
      const int64_t rq = (slices[q].n + kRoundCols - 1) / kRoundCols;
      rounds = rq > rounds ? rq : rounds;
    }
    const int64_t T = T_walk > 0 ? T_walk : 1;
    int rpi = 1;
    const int f_rpi = tuning().bgmv_rpi;
    if (f_rpi == 1 || (f_rpi == 2 && r <= 16)) rpi = f_rpi;
    int64_t cb = (rounds + (int64_t)nw * rpi - 1) / ((int64_t)nw * rpi);
    const int f_cb = tuning().bgmv_cb;
    if (f_cb >= 1 && f_cb < cb) cb = f_cb;
    a.cb = (int32_t)cb;
    int64_t grid = T * cb;
    if (grid > 8192) grid = 8192;
    if (a.short_max > 0 && grid > 1024) grid = 1024;  // one round (four per CU), as for the shrink
    const bool sh = a.short_max > 0;
#define LORA_BG_FAST(DT_, SH_)                                                                       \
  switch (r) {                                                                                      \
    case 8:                                                                                         \
      if (rpi == 2) hipLaunchKernelGGL((bgmv_expand_fast_kernel<DT_, 1, 2, SH_>), dim3(grid), dim3(kBgThreads), 0, s, a); \
      else hipLaunchKernelGGL((bgmv_expand_fast_kernel<DT_, 1, 1, SH_>), dim3(grid), dim3(kBgThreads), 0, s, a); \
      break;                                                                                        \
    case 16:                                                                                        \
      if (rpi == 2) hipLaunchKernelGGL((bgmv_expand_fast_kernel<DT_, 2, 2, SH_>), dim3(grid), dim3(kBgThreads), 0, s, a); \
      else hipLaunchKernelGGL((bgmv_expand_fast_kernel<DT_, 2, 1, SH_>), dim3(grid), dim3(kBgThreads), 0, s, a); \
      break;                                                                                        \
    case 32: hipLaunchKernelGGL((bgmv_expand_fast_kernel<DT_, 4, 1, SH_>), dim3(grid), dim3(kBgThreads), 0, s, a); break; \
    case 64: hipLaunchKernelGGL((bgmv_expand_fast_kernel<DT_, 8, 1, SH_>), dim3(grid), dim3(kBgThreads), 0, s, a); break; \
    default: hipLaunchKernelGGL((bgmv_expand_fast_kernel<DT_, 16, 1, SH_>), dim3(grid), dim3(kBgThreads), 0, s, a); break; \
  }
    if (dtype == 0) {
      if (sh) { LORA_BG_FAST(0, true) } else { LORA_BG_FAST(0, false) }
    } else {
      if (sh) { LORA_BG_FAST(1, true) } else { LORA_BG_FAST(1, false) }
    }
#undef LORA_BG_FAST
    return hipGetLastError();
  }
  int grid = bg_grid((int32_t)T_walk);
  if (a.short_max > 0 && grid > 1024) grid = 1024;
  const bool sh = a.short_max > 0;
#define LORA_BG_EXPAND(DT_, VEC_, SH_)                                                                \
  if (r <= 16)                                                                                       \
    hipLaunchKernelGGL((bgmv_expand_kernel<DT_, VEC_, 16, SH_>), dim3(grid), dim3(kBgThreads), 0, s, a); \
  else if (r <= 32)                                                                                  \
    hipLaunchKernelGGL((bgmv_expand_kernel<DT_, VEC_, 32, SH_>), dim3(grid), dim3(kBgThreads), 0, s, a); \
  else                                                                                               \
    hipLaunchKernelGGL((bgmv_expand_kernel<DT_, VEC_, 64, SH_>), dim3(grid), dim3(kBgThreads), 0, s, a);
#define LORA_BG_EXPAND_SH(DT_, VEC_) \
  if (sh) { LORA_BG_EXPAND(DT_, VEC_, true) } else { LORA_BG_EXPAND(DT_, VEC_, false) }
  if (dtype == 0) {
    if (vec) { LORA_BG_EXPAND_SH(0, true) } else { LORA_BG_EXPAND_SH(0, false) }
  } else {
    if (vec) { LORA_BG_EXPAND_SH(1, true) } else { LORA_BG_EXPAND_SH(1, false) }
  }
#undef LORA_BG_EXPAND_SH
#undef LORA_BG_EXPAND
  return hipGetLastError();
}

hipError_t launch_fused_decode(const SegView& seg, const uint16_t* x, int64_t ldx, const uint16_t* A,
                               int32_t H, int32_t r, float* v, int64_t ldv, const ExpandSliceDesc* slices,
                               int32_t num_slices, uint16_t* y, int64_t ldy, int add, int dtype,
                               hipStream_t s) {
  FusedArgs f{};
  f.x = x;
  f.ldx = ldx;
  f.A = A;
  f.H = H;
  f.v = v;
  BgExpandArgs& a = f.ex;
  a.seg = seg;
  a.v = v;
  a.ldv = ldv;
  a.v_slice_stride = 0;
  for (int q = 0; q < num_slices; ++q) a.slices[q] = slices[q];
  a.num_slices = num_slices;
  a.r = r;
  a.y = y;
  a.ldy = ldy;
  a.add = add;
  a.short_max = 0;
  // Column blocks per token as in the aligned per-token expand: one round of
  // 512 columns of the widest slice per wave.
  constexpr int nw = kBgThreads / kWave;
  int64_t rounds = 1;
  for (int q = 0; q < num_slices; ++q) {
    const int64_t rq = (slices[q].n + kRoundCols - 1) / kRoundCols;
    rounds = rq > rounds ? rq : rounds;
  }
  const int64_t cb = (rounds + nw - 1) / nw;
  a.cb = (int32_t)cb;
  int64_t grid = (int64_t)seg.T * cb;
  if (grid > 8192) grid = 8192;
  if (grid < 1) grid = 1;
#define LORA_FUSED(DT_)                                                                              \
  switch (r) {                                                                                      \
    case 8: hipLaunchKernelGGL((fused_decode_kernel<DT_, 1, 1>), dim3(grid), dim3(kBgThreads), 0, s, f); break;  \
    case 16: hipLaunchKernelGGL((fused_decode_kernel<DT_, 2, 1>), dim3(grid), dim3(kBgThreads), 0, s, f); break; \
    case 32: hipLaunchKernelGGL((fused_decode_kernel<DT_, 4, 1>), dim3(grid), dim3(kBgThreads), 0, s, f); break; \
    default: hipLaunchKernelGGL((fused_decode_kernel<DT_, 8, 1>), dim3(grid), dim3(kBgThreads), 0, s, f); break; \
  }
  if (dtype == 0) { LORA_FUSED(0) } else { LORA_FUSED(1) }
#undef LORA_FUSED
  return hipGetLastError();
}

}  // namespace lora
