// Per-token pieces shared by the per-token kernels (bgmv.hip) and the
// segment-tile expand (expand.hip), which also takes the one-token segments
// of a batch as per-token work items: the adapter-id load, the walk over
// short segments, the hi / lo split of v and the aligned per-token expand of
// one token's column block.
#pragma once

#include "lora_device.h"
#include "lora_kernels.h"

namespace lora {

constexpr int kBgThreads = 256;  // threads of a per-token workgroup

template <int DT>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  if constexpr (DT == 0) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c, false);
  } else {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c,
                                          false);
  }
}

// Adapter of token t as a uniform value; -1 when the token has none (ids
// outside [0, L) count as none).  t is the same for the whole workgroup.
// token_lora is read-only for the whole launch, so the load goes through the
// constant address space: a scalar load, counted apart from the vector loads
// in flight, so waiting for the id does not wait for them.
__device__ __forceinline__ int token_adapter(const SegView& seg, int t) {
  if (seg.dense) return 0;  // the single-adapter form: no ids to read
  typedef const __attribute__((address_space(4))) int32_t* const_ptr;
  const int l = __builtin_amdgcn_readfirstlane(*(const_ptr)(uintptr_t)(seg.token_lora + t));
  return (l >= 0 && l < seg.L) ? l : -1;
}

// Items a per-token kernel walks: every token, or, when it takes only the
// tokens of short segments (1 .. short_max tokens: the decode requests of a
// batch that mixes decode and prefill), short_max items per segment slot
// (S <= min(L, T) slots).  An item of a slot whose segment is longer, or past
// the segment's tokens, finds nothing to do after one round of loads: no
// workgroup needs a table of all segments.
__device__ __forceinline__ int bg_items(const SegView& seg, int short_max) {
  if (short_max <= 0) return seg.T;
  return min(seg.L, seg.T) * short_max;
}

// Token and adapter of slot item k (k < bg_items): token k % short_max of
// segment k / short_max, if that segment is short.  false: nothing to do (a
// longer segment, a slot past S, or invalid metadata).  Per lane.
__device__ __forceinline__ bool short_slot_token(const SegView& seg, int short_max, int k, int* t, int* l) {
  const int s = k / short_max;  // < min(L, T): the loads below are in bounds
  const int j = k - s * short_max;
  const int S = seg.counts[0];
  const int b = seg.seg_start[s];
  const int e = seg.seg_start[s + 1];
  const int lora_id = seg.seg_lora[s];
  const int len = e - b;
  if (s >= S || len < 1 || len > short_max || j >= len) return false;
  const int p = b + j;
  if (p < 0 || p >= seg.T || lora_id < 0 || lora_id >= seg.L) return false;
  const int tok = seg.sorted_token[p];
  if (tok < 0 || tok >= seg.T) return false;
  *t = tok;
  *l = lora_id;
  return true;
}

// The short-segment checks of 64 items of a workgroup's walk, one per lane,
// made in one round of loads and refreshed every 64 items: item n of the
// walk is checked by lane n % 64 of the batch loaded at item n - n % 64.
// Every wave loads the same batch, so the results are uniform.
struct ShortBatch {
  int t = 0;
  int l = -1;
  int ok = 0;
};

// For item `it`, the n-th of this workgroup's grid-stride walk over `items`
// items of `per` items per slot: false if it has no work, else its token and
// adapter.
__device__ __forceinline__ bool short_item(const SegView& seg, int short_max, int per, int items, int it,
                                           int n, ShortBatch& sb, int* t, int* l) {
  const int i = n & (kWave - 1);
  if (i == 0) {
    const int mine = it + (int)(threadIdx.x & (kWave - 1)) * (int)gridDim.x;
    sb.t = 0;
    sb.l = -1;
    sb.ok = mine < items && short_slot_token(seg, short_max, mine / per, &sb.t, &sb.l);
  }
  if (!__builtin_amdgcn_readlane(sb.ok, i)) return false;
  *t = __builtin_amdgcn_readlane(sb.t, i);
  *l = __builtin_amdgcn_readlane(sb.l, i);
  return true;
}

// Splits two fp32 values into a packed high 16-bit pair and the packed 16-bit
// rounding of the remainders (the remainder of a non-finite value is 0).
template <int DT>
__device__ __forceinline__ void split_hilo(float f0, float f1, uint32_t* hi, uint32_t* lo) {
  *hi = cvt_pack2<DT>(f0, f1);
  float h0, h1;
  unpack2<DT>(*hi, &h0, &h1);
  *lo = cvt_pack2<DT>(__builtin_isfinite(h0) ? f0 - h0 : 0.f, __builtin_isfinite(h1) ? f1 - h1 : 0.f);
}

// Products of one group of 8 ranks with one column's 8 weights: rank pairs in
// order, each pair's high part then its low part.  Both expand kernels build
// a column from these group sums and add the groups in a balanced pairwise
// tree, so a rank zero-padded to more groups gives the same bits.
template <int DT>
__device__ __forceinline__ float group_dot(const uint32_t* vh, const uint32_t* vl, u32x4 b) {
  float s = 0.f;
  s = dot2<DT>(vh[0], b.x, s);
  s = dot2<DT>(vl[0], b.x, s);
  s = dot2<DT>(vh[1], b.y, s);
  s = dot2<DT>(vl[1], b.y, s);
  s = dot2<DT>(vh[2], b.z, s);
  s = dot2<DT>(vl[2], b.z, s);
  s = dot2<DT>(vh[3], b.w, s);
  s = dot2<DT>(vl[3], b.w, s);
  return s;
}

// y[c0..c0+8) (+)= out, rounded once; yv holds the prefetched old values.
template <int DT, bool VEC>
__device__ __forceinline__ void bg_store_cols(uint16_t* yrow, int nq, int c0, int add, u32x4 yv,
                                              float out[8]) {
  if (VEC && c0 + 8 <= nq) {
    if (add) {
      const uint32_t d[4] = {yv.x, yv.y, yv.z, yv.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float y0, y1;
        unpack2<DT>(d[e], &y0, &y1);
        out[2 * e] += y0;
        out[2 * e + 1] += y1;
      }
    }
    *reinterpret_cast<u32x4*>(yrow + c0) =
        u32x4{cvt_pack2<DT>(out[0], out[1]), cvt_pack2<DT>(out[2], out[3]),
              cvt_pack2<DT>(out[4], out[5]), cvt_pack2<DT>(out[6], out[7])};
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      if (c0 + e < nq) {
        float o = out[e];
        if (add) o += to_f32<DT>(yrow[c0 + e]);
        yrow[c0 + e] = (uint16_t)(cvt_pack2<DT>(o, 0.f) & 0xffffu);
      }
    }
  }
}

constexpr int kRoundCols = kWave * 8;
// Column c of the staged sums sits at c + 4 (c / 128): each lane reads its
// 8 columns at 8 lane, and 16-byte LDS reads serve lanes 0-7 with 16-23,
// whose columns lie 128 apart -- the same banks without the 4-float shift.
constexpr int kSoRow = kRoundCols + kRoundCols / 32;

// y of rounds R0 .. R0 + RPI of a token's slice row, 8 columns a lane
// (zeros past the slice, or when y is not read).
template <int RPI>
__device__ __forceinline__ void load_round_y(const uint16_t* yrow, int nq, int add, int R0, int lane,
                                             u32x4 (&yv)[RPI]) {
#pragma unroll
  for (int u = 0; u < RPI; ++u) {
    const int c0 = (R0 + u) * kRoundCols + lane * 8;
    yv[u] = (add && c0 + 8 <= nq) ? *reinterpret_cast<const u32x4*>(yrow + c0) : u32x4{0u, 0u, 0u, 0u};
  }
}

// The first KB weight chunks of rounds R0 .. R0 + RPI for this lane.
// Chunks past the slice read chunk 0; their columns are never stored.
template <int G, int RPI, int KB>
__device__ __forceinline__ void load_round_b(const uint16_t* Bl, int64_t nchunks, int R0, int lane,
                                             u32x4 (&b)[RPI][KB]) {
#pragma unroll
  for (int u = 0; u < RPI; ++u) {
    const int64_t base = (int64_t)(R0 + u) * kRoundCols * G + lane;
#pragma unroll
    for (int k = 0; k < KB; ++k) {
      const int64_t idx = base + (int64_t)k * kWave;
      b[u][k] = *reinterpret_cast<const u32x4*>(Bl + (idx < nchunks ? idx : 0) * 8);
    }
  }
}

// One token's share of an aligned expand (r = 8 G, 16-byte aligned rows and
// sizes): the rounds of column block cb of ncb in every slice, each wave
// RPI rounds of 512 columns at a time.  Its weight block B_l is read front to
// back: load k of lane i takes 16-byte chunk 64 k + i of the current stretch,
// so each wave instruction reads 1 KB of consecutive memory; chunk c holds
// ranks 8 (c % G) .. +8 of column c / G.  The G lanes of a column add their
// group sums over DPP (a balanced tree), one of them parks the column total
// in a wave-private LDS row, and the wave reads the row back 8 columns per
// lane for 16-byte y updates.  y and v are loaded before the adapter id is
// waited for.  a: the slices (B, n, col_off), num_slices, y, ldy, add.
// vrow_of(q) points at the token's v for slice q (global memory or LDS);
// adapter() is its uniform id (-1: y stays as it is); so is this wave's
// staging row of RPI kSoRow floats.  All of the workgroup's kBgThreads
// threads call it.
template <int DT, int G, int RPI, class Args, class VRow, class Adapter>
__device__ __forceinline__ void expand_token_aligned(const Args& a, int t, int cb, int ncb, VRow vrow_of,
                                                     Adapter adapter, float* so) {
  constexpr int LG = G == 1 ? 0 : G == 2 ? 1 : G == 4 ? 2 : G == 8 ? 3 : 4;
  constexpr int K = 8 * G;                   // weight loads per lane and round
  constexpr int KB = K < 16 ? K : 16;        // loads per batch (register bound)
  constexpr int CPI = kWave / G;             // columns per load instruction
  constexpr int NW = kBgThreads / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int part = lane & (G - 1);
  for (int q = 0; q < a.num_slices; ++q) {
    const int nq = a.slices[q].n;
    const float* vrow = vrow_of(q) + part * 8;
    uint16_t* yrow = a.y + (int64_t)t * a.ldy + a.slices[q].col_off;
    for (int R0 = (cb * NW + wave) * RPI; R0 * kRoundCols < nq; R0 += ncb * NW * RPI) {
      // y and v do not depend on the adapter: they are in flight while the
      // (scalar) adapter id arrives, and only the id is waited for before
      // the weight loads go out.
      const int l = adapter();
      u32x4 yv[RPI];
      load_round_y<RPI>(yrow, nq, a.add, R0, lane, yv);
      f32x4 va = *reinterpret_cast<const f32x4*>(vrow);
      f32x4 vb = *reinterpret_cast<const f32x4*>(vrow + 4);
      if (l < 0) break;  // uniform: the row of y stays as it is
      const uint16_t* Bl = a.slices[q].B + (int64_t)l * nq * (8 * G);
      const int64_t nchunks = (int64_t)nq * G;
      u32x4 b[RPI][KB];
      load_round_b<G, RPI, KB>(Bl, nchunks, R0, lane, b);
      // All first-batch weight loads are in flight before any arithmetic;
      // the opaque moves keep the split of v from being hoisted above them.
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("" : "+v"(va), "+v"(vb));
      // Binary16 prescale of the token's v (f16_prescale): the G lanes of
      // a column group hold the whole row, so their maximum is the row's.
      float down = 1.f, up = 1.f;
      if constexpr (DT == 0) {
        float vmax = fmaxf(fmaxf(fmaxf(fabsf(va.x), fabsf(va.y)), fmaxf(fabsf(va.z), fabsf(va.w))),
                           fmaxf(fmaxf(fabsf(vb.x), fabsf(vb.y)), fmaxf(fabsf(vb.z), fabsf(vb.w))));
        if constexpr (G >= 2) vmax = fmaxf(vmax, lane_xor<0>(vmax, lane));
        if constexpr (G >= 4) vmax = fmaxf(vmax, lane_xor<1>(vmax, lane));
        if constexpr (G >= 8) vmax = fmaxf(vmax, lane_xor<2>(vmax, lane));
        if constexpr (G >= 16) vmax = fmaxf(vmax, lane_xor<3>(vmax, lane));
        f16_prescale(vmax, &down, &up);
        va *= down;
        vb *= down;
      }
      uint32_t vh[4], vl[4];
      split_hilo<DT>(va.x, va.y, &vh[0], &vl[0]);
      split_hilo<DT>(va.z, va.w, &vh[1], &vl[1]);
      split_hilo<DT>(vb.x, vb.y, &vh[2], &vl[2]);
      split_hilo<DT>(vb.z, vb.w, &vh[3], &vl[3]);
#pragma unroll
      for (int u = 0; u < RPI; ++u) {
        const int64_t base = (int64_t)(R0 + u) * kRoundCols * G + lane;
#pragma unroll
        for (int kb = 0; kb < K; kb += KB) {
          if (kb > 0) {
#pragma unroll
            for (int k = 0; k < KB; ++k) {
              const int64_t idx = base + (int64_t)(kb + k) * kWave;
              b[u][k] = *reinterpret_cast<const u32x4*>(Bl + (idx < nchunks ? idx : 0) * 8);
            }
          }
#pragma unroll
          for (int k = 0; k < KB; ++k) {
            float p = group_dot<DT>(vh, vl, b[u][k]);
            if constexpr (G >= 2) p = p + lane_xor<0>(p, lane);
            if constexpr (G >= 4) p = p + lane_xor<1>(p, lane);
            if constexpr (G >= 8) p = p + lane_xor<2>(p, lane);
            if constexpr (G >= 16) p = p + lane_xor<3>(p, lane);
            if (part == 0) {
              const int c = (kb + k) * CPI + (lane >> LG);  // a run of CPI columns in one 128
              so[u * kSoRow + c + ((c >> 7) << 2)] = DT == 0 ? p * up : p;
            }
          }
        }
      }
      // LDS operations of one wave execute in order: wave-scope fences
      // only keep the compiler from moving them.
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
      for (int u = 0; u < RPI; ++u) {
        const int c0 = (R0 + u) * kRoundCols + lane * 8;
        const float* sr = so + u * kSoRow + lane * 8 + ((lane >> 4) << 2);
        const f32x4 o0 = *reinterpret_cast<const f32x4*>(sr);
        const f32x4 o1 = *reinterpret_cast<const f32x4*>(sr + 4);
        float out[8] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w};
        if (c0 < nq) bg_store_cols<DT, true>(yrow, nq, c0, a.add, yv[u], out);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
  }
}

}  // namespace lora
