// Per-token (BGMV) shrink and expand, for decode-shaped batches.
//
// The punica issue describes BGMV as each input using its own model, with the
// speed-up coming from spreading many small products over many compute units.
// Here one workgroup takes one token at a time, in token order, and streams
// that token's adapter rows with lane-contiguous 16-byte loads: every load
// instruction of a wave covers 1 KB of one row.  These kernels read only
// token_lora: for a small batch, the sorted metadata would add dependent
// round trips before the first weight load, and every adapter of the batch
// fits in L2 anyway.  Rows that do not depend on the adapter (x, y, v) are
// loaded before the adapter id arrives.  The whole H-sum of a token stays
// inside its workgroup, so no partial sums leave it.
//
// shrink: lane i of the workgroup owns elements 8 (i + 256 k) .. +8 of H;
//   v_dot2 (two 16-bit products into fp32) accumulates x . A_l[j] for each j,
//   then a wave butterfly and an LDS step across the four waves add them up.
// expand: the token's v row is split once into hi + lo 16-bit parts (held in
//   scalar registers, as it is the same for the whole workgroup); lane i owns
//   8 consecutive output columns, whose B_l^T rows are 8 r contiguous elements,
//   and adds v_dot2(hi) + v_dot2(lo) per pair of ranks (the element-wise path
//   for unaligned shapes does the same arithmetic); y is read and written 16
//   bytes per lane and rounded once.
#include "lora_device.h"
#include "lora_kernels.h"

namespace lora {

namespace {

constexpr int kBgThreads = 256;

struct BgShrinkArgs {
  SegView seg;
  const uint16_t* x;
  int64_t ldx;
  const uint16_t* A;
  int32_t H;
  int32_t r;
  float* v;
  int64_t ldv;
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
};

template <int DT>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  if constexpr (DT == 0) {
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, a), __builtin_bit_cast(f16x2, b), c, false);
  } else {
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c,
                                          false);
  }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

// Adapter of token t as a uniform value; -1 when the token has none (ids
// outside [0, L) count as none).  t is the same for the whole workgroup.
__device__ __forceinline__ int token_adapter(const SegView& seg, int t) {
  const int l = __builtin_amdgcn_readfirstlane(seg.token_lora[t]);
  return (l >= 0 && l < seg.L) ? l : -1;
}

// RT = rows of A handled (r <= RT).  Lane i owns elements 8 (i + 256 k) .. +8
// of H; up to two blocks of 2048 elements are in flight per trip.
template <int DT, bool VEC, int RT>
__global__ __launch_bounds__(kBgThreads) void bgmv_shrink_kernel(BgShrinkArgs a) {
  constexpr int BLK = kBgThreads * 8;
  constexpr int UNR = RT <= 16 ? 2 : 1;  // blocks per trip (register bound)
  __shared__ float s_red[kBgThreads / kWave][RT];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;

  for (int t = blockIdx.x; t < a.seg.T; t += gridDim.x) {
    const uint16_t* xrow = a.x + (int64_t)t * a.ldx;
    float acc[RT];
#pragma unroll
    for (int j = 0; j < RT; ++j) acc[j] = 0.f;
    int l = 0;
    if constexpr (VEC) {
      for (int h0 = tid * 8; h0 < a.H; h0 += UNR * BLK) {
        // The x row does not depend on the adapter: its loads go first.
        u32x4 xv[UNR];
#pragma unroll
        for (int u = 0; u < UNR; ++u)
          xv[u] = h0 + u * BLK < a.H ? *reinterpret_cast<const u32x4*>(xrow + h0 + u * BLK)
                                     : u32x4{0u, 0u, 0u, 0u};
        l = token_adapter(a.seg, t);
        if (l < 0) break;
        const uint16_t* Al = a.A + (int64_t)l * a.r * a.H;
#pragma unroll
        for (int j = 0; j < RT; ++j) {
          // Rows j >= r read row 0 and are never stored.
          const uint16_t* arow = Al + (int64_t)(j < a.r ? j : 0) * a.H;
          float s = acc[j];
#pragma unroll
          for (int u = 0; u < UNR; ++u) {
            const u32x4 av = h0 + u * BLK < a.H ? *reinterpret_cast<const u32x4*>(arow + h0 + u * BLK)
                                                : u32x4{0u, 0u, 0u, 0u};
            s = dot2<DT>(xv[u].x, av.x, s);
            s = dot2<DT>(xv[u].y, av.y, s);
            s = dot2<DT>(xv[u].z, av.z, s);
            s = dot2<DT>(xv[u].w, av.w, s);
          }
          acc[j] = s;
        }
      }
      if (a.H > 0) l = token_adapter(a.seg, t);
    } else {
      l = token_adapter(a.seg, t);
      if (l >= 0) {
        const uint16_t* Al = a.A + (int64_t)l * a.r * a.H;
        for (int h = tid; h < a.H; h += kBgThreads) {
          const float xf = to_f32<DT>(xrow[h]);
#pragma unroll
          for (int j = 0; j < RT; ++j)
            if (j < a.r) acc[j] += xf * to_f32<DT>(Al[(int64_t)j * a.H + h]);
        }
      }
    }
    if (l < 0) continue;  // uniform: no adapter, v row left as it is
#pragma unroll
    for (int j = 0; j < RT; ++j) {
      const float s = wave_sum(acc[j]);
      if (lane == 0) s_red[wave][j] = s;
    }
    __syncthreads();
    if (tid < a.r && tid < RT) {
      float s = 0.f;
#pragma unroll
      for (int w = 0; w < kBgThreads / kWave; ++w) s += s_red[w][tid];
      a.v[(int64_t)t * a.ldv + tid] = s;
    }
    __syncthreads();
  }
}

// Output columns c0..c0+7 of one slice for one token: returns them in out[].
template <int DT, bool VEC, int RT>
__device__ __forceinline__ void bg_expand_cols(const uint16_t* Bl, int nq, int r, int c0,
                                               const uint32_t* vhi, const uint32_t* vlo,
                                               float out[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int c = c0 + e < nq ? c0 + e : nq - 1;  // past the slice: dropped by the caller
    const uint16_t* brow = Bl + (int64_t)c * r;
    // Same pairwise arithmetic on both paths (ranks >= r are zeros), so
    // zero-padding the rank does not change a single bit.
    float s = 0.f;
    if constexpr (VEC) {
#pragma unroll
      for (int kk = 0; kk < RT; kk += 8) {
        const u32x4 bv = load8_16<true>(brow + kk, r - kk);
        const uint32_t b4[4] = {bv.x, bv.y, bv.z, bv.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          s = dot2<DT>(vhi[kk / 2 + i], b4[i], s);
          s = dot2<DT>(vlo[kk / 2 + i], b4[i], s);
        }
      }
    } else {
      // Element-wise loads; the same pairs in the same order.
      for (int kk = 0; kk < r; kk += 2) {
        const uint32_t b = pack2(brow[kk], kk + 1 < r ? (uint32_t)brow[kk + 1] : 0u);
        s = dot2<DT>(vhi[kk / 2], b, s);
        s = dot2<DT>(vlo[kk / 2], b, s);
      }
    }
    out[e] = s;
  }
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

// RT = ranks handled (r <= RT, RT a multiple of 8).
template <int DT, bool VEC, int RT>
__global__ __launch_bounds__(kBgThreads) void bgmv_expand_kernel(BgExpandArgs a) {
  constexpr int BLK = kBgThreads * 8;
  constexpr int UNR = RT <= 16 ? 2 : 1;  // column blocks per trip (register bound)
  const int tid = threadIdx.x;

  for (int t = blockIdx.x; t < a.seg.T; t += gridDim.x) {
    const int l = token_adapter(a.seg, t);
    if (l < 0) continue;  // uniform: the row of y stays as it is
    for (int q = 0; q < a.num_slices; ++q) {
      const float* vrow = a.v + (int64_t)t * a.ldv + (int64_t)q * a.v_slice_stride;
      const int nq = a.slices[q].n;
      const uint16_t* Bl = a.slices[q].B + (int64_t)l * nq * a.r;
      uint16_t* yrow = a.y + (int64_t)t * a.ldy + a.slices[q].col_off;
      // hi / lo 16-bit pairs of v (ranks >= r are zero).
      uint32_t vhi[RT / 2], vlo[RT / 2];
#pragma unroll
      for (int k = 0; k < RT / 2; ++k) {
        const float f0 = 2 * k < a.r ? vrow[2 * k] : 0.f;
        const float f1 = 2 * k + 1 < a.r ? vrow[2 * k + 1] : 0.f;
        vhi[k] = cvt_pack2<DT>(f0, f1);
        float h0, h1;
        unpack2<DT>(vhi[k], &h0, &h1);
        vlo[k] = cvt_pack2<DT>(__builtin_isfinite(h0) ? f0 - h0 : 0.f,
                               __builtin_isfinite(h1) ? f1 - h1 : 0.f);
      }
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
          if (c0 + u * BLK < nq) bg_expand_cols<DT, VEC, RT>(Bl, nq, a.r, c0 + u * BLK, vhi, vlo, out[u]);
#pragma unroll
        for (int u = 0; u < UNR; ++u)
          if (c0 + u * BLK < nq) bg_store_cols<DT, VEC>(yrow, nq, c0 + u * BLK, a.add, yv[u], out[u]);
      }
    }
  }
}

int bg_grid(int32_t T) {
  int64_t g = T < 2048 ? T : 2048;
  return g < 1 ? 1 : (int)g;
}

}  // namespace

hipError_t launch_bgmv_shrink(const SegView& seg, const uint16_t* x, int64_t ldx, const uint16_t* A,
                              int32_t H, int32_t r, float* v, int64_t ldv, int dtype, bool vec,
                              hipStream_t s) {
  BgShrinkArgs a{seg, x, ldx, A, H, r, v, ldv};
  const int grid = bg_grid(seg.T);
#define LORA_BG_SHRINK(DT_, VEC_)                                                                     \
  if (r <= 16)                                                                                       \
    hipLaunchKernelGGL((bgmv_shrink_kernel<DT_, VEC_, 16>), dim3(grid), dim3(kBgThreads), 0, s, a);  \
  else if (r <= 32)                                                                                  \
    hipLaunchKernelGGL((bgmv_shrink_kernel<DT_, VEC_, 32>), dim3(grid), dim3(kBgThreads), 0, s, a);  \
  else                                                                                               \
    hipLaunchKernelGGL((bgmv_shrink_kernel<DT_, VEC_, 64>), dim3(grid), dim3(kBgThreads), 0, s, a);
  if (dtype == 0) {
    if (vec) { LORA_BG_SHRINK(0, true) } else { LORA_BG_SHRINK(0, false) }
  } else {
    if (vec) { LORA_BG_SHRINK(1, true) } else { LORA_BG_SHRINK(1, false) }
  }
#undef LORA_BG_SHRINK
  return hipGetLastError();
}

hipError_t launch_bgmv_expand(const SegView& seg, const float* v, int64_t ldv, int64_t v_slice_stride,
                              const ExpandSliceDesc* slices, int32_t num_slices, int32_t r,
                              uint16_t* y, int64_t ldy, int add, int dtype, bool vec, hipStream_t s) {
  BgExpandArgs a{};
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
  const int grid = bg_grid(seg.T);
#define LORA_BG_EXPAND(DT_, VEC_)                                                                     \
  if (r <= 16)                                                                                       \
    hipLaunchKernelGGL((bgmv_expand_kernel<DT_, VEC_, 16>), dim3(grid), dim3(kBgThreads), 0, s, a);  \
  else if (r <= 32)                                                                                  \
    hipLaunchKernelGGL((bgmv_expand_kernel<DT_, VEC_, 32>), dim3(grid), dim3(kBgThreads), 0, s, a);  \
  else                                                                                               \
    hipLaunchKernelGGL((bgmv_expand_kernel<DT_, VEC_, 64>), dim3(grid), dim3(kBgThreads), 0, s, a);
  if (dtype == 0) {
    if (vec) { LORA_BG_EXPAND(0, true) } else { LORA_BG_EXPAND(0, false) }
  } else {
    if (vec) { LORA_BG_EXPAND(1, true) } else { LORA_BG_EXPAND(1, false) }
  }
#undef LORA_BG_EXPAND
  return hipGetLastError();
}

}  // namespace lora
