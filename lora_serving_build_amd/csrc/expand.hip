// Expand / expand_slice on segments (SGMV form):
//   y[t, off_s + c] = (add ? y : 0) + sum_j v_s[t, j] * B_{s,l}[j, c].
//
// Work item = (64-column tile of one slice, token tile of one segment).  Four
// waves each take 16 tokens of the tile and all 64 columns; the weight rows
// of the column tile are the same for the four waves, so they meet in L1.
//
// The product is computed transposed, D[c][token] = sum_j B^T[c][j] v^T[j][token],
// with 16x16x32 matrix-core ops over 16 rank values at a time.  The fp32 v is
// split into hi = round(v) and lo = round(v - hi) in the data type: lane groups
// 0 and 1 feed hi, groups 2 and 3 feed lo, against the same 16 weights, so one
// op adds B^T (hi + lo) and v keeps about 16 significant bits.
// Output rows are mapped so that every lane owns 16 consecutive columns of one
// token: y is read and written with two 16-byte accesses per lane, and rounded
// once.
#include "lora_device.h"
#include "lora_kernels.h"
#include "tiles.h"

namespace lora {

namespace {

constexpr int kExpandThreads = 256;

struct ExpandArgs {
  SegView seg;
  const float* v;
  int64_t ldv;
  int64_t v_slice_stride;
  ExpandSliceDesc slices[kMaxSlices];
  int32_t col_tile_start[kMaxSlices + 1];  // prefix of column tiles per slice
  int32_t num_slices;
  int32_t r;
  uint16_t* y;
  int64_t ldy;
  int32_t add;
};

template <int DT, bool VEC>
__global__ __launch_bounds__(kExpandThreads) void expand_sgmv_kernel(ExpandArgs a) {
  __shared__ int32_t s_tile_start[kMaxLoras + 1];
  __shared__ int32_t s_scan[kExpandThreads / kWave + 1];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int m = lane & 15;  // token column of D / weight row index inside a 16-row tile
  const int g = lane >> 4;  // lane group

  int S;
  const int mtiles = build_tile_prefix<kExpandThreads>(a.seg, kTileTokens, s_tile_start, s_scan, &S);
  const int ctiles = a.col_tile_start[a.num_slices];
  const int n_items = mtiles * ctiles;
  const int grid = gridDim.x;

  for (int item = xcd_logical_id(blockIdx.x, grid); item < n_items; item += grid) {
    // Consecutive items walk the token tiles under one column tile, so the
    // weight tile is reused from the L2 of one XCD.
    const int ct = item / mtiles;
    const int mt = item - ct * mtiles;
    int q = 0;
    while (q + 1 < a.num_slices && a.col_tile_start[q + 1] <= ct) ++q;
    const int n0 = (ct - a.col_tile_start[q]) * kExpandCols;
    const int nq = a.slices[q].n;

    int p0 = 0, p_end = 0, l = 0;
    if (!tile_range(a.seg, kTileTokens, s_tile_start, S, mt, &p0, &p_end, &l)) continue;
    const int pw = p0 + wave * 16;
    if (pw >= p_end) continue;
    const int t_raw = (pw + m < p_end) ? a.seg.sorted_token[pw + m] : -1;
    const bool tok_ok = t_raw >= 0 && t_raw < a.seg.T;
    const int t = tok_ok ? t_raw : 0;

    const float* vrow = a.v + (int64_t)t * a.ldv + (int64_t)q * a.v_slice_stride;
    const uint16_t* Bl = a.slices[q].B + (int64_t)l * nq * a.r;
    const int c0 = n0 + g * 16;
    const int ncols = nq - c0;
    uint16_t* yrow = a.y + (int64_t)t * a.ldy + a.slices[q].col_off + c0;
    // The y row is the largest and coldest input: start its load first.
    const bool yvec = VEC && tok_ok && ncols >= 16;
    u32x4 w[2] = {u32x4{0u, 0u, 0u, 0u}, u32x4{0u, 0u, 0u, 0u}};
    if (yvec && a.add) {
      w[0] = reinterpret_cast<const u32x4*>(yrow)[0];
      w[1] = reinterpret_cast<const u32x4*>(yrow)[1];
    }

    f32x4 acc[4];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) acc[qq] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int r0 = 0; r0 < a.r; r0 += 16) {
      const int rk = r0 + (g & 1) * 8;
      float vv[8];
      if (tok_ok) {
        load8_f32<VEC>(vrow + rk, a.r - rk, vv);
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) vv[e] = 0.f;
      }
      uint32_t h[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t hi = from_f32<DT>(vv[e]);
        if (g < 2) {
          h[e] = hi;
        } else {
          const float hv = to_f32<DT>(hi);
          h[e] = __builtin_isfinite(hv) ? from_f32<DT>(vv[e] - hv) : 0u;
        }
      }
      const u32x4 bop = u32x4{pack2(h[0], h[1]), pack2(h[2], h[3]), pack2(h[4], h[5]),
                              pack2(h[6], h[7])};
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int c = n0 + (m >> 2) * 16 + qq * 4 + (m & 3);
        const u32x4 aop = (c < nq) ? load8_16<VEC>(Bl + (int64_t)c * a.r + rk, a.r - rk)
                                   : u32x4{0u, 0u, 0u, 0u};
        acc[qq] = mfma16x16x32<DT>(aop, bop, acc[qq]);
      }
    }

    // Lane (m, g) holds columns n0 + 16g + 4qq + e of token t.
    if (!tok_ok || ncols <= 0) continue;
    float out[16];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      out[qq * 4 + 0] = acc[qq].x;
      out[qq * 4 + 1] = acc[qq].y;
      out[qq * 4 + 2] = acc[qq].z;
      out[qq * 4 + 3] = acc[qq].w;
    }
    if (yvec) {
      u32x4* yp = reinterpret_cast<u32x4*>(yrow);
      if (a.add) {
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          const uint32_t d[4] = {w[hh].x, w[hh].y, w[hh].z, w[hh].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            out[hh * 8 + 2 * e] += to_f32<DT>(d[e] & 0xffffu);
            out[hh * 8 + 2 * e + 1] += to_f32<DT>(d[e] >> 16);
          }
        }
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        w[hh].x = pack2(from_f32<DT>(out[hh * 8 + 0]), from_f32<DT>(out[hh * 8 + 1]));
        w[hh].y = pack2(from_f32<DT>(out[hh * 8 + 2]), from_f32<DT>(out[hh * 8 + 3]));
        w[hh].z = pack2(from_f32<DT>(out[hh * 8 + 4]), from_f32<DT>(out[hh * 8 + 5]));
        w[hh].w = pack2(from_f32<DT>(out[hh * 8 + 6]), from_f32<DT>(out[hh * 8 + 7]));
      }
      yp[0] = w[0];
      yp[1] = w[1];
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        if (e < ncols) {
          float o = out[e];
          if (a.add) o += to_f32<DT>(yrow[e]);
          yrow[e] = (uint16_t)from_f32<DT>(o);
        }
      }
    }
  }
}

}  // namespace

hipError_t launch_expand(const SegView& seg, const float* v, int64_t ldv, int64_t v_slice_stride,
                         const ExpandSliceDesc* slices, int32_t num_slices, int32_t r,
                         uint16_t* y, int64_t ldy, int add, int dtype, bool vec, hipStream_t s) {
  ExpandArgs a{};
  a.seg = seg;
  a.v = v;
  a.ldv = ldv;
  a.v_slice_stride = v_slice_stride;
  a.num_slices = num_slices;
  a.r = r;
  a.y = y;
  a.ldy = ldy;
  a.add = add;
  int32_t ct = 0;
  for (int q = 0; q < num_slices; ++q) {
    a.slices[q] = slices[q];
    a.col_tile_start[q] = ct;
    ct += (slices[q].n + kExpandCols - 1) / kExpandCols;
  }
  a.col_tile_start[num_slices] = ct;
  const int64_t mt_max = seg.T > 0 ? (seg.T + kTileTokens - 1) / kTileTokens + (seg.L < seg.T ? seg.L : seg.T) : 0;
  int64_t items = mt_max * ct;
  int64_t grid = items < 2048 ? items : 2048;
  grid = (grid + 7) / 8 * 8;
  if (grid < 8) grid = 8;
  if (dtype == 0) {
    if (vec)
      hipLaunchKernelGGL((expand_sgmv_kernel<0, true>), dim3(grid), dim3(kExpandThreads), 0, s, a);
    else
      hipLaunchKernelGGL((expand_sgmv_kernel<0, false>), dim3(grid), dim3(kExpandThreads), 0, s, a);
  } else {
    if (vec)
      hipLaunchKernelGGL((expand_sgmv_kernel<1, true>), dim3(grid), dim3(kExpandThreads), 0, s, a);
    else
      hipLaunchKernelGGL((expand_sgmv_kernel<1, false>), dim3(grid), dim3(kExpandThreads), 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace lora
