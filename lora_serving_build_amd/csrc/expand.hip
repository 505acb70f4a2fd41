// Expand / expand_slice on segments (SGMV form):
//   y[t, off_s + c] = (add ? y : 0) + sum_j v_s[t, j] * B_{s,l}[j, c].
//
// Work item = (run of 128-column chunks of one slice, 64-token tile of one
// segment).  The four waves of a workgroup each take 16 tokens of the tile.
// Per item, each wave converts its tokens' fp32 v once into the matrix-core
// operand: v is split into hi = round(v) and lo = round(v - hi) in the data
// type, lane groups 0 and 1 carry hi and groups 2 and 3 carry lo against the
// same 16 weights, so one 16x16x32 op adds B^T (hi + lo) and v keeps about 16
// significant bits.  Per chunk, the weight block (128 rows of B_l^T, one
// contiguous 128 x r run in memory) is loaded by the whole workgroup with
// linear 16-byte loads one chunk ahead and staged in LDS, so all waves share
// one copy.  The product is computed transposed, D[c][token], and goes through
// a per-wave fp32 tile in LDS so that the read-modify-write of y -- the bulk
// of the traffic -- uses 16 lanes per row and 256 contiguous bytes per row and
// instruction.  The next chunk's y is loaded during the current chunk; y is
// rounded once, to nearest even.
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
  int32_t run_start[kMaxSlices + 1];  // prefix of chunk runs per slice
  int32_t num_slices;
  int32_t cpr;                        // chunks per run
  int32_t r;
  uint16_t* y;
  int64_t ldy;
  int32_t add;
};

constexpr int kEpiPitch = kExpandCols + 4;  // floats per row of a wave's staging tile

// NKS = 16-wide steps of r (r <= 16 * NKS).  VEC: 16-byte aligned rows, r and
// the slice offsets multiples of 8, ldy a multiple of 8.
template <int DT, bool VEC, int NKS>
__global__ __launch_bounds__(kExpandThreads) void expand_kernel(ExpandArgs a) {
  constexpr int RK = 16 * NKS;                   // padded rank
  constexpr int BP = RK + 8;                     // 16-bit elements per LDS weight row
  constexpr int PPR = RK / 8;                    // 16-byte pieces per weight row
  constexpr int BL = kExpandCols * PPR / kExpandThreads;  // pieces per thread per chunk
  constexpr int NQ = kExpandCols / 16;           // 16-column op tiles per chunk
  __shared__ __align__(16) uint16_t s_b[kExpandCols * BP];
  __shared__ __align__(16) float s_epi[kExpandThreads / kWave][16 * kEpiPitch];
  __shared__ int32_t s_tile_start[kMaxLoras + 1];
  __shared__ int32_t s_scan[kExpandThreads / kWave + 1];
  __shared__ int32_t s_tok[kTileTokens];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int m = lane & 15;  // token of the ops / weight row inside a 16-row tile
  const int g = lane >> 4;  // lane group
  const int er = lane >> 4;        // epilogue: rows er + 4 i of the wave's 16 tokens
  const int ec = (lane & 15) * 8;  // epilogue: 8 consecutive columns
  float* epi = s_epi[wave];

  int S;
  const int mtiles = build_tile_prefix<kExpandThreads>(a.seg, kTileTokens, s_tile_start, s_scan, &S);
  const int nruns = a.run_start[a.num_slices];
  const int n_items = mtiles * nruns;
  const int grid = gridDim.x;

  for (int item = xcd_logical_id(blockIdx.x, grid); item < n_items; item += grid) {
    // Consecutive items walk the token tiles under one run of columns, so
    // the weight run is reused from the L2 of one XCD.
    const int cr = item / mtiles;
    const int mt = item - cr * mtiles;
    int q = 0;
    while (q + 1 < a.num_slices && a.run_start[q + 1] <= cr) ++q;
    const int nq = a.slices[q].n;
    const int c_beg = (cr - a.run_start[q]) * a.cpr;
    const int c_end = min(c_beg + a.cpr, (nq + kExpandCols - 1) / kExpandCols);

    int p0 = 0, p_end = 0, l = 0;
    const bool ok = tile_range(a.seg, kTileTokens, s_tile_start, S, mt, &p0, &p_end, &l);
    if (tid < kTileTokens) {
      int t = -1;
      if (ok && p0 + tid < p_end) {
        t = a.seg.sorted_token[p0 + tid];
        if (t < 0 || t >= a.seg.T) t = -1;
      }
      s_tok[tid] = t;
    }
    __syncthreads();
    const bool wave_live = ok && p0 + wave * 16 < p_end;
    const uint16_t* Bl = a.slices[q].B + (int64_t)l * nq * a.r;
    uint16_t* ybase = a.y + a.slices[q].col_off;

    // v of this wave's 16 tokens as hi / lo operands, once per item.
    u32x4 bop[NKS];
    {
      const int t = s_tok[wave * 16 + m];
      const bool tok_ok = wave_live && t >= 0;
      const float* vrow = a.v + (int64_t)(tok_ok ? t : 0) * a.ldv + (int64_t)q * a.v_slice_stride;
#pragma unroll
      for (int st = 0; st < NKS; ++st) {
        const int rk = st * 16 + (g & 1) * 8;
        float vv[8];
        if (tok_ok) {
          load8_f32<VEC>(vrow + rk, a.r - rk, vv);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) vv[e] = 0.f;
        }
        uint32_t w4[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t hi = cvt_pack2<DT>(vv[2 * e], vv[2 * e + 1]);
          float h0, h1;
          unpack2<DT>(hi, &h0, &h1);
          const float l0 = __builtin_isfinite(h0) ? vv[2 * e] - h0 : 0.f;
          const float l1 = __builtin_isfinite(h1) ? vv[2 * e + 1] - h1 : 0.f;
          const uint32_t lo = cvt_pack2<DT>(l0, l1);
          w4[e] = g < 2 ? hi : lo;
        }
        bop[st] = u32x4{w4[0], w4[1], w4[2], w4[3]};
      }
    }

    // Weight chunk loader: piece p = tid + 256 i is row p / PPR, columns
    // 8 (p % PPR) .. +8 of the chunk's B_l^T rows.  Rows past the slice read
    // the last row (their outputs are dropped); ranks >= r read zero.
    u32x4 rb[BL];
    auto gload_b = [&](int c) {
#pragma unroll
      for (int i = 0; i < BL; ++i) {
        const int p = tid + kExpandThreads * i;
        const int row = p / PPR;
        const int col = (p - row * PPR) * 8;
        int n = c * kExpandCols + row;
        n = n < nq ? n : nq - 1;
        if constexpr (VEC)
          rb[i] = load8_16<true>(Bl + (int64_t)n * a.r + col, a.r - col);
        else
          rb[i] = load8_16<false>(Bl + (int64_t)n * a.r + col, a.r - col);
      }
    };
    auto swrite_b = [&]() {
#pragma unroll
      for (int i = 0; i < BL; ++i) {
        const int p = tid + kExpandThreads * i;
        const int row = p / PPR;
        const int col = (p - row * PPR) * 8;
        *reinterpret_cast<u32x4*>(&s_b[row * BP + col]) = rb[i];
      }
    };
    // y rows of this lane for chunk c (vector path only; zeros otherwise).
    auto gload_y = [&](int c, u32x4* yv) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        yv[i] = u32x4{0u, 0u, 0u, 0u};
        if constexpr (VEC) {
          const int tt = s_tok[wave * 16 + er + 4 * i];
          const int col = c * kExpandCols + ec;
          if (a.add && wave_live && tt >= 0 && nq - col >= 8)
            yv[i] = *reinterpret_cast<const u32x4*>(ybase + (int64_t)tt * a.ldy + col);
        }
      }
    };

    u32x4 ycur[4], ynext[4];
    if (c_beg < c_end) {
      gload_b(c_beg);
      swrite_b();
      gload_y(c_beg, ycur);
    }
    __syncthreads();
    for (int c = c_beg; c < c_end; ++c) {
      const bool has_next = c + 1 < c_end;
      if (has_next) {
        gload_b(c + 1);
        gload_y(c + 1, ynext);
      }
      if (wave_live) {
        f32x4 acc[NQ];
#pragma unroll
        for (int qq = 0; qq < NQ; ++qq) acc[qq] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < NKS; ++st) {
#pragma unroll
          for (int qq = 0; qq < NQ; ++qq) {
            const u32x4 aop = *reinterpret_cast<const u32x4*>(
                &s_b[(qq * 16 + m) * BP + st * 16 + (g & 1) * 8]);
            acc[qq] = mfma16x16x32<DT>(aop, bop[st], acc[qq]);
          }
        }
        // Lane (m, g) holds columns 16 qq + 4 g + e of token row m.
#pragma unroll
        for (int qq = 0; qq < NQ; ++qq)
          *reinterpret_cast<f32x4*>(epi + m * kEpiPitch + qq * 16 + 4 * g) = acc[qq];
        // Only this wave reads its staging tile; LDS operations of one wave
        // execute in order, so a wavefront-scope fence is enough.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int col = c * kExpandCols + ec;
        const int cvalid = nq - col;
        if (cvalid > 0) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int row = er + 4 * i;
            const int tt = s_tok[wave * 16 + row];
            if (tt < 0) continue;
            const f32x4 o0 = *reinterpret_cast<const f32x4*>(epi + row * kEpiPitch + ec);
            const f32x4 o1 = *reinterpret_cast<const f32x4*>(epi + row * kEpiPitch + ec + 4);
            float out[8] = {o0.x, o0.y, o0.z, o0.w, o1.x, o1.y, o1.z, o1.w};
            uint16_t* yp = ybase + (int64_t)tt * a.ldy + col;
            if (VEC && cvalid >= 8) {
              if (a.add) {
                const uint32_t d[4] = {ycur[i].x, ycur[i].y, ycur[i].z, ycur[i].w};
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                  float y0, y1;
                  unpack2<DT>(d[e], &y0, &y1);
                  out[2 * e] += y0;
                  out[2 * e + 1] += y1;
                }
              }
              *reinterpret_cast<u32x4*>(yp) =
                  u32x4{cvt_pack2<DT>(out[0], out[1]), cvt_pack2<DT>(out[2], out[3]),
                        cvt_pack2<DT>(out[4], out[5]), cvt_pack2<DT>(out[6], out[7])};
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
      }
      __syncthreads();  // every wave is done with this chunk's weights
      if (has_next) {
        swrite_b();
#pragma unroll
        for (int i = 0; i < 4; ++i) ycur[i] = ynext[i];
      }
      __syncthreads();
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
  const int64_t mt_max = seg.T > 0 ? (seg.T + kTileTokens - 1) / kTileTokens + (seg.L < seg.T ? seg.L : seg.T) : 0;
  int64_t chunks = 0;
  for (int q = 0; q < num_slices; ++q) chunks += (slices[q].n + kExpandCols - 1) / kExpandCols;
  // Chunks per run: long runs amortise an item's set-up and keep each y row
  // streaming, but leave a few items per resident workgroup.
  int64_t cpr = mt_max * chunks / 2048;
  if (cpr > 16) cpr = 16;
  if (cpr < 1) cpr = 1;
  if (const char* e = getenv("LORA_EXPAND_CPR")) {
    const long f = atol(e);
    if (f >= 1) cpr = f;
  }
  a.cpr = (int32_t)cpr;
  int32_t runs = 0;
  for (int q = 0; q < num_slices; ++q) {
    a.slices[q] = slices[q];
    a.run_start[q] = runs;
    const int64_t cq = (slices[q].n + kExpandCols - 1) / kExpandCols;
    runs += (int32_t)((cq + cpr - 1) / cpr);
  }
  a.run_start[num_slices] = runs;
  int64_t items = mt_max * runs;
  // Two resident workgroups per CU (LDS bound).
  int64_t grid = items < 512 ? items : 512;
  grid = (grid + 7) / 8 * 8;
  if (grid < 8) grid = 8;
  const int nks = r <= 16 ? 1 : r <= 32 ? 2 : r <= 64 ? 4 : 8;
#define LORA_EXPAND_LAUNCH(DT_, VEC_)                                                                \
  switch (nks) {                                                                                    \
    case 1: hipLaunchKernelGGL((expand_kernel<DT_, VEC_, 1>), dim3(grid), dim3(kExpandThreads), 0, s, a); break; \
    case 2: hipLaunchKernelGGL((expand_kernel<DT_, VEC_, 2>), dim3(grid), dim3(kExpandThreads), 0, s, a); break; \
    case 4: hipLaunchKernelGGL((expand_kernel<DT_, VEC_, 4>), dim3(grid), dim3(kExpandThreads), 0, s, a); break; \
    default: hipLaunchKernelGGL((expand_kernel<DT_, VEC_, 8>), dim3(grid), dim3(kExpandThreads), 0, s, a); break; \
  }
  if (dtype == 0) {
    if (vec) { LORA_EXPAND_LAUNCH(0, true) } else { LORA_EXPAND_LAUNCH(0, false) }
  } else {
    if (vec) { LORA_EXPAND_LAUNCH(1, true) } else { LORA_EXPAND_LAUNCH(1, false) }
  }
#undef LORA_EXPAND_LAUNCH
  return hipGetLastError();
}

}  // namespace lora
