// Shrink on segments (SGMV form): v[t, j] = sum_h x[t, h] * A_l[h, j].
//
// One workgroup of four waves owns a 64-token tile of one segment and a range
// of H (the whole of H unless the batch has too few tiles to fill the GPU).
// H is walked in blocks of 128: the block of x (64 rows x 256 B) and of A_l
// (r rows x 256 B) is loaded cooperatively -- 16 lanes per row, so one load
// instruction covers 4 rows x 256 contiguous bytes -- into registers one
// block ahead, then written to a double-buffered LDS tile.  A_l is thus read
// from L2 once per 64 tokens instead of once per 16, and the matrix cores take
// their operands from LDS (row pitch padded to 272 B, which spreads the 16 rows
// of an operand read over all banks).  Wave w multiplies tokens 16w..16w+15
// against all of r with 16x16x32 ops, accumulating the transposed product
// D[j][token] in fp32, so each lane ends with four consecutive j of one token.
//
// When H is split across workgroups (ks chunks), each chunk writes its fp32
// partial rows to the workspace (indexed by sorted position) and a second
// small kernel adds the ks partials in chunk order and writes v: the kernel
// boundary orders the two, and the sum order is fixed.
#include "lora_device.h"
#include "lora_kernels.h"
#include "tiles.h"

namespace lora {

namespace {

constexpr int kShrinkThreads = 256;
constexpr int kSkTile = 64;              // tokens per tile (4 waves x 16)
constexpr int kSkKB = kShrinkKStep;      // H elements per LDS block
constexpr int kSkPitch = kSkKB + 8;      // 16-bit elements per LDS row
constexpr int kSkChunks = kSkKB / 8;     // 16-byte chunks per row and block

struct ShrinkArgs {
  SegView seg;
  const uint16_t* x;
  int64_t ldx;
  const uint16_t* A;
  int32_t H;
  int32_t r;
  float* v;
  int64_t ldv;
  float* partial;  // [ks][T][rp] when ks > 1
  int32_t ks;
  int32_t kchunk;  // H elements per workgroup chunk (multiple of kSkKB)
  int32_t rp;      // padded rank of the partial rows (16 * NJT)
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
template <int DT, bool VEC, int NJT>
__global__ __launch_bounds__(kShrinkThreads) void shrink_kernel(ShrinkArgs a) {
  constexpr int RP = 16 * NJT;
  constexpr int XL = kSkTile * kSkChunks / kShrinkThreads;  // x chunks per thread per block (4)
  constexpr int AL = RP * kSkChunks / kShrinkThreads;       // A chunks per thread per block (NJT)
  __shared__ __align__(16) uint16_t s_x[2][kSkTile * kSkPitch];
  __shared__ __align__(16) uint16_t s_a[2][RP * kSkPitch];
  __shared__ int32_t s_tile_start[kMaxLoras + 1];
  __shared__ int32_t s_scan[kShrinkThreads / kWave + 1];
  __shared__ int32_t s_tok[kSkTile];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int m = lane & 15;  // token column of D / row of A inside a 16-row tile
  const int g = lane >> 4;  // lane group: which 8 of the 32 elements of an op
  // Cooperative load layout: chunk c = tid + 256 i, row c / 16, 16-byte column c % 16.
  const int lrow = tid >> 4;
  const int lcol = (tid & 15) * 8;

  int S;
  const int tiles = build_tile_prefix<kShrinkThreads>(a.seg, kSkTile, s_tile_start, s_scan, &S);
  const int n_items = tiles * a.ks;
  const int grid = gridDim.x;

  for (int item = xcd_logical_id(blockIdx.x, grid); item < n_items; item += grid) {
    // Consecutive items share the chunk of H and walk the tiles of a segment,
    // so neighbouring workgroups of an XCD read the same A_l block.
    const int ksi = item / tiles;
    const int tile = item - ksi * tiles;
    int p0 = 0, p_end = 0, l = 0;
    const bool ok = tile_range(a.seg, kSkTile, s_tile_start, S, tile, &p0, &p_end, &l);
    if (tid < kSkTile) {
      int t = -1;
      if (ok && p0 + tid < p_end) {
        t = a.seg.sorted_token[p0 + tid];
        if (t < 0 || t >= a.seg.T) t = -1;
      }
      s_tok[tid] = t;
    }
    __syncthreads();
    const int kbeg = ksi * a.kchunk;
    const int kend = min(a.H, kbeg + a.kchunk);
    const int t_any = s_tok[0];
    // Rows of this thread's loads.  A missing token reads some valid row: its
    // output column is dropped.  Rows j >= r read row 0: output rows dropped.
    const uint16_t* xsrc[XL];
#pragma unroll
    for (int i = 0; i < XL; ++i) {
      const int tt = s_tok[lrow + 16 * i];
      xsrc[i] = a.x + (int64_t)(tt >= 0 ? tt : (t_any >= 0 ? t_any : 0)) * a.ldx;
    }
    const uint16_t* Al = a.A + (int64_t)l * a.r * a.H;
    const uint16_t* asrc[AL];
#pragma unroll
    for (int i = 0; i < AL; ++i) {
      const int j = lrow + 16 * i;
      asrc[i] = Al + (int64_t)(j < a.r ? j : 0) * a.H;
    }

    u32x4 rx[XL], ra[AL];
    auto gload = [&](int kb) {
      // Elements at or beyond kend read as zero (only the last block has any).
      const int off = kb + lcol;
#pragma unroll
      for (int i = 0; i < XL; ++i) {
        if constexpr (VEC)
          rx[i] = load8_16_masked(xsrc[i], off, kend, ok);
        else
          rx[i] = ok ? load8_16<false>(xsrc[i] + off, kend - off) : u32x4{0u, 0u, 0u, 0u};
      }
#pragma unroll
      for (int i = 0; i < AL; ++i) {
        if constexpr (VEC)
          ra[i] = load8_16_masked(asrc[i], off, kend, ok);
        else
          ra[i] = ok ? load8_16<false>(asrc[i] + off, kend - off) : u32x4{0u, 0u, 0u, 0u};
      }
    };
    auto swrite = [&](int buf) {
#pragma unroll
      for (int i = 0; i < XL; ++i)
        *reinterpret_cast<u32x4*>(&s_x[buf][(lrow + 16 * i) * kSkPitch + lcol]) = rx[i];
#pragma unroll
      for (int i = 0; i < AL; ++i)
        *reinterpret_cast<u32x4*>(&s_a[buf][(lrow + 16 * i) * kSkPitch + lcol]) = ra[i];
    };

    f32x4 acc[NJT];
#pragma unroll
    for (int jt = 0; jt < NJT; ++jt) acc[jt] = f32x4{0.f, 0.f, 0.f, 0.f};
    const bool wave_live = ok && p0 + wave * 16 < p_end;
    const int nblk = kend > kbeg ? (kend - kbeg + kSkKB - 1) / kSkKB : 0;

    if (nblk > 0) {
      gload(kbeg);
      swrite(0);
    }
    __syncthreads();
    for (int b = 0; b < nblk; ++b) {
      const int buf = b & 1;
      if (b + 1 < nblk) gload(kbeg + (b + 1) * kSkKB);  // in flight during the ops below
      if (wave_live) {
        const uint16_t* xs = &s_x[buf][(wave * 16 + m) * kSkPitch + 8 * g];
        const uint16_t* as = &s_a[buf][m * kSkPitch + 8 * g];
#pragma unroll
        for (int kk = 0; kk < kSkKB; kk += 32) {
          const u32x4 xop = *reinterpret_cast<const u32x4*>(xs + kk);
#pragma unroll
          for (int jt = 0; jt < NJT; ++jt) {
            const u32x4 aop = *reinterpret_cast<const u32x4*>(as + jt * 16 * kSkPitch + kk);
            acc[jt] = mfma16x16x32<DT>(aop, xop, acc[jt]);
          }
        }
      }
      if (b + 1 < nblk) swrite(buf ^ 1);
      __syncthreads();
    }

    // Lane (m, g) holds D[j = 16 jt + 4 g + e][token 16 wave + m].
    const int tt = s_tok[wave * 16 + m];
    if (wave_live && tt >= 0) {
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt) {
        const int j0 = jt * 16 + 4 * g;
        if (a.ks == 1) {
          store4<VEC>(a.v + (int64_t)tt * a.ldv + j0, j0, a.r, acc[jt]);
        } else {
          float* part = a.partial + ((int64_t)ksi * a.seg.T + (p0 + wave * 16 + m)) * a.rp + j0;
          *reinterpret_cast<f32x4*>(part) = acc[jt];
        }
      }
    }
    __syncthreads();
  }
}

// v[t, :r] = sum over the ks chunks of the partial rows, in chunk order.
template <bool VEC>
__global__ __launch_bounds__(256) void shrink_reduce_kernel(SegView seg, const float* partial,
                                                            int32_t ks, int32_t rp, int32_t r,
                                                            float* v, int64_t ldv) {
  int ta = seg.counts[1];
  ta = ta < 0 ? 0 : (ta > seg.T ? seg.T : ta);
  const int per_row = rp / 4;
  const int64_t n = (int64_t)ta * per_row;
  for (int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; o < n;
       o += (int64_t)gridDim.x * blockDim.x) {
    const int p = (int)(o / per_row);
    const int j0 = (int)(o - (int64_t)p * per_row) * 4;
    if (j0 >= r) continue;
    const int t = seg.sorted_token[p];
    if (t < 0 || t >= seg.T) continue;
    f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int q = 0; q < ks; ++q)
      sum += *reinterpret_cast<const f32x4*>(partial + ((int64_t)q * seg.T + p) * rp + j0);
    store4<VEC>(v + (int64_t)t * ldv + j0, j0, r, sum);
  }
}

template <int DT, bool VEC>
hipError_t launch_typed(const ShrinkArgs& args, int njt, int grid, hipStream_t s) {
  switch (njt) {
    case 1:
      hipLaunchKernelGGL((shrink_kernel<DT, VEC, 1>), dim3(grid), dim3(kShrinkThreads), 0, s, args);
      break;
    case 2:
      hipLaunchKernelGGL((shrink_kernel<DT, VEC, 2>), dim3(grid), dim3(kShrinkThreads), 0, s, args);
      break;
    case 4:
      hipLaunchKernelGGL((shrink_kernel<DT, VEC, 4>), dim3(grid), dim3(kShrinkThreads), 0, s, args);
      break;
    default:
      hipLaunchKernelGGL((shrink_kernel<DT, VEC, 8>), dim3(grid), dim3(kShrinkThreads), 0, s, args);
      break;
  }
  return hipGetLastError();
}

int env_int(const char* name, int dflt) {
  const char* e = getenv(name);
  if (!e) return dflt;
  const long v = atol(e);
  return v > 0 ? (int)v : dflt;
}

}  // namespace

ShrinkPlan plan_shrink(int32_t T, int32_t L, int32_t H, int32_t r) {
  ShrinkPlan p{};
  const int njt0 = (r + 15) / 16;
  p.jtw = njt0 <= 1 ? 1 : njt0 <= 2 ? 2 : njt0 <= 4 ? 4 : 8;  // rank tiles (template)
  p.rp = 16 * p.jtw;
  p.mw = kSkTile / 16;
  p.jg = 1;
  p.kw = 1;
  const int64_t tiles = T > 0 ? (T + kSkTile - 1) / kSkTile + (L < T ? L : T) : 0;
  p.max_tiles = (int32_t)tiles;
  // Split H across workgroups when the tiles alone leave CUs idle; keep at
  // least two LDS blocks per chunk.
  int64_t ks = 1;
  if (tiles > 0 && tiles < 384) ks = (512 + tiles - 1) / tiles;
  const int64_t ks_max = (H + 2 * kSkKB - 1) / (2 * kSkKB);
  if (ks > ks_max) ks = ks_max;
  if (ks < 1) ks = 1;
  ks = env_int("LORA_SHRINK_KSPLIT", (int)ks);
  int64_t chunk = (H + ks - 1) / ks;
  chunk = (chunk + kSkKB - 1) / kSkKB * kSkKB;
  ks = (H + chunk - 1) / chunk;
  p.ksplit = (int32_t)ks;
  p.kchunk = (int32_t)chunk;
  p.partial_bytes = ks > 1 ? (size_t)(ks * (int64_t)T * p.rp * 4) : 0;
  p.counter_bytes = 0;
  int64_t items = tiles * ks;
  int64_t grid = items < 1024 ? items : 1024;
  grid = (grid + 7) / 8 * 8;
  if (grid < 8) grid = 8;
  p.grid = (int32_t)grid;
  return p;
}

hipError_t launch_shrink(const SegView& seg, const uint16_t* x, int64_t ldx, const uint16_t* A,
                         int32_t H, int32_t r, float* v, int64_t ldv, void* workspace,
                         const ShrinkPlan& plan, int dtype, bool vec, hipStream_t s) {
  ShrinkArgs a{};
  a.seg = seg;
  a.x = x;
  a.ldx = ldx;
  a.A = A;
  a.H = H;
  a.r = r;
  a.v = v;
  a.ldv = ldv;
  a.partial = plan.ksplit > 1 ? reinterpret_cast<float*>(workspace) : nullptr;
  a.ks = plan.ksplit;
  a.kchunk = plan.kchunk;
  a.rp = plan.rp;
  hipError_t e;
  if (dtype == 0)
    e = vec ? launch_typed<0, true>(a, plan.jtw, plan.grid, s) : launch_typed<0, false>(a, plan.jtw, plan.grid, s);
  else
    e = vec ? launch_typed<1, true>(a, plan.jtw, plan.grid, s) : launch_typed<1, false>(a, plan.jtw, plan.grid, s);
  if (e != hipSuccess || plan.ksplit == 1) return e;
  int64_t blocks = ((int64_t)seg.T * (plan.rp / 4) + 255) / 256;
  if (blocks > 1024) blocks = 1024;
  if (blocks < 1) blocks = 1;
  if (vec)
    hipLaunchKernelGGL((shrink_reduce_kernel<true>), dim3((unsigned)blocks), dim3(256), 0, s, seg,
                       a.partial, plan.ksplit, plan.rp, r, v, ldv);
  else
    hipLaunchKernelGGL((shrink_reduce_kernel<false>), dim3((unsigned)blocks), dim3(256), 0, s, seg,
                       a.partial, plan.ksplit, plan.rp, r, v, ldv);
  return hipGetLastError();
}

}  // namespace lora
