// Shrink on segments (SGMV form): v[t, j] = sum_h x[t, h] * A_l[h, j].
//
// Work item = (token tile of one segment, chunk of H).  A workgroup of four
// waves takes one item at a time from a persistent grid; wave w owns tokens
// 16w..16w+15 of the tile.  Per H step of 128 every lane loads 64 contiguous
// bytes of its token's x row and of one A_l row (lane group g = lane / 16
// covers elements 32g..32g+31), and four 16x16x32 matrix-core ops accumulate
// the transposed product D[j][token] in fp32.  Transposing puts four
// consecutive j of one token in a lane, so v is written with 16-byte stores.
//
// When H is split over several chunks (small batches need more workgroups than
// they have tiles), each item stores its fp32 partial tile in the workspace,
// and the last of the chunks of a tile to arrive (a wrapping counter,
// atomicInc) adds the partials in chunk order and stores v: one launch, a
// fixed summation order, and the counter is back at zero afterwards.
#include "lora_device.h"
#include "lora_kernels.h"
#include "tiles.h"

namespace lora {

namespace {

constexpr int kShrinkThreads = 256;

struct ShrinkArgs {
  SegView seg;
  const uint16_t* x;
  int64_t ldx;
  const uint16_t* A;
  int32_t H;
  int32_t r;
  float* v;
  int64_t ldv;
  float* partial;
  uint32_t* counter;
  int32_t ksplit;
  int32_t kchunk;
  int32_t max_tiles;
};

// Stores four consecutive j values of one v row (j0 = first), clipped at r.
template <bool VEC>
__device__ __forceinline__ void store_v4(float* p, int j0, int r, f32x4 val) {
  if (VEC && j0 + 4 <= r) {
    *reinterpret_cast<f32x4*>(p) = val;
    return;
  }
  if (j0 + 0 < r) p[0] = val.x;
  if (j0 + 1 < r) p[1] = val.y;
  if (j0 + 2 < r) p[2] = val.z;
  if (j0 + 3 < r) p[3] = val.w;
}

// NJT = number of 16-row tiles of r (r <= 16 * NJT).
template <int DT, bool VEC, int NJT>
__global__ __launch_bounds__(kShrinkThreads) void shrink_sgmv_kernel(ShrinkArgs a) {
  __shared__ int32_t s_tile_start[kMaxLoras + 1];
  __shared__ int32_t s_scan[kShrinkThreads / kWave + 1];
  __shared__ int32_t s_last;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int m = lane & 15;  // token column of the wave's 16x16 tiles / row of A
  const int g = lane >> 4;  // lane group: which 32 elements of each H step

  int S;
  const int tiles = build_tile_prefix<kShrinkThreads>(a.seg, s_tile_start, s_scan, &S);
  const int n_items = tiles * a.ksplit;
  const int grid = gridDim.x;

  for (int item = xcd_logical_id(blockIdx.x, grid); item < n_items; item += grid) {
    // Consecutive items share the chunk of H and walk the tiles of a
    // segment, so one A_l chunk serves neighbouring workgroups of an XCD.
    const int ks = item / tiles;
    const int tile = item - ks * tiles;
    int p0 = 0, p_end = 0, l = 0;
    const bool ok = tile < a.max_tiles &&
                    tile_range(a.seg, s_tile_start, S, tile, &p0, &p_end, &l);
    const int k0 = ks * a.kchunk;
    const int k1 = min(k0 + a.kchunk, a.H);
    const int pw = p0 + wave * 16;
    const bool wave_live = ok && pw < p_end;
    const int t_raw = (wave_live && pw + m < p_end) ? a.seg.sorted_token[pw + m] : -1;
    const bool tok_ok = t_raw >= 0 && t_raw < a.seg.T;
    const int t = tok_ok ? t_raw : 0;

    f32x4 acc[NJT];
#pragma unroll
    for (int jt = 0; jt < NJT; ++jt) acc[jt] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (wave_live) {
      const uint16_t* xrow = a.x + (int64_t)t * a.ldx;
      const uint16_t* Al = a.A + (int64_t)l * a.r * a.H;
      for (int k = k0; k < k1; k += kShrinkKStep) {
        const int kl = k + g * 32;
        u32x4 xv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          xv[i] = tok_ok ? load8_16<VEC>(xrow + kl + i * 8, k1 - (kl + i * 8))
                         : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int jt = 0; jt < NJT; ++jt) {
          const int j = jt * 16 + m;
          const uint16_t* arow = Al + (int64_t)j * a.H;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const u32x4 av = (j < a.r) ? load8_16<VEC>(arow + kl + i * 8, k1 - (kl + i * 8))
                                       : u32x4{0u, 0u, 0u, 0u};
            acc[jt] = mfma16x16x32<DT>(av, xv[i], acc[jt]);
          }
        }
      }
    }

    if (a.ksplit == 1) {
      if (tok_ok) {
        float* vrow = a.v + (int64_t)t * a.ldv;
#pragma unroll
        for (int jt = 0; jt < NJT; ++jt) {
          const int j0 = jt * 16 + 4 * g;
          store_v4<VEC>(vrow + j0, j0, a.r, acc[jt]);
        }
      }
      continue;
    }

    // Split H: publish the partial tile, then let the last chunk reduce.
    constexpr int RP = NJT * 16;
    if (wave_live) {
      float* part = a.partial + ((int64_t)(tile * a.ksplit + ks) * kTileTokens + wave * 16 + m) * RP;
#pragma unroll
      for (int jt = 0; jt < NJT; ++jt)
        *reinterpret_cast<f32x4*>(part + jt * 16 + 4 * g) = acc[jt];
    }
    __threadfence();
    __syncthreads();
    if (tid == 0)
      s_last = ok ? (atomicInc(&a.counter[tile], (uint32_t)(a.ksplit - 1)) ==
                     (uint32_t)(a.ksplit - 1))
                  : 0;
    __syncthreads();
    if (s_last) {
      __threadfence();
      if (tok_ok) {
        float* vrow = a.v + (int64_t)t * a.ldv;
        const float* base = a.partial + ((int64_t)tile * a.ksplit * kTileTokens + wave * 16 + m) * RP;
#pragma unroll
        for (int jt = 0; jt < NJT; ++jt) {
          f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
          for (int q = 0; q < a.ksplit; ++q) {
            sum += *reinterpret_cast<const f32x4*>(base + (int64_t)q * kTileTokens * RP + jt * 16 + 4 * g);
          }
          const int j0 = jt * 16 + 4 * g;
          store_v4<VEC>(vrow + j0, j0, a.r, sum);
        }
      }
    }
    __syncthreads();
  }
}

template <int DT, bool VEC>
hipError_t launch_typed(const ShrinkArgs& args, int njt, int grid, hipStream_t s) {
  switch (njt) {
    case 1:
      hipLaunchKernelGGL((shrink_sgmv_kernel<DT, VEC, 1>), dim3(grid), dim3(kShrinkThreads), 0, s, args);
      break;
    case 2:
      hipLaunchKernelGGL((shrink_sgmv_kernel<DT, VEC, 2>), dim3(grid), dim3(kShrinkThreads), 0, s, args);
      break;
    case 4:
      hipLaunchKernelGGL((shrink_sgmv_kernel<DT, VEC, 4>), dim3(grid), dim3(kShrinkThreads), 0, s, args);
      break;
    default:
      hipLaunchKernelGGL((shrink_sgmv_kernel<DT, VEC, 8>), dim3(grid), dim3(kShrinkThreads), 0, s, args);
      break;
  }
  return hipGetLastError();
}

int rank_tiles(int r) { return r <= 16 ? 1 : r <= 32 ? 2 : r <= 64 ? 4 : 8; }

}  // namespace

ShrinkPlan plan_shrink(int32_t T, int32_t L, int32_t H, int32_t r) {
  ShrinkPlan p{};
  const int64_t tiles = T > 0 ? (T + kTileTokens - 1) / kTileTokens + (L < T ? L : T) : 0;
  p.max_tiles = (int32_t)tiles;
  // Enough items for about two workgroups per CU, but no chunk below 256
  // elements of H.
  const int64_t want = 512;
  int64_t ks = tiles > 0 ? (want + tiles - 1) / tiles : 1;
  const int64_t ks_max = (H + 255) / 256;
  if (ks > ks_max) ks = ks_max;
  if (ks < 1) ks = 1;
  if (const char* e = getenv("LORA_SHRINK_KSPLIT")) {
    const long f = atol(e);
    if (f >= 1) ks = f;
  }
  int64_t chunk = (H + ks - 1) / ks;
  chunk = (chunk + kShrinkKStep - 1) / kShrinkKStep * kShrinkKStep;
  ks = (H + chunk - 1) / chunk;
  p.ksplit = (int32_t)ks;
  p.kchunk = (int32_t)chunk;
  const int64_t rp = 16 * rank_tiles(r);
  p.partial_bytes = ks > 1 ? (size_t)(tiles * ks * kTileTokens * rp * 4) : 0;
  p.counter_bytes = ks > 1 ? (size_t)((tiles * 4 + 255) / 256 * 256) : 0;
  int64_t items = tiles * ks;
  int64_t grid = items < 2048 ? items : 2048;
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
  a.counter = reinterpret_cast<uint32_t*>(workspace);
  a.partial = plan.ksplit > 1
                  ? reinterpret_cast<float*>(static_cast<char*>(workspace) + plan.counter_bytes)
                  : nullptr;
  a.ksplit = plan.ksplit;
  a.kchunk = plan.kchunk;
  a.max_tiles = plan.max_tiles;
  const int njt = rank_tiles(r);
  if (dtype == 0)
    return vec ? launch_typed<0, true>(a, njt, plan.grid, s) : launch_typed<0, false>(a, njt, plan.grid, s);
  return vec ? launch_typed<1, true>(a, njt, plan.grid, s) : launch_typed<1, false>(a, njt, plan.grid, s);
}

}  // namespace lora
