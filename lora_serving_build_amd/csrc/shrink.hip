// Shrink on segments (SGMV form): v[t, j] = sum_h x[t, h] * A_l[h, j].
//
// One workgroup of 16 waves takes one token tile of one segment at a time
// (persistent grid).  The 16 waves are arranged as
//   mw token groups (16 tokens each) x jg rank groups x kw slices of H,
// with mw * jg * kw = 16.  Per H step of 128 every lane loads 64 contiguous
// bytes of its token's x row and of one A_l row (lane group g = lane / 16
// covers elements 32g..32g+31) and 16x16x32 matrix-core ops accumulate the
// transposed product D[j][token] in fp32.  The kw partial tiles of a token
// group meet in LDS and are added in slice order, so the result does not
// depend on timing; there is no device-scope fence or atomic on the path.
//
// Batches with too few tiles to occupy the chip also split H across
// workgroups (ks chunks).  Each chunk then writes its fp32 partial tile to the
// workspace (indexed by sorted position) and a second small kernel adds the ks
// partials in chunk order and writes v: the kernel boundary orders the two.
#include "lora_device.h"
#include "lora_kernels.h"
#include "tiles.h"

namespace lora {

namespace {

constexpr int kShrinkWaves = 16;
constexpr int kShrinkThreads = kShrinkWaves * kWave;

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
  int32_t kchunk;  // H elements per workgroup chunk (multiple of kShrinkKStep)
  int32_t mw, jg, kw;
  int32_t rp;      // padded rank of the partial rows (= jg * JTW * 16)
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

// JTW = 16-row tiles of r per wave (1 or 2).
template <int DT, bool VEC, int JTW>
__global__ __launch_bounds__(kShrinkThreads) void shrink_kernel(ShrinkArgs a) {
  __shared__ int32_t s_tile_start[kMaxLoras + 1];
  __shared__ int32_t s_scan[kShrinkWaves + 1];
  __shared__ int32_t s_tok[kMaxShrinkTile];
  __shared__ f32x4 s_red[kShrinkWaves * 16 * JTW * 4];

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int m = lane & 15;  // token column of D / row of A inside a 16-row tile
  const int g = lane >> 4;  // lane group
  const int kw = a.kw, jg = a.jg, mw = a.mw;
  const int kg = wave % kw;
  const int jgi = (wave / kw) % jg;
  const int mg = wave / (kw * jg);
  const int tile_tokens = 16 * mw;
  constexpr int CH = JTW * 4;  // f32x4 chunks per (wave, token) row of s_red

  int S;
  const int tiles = build_tile_prefix<kShrinkThreads>(a.seg, tile_tokens, s_tile_start, s_scan, &S);
  const int n_items = tiles * a.ks;
  const int grid = gridDim.x;

  for (int item = xcd_logical_id(blockIdx.x, grid); item < n_items; item += grid) {
    // Consecutive items share the chunk of H and walk the tiles of a segment.
    const int ksi = item / tiles;
    const int tile = item - ksi * tiles;
    int p0 = 0, p_end = 0, l = 0;
    const bool ok = tile_range(a.seg, tile_tokens, s_tile_start, S, tile, &p0, &p_end, &l);
    if (tid < tile_tokens) {
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
    int wspan = (kend - kbeg + kw - 1) / kw;
    wspan = (wspan + kShrinkKStep - 1) / kShrinkKStep * kShrinkKStep;
    const int k0 = kbeg + kg * wspan;
    const int k1 = min(kend, k0 + wspan);
    const int t = s_tok[mg * 16 + m];
    const bool tok_ok = t >= 0;
    const bool wave_live = ok && p0 + mg * 16 < p_end;

    f32x4 acc[JTW];
#pragma unroll
    for (int jj = 0; jj < JTW; ++jj) acc[jj] = f32x4{0.f, 0.f, 0.f, 0.f};

    if (wave_live) {
      const uint16_t* xrow = a.x + (int64_t)(tok_ok ? t : 0) * a.ldx;
      const uint16_t* Al = a.A + (int64_t)l * a.r * a.H;
      for (int k = k0; k < k1; k += kShrinkKStep) {
        const int kl = k + g * 32;
        u32x4 xv[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          xv[i] = tok_ok ? load8_16<VEC>(xrow + kl + i * 8, k1 - (kl + i * 8))
                         : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int jj = 0; jj < JTW; ++jj) {
          const int j = (jgi * JTW + jj) * 16 + m;
          const uint16_t* arow = Al + (int64_t)j * a.H;
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const u32x4 av = (j < a.r) ? load8_16<VEC>(arow + kl + i * 8, k1 - (kl + i * 8))
                                       : u32x4{0u, 0u, 0u, 0u};
            acc[jj] = mfma16x16x32<DT>(av, xv[i], acc[jj]);
          }
        }
      }
    }
    // Lane (m, g) holds D[j = 16 jj + 4 g + e][token m] of its rank group.
#pragma unroll
    for (int jj = 0; jj < JTW; ++jj) s_red[(wave * 16 + m) * CH + jj * 4 + g] = acc[jj];
    __syncthreads();

    // Add the kw slices of H in order and write v (or the chunk's partial).
    const int chunks_per_tok = jg * CH;
    const int n_out = tile_tokens * chunks_per_tok;
    for (int o = tid; o < n_out; o += kShrinkThreads) {
      const int tokl = o / chunks_per_tok;
      const int c = o - tokl * chunks_per_tok;
      const int jgo = c / CH;
      const int cc = c - jgo * CH;
      const int mgo = tokl >> 4;
      const int mm = tokl & 15;
      const int tt = s_tok[tokl];
      if (tt < 0) continue;
      f32x4 sum = f32x4{0.f, 0.f, 0.f, 0.f};
      const int wbase = (mgo * jg + jgo) * kw;
      for (int q = 0; q < kw; ++q) sum += s_red[((wbase + q) * 16 + mm) * CH + cc];
      const int j0 = jgo * JTW * 16 + (cc >> 2) * 16 + (cc & 3) * 4;
      if (a.ks == 1) {
        store4<VEC>(a.v + (int64_t)tt * a.ldv + j0, j0, a.r, sum);
      } else {
        float* part = a.partial + ((int64_t)ksi * a.seg.T + (p0 + tokl)) * a.rp + j0;
        *reinterpret_cast<f32x4*>(part) = sum;
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
hipError_t launch_typed(const ShrinkArgs& args, int jtw, int grid, hipStream_t s) {
  if (jtw == 1)
    hipLaunchKernelGGL((shrink_kernel<DT, VEC, 1>), dim3(grid), dim3(kShrinkThreads), 0, s, args);
  else
    hipLaunchKernelGGL((shrink_kernel<DT, VEC, 2>), dim3(grid), dim3(kShrinkThreads), 0, s, args);
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
  const int njt = (r + 15) / 16;
  p.jtw = njt == 1 ? 1 : 2;
  const int need_jg = (njt + p.jtw - 1) / p.jtw;
  p.jg = need_jg <= 1 ? 1 : need_jg <= 2 ? 2 : 4;
  p.rp = p.jg * p.jtw * 16;
  // Token groups per workgroup: larger tiles reuse A_l across more tokens;
  // keep about one workgroup per CU or more.
  int mw = 1;
  while (mw * 2 * p.jg <= kShrinkWaves && mw * 2 <= kMaxShrinkTile / 16 &&
         (int64_t)T >= (int64_t)4096 * mw * 2)
    mw *= 2;
  mw = env_int("LORA_SHRINK_MW", mw);
  while (mw & (mw - 1)) mw &= mw - 1;  // powers of two only: mw * jg * kw must be 16
  if (mw > kMaxShrinkTile / 16) mw = kMaxShrinkTile / 16;
  if (mw * p.jg > kShrinkWaves) mw = kShrinkWaves / p.jg;
  p.mw = mw;
  p.kw = kShrinkWaves / (p.mw * p.jg);
  const int64_t tt = 16 * (int64_t)p.mw;
  const int64_t tiles = T > 0 ? (T + tt - 1) / tt + (L < T ? L : T) : 0;
  p.max_tiles = (int32_t)tiles;
  // Split H across workgroups only when the tiles alone leave most CUs idle,
  // and never below one H step per wave.
  int64_t ks = 1;
  if (tiles > 0 && tiles < 128) ks = (256 + tiles - 1) / tiles;
  const int64_t ks_max = H / ((int64_t)p.kw * kShrinkKStep);
  if (ks > ks_max) ks = ks_max;
  if (ks < 1) ks = 1;
  ks = env_int("LORA_SHRINK_KSPLIT", (int)ks);
  int64_t chunk = (H + ks - 1) / ks;
  chunk = (chunk + kShrinkKStep - 1) / kShrinkKStep * kShrinkKStep;
  ks = (H + chunk - 1) / chunk;
  p.ksplit = (int32_t)ks;
  p.kchunk = (int32_t)chunk;
  p.partial_bytes = ks > 1 ? (size_t)(ks * (int64_t)T * p.rp * 4) : 0;
  p.counter_bytes = 0;
  int64_t items = tiles * ks;
  int64_t grid = items < 512 ? items : 512;
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
  a.mw = plan.mw;
  a.jg = plan.jg;
  a.kw = plan.kw;
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
