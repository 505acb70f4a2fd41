// Device-side building blocks shared by the gfx950 kernels: vector types,
// 16-bit conversions, the 16x16x32 matrix-core op and wave/block scans.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lora {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- 16-bit <-> fp32
// DT 0 = IEEE binary16, DT 1 = bfloat16.  Widening is exact; narrowing rounds
// to nearest even (bf16 by rounding the binary32 pattern; NaN stays NaN).
template <int DT>
__device__ __forceinline__ float to_f32(uint32_t bits16) {
  if constexpr (DT == 0) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
  } else {
    return __uint_as_float(bits16 << 16);
  }
}

template <int DT>
__device__ __forceinline__ uint32_t from_f32(float f) {
  if constexpr (DT == 0) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
  } else {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
  }
}

// Packs two 16-bit patterns into one dword (lo = first element).
__device__ __forceinline__ uint32_t pack2(uint32_t a, uint32_t b) { return a | (b << 16); }

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

// Rounds two floats to nearest even and packs them (a in the low half): one
// v_cvt_pk_{bf16,f16}_f32 on gfx950.
template <int DT>
__device__ __forceinline__ uint32_t cvt_pack2(float a, float b) {
  const f32x2 f = f32x2{a, b};
  if constexpr (DT == 0) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2));
  } else {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
  }
}

// Widens the two 16-bit values of a packed dword.
template <int DT>
__device__ __forceinline__ void unpack2(uint32_t d, float* lo, float* hi) {
  if constexpr (DT == 0) {
    const f16x2 h = __builtin_bit_cast(f16x2, d);
    *lo = (float)h.x;
    *hi = (float)h.y;
  } else {
    *lo = __uint_as_float(d << 16);
    *hi = __uint_as_float(d & 0xffff0000u);
  }
}

// ---------------------------------------------------------------- binary16 range of v
// expand feeds the fp32 v to 16-bit products as hi = round16(v) plus
// lo = round16(v - hi).  In binary16 a |v| of 65520 or more would round to
// infinity, and values below 2^-14 lose bits to subnormals.  A power of two
// 2^-k taken per token moves the token's largest |v| into [2^13, 2^14) before
// the split, and the fp32 product is multiplied by 2^k afterwards: both are
// exact, so the result is the unscaled one wherever that one is in range.
// k = 0 for a zero, fp32-subnormal or non-finite maximum; |k| <= 100 keeps
// both factors normal fp32 numbers.
__device__ __forceinline__ void f16_prescale(float maxabs, float* down, float* up) {
  const uint32_t e = (__float_as_uint(maxabs) >> 23) & 0xffu;
  int k = (e == 0u || e == 255u) ? 0 : (int)e - 127 - 13;
  k = k < -100 ? -100 : (k > 100 ? 100 : k);
  *down = __uint_as_float((uint32_t)(127 - k) << 23);
  *up = __uint_as_float((uint32_t)(127 + k) << 23);
}

// Maximum of x over the four lanes l, l ^ 16, l ^ 32 and l ^ 48 (the four
// lane groups of one row position), with the gfx950 lane-swap instructions:
// called with both operands equal, each returns the lane's own value and that
// of its partner row.  Every lane of the wave must be active.
__device__ __forceinline__ float max_over_lane_groups(float x) {
  auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
  s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(s[0]), __uint_as_float(s[1]));
}

// ---------------------------------------------------------------- matrix core
// D(16x16, fp32) += A(16x32) * B(32x16) with 8 elements of A and B per lane.
// Whatever the hardware's internal k numbering, slot (lane / 16, element e) of
// A meets slot (lane / 16, element e) of B, so both operands only have to
// place the same k in the same slot.  Lane i of D holds rows 4 * (i / 16) + 0..3
// of column i % 16.
template <int DT>
__device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (DT == 0) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                  __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
}

// ---------------------------------------------------------------- loads
// Loads 8 consecutive 16-bit elements p[0..8) as 4 dwords.  Elements at or
// beyond `limit` (counted from p) read as zero.  VEC: p is 16-byte aligned
// and limit is a multiple of 8, so a chunk is either whole or absent.
template <bool VEC>
__device__ __forceinline__ u32x4 load8_16(const uint16_t* __restrict__ p, int limit) {
  if constexpr (VEC) {
    return limit >= 8 ? *reinterpret_cast<const u32x4*>(p) : u32x4{0u, 0u, 0u, 0u};
  }
  uint32_t e[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) e[i] = (i < limit) ? (uint32_t)p[i] : 0u;
  u32x4 r;
  r.x = pack2(e[0], e[1]);
  r.y = pack2(e[2], e[3]);
  r.z = pack2(e[4], e[5]);
  r.w = pack2(e[6], e[7]);
  return r;
}

// Branch-free load of the 8 16-bit elements row[off..off+8) for the vector
// path: the address is clamped into [0, end - 8] so the load is always legal,
// and the value is replaced by zeros when !ok or off >= end.  Keeping loads
// out of divergent branches lets the compiler count outstanding loads instead
// of draining them all before the matrix ops.  Needs end >= 8 and 16-byte
// aligned chunks (end, off multiples of 8).
__device__ __forceinline__ u32x4 load8_16_masked(const uint16_t* __restrict__ row, int off,
                                                 int end, bool ok) {
  const int safe = off < end ? off : end - 8;
  const u32x4 v = *reinterpret_cast<const u32x4*>(row + safe);
  const bool keep = ok && off < end;
  return u32x4{keep ? v.x : 0u, keep ? v.y : 0u, keep ? v.z : 0u, keep ? v.w : 0u};
}

// Loads 8 consecutive floats (elements beyond `limit` read as zero).  VEC: p
// is 16-byte aligned and limit is a multiple of 8.
template <bool VEC>
__device__ __forceinline__ void load8_f32(const float* __restrict__ p, int limit, float out[8]) {
  if constexpr (VEC) {
    if (limit < 8) {
#pragma unroll
      for (int i = 0; i < 8; ++i) out[i] = 0.0f;
      return;
    }
    f32x4 a = *reinterpret_cast<const f32x4*>(p);
    f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
    out[0] = a.x; out[1] = a.y; out[2] = a.z; out[3] = a.w;
    out[4] = b.x; out[5] = b.y; out[6] = b.z; out[7] = b.w;
    return;
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) out[i] = (i < limit) ? p[i] : 0.0f;
}

// ---------------------------------------------------------------- scans
// Inclusive prefix sum across the 64 lanes of a wave, in six DPP moves with
// no LDS round trip: shifts right by 1, 2, 4 and 8 lanes inside each row of
// 16 build the row sums, then the last lane of row 0 is added into row 1 and
// that of row 2 into row 3 (row_bcast:15), and lane 31 into rows 2 and 3
// (row_bcast:31).  A lane whose source lies outside its row, or whose row is
// masked off, adds the tied old value, 0.
__device__ __forceinline__ int wave_inclusive_sum(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return x;
}

// Running maximum across the lanes of a wave for values >= 0 (same moves as
// wave_inclusive_sum; 0 is the identity).  Lane 63 holds the wave maximum.
__device__ __forceinline__ int wave_inclusive_max(int x) {
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false));
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false));
  return x;
}

// Exclusive prefix sum over all threads of a block of NT threads.  `scratch`
// holds NT / 64 + 1 ints of LDS.  Returns the exclusive prefix; *total gets the
// block total.  Contains __syncthreads(); every thread must call it.
template <int NT>
__device__ __forceinline__ int block_exclusive_sum(int x, int* scratch, int* total) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  int inc = wave_inclusive_sum(x);
  if (lane == kWave - 1) scratch[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    int w = (lane < NW) ? scratch[lane] : 0;
    int wi = wave_inclusive_sum(w);
    if (lane < NW) scratch[lane] = wi - w;
    if (lane == NW - 1) scratch[NW] = wi;
  }
  __syncthreads();
  int excl = scratch[wave] + inc - x;
  *total = scratch[NW];
  __syncthreads();
  return excl;
}

// ---------------------------------------------------------------- wave reductions
// Value of lane (lane ^ (1 << B)) for B <= 3, i.e. inside one row of 16 lanes,
// through DPP: quad permutations for bits 0 and 1, two row shifts for bit 2,
// a row rotation by 8 for bit 3.
template <int B>
__device__ __forceinline__ float lane_xor(float v, int lane) {
  static_assert(B >= 0 && B <= 3, "DPP exchange stays inside a row");
  const int i = __float_as_int(v);
  if constexpr (B == 0) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, i, 0xB1, 0xF, 0xF, true));  // [1,0,3,2]
  } else if constexpr (B == 1) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, i, 0x4E, 0xF, 0xF, true));  // [2,3,0,1]
  } else if constexpr (B == 2) {
    const int up = __builtin_amdgcn_update_dpp(0, i, 0x104, 0xF, 0xF, true);    // from lane + 4
    const int down = __builtin_amdgcn_update_dpp(0, i, 0x114, 0xF, 0xF, true);  // from lane - 4
    return __int_as_float((lane & 4) ? down : up);
  } else {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, i, 0x128, 0xF, 0xF, true));  // rotate 8
  }
}

// One step of a transposing reduction over lane bit B: lanes with bit B clear
// keep (a + a of the partner lane), lanes with it set keep (b + b of the
// partner).  Bits 5 and 4 use the gfx950 lane-swap instructions, which move
// half of each operand across 32- or 16-lane boundaries in one VALU op.
template <int B>
__device__ __forceinline__ float pair_step(float a, float b, int lane) {
  if constexpr (B == 5 || B == 4) {
    const auto s = B == 5 ? __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false)
                          : __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(s[0]) + __uint_as_float(s[1]);
  } else {
    const bool hi = (lane >> B) & 1;
    const float keep = hi ? b : a;
    const float send = hi ? a : b;
    return keep + lane_xor<B>(send, lane);
  }
}

template <int B, int M>
__device__ __forceinline__ void transpose_step(float* x, int lane) {
  if constexpr (M >= 2) {
#pragma unroll
    for (int i = 0; i < M / 2; ++i) x[i] = pair_step<B>(x[i], x[i + M / 2], lane);
  } else {
    static_assert(B <= 3, "at least four values per lane");
    x[0] = x[0] + lane_xor<B>(x[0], lane);
  }
}

// Sums each of the N per-lane values x[0..N) over the 64 lanes of a wave
// (N a power of two, 4 <= N <= 64), in about N + 6 cross-lane operations
// instead of 6 N.  Afterwards x[0] of lane l holds the wave total of value
// (l >> (6 - log2 N)) & (N - 1); the lanes that share those bits hold the same
// total.  The order of the additions is fixed, so the result is reproducible.
template <int N>
__device__ __forceinline__ void wave_transpose_sum(float (&x)[N]) {
  static_assert(N >= 4 && N <= 64 && (N & (N - 1)) == 0, "N: power of two in [4, 64]");
  const int lane = threadIdx.x & (kWave - 1);
  transpose_step<5, N>(x, lane);
  transpose_step<4, N / 2>(x, lane);
  transpose_step<3, (N / 4 > 1 ? N / 4 : 1)>(x, lane);
  transpose_step<2, (N / 8 > 1 ? N / 8 : 1)>(x, lane);
  transpose_step<1, (N / 16 > 1 ? N / 16 : 1)>(x, lane);
  transpose_step<0, (N / 32 > 1 ? N / 32 : 1)>(x, lane);
}

template <int N>
constexpr int log2_of() {
  return N <= 1 ? 0 : 1 + log2_of<N / 2>();
}

// First work item of workgroup wg in a persistent grid that then steps by
// the grid size.  Workgroups are dispatched round-robin over the 8 XCDs, so
// XCD x runs workgroups x, x + 8, ...; numbering them x per + (wg >> 3) gives
// each XCD a contiguous block of items per round (neighbouring items share
// one L2), while the items of one round stay one contiguous window of the
// item order across the chip (measured: 20-27% faster on large expands than
// per-XCD blocks of the whole item range).  With fewer items than workgroups
// (the grid is sized on the host from an upper bound), per shrinks to
// ceil(n_items / 8) so that every XCD gets an equal share.  A grid that is not
// a multiple of 8 keeps plain order.
__device__ __forceinline__ int xcd_first_item(int wg, int grid, int n_items) {
  if ((grid & 7) != 0) return wg;
  int per = grid >> 3;
  if (n_items < grid) per = (n_items + 7) >> 3;
  const int local = wg >> 3;
  return local < per ? (wg & 7) * per + local : n_items;
}

}  // namespace lora
