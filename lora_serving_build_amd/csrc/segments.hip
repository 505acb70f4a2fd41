// Segment metadata builder: a stable counting sort of token indices by
// adapter id (punica issue: tokens sharing an adapter form one SGMV segment).
//
// One workgroup (4 or 16 waves) does the whole batch.  Wave w owns the
// contiguous block of tokens [w * span, (w + 1) * span), walked in chunks of
// 64 (lane i takes token chunk_start + i), and keeps its keys in registers
// (key = adapter id, or L for "no adapter"):
//   1. each wave counts its keys into its own LDS row cnt[w][key] -- up to
//      128 keys, into two registers per lane instead (lane k holds keys k
//      and k + 64) -- : lanes with equal keys are grouped with ballots and
//      one lane adds the group size;
//   2. one block scan over the keys gives every key its start; each row entry
//      then becomes the first position of that wave's tokens of that key
//      (start + the key's tokens in earlier waves); segments, tails and the
//      counts record are written here;
//   3. each wave walks its chunks again and sends every token to its row
//      entry + the group members in earlier lanes, bumping the entry.  Token
//      order is kept inside a wave (chunks in order, lanes in order) and
//      across waves (bases), so the result is the unique stable order.
// Rows are private to their wave and the LDS operations of a wave execute in
// order, so only the scan needs barriers.  The ids are read in one round of
// loads; metadata is a few KB, so the kernel is latency-bound.
#include "lora_device.h"
#include "lora_kernels.h"

namespace lora {

namespace {

constexpr size_t kSegMaxLds = 64 * 1024;  // bytes of per-wave rows a launch may take

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & (kWave - 1);
  return (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
}

// Exclusive prefix sums of two values over a block of NW waves (one pass).
template <int NW>
__device__ __forceinline__ void block_exclusive_sum2(int a, int b, int* scratch, int* ea, int* eb,
                                                     int* ta, int* tb) {
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  int ia = a, ib = b;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int ya = __shfl_up(ia, d, kWave);
    const int yb = __shfl_up(ib, d, kWave);
    if (lane >= d) {
      ia += ya;
      ib += yb;
    }
  }
  if (lane == kWave - 1) {
    scratch[2 * wave] = ia;
    scratch[2 * wave + 1] = ib;
  }
  __syncthreads();
  int pa = 0, pb = 0, sa = 0, sb = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const int wa = scratch[2 * w], wb = scratch[2 * w + 1];
    if (w < wave) {
      pa += wa;
      pb += wb;
    }
    sa += wa;
    sb += wb;
  }
  *ea = pa + ia - a;
  *eb = pb + ib - b;
  *ta = sa;
  *tb = sb;
}

// Key of token t (L = no adapter), or -1 past the batch; *bad is set for ids
// outside [-1, L).
__device__ __forceinline__ int key_of(int id, int L, bool* bad) {
  const bool act = id >= 0 && id < L;
  *bad = !act && id != -1;
  return act ? id : L;
}

// NW = waves (16 when the batch is large and their rows fit, so that the
// ballot chains of several waves overlap on each SIMD; else 4).  KR = chunks
// of keys a lane keeps in registers (chosen from T, so small batches run a
// short kernel); waves with more chunks reload their ids.
template <int NW, int KR>
__global__ __launch_bounds__(NW * kWave) void build_segments_kernel(
    const int32_t* __restrict__ ids, int32_t T, int32_t L, int32_t* __restrict__ sorted_token,
    int32_t* __restrict__ seg_lora, int32_t* __restrict__ seg_start,
    int32_t* __restrict__ counts) {
  // LDS: cnt[NW][L + 1], first counts, then per-wave positions.
  extern __shared__ int32_t cnt[];
  __shared__ int32_t scan_scratch[2 * NW];
  __shared__ int32_t s_bad[NW], s_longest[NW], s_ta, s_nseg;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int nkeys = L + 1;
  int32_t* row = cnt + wave * nkeys;

  // Tokens of this wave: [t0, t0 + span), nch chunks of 64.
  const int span = (((T + NW - 1) / NW) + kWave - 1) / kWave * kWave;
  const int t0 = wave * span;
  const int nch = span / kWave;
  const bool in_regs = nch <= KR;

  int keys[KR];
  int nbad = 0;  // ids outside [-1, L) seen by this lane in phase 1
  // Loads every id of a block of chunks at once (addresses clamped into the
  // batch, so no load sits in a branch), then turns them into keys.
  auto load_keys = [&](int cb, bool count) {
    if (T == 0) return;
#pragma unroll
    for (int c = 0; c < KR; ++c) {
      const int t = t0 + (cb + c) * kWave + lane;
      keys[c] = ids[t < T ? t : T - 1];
    }
#pragma unroll
    for (int c = 0; c < KR; ++c) {
      const int t = t0 + (cb + c) * kWave + lane;
      bool bad = false;
      const int key = key_of(keys[c], L, &bad);
      const bool valid = cb + c < nch && t < T;
      keys[c] = valid ? key : -1;
      if (count && valid && bad) ++nbad;
    }
  };

  // Up to 128 keys, a wave keeps its per-key counts (later: positions) in two
  // registers per lane, lane k holding keys k and k + 64; otherwise in its LDS
  // row, added to with LDS atomics that nothing waits for.
  const bool kreg = nkeys <= 2 * kWave;
  int kr0 = 0, kr1 = 0;

  // The id loads go out first; the row is cleared while they are in flight.
  load_keys(0, true);
  if (!kreg)
    for (int k = lane; k < nkeys; k += kWave) row[k] = 0;

  // ---- 1. per-wave histogram
  for (int cb = 0; cb < nch; cb += KR) {
    if (cb > 0) load_keys(cb, true);
    const int cend = min(KR, nch - cb);
#pragma unroll 1
    for (int c = 0; c < cend; ++c) {
      const int key = keys[c];  // -1 for tokens past the batch
      uint64_t todo = __ballot(key >= 0);
      while (todo) {
        const int leader = __ffsll((unsigned long long)todo) - 1;
        const int lkey = __builtin_amdgcn_readlane(key, leader);
        const uint64_t same = __ballot(key == lkey);
        const int n = __popcll(same);
        if (kreg) {
          if (lane == (lkey & (kWave - 1))) {
            if (lkey < kWave) kr0 += n; else kr1 += n;
          }
        } else if (lane == leader) {
          atomicAdd(&row[lkey], n);
        }
        todo &= ~same;
      }
    }
  }
  if (kreg) {
    if (lane < nkeys) row[lane] = kr0;
    if (lane + kWave < nkeys) row[lane + kWave] = kr1;
  }
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) nbad += __shfl_xor(nbad, d, kWave);
  if (lane == 0) s_bad[wave] = nbad;
  __syncthreads();

  // ---- 2. scan over keys: starts, per-wave bases, segments, tails, counts
  const int per = (nkeys + (NW * kWave) - 1) / (NW * kWave);
  const int k_lo = min(tid * per, nkeys);
  const int k_hi = min(k_lo + per, nkeys);
  int my_tokens = 0, my_segs = 0, my_long = 0;
  for (int k = k_lo; k < k_hi; ++k) {
    int c = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) c += cnt[w * nkeys + k];
    my_tokens += c;
    if (k < L && c > 0) {
      ++my_segs;
      my_long = max(my_long, c);
    }
  }
  int tok_before, seg_before, tok_total, seg_total;
  block_exclusive_sum2<NW>(my_tokens, my_segs, scan_scratch, &tok_before, &seg_before, &tok_total,
                       &seg_total);
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) my_long = max(my_long, __shfl_xor(my_long, d, kWave));
  if (lane == 0) s_longest[wave] = my_long;
  for (int k = k_lo; k < k_hi; ++k) {
    int b = tok_before;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const int c = cnt[w * nkeys + k];
      cnt[w * nkeys + k] = b;
      b += c;
    }
    const int c = b - tok_before;
    if (k < L && c > 0) {
      seg_lora[seg_before] = k;
      seg_start[seg_before] = tok_before;
      ++seg_before;
    }
    if (k == L) s_ta = tok_before;
    tok_before = b;
  }
  if (tid == 0) s_nseg = seg_total;
  __syncthreads();
  const int S = s_nseg;
  const int t_active = s_ta;
  for (int s = S + tid; s < L; s += (NW * kWave)) seg_lora[s] = -1;
  for (int s = S + tid; s <= L; s += (NW * kWave)) seg_start[s] = t_active;

  // ---- 3. stable scatter (wave-private rows: no barriers)
  if (kreg) {
    kr0 = lane < nkeys ? row[lane] : 0;
    kr1 = lane + kWave < nkeys ? row[lane + kWave] : 0;
  }
  int ck = -1, cpos = 0;  // LDS rows: the position of key ck, held in a scalar
  for (int cb = 0; cb < nch; cb += KR) {
    if (!in_regs) load_keys(cb, false);
    const int cend = min(KR, nch - cb);
#pragma unroll 1
    for (int c = 0; c < cend; ++c) {
      const int key = keys[c];
      const int t = t0 + (cb + c) * kWave + lane;
      uint64_t todo = __ballot(key >= 0);
      while (todo) {
        const int leader = __ffsll((unsigned long long)todo) - 1;
        const int lkey = __builtin_amdgcn_readlane(key, leader);
        const uint64_t same = __ballot(key == lkey);
        const int n = __popcll(same);
        int b;
        if (kreg) {
          b = lkey < kWave ? __builtin_amdgcn_readlane(kr0, lkey)
                           : __builtin_amdgcn_readlane(kr1, lkey - kWave);
          if (lane == (lkey & (kWave - 1))) {
            if (lkey < kWave) kr0 = b + n; else kr1 = b + n;
          }
        } else {
          if (lkey != ck) {
            if (ck >= 0 && lane == 0) row[ck] = cpos;
            b = row[lkey];  // same address in every lane: a broadcast
            ck = lkey;
          } else {
            b = cpos;
          }
          cpos = b + n;
        }
        const int pos = b + __popcll(same & lanemask_lt());
        if (key == lkey && pos < T) sorted_token[pos] = t;  // pos < T always; kept as a guard
        todo &= ~same;
      }
    }
  }
  __syncthreads();
  if (tid == 0) {
    int bad = 0, longest = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      bad += s_bad[w];
      longest = max(longest, s_longest[w]);
    }
    counts[0] = S;
    counts[1] = t_active;
    counts[2] = longest;
    counts[3] = bad;
  }
}

}  // namespace

hipError_t launch_build_segments(const int32_t* token_lora, int32_t T, int32_t L,
                                 int32_t* sorted_token, int32_t* seg_lora, int32_t* seg_start,
                                 int32_t* counts, hipStream_t s) {
  const size_t row_bytes = sizeof(int32_t) * (size_t)(L + 1);
  const bool wide = T > 256 && 16 * row_bytes <= kSegMaxLds;
  const int nw = wide ? 16 : 4;
  const size_t lds = (size_t)nw * row_bytes;
  const int chunks = ((T + nw - 1) / nw + kWave - 1) / kWave;  // per wave
#define LORA_SEG_LAUNCH(NW_, KR_)                                                                  \
  hipLaunchKernelGGL((build_segments_kernel<NW_, KR_>), dim3(1), dim3(NW_ * kWave), lds, s,        \
                     token_lora, T, L, sorted_token, seg_lora, seg_start, counts)
  if (wide) {
    if (chunks <= 1) LORA_SEG_LAUNCH(16, 1);
    else if (chunks <= 4) LORA_SEG_LAUNCH(16, 4);
    else if (chunks <= 8) LORA_SEG_LAUNCH(16, 8);
    else LORA_SEG_LAUNCH(16, 32);
  } else {
    if (chunks <= 1) LORA_SEG_LAUNCH(4, 1);
    else if (chunks <= 4) LORA_SEG_LAUNCH(4, 4);
    else if (chunks <= 8) LORA_SEG_LAUNCH(4, 8);
    else LORA_SEG_LAUNCH(4, 32);
  }
#undef LORA_SEG_LAUNCH
  return hipGetLastError();
}

}  // namespace lora
