// Segment metadata builder: a stable counting sort of token indices by
// adapter id (punica issue: tokens sharing an adapter form one SGMV segment).
//
// One workgroup of 1024 threads (16 waves) does the whole batch in LDS:
//   1. histogram of the keys (key = adapter id, or L for "no adapter"); each
//      wave groups equal keys with ballots and adds one count per key,
//   2. exclusive scan of the histogram: segment starts, segment numbering,
//      tails, the counts record,
//   3. ranking in rounds of 1024 tokens: a token's destination is the start of
//      its key + tokens of that key in earlier rounds + in earlier waves of the
//      round + in earlier lanes of its wave.  Equal keys keep token order, so
//      the result is the unique stable order.
// Metadata is a few KB, so the kernel is latency-bound; a single workgroup
// avoids any inter-workgroup handshake.
#include "lora_device.h"
#include "lora_kernels.h"

namespace lora {

namespace {

constexpr int kSegThreads = 1024;
constexpr int kSegWaves = kSegThreads / kWave;

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & (kWave - 1);
  return (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
}

__global__ __launch_bounds__(kSegThreads) void build_segments_kernel(
    const int32_t* __restrict__ ids, int32_t T, int32_t L, int32_t* __restrict__ sorted_token,
    int32_t* __restrict__ seg_lora, int32_t* __restrict__ seg_start,
    int32_t* __restrict__ counts) {
  // LDS: key_pos[L + 1] (histogram, then running positions) followed by the
  // per-round table cnt[kSegWaves][L + 1] of 8-bit counts.
  extern __shared__ int32_t smem[];
  int32_t* key_pos = smem;
  uint8_t* cnt = reinterpret_cast<uint8_t*>(smem + (L + 1));
  __shared__ int32_t scan_scratch[kSegWaves + 1];
  __shared__ int32_t s_bad, s_longest, s_ta, s_nseg;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int nkeys = L + 1;

  for (int k = tid; k < nkeys; k += kSegThreads) key_pos[k] = 0;
  for (int k = tid; k < kSegWaves * nkeys; k += kSegThreads) cnt[k] = 0;
  if (tid == 0) {
    s_bad = 0;
    s_longest = 0;
  }
  __syncthreads();

  // ---- 1. histogram
  for (int base = 0; base < T; base += kSegThreads) {
    const int t = base + tid;
    const bool valid = t < T;
    int key = L;
    bool bad = false;
    if (valid) {
      const int id = ids[t];
      const bool act = id >= 0 && id < L;
      key = act ? id : L;
      bad = !act && id != -1;
    }
    const uint64_t live = __ballot(valid);
    const uint64_t badm = __ballot(bad);
    if (lane == 0 && badm) atomicAdd(&s_bad, __popcll(badm));
    uint64_t todo = live;
    while (todo) {
      const int leader = __ffsll((unsigned long long)todo) - 1;
      const int lkey = __shfl(key, leader, kWave);
      const uint64_t same = __ballot(valid && key == lkey) & live;
      if (lane == leader) atomicAdd(&key_pos[lkey], __popcll(same));
      todo &= ~same;
    }
  }
  __syncthreads();

  // ---- 2. scan: starts, segment numbering, tails, counts
  const int per = (nkeys + kSegThreads - 1) / kSegThreads;
  const int k_lo = min(tid * per, nkeys);
  const int k_hi = min(k_lo + per, nkeys);
  int my_tokens = 0, my_segs = 0, my_long = 0;
  for (int k = k_lo; k < k_hi; ++k) {
    const int c = key_pos[k];
    my_tokens += c;
    if (k < L && c > 0) {
      ++my_segs;
      my_long = max(my_long, c);
    }
  }
  if (my_long) atomicMax(&s_longest, my_long);
  int tok_total, seg_total;
  int tok_before = block_exclusive_sum<kSegThreads>(my_tokens, scan_scratch, &tok_total);
  int seg_before = block_exclusive_sum<kSegThreads>(my_segs, scan_scratch, &seg_total);
  for (int k = k_lo; k < k_hi; ++k) {
    const int c = key_pos[k];
    key_pos[k] = tok_before;
    if (k < L && c > 0) {
      seg_lora[seg_before] = k;
      seg_start[seg_before] = tok_before;
      ++seg_before;
    }
    if (k == L) s_ta = tok_before;
    tok_before += c;
  }
  if (tid == 0) s_nseg = seg_total;
  __syncthreads();
  const int S = s_nseg;
  const int t_active = s_ta;
  for (int s = S + tid; s < L; s += kSegThreads) seg_lora[s] = -1;
  for (int s = S + tid; s <= L; s += kSegThreads) seg_start[s] = t_active;
  if (tid == 0) {
    counts[0] = S;
    counts[1] = t_active;
    counts[2] = s_longest;
    counts[3] = s_bad;
  }

  // ---- 3. stable ranking
  for (int base = 0; base < T; base += kSegThreads) {
    const int t = base + tid;
    const bool valid = t < T;
    int key = L;
    if (valid) {
      const int id = ids[t];
      key = (id >= 0 && id < L) ? id : L;
    }
    const uint64_t live = __ballot(valid);
    int rank_in_wave = 0, lead_count = 0;
    uint64_t todo = live;
    while (todo) {
      const int leader = __ffsll((unsigned long long)todo) - 1;
      const int lkey = __shfl(key, leader, kWave);
      const uint64_t same = __ballot(valid && key == lkey) & live;
      if (valid && key == lkey) rank_in_wave = __popcll(same & lanemask_lt());
      if (lane == leader) {
        lead_count = __popcll(same);
        cnt[wave * nkeys + lkey] = (uint8_t)lead_count;
      }
      todo &= ~same;
    }
    __syncthreads();
    if (valid) {
      int before = 0;
      for (int w = 0; w < wave; ++w) before += cnt[w * nkeys + key];
      sorted_token[key_pos[key] + before + rank_in_wave] = t;
    }
    __syncthreads();
    if (lead_count) {
      atomicAdd(&key_pos[key], lead_count);
      cnt[wave * nkeys + key] = 0;
    }
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_build_segments(const int32_t* token_lora, int32_t T, int32_t L,
                                 int32_t* sorted_token, int32_t* seg_lora, int32_t* seg_start,
                                 int32_t* counts, hipStream_t s) {
  const size_t lds = sizeof(int32_t) * (size_t)(L + 1) + (size_t)kSegWaves * (size_t)(L + 1);
  hipLaunchKernelGGL(build_segments_kernel, dim3(1), dim3(kSegThreads), lds, s, token_lora, T, L,
                     sorted_token, seg_lora, seg_start, counts);
  return hipGetLastError();
}

}  // namespace lora
