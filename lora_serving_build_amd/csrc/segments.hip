// Segment metadata builder: a stable counting sort of token indices by
// adapter id (punica issue: tokens sharing an adapter form one SGMV segment).
//
// One workgroup (4 or 16 waves) does the whole batch.  Wave w owns the
// contiguous block of tokens [w * span, (w + 1) * span), walked in chunks of
// 64 (lane i takes token chunk_start + i), and keeps its keys in registers
// (key = adapter id, or L for "no adapter").  Inside a chunk the lanes that
// hold one key form a group, found with one ballot per key bit: a lane's
// group is the AND, over the bits, of that bit's ballot where its own bit is
// set and of the complement where it is clear.  A chunk thus costs
// O(log2 L) instructions whatever the mix of keys in it.
//   1. the first lane of each group adds the group size to the wave's LDS
//      row cnt[w][key];
//   2. one block scan over the keys gives every key its start; each row entry
//      then becomes the first position of that wave's tokens of that key
//      (start + the key's tokens in earlier waves); segments, tails and the
//      counts record are written here;
//   3. each wave walks its chunks again: a token goes to its row entry plus
//      the group members in lower lanes, and the group's first lane moves the
//      entry past the group.  Order is kept inside a wave (chunks in order,
//      lanes in order) and across waves (bases), so the result is the unique
//      stable order.
// Rows are private to their wave and the LDS operations of a wave execute in
// order, so only the scan needs barriers.  Sums and maxima across lanes are
// DPP moves.  The ids are read in one round of loads; metadata is a few KB,
// so the kernel is latency-bound.
#include "lora_device.h"
#include "lora_kernels.h"

namespace lora {

namespace {

constexpr size_t kSegMaxLds = 64 * 1024;  // bytes of per-wave rows a launch may take

// Lanes of the wave whose key equals this lane's, for keys in [0, 2^nbits);
// `live` is the ballot of the lanes that hold a key at all.  A chunk whose
// live lanes all hold one key (the common case inside long sequences) is one
// group, found with one compare.
__device__ __forceinline__ uint64_t key_group(int key, uint64_t live, int nbits) {
  const int k0 = __builtin_amdgcn_readlane(key, (int)__builtin_ctzll(live));
  if (__ballot(key == k0) == live) return live;  // uniform
  uint64_t m = live;
  for (int i = 0; i < nbits; ++i) {
    const bool bit = (key >> i) & 1;
    const uint64_t b = __ballot(bit);
    m &= bit ? b : ~b;
  }
  return m;
}

// Set bits of m in lanes below this one.
__device__ __forceinline__ int lanes_below(uint64_t m) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                        __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// NW = waves (16 when the batch is large and their rows fit, so that the
// chunk loops of several waves overlap on each SIMD; else 4).  KR = chunks
// of keys a lane keeps in registers (chosen from T, so small batches run a
// short kernel); waves with more chunks reload their ids.
template <int NW, int KR>
__global__ __launch_bounds__(NW * kWave) void build_segments_kernel(
    const int32_t* __restrict__ ids, int32_t T, int32_t L, int32_t* __restrict__ sorted_token,
    int32_t* __restrict__ seg_lora, int32_t* __restrict__ seg_start,
    int32_t* __restrict__ counts) {
  // LDS: cnt[NW][L + 1], first counts, then per-wave positions.
  extern __shared__ int32_t cnt[];
  __shared__ int4 s_scan[NW];
  __shared__ int2 s_wave[NW];  // per wave: ids outside [-1, L), tokens without an adapter

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = tid / kWave;
  const int nkeys = L + 1;
  const int nbits = 32 - __clz(L);  // keys are 0..L
  int32_t* row = cnt + wave * nkeys;

  // Tokens of this wave: [t0, t0 + span), nch chunks of 64.
  const int span = (((T + NW - 1) / NW) + kWave - 1) / kWave * kWave;
  const int t0 = wave * span;
  const int nch = span / kWave;
  const bool in_regs = nch <= KR;

  int keys[KR];
#pragma unroll
  for (int c = 0; c < KR; ++c) keys[c] = -1;
  int nbad = 0;  // ids outside [-1, L) seen by this lane in phase 1
  // Loads every id of a block of chunks at once (addresses clamped into the
  // batch, so no load sits in a branch), then turns them into keys; -1 marks
  // lanes past the batch.
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
      const int id = keys[c];
      const bool valid = cb + c < nch && t < T;
      const bool act = id >= 0 && id < L;
      keys[c] = !valid ? -1 : (act ? id : L);
      if (count && valid && !act && id != -1) ++nbad;
    }
  };

  // The id loads go out first; the row is cleared while they are in flight.
  load_keys(0, true);
  for (int k = lane; k < nkeys; k += kWave) row[k] = 0;

  // ---- 1. per-wave histogram
  int none = 0;  // tokens of this wave without an adapter (uniform)
  for (int cb = 0; cb < nch; cb += KR) {
    if (cb > 0) load_keys(cb, true);
    const int cend = min(KR, nch - cb);
#pragma unroll
    for (int c = 0; c < KR; ++c) {
      if (c >= cend) break;
      const int key = keys[c];
      const uint64_t live = __ballot(key >= 0);
      if (live == 0) continue;
      none += __popcll(__ballot(key == L));
      const uint64_t grp = key_group(key, live, nbits);
      if (key >= 0 && lanes_below(grp) == 0) atomicAdd(&row[key], __popcll(grp));
    }
  }
  nbad = __builtin_amdgcn_readlane(wave_inclusive_sum(nbad), kWave - 1);
  if (lane == 0) s_wave[wave] = make_int2(nbad, none);
  __syncthreads();

  // ---- 2. scan over keys: starts, per-wave bases, segments, tails, counts
  // Only the KW waves that own keys take part (one wave up to 64 keys); the
  // others wait at the barriers, so the scan's instructions are not issued
  // by every wave of a SIMD.  KW and per are uniform.
  const int KW = min(NW, (nkeys + kWave - 1) / kWave);
  const int per = (nkeys + (KW * kWave) - 1) / (KW * kWave);
  const int k_lo = min(tid * per, nkeys);
  const int k_hi = min(k_lo + per, nkeys);
  int my_tokens = 0, my_segs = 0, my_long = 0;
  int wave_segs = 0, wave_long = 0;  // totals of this wave (lane 63)
  if (wave < KW) {
    for (int k = k_lo; k < k_hi; ++k) {
      int c = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) c += cnt[w * nkeys + k];  // independent reads, issued together
      my_tokens += c;
      if (k < L && c > 0) {
        ++my_segs;
        my_long = max(my_long, c);
      }
    }
    // Block scan of (tokens, segments) and maximum of the segment lengths.
    const int inc_t = wave_inclusive_sum(my_tokens);
    const int inc_s = wave_inclusive_sum(my_segs);
    const int max_l = wave_inclusive_max(my_long);
    if (KW > 1 && lane == kWave - 1) s_scan[wave] = make_int4(inc_t, inc_s, max_l, 0);
    wave_segs = __builtin_amdgcn_readlane(inc_s, kWave - 1);
    wave_long = __builtin_amdgcn_readlane(max_l, kWave - 1);
    my_tokens = inc_t - my_tokens;  // now exclusive, inside the wave
    my_segs = inc_s - my_segs;
  }
  // One key wave (up to 64 keys) needs no exchange between waves.  KW is
  // uniform, so every wave takes the same side of this barrier.
  if (KW > 1) __syncthreads();
  if (wave < KW) {
    // Per-wave records are combined across lanes (lane w takes wave w's).
    const int2 qw = lane < NW ? s_wave[lane] : make_int2(0, 0);
    const int bad = __builtin_amdgcn_readlane(wave_inclusive_sum(qw.x), kWave - 1);
    const int t_active = T - __builtin_amdgcn_readlane(wave_inclusive_sum(qw.y), kWave - 1);
    int S = wave_segs, longest = wave_long;
    int tok_before = my_tokens, seg_before = my_segs;
    if (KW > 1) {
      const int4 q = lane < KW ? s_scan[lane] : make_int4(0, 0, 0, 0);
      const int qt = wave_inclusive_sum(q.x);
      const int qs = wave_inclusive_sum(q.y);
      S = __builtin_amdgcn_readlane(qs, kWave - 1);
      longest = __builtin_amdgcn_readlane(wave_inclusive_max(q.z), kWave - 1);
      // Tokens and segments of the key waves before this one.
      tok_before += __builtin_amdgcn_readlane(qt - q.x, wave);
      seg_before += __builtin_amdgcn_readlane(qs - q.y, wave);
    }
    for (int k = k_lo; k < k_hi; ++k) {
      // All of the key's row entries are read before any is rewritten, so the
      // reads go out together instead of one round trip per wave.
      int cw[NW];
#pragma unroll
      for (int w = 0; w < NW; ++w) cw[w] = cnt[w * nkeys + k];
      int b = tok_before;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        cnt[w * nkeys + k] = b;
        b += cw[w];
      }
      const int c = b - tok_before;
      if (k < L && c > 0 && seg_before < L) {
        seg_lora[seg_before] = k;
        seg_start[seg_before] = tok_before;
        ++seg_before;
      }
      tok_before = b;
    }
    for (int s = S + tid; s < L; s += (KW * kWave)) seg_lora[s] = -1;
    for (int s = S + tid; s <= L; s += (KW * kWave)) seg_start[s] = t_active;
    if (tid == 0) {
      counts[0] = S;
      counts[1] = t_active;
      counts[2] = longest;
      counts[3] = bad;
    }
  }
  __syncthreads();

  // ---- 3. stable scatter (wave-private rows: no barriers)
  for (int cb = 0; cb < nch; cb += KR) {
    if (!in_regs) load_keys(cb, false);
    const int cend = min(KR, nch - cb);
#pragma unroll
    for (int c = 0; c < KR; ++c) {
      if (c >= cend) break;
      const int key = keys[c];
      const uint64_t live = __ballot(key >= 0);
      if (live == 0) continue;
      const uint64_t grp = key_group(key, live, nbits);
      const int below = lanes_below(grp);
      if (key >= 0) {
        const int b = row[key];
        if (below == 0) row[key] = b + __popcll(grp);  // after every lane's read
        const int pos = b + below;
        if (pos < T) sorted_token[pos] = t0 + (cb + c) * kWave + lane;  // pos < T always; a guard
      }
    }
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
