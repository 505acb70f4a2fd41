// C-ABI of liblora_mi355x (declared in include/lora.h): argument validation,
// dispatch to the gfx950 kernels, error reporting.  Nothing here allocates,
// copies between host and device or synchronises.
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>
#include <mutex>

#include "lora.h"
#include "lora_kernels.h"

namespace {

thread_local char g_error[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_error, sizeof g_error, fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_error[0] = '\0';
  return LORA_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(LORA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int check_dtype(int dtype, const char* fn) {
  if (dtype != LORA_F16 && dtype != LORA_BF16)
    return fail(LORA_ERR_INVALID_ARG, "%s: dtype %d is neither LORA_F16 nor LORA_BF16", fn, dtype);
  return LORA_OK;
}

// Validates the metadata struct that shrink / expand read.
int check_segments(const lora_segments* seg, const char* fn) {
  if (!seg) return fail(LORA_ERR_INVALID_ARG, "%s: seg is NULL", fn);
  if (seg->num_tokens < 0) return fail(LORA_ERR_INVALID_ARG, "%s: num_tokens %d < 0", fn, seg->num_tokens);
  if (seg->num_loras < 1 || seg->num_loras > LORA_MAX_LORAS)
    return fail(LORA_ERR_UNSUPPORTED, "%s: num_loras %d outside [1, %d]", fn, seg->num_loras,
                LORA_MAX_LORAS);
  if (!seg->seg_lora || !seg->seg_start || !seg->counts)
    return fail(LORA_ERR_INVALID_ARG, "%s: segment buffers must not be NULL", fn);
  if (seg->num_tokens > 0 && (!seg->token_lora || !seg->sorted_token))
    return fail(LORA_ERR_INVALID_ARG, "%s: token buffers must not be NULL", fn);
  return LORA_OK;
}

int check_rank(int32_t r, const char* fn) {
  if (r < 1 || r > LORA_MAX_RANK)
    return fail(LORA_ERR_UNSUPPORTED, "%s: rank %d outside [1, %d]", fn, r, LORA_MAX_RANK);
  return LORA_OK;
}

// Kernel path: 0 = automatic, 1 = per-token (BGMV), 2 = segment tiles (SGMV).
std::atomic<int> g_path{0};


// Automatic choice between the kernel families, from timings of both on
// decode-sized batches (T = 16 .. 512, H = 4096 and 16384, r = 16 .. 64, 4
// adapters, MI355X).
//
// Shrink: the per-token kernel needs one launch and no partial sums, but
// re-reads the adapter's A (and, with several rank blocks, x) from L2 for
// every token; the tiles read A once per 64-token tile but split the H-sum
// over workgroups and add a second launch.  Fitted costs (microseconds):
//   per-token  3 + (bytes read by its workgroups) / 22e6
//   tiles      7 + H / 1600 + T H / 1.6e6
// and the cheaper one is taken (at most 512 tokens for the per-token kernel).
//
// Expand: the per-token kernel streams a token's whole B_l, so it wins only
// while the batch is small and the rank low (r <= 16 up to T n = 4M output
// elements, r <= 32 up to 1M); a 64-token tile shares one staged weight block.
enum class Op { kShrink, kExpand };

bool use_bgmv(Op op, int32_t T, int32_t r, int64_t width, bool vec) {
  const int mode = g_path.load(std::memory_order_relaxed);
  if (!lora::bgmv_supports(op == Op::kExpand, r, vec)) return false;
  if (mode == 1) return true;
  if (mode == 2) return false;
  if (T > 512) return false;
  if (op == Op::kShrink) {
    const int rt = lora::bgmv_shrink_ranks(T, r, (int32_t)width);
    const double bytes = (double)T * ((r + rt - 1) / rt) * (rt + 1) * (double)width * 2.0;
    const double t_token = 3.0 + bytes / 22e6;
    const double t_tile = 7.0 + (double)width / 1600.0 + (double)T * (double)width / 1.6e6;
    return t_token < t_tile;
  }
  if (!vec) return r <= 16;
  const int64_t elems = (int64_t)T * width;
  if (r <= 16) return elems <= ((int64_t)4 << 20);
  if (r <= 32) return elems <= ((int64_t)1 << 20);
  return false;
}

int read_env_int(const char* name) {
  const char* e = getenv(name);
  if (!e) return 0;
  const long v = atol(e);
  return v > 0 && v < (1 << 20) ? (int)v : 0;
}

lora::Tuning read_tuning() {
  lora::Tuning t;
  t.shrink_ksplit = read_env_int("LORA_SHRINK_KSPLIT");
  t.expand_tb = read_env_int("LORA_EXPAND_TB");
  t.expand_cpr = read_env_int("LORA_EXPAND_CPR");
  t.bgmv_shrink_rt = read_env_int("LORA_BGMV_SHRINK_RT");
  t.bgmv_rpi = read_env_int("LORA_BGMV_RPI");
  t.bgmv_cb = read_env_int("LORA_BGMV_CB");
  t.expand_wgs_per_cu = read_env_int("LORA_EXPAND_WGS_PER_CU");
  t.expand_balance = read_env_int("LORA_EXPAND_BALANCE");
  t.shrink_tb = read_env_int("LORA_SHRINK_TB");
  t.shrink_group = read_env_int("LORA_SHRINK_GROUP");
  t.expand_line_y = read_env_int("LORA_EXPAND_LINE_Y");
  return t;
}

// Read once, when the library is loaded.
lora::Tuning g_tuning = read_tuning();

lora::SegView view(const lora_segments* seg) {
  lora::SegView s;
  s.token_lora = seg->token_lora;
  s.sorted_token = seg->sorted_token;
  s.seg_lora = seg->seg_lora;
  s.seg_start = seg->seg_start;
  s.counts = seg->counts;
  s.lora_rank = seg->lora_rank;
  s.T = seg->num_tokens;
  s.L = seg->num_loras;
  s.dense = 0;
  return s;
}

}  // namespace

namespace lora {
const Tuning& tuning() { return g_tuning; }
void reload_tuning() { g_tuning = read_tuning(); }
}  // namespace lora

// Scratch of lora_shrink_noalloc: the partial rows of the shrink's H split.
// Each GPU the library runs on holds its own copy from module load until the
// process ends.  Host code never uses this name as an address: the device
// address of the current GPU's copy comes from hipGetSymbolAddress.
static __device__ __align__(256) unsigned char scratch[LORA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of scratch on the GPU that runs `stream` (which must be the
// current device), looked up once per device.
int scratch_address(const char* fn, void* stream, void** out) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return fail(LORA_ERR_HIP, "%s: hipGetDevice: %s", fn, hipGetErrorString(e));
  if (stream) {
    hipDevice_t sd = 0;
    e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &sd);
    if (e != hipSuccess) return fail(LORA_ERR_HIP, "%s: hipStreamGetDevice: %s", fn, hipGetErrorString(e));
    if ((int)sd != cur)
      return fail(LORA_ERR_INVALID_ARG, "%s: the stream belongs to device %d but device %d is current", fn,
                  (int)sd, cur);
  }
  if (cur < 0 || cur >= kMaxDevices)
    return fail(LORA_ERR_UNSUPPORTED, "%s: device %d beyond the %d devices supported", fn, cur, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[cur]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      return fail(LORA_ERR_HIP, "%s: hipGetSymbolAddress(scratch): %s", fn, hipGetErrorString(e));
    g_scratch_ptr[cur] = p;
  }
  *out = g_scratch_ptr[cur];
  return LORA_OK;
}

// Whether a segment-tile shrink hands its one-token segments to the
// per-token kernel (the device-side per-segment choice): automatic path,
// metadata present, and enough adapters for many one-token segments.  The
// per-token shrink takes every rank.
bool shrink_split(const lora::SegView& sv) {
  return g_path.load(std::memory_order_relaxed) == 0 && !sv.dense && sv.L >= 256;
}

// lora_shrink, lora_shrink_noalloc and lora_shrink_single, after their
// batch description (sv) has been checked.  With use_scratch, the H-split
// partial rows go to this device's static scratch instead of a workspace.
int shrink_core(const char* fn, const void* x, int64_t ldx, const void* A, int32_t H, int32_t r,
                const lora::SegView& sv, float* v, int64_t ldv, void* workspace, size_t workspace_bytes,
                bool use_scratch, int dtype, void* stream) {
  if (int e = check_dtype(dtype, fn)) return e;
  if (int e = check_rank(r, fn)) return e;
  if (H < 1) return fail(LORA_ERR_INVALID_ARG, "%s: H %d < 1", fn, H);
  if (ldx < H) return fail(LORA_ERR_INVALID_ARG, "%s: ldx %lld < H %d", fn, (long long)ldx, H);
  if (ldv < r) return fail(LORA_ERR_INVALID_ARG, "%s: ldv %lld < r %d", fn, (long long)ldv, r);
  const int32_t T = sv.T;
  if (T == 0) return ok();
  if (!x || !A || !v) return fail(LORA_ERR_INVALID_ARG, "%s: x, A and v must not be NULL", fn);
  const bool vec = (H % 8 == 0) && (ldx % 8 == 0) && aligned16(x) && aligned16(A) &&
                   (ldv % 4 == 0) && aligned16(v);
  if (use_bgmv(Op::kShrink, T, r, H, vec)) {
    hipError_t err = lora::launch_bgmv_shrink(sv, static_cast<const uint16_t*>(x), ldx,
                                              static_cast<const uint16_t*>(A), H, r, v, ldv, dtype,
                                              vec, static_cast<hipStream_t>(stream));
    return hip_status(err, fn);
  }
  // The static scratch bounds how far the kernel may raise the H split.
  const lora::ShrinkPlan plan =
      lora::plan_shrink(T, sv.L, H, r, use_scratch ? (size_t)LORA_NOALLOC_SCRATCH_BYTES : 0);
  const size_t need = plan.partial_bytes;
  if (use_scratch && need > 0) {
    if (need > (size_t)LORA_NOALLOC_SCRATCH_BYTES)
      return fail(LORA_ERR_UNSUPPORTED,
                  "%s: this shrink needs %zu bytes of scratch, more than the %zu of the static scratch "
                  "(LORA_NOALLOC_SCRATCH_BYTES); use lora_shrink with a workspace",
                  fn, need, (size_t)LORA_NOALLOC_SCRATCH_BYTES);
    if (int e = scratch_address(fn, stream, &workspace)) return e;
    workspace_bytes = LORA_NOALLOC_SCRATCH_BYTES;
  }
  if (need > 0) {
    if (!workspace || workspace_bytes < need)
      return fail(LORA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                  workspace ? workspace_bytes : (size_t)0);
    if (!aligned16(workspace))
      return fail(LORA_ERR_WORKSPACE, "%s: workspace must be 16-byte aligned", fn);
  }
  // The per-segment choice of the expand (below) applies to the shrink too:
  // in a batch of at least 256 adapters, one-token segments go to the
  // per-token kernel, launched last so that the split-H reduce (which writes
  // every active row from the partial rows) cannot overwrite them.  Measured
  // on MI355X, 7168 prefill + 1024 decode tokens over 1040 adapters, H =
  // 4096, tiles alone against tiles on the prefill + per-token on the decode
  // tokens: 119 -> 52 us at r = 16, 184 -> 132 at r = 64, 268 -> 230 at
  // r = 128; with no one-token segment the empty per-token pass adds 2.5-4 us.
  const bool split = shrink_split(sv);
  hipError_t err = lora::launch_shrink(sv, static_cast<const uint16_t*>(x), ldx,
                                       static_cast<const uint16_t*>(A), H, r, v, ldv, workspace,
                                       plan, dtype, vec, static_cast<hipStream_t>(stream), split ? 2 : 1);
  if (err == hipSuccess && split)
    err = lora::launch_bgmv_shrink(sv, static_cast<const uint16_t*>(x), ldx, static_cast<const uint16_t*>(A),
                                   H, r, v, ldv, dtype, vec, static_cast<hipStream_t>(stream), 1);
  return hip_status(err, fn);
}

int shrink_call(const char* fn, const void* x, int64_t ldx, const void* A, int32_t H, int32_t r,
                const lora_segments* seg, float* v, int64_t ldv, void* workspace, size_t workspace_bytes,
                bool use_scratch, int dtype, void* stream) {
  if (int e = check_segments(seg, fn)) return e;
  return shrink_core(fn, x, ldx, A, H, r, view(seg), v, ldv, workspace, workspace_bytes, use_scratch,
                     dtype, stream);
}

// The batch of the single-adapter entry points: T tokens, all on adapter 0.
lora::SegView dense_view(int32_t T) {
  lora::SegView s{};
  s.T = T;
  s.L = 1;
  s.dense = 1;
  return s;
}

}  // namespace

extern "C" {

size_t lora_segments_workspace_bytes(int32_t T, int32_t L) {
  // The builder is one workgroup whose histogram, scans and scatter cursors
  // all live in LDS: it needs no device scratch for any T and L in range.
  (void)T;
  (void)L;
  return 0;
}

int lora_build_segments(const int32_t* token_lora, int32_t T, int32_t L, lora_segments* seg,
                        void* workspace, size_t workspace_bytes, void* stream) {
  static const char* fn = "lora_build_segments";
  if (!seg) return fail(LORA_ERR_INVALID_ARG, "%s: seg is NULL", fn);
  if (T < 0) return fail(LORA_ERR_INVALID_ARG, "%s: num_tokens %d < 0", fn, T);
  if (L < 1 || L > LORA_MAX_LORAS)
    return fail(LORA_ERR_UNSUPPORTED, "%s: num_loras %d outside [1, %d]", fn, L, LORA_MAX_LORAS);
  if (T > 0 && !token_lora) return fail(LORA_ERR_INVALID_ARG, "%s: token buffers must not be NULL", fn);
  const size_t need = lora_segments_workspace_bytes(T, L);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(LORA_ERR_WORKSPACE, "%s: workspace of %zu bytes needed, %zu given", fn, need,
                workspace ? workspace_bytes : (size_t)0);
  seg->num_tokens = T;
  seg->num_loras = L;
  seg->token_lora = token_lora;
  if (int e = check_segments(seg, fn)) return e;
  hipError_t err = lora::launch_build_segments(seg->token_lora, seg->num_tokens, seg->num_loras,
                                               seg->sorted_token, seg->seg_lora, seg->seg_start,
                                               seg->counts, static_cast<hipStream_t>(stream));
  return hip_status(err, fn);
}

size_t lora_shrink_workspace_bytes(int32_t T, int32_t L, int32_t H, int32_t r) {
  if (T <= 0 || L < 1 || H < 1 || r < 1 || r > LORA_MAX_RANK) return 0;
  const lora::ShrinkPlan p = lora::plan_shrink(T, L, H, r);
  return p.partial_bytes;
}

int lora_shrink(const void* x, int64_t ldx, const void* A, int32_t H, int32_t r,
                const lora_segments* seg, float* v, int64_t ldv, void* workspace,
                size_t workspace_bytes, int dtype, void* stream) {
  return shrink_call("lora_shrink", x, ldx, A, H, r, seg, v, ldv, workspace, workspace_bytes, false,
                     dtype, stream);
}

int lora_shrink_noalloc(const void* x, int64_t ldx, const void* A, int32_t H, int32_t r,
                        const lora_segments* seg, float* v, int64_t ldv, int dtype, void* stream) {
  return shrink_call("lora_shrink_noalloc", x, ldx, A, H, r, seg, v, ldv, nullptr, 0, true, dtype,
                     stream);
}

}  // extern "C"

namespace {

// Checks the slices of an expand_slice and fills their descriptors: none
// NULL or empty, inside [0, ldy), none overlapping another.
int check_slices(const char* fn, const void* const* B, const int32_t* n_s, const int64_t* col_off,
                 int32_t num_slices, int64_t ldy, lora::ExpandSliceDesc* desc) {
  if (num_slices < 1 || num_slices > LORA_MAX_SLICES)
    return fail(LORA_ERR_UNSUPPORTED, "%s: num_slices %d outside [1, %d]", fn, num_slices,
                LORA_MAX_SLICES);
  if (!B || !n_s || !col_off)
    return fail(LORA_ERR_INVALID_ARG, "%s: B, n_s and col_off must not be NULL", fn);
  int order[LORA_MAX_SLICES];
  for (int s = 0; s < num_slices; ++s) {
    if (!B[s]) return fail(LORA_ERR_INVALID_ARG, "%s: B[%d] is NULL", fn, s);
    if (n_s[s] < 1) return fail(LORA_ERR_INVALID_ARG, "%s: n_s[%d] = %d < 1", fn, s, n_s[s]);
    if (col_off[s] < 0 || col_off[s] + n_s[s] > ldy)
      return fail(LORA_ERR_INVALID_ARG, "%s: slice %d columns [%lld, %lld) outside [0, ldy=%lld)",
                  fn, s, (long long)col_off[s], (long long)(col_off[s] + n_s[s]), (long long)ldy);
    desc[s].B = static_cast<const uint16_t*>(B[s]);
    desc[s].n = n_s[s];
    desc[s].col_off = col_off[s];
    order[s] = s;
  }
  std::sort(order, order + num_slices, [&](int a, int b) { return col_off[a] < col_off[b]; });
  for (int i = 1; i < num_slices; ++i) {
    const int a = order[i - 1], b = order[i];
    if (col_off[a] + n_s[a] > col_off[b])
      return fail(LORA_ERR_INVALID_ARG, "%s: slices %d and %d overlap", fn, a, b);
  }
  return LORA_OK;
}

// lora_expand_slice and lora_expand_slice_single after their batch
// description (sv) has been checked.
int expand_core(const char* fn, const float* v, int64_t ldv, int64_t v_slice_stride, const void* const* B,
                const int32_t* n_s, const int64_t* col_off, int32_t num_slices, int32_t r,
                const lora::SegView& sv, void* y, int64_t ldy, int add_inputs, int dtype, void* stream) {
  if (int e = check_dtype(dtype, fn)) return e;
  if (int e = check_rank(r, fn)) return e;
  if (ldv < r) return fail(LORA_ERR_INVALID_ARG, "%s: ldv %lld < r %d", fn, (long long)ldv, r);
  if (v_slice_stride < 0)
    return fail(LORA_ERR_INVALID_ARG, "%s: v_slice_stride %lld < 0", fn, (long long)v_slice_stride);
  lora::ExpandSliceDesc desc[LORA_MAX_SLICES];
  if (int e = check_slices(fn, B, n_s, col_off, num_slices, ldy, desc)) return e;
  const int32_t T = sv.T;
  if (T == 0) return ok();
  if (!v || !y) return fail(LORA_ERR_INVALID_ARG, "%s: v and y must not be NULL", fn);
  bool vec = (r % 8 == 0) && (ldv % 4 == 0) && (v_slice_stride % 4 == 0) && aligned16(v) &&
             (ldy % 8 == 0) && aligned16(y);
  for (int s = 0; s < num_slices; ++s)
    vec = vec && aligned16(B[s]) && (col_off[s] % 8 == 0) && (n_s[s] % 8 == 0);
  if (g_path.load(std::memory_order_relaxed) == 1 && !lora::bgmv_supports(true, r, vec))
    return fail(LORA_ERR_UNSUPPORTED,
                "%s: the per-token path takes r <= %d, or r = 128 with 16-byte aligned rows and sizes "
                "that are multiples of 8", fn, lora::kBgmvMaxRank);
  int64_t ncols = 0;
  for (int s = 0; s < num_slices; ++s) ncols += n_s[s];
  if (use_bgmv(Op::kExpand, T, r, ncols, vec)) {
    hipError_t err = lora::launch_bgmv_expand(sv, v, ldv, v_slice_stride, desc, num_slices, r,
                                              static_cast<uint16_t*>(y), ldy, add_inputs ? 1 : 0,
                                              dtype, vec, static_cast<hipStream_t>(stream));
    return hip_status(err, fn);
  }
  // Per-segment choice on the device (punica issue: BGMV for inputs with
  // their own adapter, SGMV for segments sharing one): in a batch that mixes
  // prefill segments with one-token (decode) segments, the tile kernel takes
  // the segments of two tokens and more and the per-token kernel takes the
  // one-token segments, each finding its own from the metadata.  Measured on
  // MI355X (7168 prefill tokens over 16 adapters plus 1024 decode tokens with
  // an adapter each, H = n = 4096): tiles alone 174 us (r = 16) and 219 us
  // (r = 64), tiles on the prefill + per-token on the decode tokens 81 and
  // 158 us.  Segments of 2 to 7 tokens measured faster on tiles at r = 64, so
  // only one-token segments move; at r = 128 the per-token expand is about
  // twice as slow as the tiles on small batches (16-512 tokens: 15-20 us
  // against 10-12), so the split stops at r = 64.  The second launch costs
  // 2.5-4 us when it finds nothing, so it is made only when the batch can
  // hold many one-token segments: at least 256 adapters.
  // With aligned data and r = 8, 16, 32 or 64 the tile launch itself takes
  // the one-token segments as per-token work items (the aligned per-token
  // expand's body), so both kinds of segment share one launch; other shapes
  // take a second, per-token launch.
  const bool split = g_path.load(std::memory_order_relaxed) == 0 && !sv.dense && sv.L >= 256 &&
                     r <= lora::kBgmvMaxRank;
  const bool one_launch = split && vec && (r == 8 || r == 16 || r == 32 || r == 64);
  hipError_t err = lora::launch_expand(sv, v, ldv, v_slice_stride, desc, num_slices, r,
                                       static_cast<uint16_t*>(y), ldy, add_inputs ? 1 : 0, dtype,
                                       vec, static_cast<hipStream_t>(stream), split ? 2 : 1, one_launch);
  if (err == hipSuccess && split && !one_launch)
    err = lora::launch_bgmv_expand(sv, v, ldv, v_slice_stride, desc, num_slices, r,
                                   static_cast<uint16_t*>(y), ldy, add_inputs ? 1 : 0, dtype, vec,
                                   static_cast<hipStream_t>(stream), 1);
  return hip_status(err, fn);
}

}  // namespace

extern "C" {

int lora_expand_slice(const float* v, int64_t ldv, int64_t v_slice_stride, const void* const* B,
                      const int32_t* n_s, const int64_t* col_off, int32_t num_slices, int32_t r,
                      const lora_segments* seg, void* y, int64_t ldy, int add_inputs, int dtype,
                      void* stream) {
  static const char* fn = "lora_expand_slice";
  if (int e = check_segments(seg, fn)) return e;
  return expand_core(fn, v, ldv, v_slice_stride, B, n_s, col_off, num_slices, r, view(seg), y, ldy,
                     add_inputs, dtype, stream);
}

int lora_shrink_expand(const void* x, int64_t ldx, const void* A, int32_t H, int32_t r, const void* const* B,
                       const int32_t* n_s, const int64_t* col_off, int32_t num_slices,
                       const lora_segments* seg, float* v, int64_t ldv, void* y, int64_t ldy, int add_inputs,
                       int dtype, void* stream) {
  static const char* fn = "lora_shrink_expand";
  if (int e = check_segments(seg, fn)) return e;
  if (int e = check_dtype(dtype, fn)) return e;
  if (int e = check_rank(r, fn)) return e;
  if (r != 8 && r != 16 && r != 32 && r != 64)
    return fail(LORA_ERR_UNSUPPORTED,
                "%s: rank %d is not 8, 16, 32 or 64 (use lora_shrink and lora_expand_slice)", fn, r);
  if (H < 1) return fail(LORA_ERR_INVALID_ARG, "%s: H %d < 1", fn, H);
  if (ldx < H) return fail(LORA_ERR_INVALID_ARG, "%s: ldx %lld < H %d", fn, (long long)ldx, H);
  if (ldv < r) return fail(LORA_ERR_INVALID_ARG, "%s: ldv %lld < r %d", fn, (long long)ldv, r);
  lora::ExpandSliceDesc desc[LORA_MAX_SLICES];
  if (int e = check_slices(fn, B, n_s, col_off, num_slices, ldy, desc)) return e;
  const lora::SegView sv = view(seg);
  if (sv.T == 0) return ok();
  if (!x || !A || !v || !y) return fail(LORA_ERR_INVALID_ARG, "%s: x, A, v and y must not be NULL", fn);
  bool aligned = (H % 8 == 0) && (ldx % 8 == 0) && aligned16(x) && aligned16(A) && (ldy % 8 == 0) &&
                 aligned16(y);
  for (int q = 0; q < num_slices; ++q)
    aligned = aligned && aligned16(B[q]) && (col_off[q] % 8 == 0) && (n_s[q] % 8 == 0);
  if (!aligned)
    return fail(LORA_ERR_UNSUPPORTED,
                "%s: needs 16-byte aligned x, A, B and y with H, ldx, ldy, the slice widths and offsets "
                "multiples of 8 (use lora_shrink and lora_expand_slice)", fn);
  hipError_t err = lora::launch_fused_decode(sv, static_cast<const uint16_t*>(x), ldx,
                                             static_cast<const uint16_t*>(A), H, r, v, ldv, desc, num_slices,
                                             static_cast<uint16_t*>(y), ldy, add_inputs ? 1 : 0, dtype,
                                             static_cast<hipStream_t>(stream));
  return hip_status(err, fn);
}

int lora_expand_slice_single(const float* v, int64_t ldv, int64_t v_slice_stride, const void* const* B,
                             const int32_t* n_s, const int64_t* col_off, int32_t num_slices, int32_t r,
                             int32_t T, void* y, int64_t ldy, int add_inputs, int dtype, void* stream) {
  static const char* fn = "lora_expand_slice_single";
  if (T < 0) return fail(LORA_ERR_INVALID_ARG, "%s: T %d < 0", fn, T);
  return expand_core(fn, v, ldv, v_slice_stride, B, n_s, col_off, num_slices, r, dense_view(T), y, ldy,
                     add_inputs, dtype, stream);
}

int lora_expand_single(const float* v, int64_t ldv, const void* B, int32_t r, int32_t n, int32_t T,
                       void* y, int64_t ldy, int add_inputs, int dtype, void* stream) {
  const void* Bs[1] = {B};
  const int32_t ns[1] = {n};
  const int64_t off[1] = {0};
  int rc = lora_expand_slice_single(v, ldv, 0, Bs, ns, off, 1, r, T, y, ldy, add_inputs, dtype, stream);
  if (rc != LORA_OK) {
    char tmp[512];
    snprintf(tmp, sizeof tmp, "lora_expand_single: %s", g_error);
    snprintf(g_error, sizeof g_error, "%s", tmp);
  }
  return rc;
}

size_t lora_shrink_single_workspace_bytes(int32_t T, int32_t H, int32_t r) {
  return lora_shrink_workspace_bytes(T, 1, H, r);
}

int lora_shrink_single(const void* x, int64_t ldx, const void* A, int32_t H, int32_t r, int32_t T,
                       float* v, int64_t ldv, void* workspace, size_t workspace_bytes, int dtype,
                       void* stream) {
  static const char* fn = "lora_shrink_single";
  if (T < 0) return fail(LORA_ERR_INVALID_ARG, "%s: T %d < 0", fn, T);
  return shrink_core(fn, x, ldx, A, H, r, dense_view(T), v, ldv, workspace, workspace_bytes, false, dtype,
                     stream);
}

int lora_expand(const float* v, int64_t ldv, const void* B, int32_t r, int32_t n,
                const lora_segments* seg, void* y, int64_t ldy, int add_inputs, int dtype,
                void* stream) {
  const void* Bs[1] = {B};
  const int32_t ns[1] = {n};
  const int64_t off[1] = {0};
  int rc = lora_expand_slice(v, ldv, 0, Bs, ns, off, 1, r, seg, y, ldy, add_inputs, dtype, stream);
  if (rc != LORA_OK) {
    // Report under this entry point's name.
    char tmp[512];
    snprintf(tmp, sizeof tmp, "lora_expand: %s", g_error);
    snprintf(g_error, sizeof g_error, "%s", tmp);
  }
  return rc;
}

int lora_set_path(int mode) {
  if (mode < 0 || mode > 2)
    return fail(LORA_ERR_INVALID_ARG, "lora_set_path: mode %d is not 0, 1 or 2", mode);
  return g_path.exchange(mode);
}

void lora_reload_tuning(void) { lora::reload_tuning(); }

const char* lora_last_error(void) { return g_error; }

}  // extern "C"
