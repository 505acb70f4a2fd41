/*
 * liblora_mi355x: multi-LoRA gather-matmul (shrink / expand / expand_slice)
 * for AMD Instinct MI355X (gfx950).
 *
 * Problem statement (from the pages this library follows):
 *  - vLLM PR "[misc] Add LoRA kernel micro benchmarks": one call computes a
 *    whole m x k x n product in which every token uses the weight matrix that
 *    its LoRA id selects out of num_loras; the ops are shrink, expand and
 *    expand_slice in BGMV (one token per sequence) and SGMV (segments)
 *    forms; expand optionally adds to the existing output (add_inputs); its
 *    input is fp32 and its weights and output are fp16/bf16; expand_slice is
 *    equivalent to one expand per output slice; shrink with split-K either
 *    stores or accumulates, which makes repeated calls hard to check.
 *  - vLLM PR "[Hardware][TPU][V1] Multi-LoRA Optimisations for the V1 TPU
 *    backend", summary: shrink and expand as separate kernels; adapters used
 *    by expand are pre-transposed once at load time.
 *  - punica issue "The smallest rank supported is 16?": segments of tokens
 *    sharing one adapter (SGMV) with BGMV as a strict subset; ranks other
 *    than the supported bins are handled by zero padding.
 *
 * Mathematics.  For token t with adapter l = lora(t):
 *   shrink:  v[t, j] = sum_{h < H} x[t, h] * A_l[h, j]            j < r
 *   expand:  y[t, c] = (add_inputs ? y[t, c] : 0) + sum_{j < r} v[t, j] * B_l[j, c]
 * lora(t) = -1 means "no adapter": such rows of v and y are never written.
 *
 * Memory layouts (all row-major, every pointer below is DEVICE memory unless
 * marked host; the contraction index of both weights is contiguous):
 *   x  [T][ldx]        fp16/bf16
 *   A  [L][r][H]       fp16/bf16   (A_l stored transposed: row j holds A_l[:, j])
 *   v  [T][ldv]        fp32
 *   B  [L][n][r]       fp16/bf16   (B_l stored transposed: row c holds B_l[:, c])
 *   y  [T][ldy]        fp16/bf16
 * x, A, B and y share one dtype.
 *
 * Calls.  Every call is asynchronous on the given stream (a hipStream_t passed
 * as void*; NULL = the default stream), copies nothing between host and device,
 * never synchronises, and launches a fixed number of kernels whose geometry
 * depends only on the scalar arguments, so calls can be captured in a HIP
 * graph.  Host-checkable errors return a negative status before anything is
 * launched; lora_last_error() then describes the problem.  Data-dependent
 * problems (adapter ids outside [-1, L)) are not errors: such tokens are
 * treated as -1 and counted.
 *
 * Precision.  Products are accumulated in fp32.  expand rounds once, to
 * nearest even, when it writes y.  Inside expand the fp32 v is split into a
 * high and a low 16-bit part, hi = round(v) and lo = round(v - hi), so that
 * the matrix cores see v to about 16 significant bits (bf16) or 22 (fp16).
 * With fp16 data each token's v is first multiplied by a power of two that
 * brings its largest |v| into [2^13, 2^14), and the fp32 products are
 * multiplied back before y is added: any finite fp32 v is accepted, also
 * beyond the fp16 range.
 */
#ifndef LORA_MI355X_H
#define LORA_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define LORA_OK 0
#define LORA_ERR_INVALID_ARG (-1)  /* bad pointer, size, stride or slice layout      */
#define LORA_ERR_UNSUPPORTED (-2)  /* outside the supported envelope (limits below)  */
#define LORA_ERR_WORKSPACE (-3)    /* workspace missing or too small                 */
#define LORA_ERR_HIP (-4)          /* the HIP runtime reported an error at launch    */

/* Element types of x, A, B and y. */
#define LORA_F16 0
#define LORA_BF16 1

/* Limits. */
#define LORA_MAX_RANK 128     /* r in [1, 128]                                      */
#define LORA_MAX_LORAS 2048   /* L in [1, 2048]                                     */
#define LORA_MAX_SLICES 8     /* expand_slice: 1..8 slices                          */

/* Segment metadata of one batch: tokens grouped by adapter (SGMV segments).
 * A host struct whose pointers are caller-owned device buffers.  Built once
 * per batch by lora_build_segments and then read by every shrink / expand
 * of that batch.  Contents after a build:
 *   sorted_token[T]  active tokens ordered by (adapter id, token index), then
 *                    the tokens without an adapter in ascending order
 *   seg_lora[L]      adapter id of segment s for s < S, then -1
 *   seg_start[L+1]   first position in sorted_token of segment s; entries
 *                    S..L hold T_a (the number of active tokens)
 *   counts[4]        {S, T_a, longest segment, number of ids outside [-1, L)}
 * Callers that already hold grouped batches may fill these buffers (and the
 * three fields that lora_build_segments sets) themselves, as long as they
 * respect exactly these invariants. */
typedef struct lora_segments {
  int32_t num_tokens;          /* T >= 0 (set by lora_build_segments)            */
  int32_t num_loras;           /* L in [1, LORA_MAX_LORAS] (set by the build)     */
  const int32_t *token_lora;   /* [T] adapter id of each token, -1 = none (set by
                                * the build to the pointer it was given)         */
  int32_t *sorted_token;       /* [T]                                           */
  int32_t *seg_lora;           /* [L]                                           */
  int32_t *seg_start;          /* [L + 1]                                       */
  int32_t *counts;             /* [4]                                           */
  const int32_t *lora_rank;    /* [L] optional (NULL = every adapter has rank r):
                                * live rank of each adapter, read by the segment
                                * (SGMV) kernels, which then skip A rows and B rank
                                * pieces at or beyond it; those must hold zeros
                                * (the issue's rank padding), since the per-token
                                * kernels read the padded weights as they are.
                                * Values are clamped to [0, r].                   */
} lora_segments;

/* Device scratch bytes lora_build_segments needs for T tokens and L
 * adapters.  The builder is one workgroup whose histogram, scans and scatter
 * cursors live in LDS, so this is 0 for every T and L in range; callers that
 * size a workspace from it stay correct if that changes. */
size_t lora_segments_workspace_bytes(int32_t T, int32_t L);

/* Builds the segment metadata of one batch (punica issue: SGMV segments of
 * tokens that share an adapter; TPU PR summary: tokens without an adapter
 * are skipped) with one kernel of one workgroup.
 *   token_lora  [T] device, adapter id per token; -1 = no adapter; ids outside
 *               [-1, L) are treated as -1 and counted in counts[3]
 *   seg         host struct whose four output pointers (sorted_token,
 *               seg_lora, seg_start, counts) the caller has set to device
 *               buffers of the sizes above; the call sets num_tokens = T,
 *               num_loras = L and token_lora, and leaves lora_rank alone
 *   workspace   device scratch of lora_segments_workspace_bytes(T, L) bytes
 *               (may be NULL when that is 0)
 * The order inside a segment is ascending token index, so the result is
 * unique.  T = 0 and all-(-1) batches are valid.
 * Errors: LORA_ERR_INVALID_ARG for a NULL seg or buffer (with T > 0) or
 * T < 0; LORA_ERR_UNSUPPORTED for L outside [1, LORA_MAX_LORAS];
 * LORA_ERR_WORKSPACE; LORA_ERR_HIP. */
int lora_build_segments(const int32_t *token_lora, int32_t T, int32_t L, lora_segments *seg,
                        void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes that lora_shrink needs for T tokens, L adapters, hidden
 * size H and rank r (0 if it needs none).  Only batches with too few token
 * tiles to occupy the GPU split the H-sum across workgroups (mid-size
 * batches at r <= 32 and small H split it across the waves of one workgroup
 * instead, and need none); the workspace
 * then holds a 256-byte header (the split the kernel chose) and one fp32
 * partial row per token and H chunk, for as many chunks as the kernel may
 * choose for the fewest tiles T tokens can make.  The host sees only an
 * upper bound on the tiles (one partial tile per adapter of the pool); the
 * kernel sets the split from the true count, so a batch that uses few
 * adapters of a large pool still fills the GPU. */
size_t lora_shrink_workspace_bytes(int32_t T, int32_t L, int32_t H, int32_t r);

/* Shrink (micro-benchmark PR: bgmv_shrink / sgmv_shrink; TPU PR: the
 * separate shrink kernel):  v[t, j] = sum_h x[t, h] * A_l[h, j], j < r, for
 * every active token t, fp32 accumulation, fp32 result.  v rows of tokens
 * without an adapter are not written.  The result overwrites v: any split of
 * the H-sum across waves or workgroups is reduced inside the call in a
 * fixed order, so repeated calls give identical bits.  When the H-sum is
 * split across workgroups the call launches a second, small kernel.
 *   x          [T][ldx] device, ldx >= H
 *   A          [L][r][H] device
 *   seg        metadata built for this batch (T, L taken from it)
 *   v          [T][ldv] fp32 device, ldv >= r
 *   workspace  device buffer of >= lora_shrink_workspace_bytes(T, L, H, r)
 *              bytes, 16-byte aligned (may be NULL when that size is 0); its
 *              contents need no initialisation.  Calls that run concurrently
 *              must not share a workspace.
 * Errors: INVALID_ARG (NULL pointers, H < 1, ld too small, bad dtype),
 * UNSUPPORTED (r outside [1, LORA_MAX_RANK]), WORKSPACE, HIP. */
int lora_shrink(const void *x, int64_t ldx, const void *A, int32_t H, int32_t r,
                const lora_segments *seg, float *v, int64_t ldv, void *workspace,
                size_t workspace_bytes, int dtype, void *stream);

/* Size of the static device scratch of lora_shrink_noalloc (16 MiB per GPU). */
#define LORA_NOALLOC_SCRATCH_BYTES (16u << 20)

/* lora_shrink without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc.  Same arguments,
 * kernels as lora_shrink; the partial rows of an H split go to a
 * static device array of LORA_NOALLOC_SCRATCH_BYTES that each GPU holds from
 * the library's load until the process ends (its address is looked up once
 * per device, on the first call that needs it, with the stream's device
 * current).  Every partial row is written before it is read, so nothing has
 * to be cleared between calls; the array keeps the last call's contents.
 * All calls on one GPU share the array: calls that overlap in time on one
 * GPU (different streams, or host threads) race and must be serialised by
 * the caller; calls on one stream are ordered and safe.  The results are
 * lora_shrink's bits except where the kernel would split H into more chunks
 * than the array holds: then it takes fewer, and v may differ in the last
 * bits (fp32 sums in another grouping), within the same tolerance.
 * Errors: those of lora_shrink; LORA_ERR_UNSUPPORTED when the split the host
 * chooses from the tile bound needs more than LORA_NOALLOC_SCRATCH_BYTES --
 * reported before anything is launched; LORA_ERR_INVALID_ARG
 * when the stream belongs to a device other than the current one. */
int lora_shrink_noalloc(const void *x, int64_t ldx, const void *A, int32_t H, int32_t r,
                        const lora_segments *seg, float *v, int64_t ldv, int dtype, void *stream);

/* Expand (micro-benchmark PR: bgmv_expand / sgmv_expand, add_inputs):
 *   y[t, c] = (add_inputs ? y[t, c] : 0) + sum_{j<r} v[t, j] * B_l[j, c],  c < n
 * for every active token; rows of tokens without an adapter and columns
 * c >= n are not touched.  One rounding to the output type per element.
 *   v  [T][ldv] fp32 device;  B  [L][n][r] device;  y  [T][ldy] device, ldy >= n.
 * Same as lora_expand_slice with one slice at column 0. */
int lora_expand(const float *v, int64_t ldv, const void *B, int32_t r, int32_t n,
                const lora_segments *seg, void *y, int64_t ldy, int add_inputs,
                int dtype, void *stream);

/* Expand into column slices of a fused output (micro-benchmark PR:
 * expand_slice, num_slices; equivalent to one expand per slice issued back to
 * back).  Slice s uses weights B[s] ([L][n_s[s]][r], device), input
 * v + s * v_slice_stride (elements; 0 = all slices share one v) and writes
 * columns [col_off[s], col_off[s] + n_s[s]) of y.  B, n_s and col_off are
 * HOST arrays of num_slices entries.  Slices must lie inside [0, ldy) and must
 * not overlap; columns outside every slice are not touched.
 * Errors: INVALID_ARG (NULL pointers, n_s < 1, overlapping or out-of-range
 * slices), UNSUPPORTED (num_slices outside [1, LORA_MAX_SLICES], r range), HIP. */
int lora_expand_slice(const float *v, int64_t ldv, int64_t v_slice_stride,
                      const void *const *B, const int32_t *n_s, const int64_t *col_off,
                      int32_t num_slices, int32_t r, const lora_segments *seg, void *y,
                      int64_t ldy, int add_inputs, int dtype, void *stream);

/* Shrink then expand_slice in one launch, for decode batches (TPU PR summary:
 * the Pallas kernel was split into separate shrink and expand kernels;
 * which form is faster depends on the shape -- one launch instead of two
 * pays where a decode step's calls are bound by their launch and round
 * trips).  Computes v = x . A_l as lora_shrink (v is written, the same
 * values up to the order of the fp32 sums) and y (+)= v . B_s[l] for every
 * slice as lora_expand_slice with v_slice_stride 0.  Each token is handled by
 * its own workgroups, so the cost grows with T times the adapter's weight
 * bytes: meant for decode batches (up to a few hundred tokens); larger
 * batches belong to the separate calls.  Reads token_lora only (the sorted
 * metadata need not be built).
 *   r          8, 16, 32 or 64
 *   x, A       as lora_shrink;  B, n_s, col_off, num_slices, y, ldy as
 *              lora_expand_slice;  v  [T][ldv] fp32 device, ldv >= r, written
 * Every row and size must be 16-byte aligned: x, A, B, y 16-byte aligned; H,
 * ldx, ldy, n_s[] and col_off[] multiples of 8.
 * Errors: INVALID_ARG (NULL pointers, H < 1, ld too small, bad dtype, slice
 * errors as lora_expand_slice), UNSUPPORTED (another rank, unaligned data,
 * num_slices), HIP. */
int lora_shrink_expand(const void *x, int64_t ldx, const void *A, int32_t H, int32_t r,
                       const void *const *B, const int32_t *n_s, const int64_t *col_off,
                       int32_t num_slices, const lora_segments *seg, float *v, int64_t ldv,
                       void *y, int64_t ldy, int add_inputs, int dtype, void *stream);

/* Single-adapter forms (TPU PR summary: the masking is removed when only one
 * adapter is in use; micro-benchmark PR review thread: with few adapters the
 * kernels should match torch.mm).  Every token t in [0, T) uses the one
 * adapter, so no segment metadata exists and none is read: token index =
 * row, as in a plain dense product.  Same results as the segment forms with
 * every id 0 and L = 1; same validation, except that T >= 0 replaces the
 * metadata checks.
 *   A  [r][H] device (the adapter's H x r matrix stored transposed)
 *   B  [n][r] device, per slice (the adapter's r x n matrix stored transposed)
 * lora_shrink_single needs a workspace of lora_shrink_single_workspace_bytes
 * (T, H, r) bytes (0 when its H-sum is not split). */
size_t lora_shrink_single_workspace_bytes(int32_t T, int32_t H, int32_t r);
int lora_shrink_single(const void *x, int64_t ldx, const void *A, int32_t H, int32_t r, int32_t T,
                       float *v, int64_t ldv, void *workspace, size_t workspace_bytes, int dtype,
                       void *stream);
int lora_expand_single(const float *v, int64_t ldv, const void *B, int32_t r, int32_t n, int32_t T,
                       void *y, int64_t ldy, int add_inputs, int dtype, void *stream);
int lora_expand_slice_single(const float *v, int64_t ldv, int64_t v_slice_stride,
                             const void *const *B, const int32_t *n_s, const int64_t *col_off,
                             int32_t num_slices, int32_t r, int32_t T, void *y, int64_t ldy,
                             int add_inputs, int dtype, void *stream);

/* Kernel path (punica issue: BGMV, one adapter per input, is a strict subset
 * of SGMV, segments of inputs sharing an adapter; both compute the same
 * result).  0 = automatic: batches of at most 512 tokens may take the
 * per-token (BGMV) kernels -- a shrink when a cost fitted to measured times of
 * both families (from T, H and r) favours it, an expand when r <= 16 and
 * T n <= 4M or r <= 32 and T n <= 1M -- everything else the segment-tile
 * (SGMV) kernels.  In automatic mode, a segment-tile call of at least 256
 * adapters also chooses per segment on the device (punica issue, BGMV vs
 * SGMV): its one-token segments go to per-token work (the shrink at every
 * rank, the expand up to r = 64), its longer segments to the tiles.
 * 1 = always per-token (shrink: any r; expand: r <= 64, or r = 128 with
 * 16-byte aligned rows and sizes that are multiples of 8, else
 * LORA_ERR_UNSUPPORTED); 2 = always segment tiles, every segment.
 * Process-wide, meant for tests and measurement.  Returns the previous mode,
 * or LORA_ERR_INVALID_ARG for an unknown mode. */
int lora_set_path(int mode);

/* Re-reads the launch-plan overrides (LORA_SHRINK_KSPLIT, LORA_EXPAND_TB,
 * LORA_EXPAND_CPR, LORA_BGMV_SHRINK_RT, LORA_BGMV_RPI, LORA_BGMV_CB) from the
 * environment.  They are read once when the library is loaded; this is for
 * tests and measurement that change them within one process, and must not
 * run concurrently with other calls.  Every plan they select computes the
 * same result. */
void lora_reload_tuning(void);

/* Message describing the last non-OK status returned on this thread. */
const char *lora_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* LORA_MI355X_H */
