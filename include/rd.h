/*
 * rd.h -- C ABI of librd.so: ragged dot (grouped GEMM) for mixture-of-experts
 * expert FFNs, and the limit-aware silu(gate) * up GLU, on MI355X (gfx950).
 *
 * Sources of the operations (the pages these entry points implement):
 *   [SkyRL]   SkyRL-tx PR #867, "Integrate ragged_dot pallas kernel with
 *             group_offset support": ragged_dot, its trans_rhs form,
 *             trans_ragged_dot, the VJP rules in the review, and the
 *             group_offset window of the suggested fast_ragged_dot.
 *   [MaxText] MaxText PR #5760, "397B v7x trainer: MoE wo FSDP sharding and
 *             valid-rows-only MoE kernels", commit on valid rows: the
 *             packed-buffer row limit, the glu_rows forward/backward and the
 *             weighted unsort backward (unsort_bwd_rows).
 *   [TE]      TransformerEngine PR #2213, "Async issuing D2H memcpy for
 *             grouped_gemm group_sizes array", Description: copying
 *             group_sizes to the host stalls the GPU and breaks graph capture.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensors are device pointers to contiguous row-major arrays, 16-byte
 *   aligned, owned by the caller.  The library allocates nothing per call,
 *   keeps no per-call state, and is reentrant.
 * - bf16 means IEEE binary32 truncated to its high 16 bits (bfloat16).
 * - group_sizes, group_offset and limit are DEVICE scalars/arrays (int32).
 *   The host never reads them: no device-to-host copy and no synchronisation
 *   happens inside any call ([TE]), so every call may be captured in a HIP
 *   graph and replayed after group_sizes changes on the device.
 * - Every call enqueues its kernels on `stream` (a hipStream_t; NULL is the
 *   legacy default stream) and returns without waiting.
 * - Return value: RD_OK, or a nonzero status.  Problems visible on the host
 *   (null pointers, bad sizes, misalignment, unknown dtype) are reported
 *   before anything is launched; a launch failure reports RD_EHIP.  Faults
 *   of enqueued work surface at the caller's next synchronisation, as usual
 *   for HIP.  Device-side values never cause out-of-bounds accesses; they
 *   are clamped as follows:
 *     * a negative group size counts as 0;
 *     * L = clamp(*limit, 0, m) (m when limit is NULL);
 *     * group boundaries are the exclusive prefix sums of the sizes,
 *       clamped to [0, L]; rows beyond the sum of the sizes belong to no
 *       group;
 *     * a window that does not fit (offset < 0 or offset + num_local >
 *       num_groups) is empty.
 */
#ifndef RD_H
#define RD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RD_ABI_VERSION 8

/* status codes */
#define RD_OK 0
#define RD_EINVAL 1        /* a host-visible argument is invalid           */
#define RD_EUNSUPPORTED 2  /* valid but outside what the kernels support   */
#define RD_EHIP 3          /* the HIP runtime reported an error            */
#define RD_ESCRATCH 4      /* rd_forward_noalloc: sizes need more scratch  */

/* element types */
#define RD_BF16 0
#define RD_F32 1

/* largest num_groups (and num_local) the device-side schedule handles */
#define RD_MAX_GROUPS 1024

/* Version of this ABI (RD_ABI_VERSION). */
int rd_abi_version(void);

/* Static, NUL-terminated description of a status code. */
const char* rd_status_string(int status);

/*
 * Workspace (device scratch, caller-owned) that rd_forward (trans_rhs == 0)
 * or rd_forward_trans_rhs (trans_rhs != 0) can use for these sizes: 0 when
 * the call needs none.  Currently nonzero only for decode-sized forward calls
 * (at most 24 rows per local group on average, k a multiple of 16, n a
 * multiple of 256), where every CU streams an equal share of the weight
 * bytes and the fp32 partial sums of blocks shared by two CUs are added in a
 * second, fixed-order pass.  The size (at most 256 MiB) grows with
 * (m / 32 + num_local) and depends on the current device's CU count.
 * Returns 0 for sizes the entry points would reject.
 */
size_t rd_forward_workspace_size(int64_t m, int64_t k, int64_t n, int32_t num_local, int32_t trans_rhs);

/*
 * ragged_dot ([SkyRL]; window from fast_ragged_dot; limit from [MaxText]).
 *
 *   x            [m, k] bf16: rows sorted by group.
 *   w            [num_local, k, n] bf16: one matrix per LOCAL group.
 *   group_sizes  [num_groups] int32 on the device.
 *   group_offset NULL, or [1] int32 on the device: index of the first local
 *                group.  NULL means offset 0 and requires
 *                num_local == num_groups.
 *   limit        NULL, or [1] int32 on the device: only rows [0, L) of x
 *                and out are valid (a packed expert buffer).
 *   out          [m, n], out_dtype RD_BF16 or RD_F32.
 *
 * With b[] the clamped boundaries and off the offset, rows r in
 * [b[off+j], b[off+j+1]) get out[r,:] = x[r,:] @ w[j] (fp32 accumulation,
 * then one rounding to out_dtype, round-to-nearest-even for bf16).  Every
 * other row below L is written as +0.  Rows >= L are neither read (in x)
 * nor written (in out).
 *
 * workspace/workspace_bytes: NULL/0, or device scratch of at least
 * rd_forward_workspace_size(m, k, n, num_local, 0) bytes, 16-byte aligned,
 * not shared with a concurrently running call.  With less than that size the
 * call runs without the split-contraction path (same results within the
 * GEMM tolerance, slower for decode shapes).  Its contents on entry do not
 * matter and are undefined on return.
 *
 * Requirements: m >= 0; k, n > 0 and multiples of 8; 1 <= num_local <=
 * num_groups <= RD_MAX_GROUPS; m, k, n < 2^31.  With m == 0 nothing is
 * launched and x, out may be NULL.
 */
int rd_forward(const void* x, const void* w, const int32_t* group_sizes, int32_t num_groups,
               const int32_t* group_offset, int32_t num_local, const int32_t* limit, void* out,
               int32_t out_dtype, int64_t m, int64_t k, int64_t n, void* workspace, size_t workspace_bytes,
               void* stream);

/*
 * rd_forward for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc.  The
 * same computation and results as rd_forward with a workspace of
 * rd_forward_workspace_size(m, k, n, num_local, 0) bytes, but the
 * split-contraction decode path keeps its fp32 partial sums in a static
 * device array of RD_NOALLOC_SCRATCH_BYTES per GPU, reserved when the library
 * is loaded and held until the process ends; no call allocates or frees
 * anything.  Calls whose sizes need more scratch than that return
 * RD_ESCRATCH before anything is launched (the 64-token top-8 decode step
 * over 128 experts of k 4096, n 1536 needs 72 MiB on a 256-CU device).
 * Every call on a GPU uses that GPU's one array, whose contents are left
 * over from the last call (every location a call reads it has written
 * first): calls that overlap on one GPU, from several streams or threads,
 * race and must be serialised by the caller.  The first call on a device
 * looks the array's address up (not inside a graph capture: make one call
 * on the device before capturing).
 */
#define RD_NOALLOC_SCRATCH_BYTES (80u << 20)
int rd_forward_noalloc(const void* x, const void* w, const int32_t* group_sizes, int32_t num_groups,
                       const int32_t* group_offset, int32_t num_local, const int32_t* limit, void* out,
                       int32_t out_dtype, int64_t m, int64_t k, int64_t n, void* stream);

/*
 * ragged_dot with trans_rhs ([SkyRL], the dx rule of the backward):
 * identical to rd_forward except that w is [num_local, n, k] and
 * out[r,:] = x[r,:] @ w[j]^T, i.e. the contraction runs over w's last dim.
 * Its workspace size is rd_forward_workspace_size(m, k, n, num_local, 1).
 */
int rd_forward_trans_rhs(const void* x, const void* w, const int32_t* group_sizes,
                         int32_t num_groups, const int32_t* group_offset, int32_t num_local,
                         const int32_t* limit, void* out, int32_t out_dtype, int64_t m, int64_t k,
                         int64_t n, void* workspace, size_t workspace_bytes, void* stream);

/*
 * ragged_dot with trans_rhs on fp8 operands ([SkyRL]: the kernels take a
 * compute_dtype; the pages report nothing for fp8, so this is the plainest
 * form): x [m, k] and w [num_local, n, k] hold OCP FP8 E4M3 values (1 sign,
 * 4 exponent bits with bias 7, 3 mantissa bits; no infinities, S.1111.111 is
 * NaN), out[r,:] = x[r,:] @ w[j]^T with float32 accumulation of the exact
 * products, then one rounding to out_dtype.  No scaling factors are applied
 * (fold them into the inputs or the output).  Window, limit and row rules
 * are those of rd_forward.  Requires k a multiple of 128 and
 * k * max(m, n) < 2^32 (else RD_EUNSUPPORTED).
 */
int rd_forward_trans_rhs_fp8(const void* x, const void* w, const int32_t* group_sizes, int32_t num_groups,
                             const int32_t* group_offset, int32_t num_local, const int32_t* limit, void* out,
                             int32_t out_dtype, int64_t m, int64_t k, int64_t n, void* stream);

/*
 * ragged_dot on fp8 operands in the plain form ([SkyRL] ragged_dot with a
 * compute_dtype, as rd_forward_trans_rhs_fp8): x [m, k] and
 * w [num_local, k, n] hold OCP FP8 E4M3 values, out[r,:] = x[r,:] @ w[j]
 * with float32 accumulation of the exact products, one rounding to
 * out_dtype, no scaling factors.  Window, limit and row rules are those of
 * rd_forward.  Requires k a multiple of 128, n a multiple of 16 and
 * k * max(m, n) < 2^32 (else RD_EUNSUPPORTED).
 */
int rd_forward_fp8(const void* x, const void* w, const int32_t* group_sizes, int32_t num_groups,
                   const int32_t* group_offset, int32_t num_local, const int32_t* limit, void* out,
                   int32_t out_dtype, int64_t m, int64_t k, int64_t n, void* stream);

/*
 * trans_ragged_dot ([SkyRL], _gpu_trans_ragged_dot_fwd; the weight
 * gradient): dw[j] = x_j^T @ dy_j over the rows of local group j.
 *
 *   x   [m, k] bf16,  dy [m, n] bf16,  dw [num_local, k, n] (RD_BF16 or RD_F32).
 *   group_sizes, group_offset, limit: as for rd_forward.
 *
 * Rows outside a group's [b[off+j], b[off+j+1]) contribute nothing: they are
 * removed by selection, so NaN or garbage there (e.g. rows >= L of a packed
 * buffer, [MaxText]) cannot reach dw.  A local group with no rows gets an
 * all +0 dw[j].  Rows >= L are never read.
 *
 * With m == 0, x and dy may be NULL and every dw[j] is written as +0.
 *
 * Row split: with a workspace, a group whose rows cost at least the mean
 * work per CU (and more than one chunk) is cut into row chunks of equal
 * length, decided on the device from group_sizes.  Each chunk's tile
 * goes to the workspace as an fp32 partial, and a second kernel adds a
 * tile's partials in chunk order and rounds once (per-block partials summed
 * after the pass, never a read-modify-write shared by workgroups: the race
 * lesson of [MaxText]'s unsort review).  Results are deterministic: the same
 * inputs, sizes and workspace_bytes give the same bits; a different
 * workspace_bytes may change which groups are split, and with it the
 * float32 summation order (within rounding).  The bf16 result is the RNE
 * rounding of the f32 result of the same call shape.
 *
 * workspace/workspace_bytes: NULL/0 (no split), or caller-owned device
 * scratch, 16-byte aligned; rd_trans_workspace_size(m, k, n, num_local)
 * bytes let every qualifying group split (0 when the sizes never split:
 * m == 0, or operands past 4 GiB), a smaller size splits fewer groups.  The
 * workspace must not be in use by another call on another stream.
 * RD_EINVAL for workspace_bytes > 0 with a NULL or misaligned workspace.
 */
size_t rd_trans_workspace_size(int64_t m, int64_t k, int64_t n, int32_t num_local);
int rd_trans(const void* x, const void* dy, const int32_t* group_sizes, int32_t num_groups,
             const int32_t* group_offset, int32_t num_local, const int32_t* limit, void* dw,
             int32_t dw_dtype, int64_t m, int64_t k, int64_t n, void* workspace,
             size_t workspace_bytes, void* stream);

/*
 * trans_ragged_dot on fp8 operands (as rd_trans; [SkyRL] compute_dtype, the
 * reading of rd_forward_trans_rhs_fp8): x [m, k] and dy [m, n] hold OCP FP8
 * E4M3 values, dw[j] = x_j^T @ dy_j with float32 accumulation of the exact
 * products over the group's rows, one rounding to dw_dtype; rows outside a
 * group removed by selection, an empty group +0, rows >= L never read.
 * Requires k and n multiples of 16 and m * max(k, n) < 2^32 (else
 * RD_EUNSUPPORTED).  workspace/workspace_bytes as for rd_trans, with the
 * same row split of long groups (fp32 partials added in chunk order, the
 * same determinism), from 1.3 times the mean work per CU: these tiles take
 * half the steps for the same partial traffic.
 * rd_trans_workspace_size(m, k, n, num_local) bytes let every qualifying
 * group split (0 from it: no split).  RD_EINVAL for workspace_bytes > 0 with
 * a NULL or misaligned workspace.
 */
int rd_trans_fp8(const void* x, const void* dy, const int32_t* group_sizes, int32_t num_groups,
                 const int32_t* group_offset, int32_t num_local, const int32_t* limit, void* dw,
                 int32_t dw_dtype, int64_t m, int64_t k, int64_t n, void* workspace, size_t workspace_bytes,
                 void* stream);

/*
 * The MoE up-projection with the GLU as its epilogue ([MaxText]: the expert
 * FFN computes fused = ragged_dot(x, wi) as [gate | up] and then
 * silu(gate) * up; [SkyRL] ragged_dot and the group_offset window).  One
 * kernel computes
 *
 *   fused = bf16(ragged_dot(x, wi))           (as rd_forward, out_dtype bf16)
 *   act   = the rd_glu_fwd result on fused     (same float32 evaluation)
 *
 * and is bit-identical to rd_forward without a workspace followed by
 * rd_glu_fwd: each tile pairs gate columns [c, c + 128) with up columns
 * [h + c, h + c + 128), rounds both to bf16 as the [gate | up] buffer holds
 * them, and evaluates the GLU on them.  (rd_forward's split-contraction
 * decode path, taken only with a workspace, sums in another order.)
 *
 *   x     [m, k] bf16.
 *   wi    [num_local, k, 2h] bf16: columns [0, h) gate, [h, 2h) up.
 *   act   [m, h] bf16 (output).
 *   fused [m, 2h] bf16 (output) or NULL: the [gate | up] buffer (the
 *         backward's residual) is then not written at all.
 *
 * group_sizes, group_offset, num_local and limit as rd_forward: rows below L
 * outside the window are +0 in act (and fused), rows >= L are neither read
 * nor written.  Requires k a multiple of 64, h a multiple of 128, and every
 * operand under 4 GiB (else RD_EUNSUPPORTED).  With m == 0 nothing is
 * launched and x, act, fused may be NULL.
 */
int rd_forward_glu(const void* x, const void* wi, const int32_t* group_sizes, int32_t num_groups,
                   const int32_t* group_offset, int32_t num_local, const int32_t* limit, void* act,
                   void* fused, int64_t m, int64_t k, int64_t h, void* stream);

/*
 * GLU forward over the valid rows ([MaxText], glu_rows forward).
 *
 *   fused [rows, 2h] bf16 laid out as [gate | up] along the columns.
 *   out   [rows, h] bf16.
 *   limit NULL (all rows) or [1] int32 on the device.
 *
 * For r < L: out[r,c] = bf16(g / (1 + exp(-g)) * u), g = fused[r,c],
 * u = fused[r,h+c], evaluated in float32 in that order (negate, exp, +1,
 * divide, multiply), no denormal flushing and no contraction into FMA; only
 * the result is rounded (RNE).  exp and the divide use the hardware base-2
 * exponential and (range-scaled) reciprocal, which keeps every output within
 * one bf16 ulp of the correctly rounded float32 evaluation.  Rows >= L are neither read nor written.
 * h > 0, multiple of 8.
 */
int rd_glu_fwd(const void* fused, const int32_t* limit, void* out, int64_t rows, int64_t h,
               void* stream);

/*
 * GLU backward over the valid rows ([MaxText], glu_rows backward).
 *
 *   fused   [rows, 2h] bf16 [gate | up];  d_out [rows, h] bf16.
 *   d_fused [rows, 2h] bf16 written as [d_gate | d_up] in one pass.
 *
 * For r < L, in float32 with s = 1 / (1 + exp(-g)):
 *   d_up   = d * (g / (1 + exp(-g)))
 *   d_gate = ((d * u) * s) * (1 + g * (1 - s))
 * each rounded once (RNE), then -0 is written as +0 in both halves; exp and
 * the divides as in rd_glu_fwd (within one bf16 ulp).
 * Rows >= L are neither read nor written.  h > 0, multiple of 8.
 */
int rd_glu_bwd(const void* fused, const void* d_out, const int32_t* limit, void* d_fused,
               int64_t rows, int64_t h, void* stream);

/*
 * Weighted unsort backward over the valid rows ([MaxText], unsort_bwd_rows:
 * the buffered branch of the ring unsort backward).
 *
 *   g     [rows, hidden] bf16: the incoming gradient gathered into the packed
 *         expert buffer's (sorted) row order.
 *   y     [rows, hidden] bf16: the expert outputs in the same order.
 *   w     [rows] float32: each row's routing weight.
 *   limit NULL (all rows) or [1] int32 on the device.
 *   grad  [rows, hidden] bf16: grad[r, c] = bf16(f32(g[r, c]) * w[r]), a
 *         float32 product rounded once to bf16 (RNE).
 *   dot   [rows] float32: dot[r] = sum_c f32(g[r, c]) * f32(y[r, c]), the
 *         routing-weight gradient: exact products summed in float64 in a
 *         fixed order and rounded once to float32 (within half a float32
 *         ulp of the exact dot; the same on every run; the page leaves the
 *         summation free and checks it with an absolute tolerance of 1e-4).
 *
 * Rows r >= L = clamp(*limit, 0, rows) are neither read nor written (in any
 * of the five arrays).  hidden > 0 and a multiple of 8; g, y, grad 16-byte
 * aligned; w, dot 4-byte aligned.  With rows == 0 nothing is launched and the
 * pointers may be NULL.
 */
int rd_unsort_bwd_rows(const void* g, const void* y, const float* w, const int32_t* limit, void* grad, float* dot,
                       int64_t rows, int64_t hidden, void* stream);

/*
 * Rows at or past the valid-row limit set to +0 ([MaxText]: the packed
 * expert buffer's kernels touch only rows [0, limit), limit a device
 * scalar).  Rows r >= L = clamp(*limit, 0, rows) of the [rows, row_bytes]
 * buffer buf get all-zero bytes; rows below L are not touched.  Used for the
 * gradients of a packed buffer's inputs, which are exactly zero past the
 * limit (those rows take no part in the computation).  limit NULL means
 * L = rows: nothing is written or launched.  row_bytes > 0 and a multiple of
 * 16 (else RD_EUNSUPPORTED); buf 16-byte aligned; with rows == 0 nothing is
 * launched and buf may be NULL.
 */
int rd_zero_rows_from_limit(void* buf, const int32_t* limit, int64_t rows, int64_t row_bytes, void* stream);

/*
 * Tuning hook, for tile sweeps (the pages ask whether benchmarking and
 * tuning code should ship with the kernels: SkyRL-tx PR #867, "Todo /
 * Questions"); not needed for correct results.  Sets a process-wide override
 * read by later calls:
 *   RD_TUNE_FWD_TILE   the grouped-GEMM tile shape of rd_forward,
 *                      rd_forward_trans_rhs and rd_forward_glu (value in
 *                      [0, rd_tune_tile_count()), or -1 for the built-in
 *                      choice from m, k, n and num_local);
 *   RD_TUNE_TRANS_TILE the same for rd_trans;
 *   RD_TUNE_DECODE     1 (default) allows the split-contraction decode path
 *                      of rd_forward, 0 turns it off.
 * Every shape computes the same results within the GEMM tolerance (the
 * contraction order within a tile is the same, so outputs agree bitwise in
 * practice).  rd_forward_glu ignores forced shapes it has no fused form of.
 * Returns RD_OK, or RD_EINVAL for an unknown key or an out-of-range value.
 * Thread-safe; a call in flight on another thread sees the old or the new
 * value.
 */
#define RD_TUNE_FWD_TILE 0
#define RD_TUNE_TRANS_TILE 1
#define RD_TUNE_DECODE 2
int rd_tune_set(int32_t which, int32_t value);

/* Number of grouped-GEMM tile shapes RD_TUNE_FWD_TILE / RD_TUNE_TRANS_TILE accept. */
int rd_tune_tile_count(void);

#ifdef __cplusplus
}
#endif

#endif /* RD_H */
