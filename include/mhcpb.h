/*
 * mhcpb.h -- C-ABI of the DSv4.1 mHC projection/RMS backward for MI355X
 * (gfx950).
 *
 * The operation ("DSv4.1 mHC projection/RMS backward", cuDNN Frontend page,
 * introduction): with P = grad_proj[:, :24],
 *
 *     dX = P W + grad_r / (r K) * X        stored as BF16
 *     dW = P^T X                           stored as FP32
 *
 * over X of shape [T, K], K = streams * hidden.  Both matrix products round
 * their operands to TF32 (round to nearest even of the FP32 fraction at 10
 * bits) and sum in FP32; the RMS term is computed in FP32 from the raw x.
 * dW is the sum of per-slab partial sums added in an order fixed in advance,
 * with no atomic operations, so its bits depend only on (T, K) and this
 * library, never on the CU count, the launch timing or the run.  dX and dW
 * are written, never added to (same page, introduction).
 *
 * Tensor contract (same page, "Requirements and tensor contract"): compact
 * row-major tensors, columns 24..31 of grad_proj are never read, r holds the
 * positive forward RMS values, every operand, output and the workspace are
 * disjoint and 16-byte aligned.  Anything else is rejected; nothing is
 * converted or repacked.
 *
 * All device pointers are plain HIP device addresses owned by the caller.
 * The library never allocates, frees or synchronizes device memory; a plan
 * holds host metadata only ("Prepared class API" section: compile() does no
 * tensor work, execute() allocates no tensor storage and enqueues exactly two
 * kernels).  Every function returns a status and never throws.  Arguments
 * are validated before anything is enqueued: on a validation error no kernel
 * is launched and no output is written.  MHCPB_ERROR_LAUNCH reports a launch
 * the runtime refused; when that is a call's second kernel, the first one is
 * already enqueued and its outputs (dX, the workspace) are to be treated as
 * undefined.
 */
#ifndef MHCPB_H
#define MHCPB_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Opaque plan: host memory only, immutable after creation. */
typedef struct mhcpb_plan_s *mhcpb_plan_t;

typedef enum mhcpb_status {
    MHCPB_SUCCESS = 0,
    MHCPB_ERROR_INVALID_ARGUMENT = 1, /* NULL plan or pointer, T < 1          */
    MHCPB_ERROR_UNSUPPORTED = 2,      /* streams != 4, hidden odd or < 2,
                                         sizes beyond the supported range     */
    MHCPB_ERROR_MISALIGNED = 3,       /* a pointer not 16-byte aligned        */
    MHCPB_ERROR_OVERLAP = 4,          /* two byte ranges intersect            */
    MHCPB_ERROR_WORKSPACE = 5,        /* workspace smaller than required      */
    MHCPB_ERROR_LAUNCH = 6            /* the HIP runtime refused a launch     */
} mhcpb_status_t;

/*
 * Create a plan for X of shape [T, streams * hidden].
 *   T       tokens, 1 <= T <= 2^31 - 1
 *   streams residual streams; must be 4 (the page's supported profile)
 *   hidden  hidden size per stream; even, 2 <= hidden <= 2^20, so that every
 *           BF16 row of dX is a multiple of 16 bytes
 * Host work only: the split schedule, the grid and the workspace size.  The
 * split count S depends on T alone (S = min(32, max(ceil(T / 512),
 * min(8, ceil(T / 64))))), which is what makes dW bitwise reproducible across
 * devices with different CU counts.
 * On success *plan receives a new plan; on error *plan is set to NULL.
 */
mhcpb_status_t mhcpb_plan_create(mhcpb_plan_t *plan, int64_t T, int32_t streams,
                                 int32_t hidden);

/* Free a plan (host memory).  NULL is accepted and ignored. */
mhcpb_status_t mhcpb_plan_destroy(mhcpb_plan_t plan);

/*
 * Bytes of device workspace execute() needs: S * 24 * K * 4, one FP32 [24, K]
 * partial dW slab per split ("Prepared class API": 15,728,640 bytes at T =
 * 4096, 4 streams, hidden 5120, i.e. S = 8).  Contents are undefined on entry
 * and on exit; the workspace is caller-owned.
 */
mhcpb_status_t mhcpb_workspace_bytes(mhcpb_plan_t plan, size_t *bytes);

/* The split count S(T) of the plan (for schedule inspection). */
mhcpb_status_t mhcpb_plan_split_count(mhcpb_plan_t plan, int32_t *splits);

/*
 * The number of partial dW slabs an execute() call of the plan writes to the
 * workspace and reads back (for byte accounting): S, less the slabs whose
 * sum kernel 1 forms before it stores them.  Kernel 1's workgroups walk runs
 * of consecutive slabs; the one that holds slabs 0 .. n-1 of a column tile
 * adds their partials up in ascending order, as kernel 2 would, and stores
 * only the sum (in slab n - 1, where kernel 2 then starts), so n - 1 slabs
 * are neither written nor read.  n depends on the launch shape (T and K), never
 * on the device; dW bits do not depend on it.  Host work only.
 */
mhcpb_status_t mhcpb_plan_partial_slabs(mhcpb_plan_t plan, int32_t *slabs);

/*
 * Enqueue the stage on `stream` (0 = the null stream): kernel 1 streams X
 * once, writes dX and the partial dW slabs (mhcpb_plan_partial_slabs of the
 * S, the first of them holding the sum of the slabs before it) into the
 * workspace; kernel 2 sums them in ascending split order into dW.
 *
 *   x              [T, K]  FP32 input
 *   w              [24, K] FP32 projection weight
 *   grad_proj      [T, 32] FP32; columns 24..31 are never read (NaN is fine)
 *   grad_r         [T]     FP32 gradient of the RMS value
 *   r              [T]     FP32 forward RMS, positive (not checked on device;
 *                          other values follow IEEE arithmetic)
 *   dx             [T, K]  BF16 bit patterns, overwritten
 *   dw             [24, K] FP32, overwritten
 *   grad_x_addend  [T, K]  BF16 or NULL.  When given it is added to the FP32
 *                          dX value before the single rounding to BF16 (the
 *                          fused stream gradient of prime-kernels pull
 *                          request 15, "fused mHC stream gradient" item)
 *   workspace      >= mhcpb_workspace_bytes(plan) bytes of device memory
 *   workspace_size the size of that buffer in bytes
 *
 * Every pointer must be 16-byte aligned and every byte range disjoint from
 * the others.  The call only validates and launches: it returns before the
 * kernels finish, and the caller keeps every buffer alive until the stream
 * work completes.  Concurrent calls are safe when they use separate outputs
 * and workspaces ("Prepared class API").  Because the call is launch-only it
 * can be recorded into a HIP graph.
 */
mhcpb_status_t mhcpb_execute(mhcpb_plan_t plan, const float *x, const float *w,
                             const float *grad_proj, const float *grad_r,
                             const float *r, uint16_t *dx, float *dw,
                             const uint16_t *grad_x_addend, void *workspace,
                             size_t workspace_size, hipStream_t stream);

/*
 * Same as mhcpb_execute, and attaches caller events to the kernel launches
 * (any of them may be NULL): `before_k1` takes the start time of kernel 1,
 * `after_k1` its end time, `after_k2` the end time of kernel 2.  The times
 * come from the dispatches themselves (hipExtLaunchKernel), so no marker is
 * inserted between the kernels: hipEventElapsedTime(before_k1, after_k1) is
 * kernel 1's execution time and (after_k1, after_k2) kernel 2's plus the gap
 * between them.  The events are created and owned by the caller.
 */
mhcpb_status_t mhcpb_execute_with_events(
    mhcpb_plan_t plan, const float *x, const float *w, const float *grad_proj,
    const float *grad_r, const float *r, uint16_t *dx, float *dw,
    const uint16_t *grad_x_addend, void *workspace, size_t workspace_size,
    hipStream_t stream, hipEvent_t before_k1, hipEvent_t after_k1,
    hipEvent_t after_k2);

/*
 * mhcpb_execute without a caller workspace, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc).  The partial dW slabs go to a static workspace of
 * 64 MiB (67,108,864 bytes) per GPU that the library holds from its load
 * until the process ends; the call allocates nothing.  Arguments, results and
 * errors are those of mhcpb_execute, plus MHCPB_ERROR_WORKSPACE when the
 * plan's workspace (mhcpb_workspace_bytes, S * 24 * K * 4) exceeds 64 MiB
 * (every T fits at K = 20480; with 32 slabs, T > 15872, K must stay within
 * 21,845) and MHCPB_ERROR_LAUNCH when the static workspace cannot be
 * located on the current device.  The device is the calling thread's current
 * one (hipGetDevice), which must be the device of `stream` and the buffers.
 * Every such call on one GPU shares that workspace: calls that overlap in
 * time on one GPU (other streams, other threads) race and may give wrong
 * results; serialise them or use mhcpb_execute with separate workspaces.
 */
mhcpb_status_t mhcpb_execute_noalloc(mhcpb_plan_t plan, const float *x, const float *w,
                                     const float *grad_proj, const float *grad_r,
                                     const float *r, uint16_t *dx, float *dw,
                                     const uint16_t *grad_x_addend, hipStream_t stream);

/*
 * The split backward ("FP8 weight cache, split backward, fused mHC stream
 * gradient" on the prime-kernels page: dX is produced by its own call, so
 * that it can be handed on while dW is still to be computed).  Each
 * form reads X once, so the pair reads it twice; each output has exactly the
 * bits mhcpb_execute gives it.
 *
 * mhcpb_execute_dx: one kernel writing dX only (arguments as in
 * mhcpb_execute; no dW, no workspace).  Required: x, w, grad_proj, grad_r, r,
 * dx; grad_x_addend may be NULL.
 */
mhcpb_status_t mhcpb_execute_dx(mhcpb_plan_t plan, const float *x, const float *w,
                                const float *grad_proj, const float *grad_r,
                                const float *r, uint16_t *dx,
                                const uint16_t *grad_x_addend, hipStream_t stream);

/*
 * mhcpb_execute_dw: kernel 1 writing the partial dW slabs only, then kernel 2
 * (arguments as in mhcpb_execute).  Required: x, grad_proj, dw, a workspace
 * of at least mhcpb_workspace_bytes(plan) bytes.
 */
mhcpb_status_t mhcpb_execute_dw(mhcpb_plan_t plan, const float *x, const float *grad_proj,
                                float *dw, void *workspace, size_t workspace_size,
                                hipStream_t stream);

/*
 * The forward map of the stage: for every row t of X [T, K] and gate j < 24,
 *
 *     proj[t, j] = sum_k TF32(X[t, k]) TF32(W[j, k])     FP32 accumulation
 *     r[t]       = sqrt(sum_k X[t, k]^2 / K + eps)        FP32, raw x
 *
 * in one read of X.  dX and dW of mhcpb_execute are exactly the gradient of
 * this map for the cotangents (grad_proj[:, :24], grad_r): the backward page
 * ("DSv4.1 mHC projection/RMS backward", introduction and "Requirements and
 * tensor contract") takes r as the RMS of the forward, and the prime-kernels
 * pull request 15 page lists the RMS and the gate logits of the streams as
 * one pass ("mhc_projection").  The logits leave unnormalised (the division
 * by r, the gate activations and the stream collapse belong to the caller).
 *
 *   x        [T, K]  FP32, the plan's shape
 *   w        [24, K] FP32
 *   eps      finite and >= 0 (else MHCPB_ERROR_INVALID_ARGUMENT)
 *   proj     [T, 32] FP32 out: logits in columns 0..23, +0 in 24..31 (the
 *            row layout of grad_proj), overwritten
 *   r        [T] FP32 out, overwritten
 *   workspace at least mhcpb_forward_workspace_bytes(plan) bytes: ceil(K /
 *            1024) x ceil(T / 16) x 2048, the partial logits and sums of
 *            squares of each 1024-column tile (32 FP32 per token); contents
 *            undefined on entry and on exit
 *
 * Two kernels on `stream`: one pass over X writing a partial per 1024-column
 * tile and token, then their sum in tile order.  Each row's results depend
 * only on that row, W, eps and K (not on T or other rows).  ceil(K / 1024) x
 * ceil(T / 16) must stay below 2^31 (else MHCPB_ERROR_UNSUPPORTED).
 * Non-finite inputs give non-finite outputs where IEEE arithmetic on the TF32
 * operands does (a NaN in a row makes its 24 logits and r NaN); whether such
 * a logit is +-inf or NaN is not promised.  A sum of squares beyond the FP32
 * range gives r = +inf.  Alignment, overlap and status codes as for
 * mhcpb_execute.
 */
mhcpb_status_t mhcpb_forward_workspace_bytes(mhcpb_plan_t plan, size_t *bytes);

mhcpb_status_t mhcpb_forward(mhcpb_plan_t plan, const float *x, const float *w, float eps,
                             float *proj, float *r, void *workspace, size_t workspace_size,
                             hipStream_t stream);

/*
 * mhcpb_forward with caller-owned events attached to the dispatches:
 * `before_k1` and `after_k1` take the start and end times of the pass over X,
 * `after_k2` the end time of the sum of the tiles.  Any may be NULL.
 */
mhcpb_status_t mhcpb_forward_with_events(mhcpb_plan_t plan, const float *x, const float *w,
                                         float eps, float *proj, float *r, void *workspace,
                                         size_t workspace_size, hipStream_t stream,
                                         hipEvent_t before_k1, hipEvent_t after_k1,
                                         hipEvent_t after_k2);

/*
 * A second workload: the deterministic BF16 RMSNorm backward of the
 * "flashinfer.cake_rmsnorm_det_train.cake_rmsnorm_det_train_backward" page
 * (its signature, parameters and the notes on program selection).  For
 * y = x * rstd * w per row of x [T, H],
 *
 *     c1[t]   = sum_h w[h] g[t, h] x[t, h] / H
 *     dx[t, h] = rstd[t] w[h] g[t, h] - rstd[t]^3 c1[t] x[t, h]
 *                (+ g_residual[t, h])                      BF16, one rounding
 *     dw[h]   = sum_t g[t, h] x[t, h] rstd[t]               FP32
 *
 * (the page prints no formula: this is the gradient of that map with rstd
 * taken as the forward returned it).  dx is computed in FP32 and rounded to
 * BF16 once, the residual gradient added a single time, before that rounding.
 * dw is reduced from per-block partials in a fixed order: the rows are dealt
 * round-robin to S = min(ceil(T / 16), 256 * max(1, 12 / ceil(H / 512)))
 * blocks, a function of (T, H) alone, so dw is bitwise reproducible for a
 * given (T, H) on any device, whatever its CU count; each row's dx depends
 * on that row alone.
 *
 * Workspace: S * H * 4 bytes (one FP32 partial dw per block; 0 when T = 0).
 */
typedef enum mhcpb_dtype {
    MHCPB_DTYPE_BF16 = 0,
    MHCPB_DTYPE_F32 = 1
} mhcpb_dtype_t;

/*
 * Bytes of workspace mhcpb_rmsnorm_backward needs for T rows of width H.
 * MHCPB_ERROR_INVALID_ARGUMENT for T < 0, H < 1 or a NULL `bytes`;
 * MHCPB_ERROR_UNSUPPORTED for a shape mhcpb_rmsnorm_backward rejects as such.
 */
mhcpb_status_t mhcpb_rmsnorm_backward_workspace_bytes(int64_t T, int32_t H, size_t *bytes);

/*
 * Enqueue the RMSNorm backward on `stream`: kernel 1 reads g, x (and
 * g_residual) once, writes dx and one partial dw per block; kernel 2 adds the
 * partials in a fixed order into dw.  With T = 0 only kernel 2 runs and dw
 * becomes +0.
 *
 *   T, H        rows and width; 0 <= T <= 2^31 - 1; H a multiple of 8 (rows of
 *               16-byte multiples, as the page requires for in-place reads)
 *               with 8 <= H <= 6144 (the page's widths go up to 6144), else
 *               MHCPB_ERROR_UNSUPPORTED
 *   g, x        [T, H] BF16 bit patterns, row-major and compact
 *   w           [H] BF16 (w_dtype MHCPB_DTYPE_BF16) or FP32 (MHCPB_DTYPE_F32)
 *   rstd        [T] FP32 reciprocal RMS of the forward (any value; IEEE
 *               arithmetic follows)
 *   g_residual  [T, H] BF16 or NULL
 *   dx          [T, H] BF16 out, overwritten
 *   dw          [H] FP32 out, overwritten
 *   workspace   >= mhcpb_rmsnorm_backward_workspace_bytes(T, H) bytes of
 *               device memory (may be NULL when that is 0); contents
 *               undefined on entry and exit
 *
 * Pointers that take part must be 16-byte aligned and their byte ranges
 * disjoint (MHCPB_ERROR_MISALIGNED, MHCPB_ERROR_OVERLAP); g, x, rstd and dx
 * may be NULL only when T = 0; w and dw are always required.  Like
 * mhcpb_execute it only validates and launches, allocates nothing, and on a
 * validation error launches nothing.
 */
mhcpb_status_t mhcpb_rmsnorm_backward(int64_t T, int32_t H, const uint16_t *g, const uint16_t *x,
                                      const void *w, mhcpb_dtype_t w_dtype, const float *rstd,
                                      const uint16_t *g_residual, uint16_t *dx, float *dw,
                                      void *workspace, size_t workspace_size, hipStream_t stream);

/*
 * mhcpb_rmsnorm_backward with caller-owned events: `before_k1` and `after_k1`
 * take the start and end times of kernel 1, `after_k2` the end time of
 * kernel 2 (when T = 0 the first two are recorded just before kernel 2).
 * Any may be NULL.
 */
mhcpb_status_t mhcpb_rmsnorm_backward_with_events(
    int64_t T, int32_t H, const uint16_t *g, const uint16_t *x, const void *w,
    mhcpb_dtype_t w_dtype, const float *rstd, const uint16_t *g_residual, uint16_t *dx,
    float *dw, void *workspace, size_t workspace_size, hipStream_t stream,
    hipEvent_t before_k1, hipEvent_t after_k1, hipEvent_t after_k2);

/* A static, human-readable name for a status code. */
const char *mhcpb_status_string(mhcpb_status_t status);

#ifdef __cplusplus
}
#endif

#endif /* MHCPB_H */
