// Plan creation, argument validation and the C-ABI entry points.
//
// Follows the "Prepared class API" and "Requirements and tensor contract"
// sections of the "DSv4.1 mHC projection/RMS backward" page: a plan is host
// metadata; execute() checks the operands (alignment, disjointness), then
// puts the two kernels on the stream and allocates no memory.  The split forms (dX
// only, dW only) follow the split backward of the prime-kernels page ("FP8
// weight cache, split backward, fused mHC stream gradient").  The forward
// entry points (the map the stage differentiates) use the same plan.
#include <algorithm>
#include <cstdint>
#include <cstdlib>
#include <new>

#include "../../include/mhcpb.h"
#include "mhcpb_internal.h"

namespace {

constexpr int64_t kMaxT = (int64_t{1} << 31) - 1;
constexpr int32_t kMaxHidden = 1 << 20;
constexpr uintptr_t kAlign = 16;

struct Range {
    uintptr_t lo;
    uintptr_t hi;  // one past the end
};

bool aligned(const void *p) { return (reinterpret_cast<uintptr_t>(p) % kAlign) == 0; }

bool overlap(const Range &a, const Range &b) { return a.lo < b.hi && b.lo < a.hi; }

// One operand or output of a call: its address, its size in bytes, and
// whether the call needs it (an optional one may be NULL).
struct Operand {
    const void *ptr;
    uint64_t bytes;
    bool required;
};

// Alignment, address wrap-around and pairwise overlap of the byte ranges of
// the operands that are present, before any HIP call.
mhcpb_status_t validate_ranges(const Operand *ops, int n) {
    for (int i = 0; i < n; ++i)
        if (ops[i].ptr && !aligned(ops[i].ptr))
            return MHCPB_ERROR_MISALIGNED;
    Range rs[10];
    int m = 0;
    for (int i = 0; i < n; ++i) {
        if (!ops[i].ptr)
            continue;
        const uintptr_t lo = reinterpret_cast<uintptr_t>(ops[i].ptr);
        const Range r{lo, lo + static_cast<uintptr_t>(ops[i].bytes)};
        if (r.hi < r.lo)  // address wrap-around
            return MHCPB_ERROR_INVALID_ARGUMENT;
        rs[m++] = r;
    }
    for (int i = 0; i < m; ++i)
        for (int j = i + 1; j < m; ++j)
            if (overlap(rs[i], rs[j]))
                return MHCPB_ERROR_OVERLAP;
    return MHCPB_SUCCESS;
}

// Validates the operands the requested outputs need, then enqueues kernel 1
// (and kernel 2 when dW is produced).
mhcpb_status_t run(mhcpb_plan_t plan, mhcpb::Outputs out, const float *x, const float *w,
                   const float *grad_proj, const float *grad_r, const float *r,
                   uint16_t *dx, float *dw, const uint16_t *addend, void *ws,
                   size_t ws_size, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1,
                   hipEvent_t ev2) {
    if (!plan)
        return MHCPB_ERROR_INVALID_ARGUMENT;
    const mhcpb::Plan &p = plan->plan;
    const bool want_dx = out != mhcpb::Outputs::kDwOnly;
    const bool want_dw = out != mhcpb::Outputs::kDxOnly;
    const uint64_t T = static_cast<uint64_t>(p.T), K = static_cast<uint64_t>(p.K);
    const Operand ops[] = {
        {x, T * K * 4, true},
        {grad_proj, T * 32 * 4, true},
        {w, 24 * K * 4, want_dx},
        {grad_r, T * 4, want_dx},
        {r, T * 4, want_dx},
        {dx, T * K * 2, want_dx},
        {addend, T * K * 2, false},
        {dw, 24 * K * 4, want_dw},
        {ws, p.ws_bytes, want_dw},
    };
    constexpr int n = static_cast<int>(sizeof(ops) / sizeof(ops[0]));
    for (int i = 0; i < n; ++i)
        if (ops[i].required && !ops[i].ptr)
            return MHCPB_ERROR_INVALID_ARGUMENT;
    if (want_dw && ws_size < p.ws_bytes)
        return MHCPB_ERROR_WORKSPACE;
    const mhcpb_status_t st = validate_ranges(ops, n);
    if (st != MHCPB_SUCCESS)
        return st;
    mhcpb::Args a{x, w, grad_proj, grad_r, r, dx, dw, addend, static_cast<float *>(ws)};
    if (mhcpb::launch_projection(p, a, out, stream, ev0, ev1) != hipSuccess)
        return MHCPB_ERROR_LAUNCH;
    if (want_dw && mhcpb::launch_reduce(p, a, stream, ev2) != hipSuccess)
        return MHCPB_ERROR_LAUNCH;
    return MHCPB_SUCCESS;
}

// The forward: validates every operand, then enqueues its two kernels.
mhcpb_status_t run_forward(mhcpb_plan_t plan, const float *x, const float *w, float eps,
                           float *proj, float *r, void *ws, size_t ws_size, hipStream_t stream,
                           hipEvent_t ev0, hipEvent_t ev1, hipEvent_t ev2) {
    if (!plan)
        return MHCPB_ERROR_INVALID_ARGUMENT;
    const mhcpb::Plan &p = plan->plan;
    const uint64_t T = static_cast<uint64_t>(p.T), K = static_cast<uint64_t>(p.K);
    const uint64_t wsb = mhcpb::forward_workspace_bytes(p.T, p.K);
    const Operand ops[] = {
        {x, T * K * 4, true},     {w, 24 * K * 4, true}, {proj, T * 32 * 4, true},
        {r, T * 4, true},         {ws, wsb, true},
    };
    constexpr int n = static_cast<int>(sizeof(ops) / sizeof(ops[0]));
    for (int i = 0; i < n; ++i)
        if (!ops[i].ptr)
            return MHCPB_ERROR_INVALID_ARGUMENT;
    // eps must be a finite, non-negative FP32 value (a NaN eps would make
    // every RMS NaN).
    if (!(eps >= 0.0f && eps <= 3.4028234663852886e38f))
        return MHCPB_ERROR_INVALID_ARGUMENT;
    if (mhcpb::forward_units(p.T, p.K) >= (int64_t{1} << 31))
        return MHCPB_ERROR_UNSUPPORTED;
    if (ws_size < wsb)
        return MHCPB_ERROR_WORKSPACE;
    const mhcpb_status_t st = validate_ranges(ops, n);
    if (st != MHCPB_SUCCESS)
        return st;
    if (mhcpb::launch_forward(p, x, w, proj, r, eps, static_cast<float *>(ws), stream, ev0, ev1,
                              ev2) != hipSuccess)
        return MHCPB_ERROR_LAUNCH;
    return MHCPB_SUCCESS;
}

// Shape check of the RMSNorm backward: status, and the block schedule.
mhcpb_status_t rmsnorm_shape(int64_t T, int32_t H, mhcpb::RmsPlan *p) {
    if (T < 0 || H < 1)
        return MHCPB_ERROR_INVALID_ARGUMENT;
    if (T > kMaxT || H > mhcpb::kRmsMaxH || H < 8 || (H % 8) != 0)
        return MHCPB_ERROR_UNSUPPORTED;
    *p = mhcpb::rmsnorm_plan(T, H);
    return MHCPB_SUCCESS;
}

mhcpb_status_t run_rmsnorm(int64_t T, int32_t H, const uint16_t *g, const uint16_t *x,
                           const void *w, mhcpb_dtype_t w_dtype, const float *rstd,
                           const uint16_t *res, uint16_t *dx, float *dw, void *ws,
                           size_t ws_size, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1,
                           hipEvent_t ev2) {
    mhcpb::RmsPlan p{};
    const mhcpb_status_t shape = rmsnorm_shape(T, H, &p);
    if (shape != MHCPB_SUCCESS)
        return shape;
    if (w_dtype != MHCPB_DTYPE_BF16 && w_dtype != MHCPB_DTYPE_F32)
        return MHCPB_ERROR_INVALID_ARGUMENT;
    const uint64_t rows = static_cast<uint64_t>(T), h = static_cast<uint64_t>(H);
    const uint64_t wsb = mhcpb::rmsnorm_workspace_bytes(p);
    const bool any = T > 0;
    const Operand ops[] = {
        {g, rows * h * 2, any},
        {x, rows * h * 2, any},
        {w, h * (w_dtype == MHCPB_DTYPE_F32 ? 4 : 2), true},
        {rstd, rows * 4, any},
        {res, rows * h * 2, false},
        {dx, rows * h * 2, any},
        {dw, h * 4, true},
        {ws, wsb, wsb > 0},
    };
    constexpr int n = static_cast<int>(sizeof(ops) / sizeof(ops[0]));
    for (int i = 0; i < n; ++i)
        if (ops[i].required && !ops[i].ptr)
            return MHCPB_ERROR_INVALID_ARGUMENT;
    if (ws_size < wsb)
        return MHCPB_ERROR_WORKSPACE;
    // With no rows only w, dw and the workspace take part.
    const Operand used[] = {ops[2], ops[6], ops[7]};
    const mhcpb_status_t st = any ? validate_ranges(ops, n) : validate_ranges(used, 3);
    if (st != MHCPB_SUCCESS)
        return st;
    if (mhcpb::launch_rmsnorm_backward(p, g, x, w, w_dtype == MHCPB_DTYPE_F32, rstd, res, dx, dw,
                                       static_cast<float *>(ws), stream, ev0, ev1,
                                       ev2) != hipSuccess)
        return MHCPB_ERROR_LAUNCH;
    return MHCPB_SUCCESS;
}

// The bound of the kernels' LDS counter waits for a new plan: the default,
// or the value of the environment variable when it holds a decimal integer in
// [0, 2^20] (anything else is ignored).
int32_t wait_polls_setting() {
    const char *v = std::getenv(mhcpb::kWaitPollsEnv);
    if (!v || !*v)
        return mhcpb::kDefaultWaitPolls;
    char *end = nullptr;
    const long n = std::strtol(v, &end, 10);
    if (*end != '\0' || n < 0 || n > (1L << 20))
        return mhcpb::kDefaultWaitPolls;
    return static_cast<int32_t>(n);
}

}  // namespace

extern "C" {

mhcpb_status_t mhcpb_plan_create(mhcpb_plan_t *plan, int64_t T, int32_t streams,
                                 int32_t hidden) {
    if (!plan)
        return MHCPB_ERROR_INVALID_ARGUMENT;
    *plan = nullptr;
    if (T < 1)
        return MHCPB_ERROR_INVALID_ARGUMENT;
    if (T > kMaxT || streams != 4 || hidden < 2 || hidden > kMaxHidden || (hidden % 2) != 0)
        return MHCPB_ERROR_UNSUPPORTED;
    mhcpb::Plan p{};
    p.T = T;
    p.streams = streams;
    p.hidden = hidden;
    p.K = static_cast<int64_t>(streams) * hidden;
    p.S = mhcpb::split_count(T);
    p.L = (T + p.S - 1) / p.S;
    p.ws_bytes = static_cast<size_t>(p.S) * mhcpb::kProjCols * static_cast<size_t>(p.K) * 4;
    p.wait_polls = wait_polls_setting();
    p.shape = mhcpb::projection_shape(p.K, p.S);
    auto *h = new (std::nothrow) mhcpb_plan_s{p};
    if (!h)
        return MHCPB_ERROR_INVALID_ARGUMENT;
    *plan = h;
    return MHCPB_SUCCESS;
}

mhcpb_status_t mhcpb_plan_destroy(mhcpb_plan_t plan) {
    delete plan;
    return MHCPB_SUCCESS;
}

mhcpb_status_t mhcpb_workspace_bytes(mhcpb_plan_t plan, size_t *bytes) {
    if (!plan || !bytes)
        return MHCPB_ERROR_INVALID_ARGUMENT;
    *bytes = plan->plan.ws_bytes;
    return MHCPB_SUCCESS;
}

mhcpb_status_t mhcpb_plan_split_count(mhcpb_plan_t plan, int32_t *splits) {
    if (!plan || !splits)
        return MHCPB_ERROR_INVALID_ARGUMENT;
    *splits = plan->plan.S;
    return MHCPB_SUCCESS;
}

mhcpb_status_t mhcpb_plan_partial_slabs(mhcpb_plan_t plan, int32_t *slabs) {
    if (!plan || !slabs)
        return MHCPB_ERROR_INVALID_ARGUMENT;
    *slabs = plan->plan.S - plan->plan.shape.first_slab;
    return MHCPB_SUCCESS;
}

mhcpb_status_t mhcpb_execute(mhcpb_plan_t plan, const float *x, const float *w,
                             const float *grad_proj, const float *grad_r, const float *r,
                             uint16_t *dx, float *dw, const uint16_t *grad_x_addend,
                             void *workspace, size_t workspace_size, hipStream_t stream) {
    return run(plan, mhcpb::Outputs::kBoth, x, w, grad_proj, grad_r, r, dx, dw, grad_x_addend,
               workspace, workspace_size, stream, nullptr, nullptr, nullptr);
}

mhcpb_status_t mhcpb_execute_with_events(mhcpb_plan_t plan, const float *x, const float *w,
                                         const float *grad_proj, const float *grad_r,
                                         const float *r, uint16_t *dx, float *dw,
                                         const uint16_t *grad_x_addend, void *workspace,
                                         size_t workspace_size, hipStream_t stream,
                                         hipEvent_t before_k1, hipEvent_t after_k1,
                                         hipEvent_t after_k2) {
    return run(plan, mhcpb::Outputs::kBoth, x, w, grad_proj, grad_r, r, dx, dw, grad_x_addend,
               workspace, workspace_size, stream, before_k1, after_k1, after_k2);
}

mhcpb_status_t mhcpb_execute_noalloc(mhcpb_plan_t plan, const float *x, const float *w,
                                     const float *grad_proj, const float *grad_r, const float *r,
                                     uint16_t *dx, float *dw, const uint16_t *grad_x_addend,
                                     hipStream_t stream) {
    if (!plan)
        return MHCPB_ERROR_INVALID_ARGUMENT;
    if (plan->plan.ws_bytes > mhcpb::kStaticWorkspaceBytes)
        return MHCPB_ERROR_WORKSPACE;
    void *ws = nullptr;
    if (mhcpb::static_workspace(&ws) != hipSuccess)
        return MHCPB_ERROR_LAUNCH;
    return run(plan, mhcpb::Outputs::kBoth, x, w, grad_proj, grad_r, r, dx, dw, grad_x_addend, ws,
               mhcpb::kStaticWorkspaceBytes, stream, nullptr, nullptr, nullptr);
}

mhcpb_status_t mhcpb_execute_dx(mhcpb_plan_t plan, const float *x, const float *w,
                                const float *grad_proj, const float *grad_r, const float *r,
                                uint16_t *dx, const uint16_t *grad_x_addend,
                                hipStream_t stream) {
    return run(plan, mhcpb::Outputs::kDxOnly, x, w, grad_proj, grad_r, r, dx, nullptr,
               grad_x_addend, nullptr, 0, stream, nullptr, nullptr, nullptr);
}

mhcpb_status_t mhcpb_execute_dw(mhcpb_plan_t plan, const float *x, const float *grad_proj,
                                float *dw, void *workspace, size_t workspace_size,
                                hipStream_t stream) {
    return run(plan, mhcpb::Outputs::kDwOnly, x, nullptr, grad_proj, nullptr, nullptr, nullptr,
               dw, nullptr, workspace, workspace_size, stream, nullptr, nullptr, nullptr);
}

mhcpb_status_t mhcpb_forward_workspace_bytes(mhcpb_plan_t plan, size_t *bytes) {
    if (!plan || !bytes)
        return MHCPB_ERROR_INVALID_ARGUMENT;
    *bytes = static_cast<size_t>(mhcpb::forward_workspace_bytes(plan->plan.T, plan->plan.K));
    return MHCPB_SUCCESS;
}

mhcpb_status_t mhcpb_forward(mhcpb_plan_t plan, const float *x, const float *w, float eps,
                             float *proj, float *r, void *workspace, size_t workspace_size,
                             hipStream_t stream) {
    return run_forward(plan, x, w, eps, proj, r, workspace, workspace_size, stream, nullptr,
                       nullptr, nullptr);
}

mhcpb_status_t mhcpb_forward_with_events(mhcpb_plan_t plan, const float *x, const float *w,
                                         float eps, float *proj, float *r, void *workspace,
                                         size_t workspace_size, hipStream_t stream,
                                         hipEvent_t before_k1, hipEvent_t after_k1,
                                         hipEvent_t after_k2) {
    return run_forward(plan, x, w, eps, proj, r, workspace, workspace_size, stream, before_k1,
                       after_k1, after_k2);
}

mhcpb_status_t mhcpb_rmsnorm_backward_workspace_bytes(int64_t T, int32_t H, size_t *bytes) {
    if (!bytes)
        return MHCPB_ERROR_INVALID_ARGUMENT;
    mhcpb::RmsPlan p{};
    const mhcpb_status_t st = rmsnorm_shape(T, H, &p);
    if (st != MHCPB_SUCCESS)
        return st;
    *bytes = static_cast<size_t>(mhcpb::rmsnorm_workspace_bytes(p));
    return MHCPB_SUCCESS;
}

mhcpb_status_t mhcpb_rmsnorm_backward(int64_t T, int32_t H, const uint16_t *g, const uint16_t *x,
                                      const void *w, mhcpb_dtype_t w_dtype, const float *rstd,
                                      const uint16_t *g_residual, uint16_t *dx, float *dw,
                                      void *workspace, size_t workspace_size,
                                      hipStream_t stream) {
    return run_rmsnorm(T, H, g, x, w, w_dtype, rstd, g_residual, dx, dw, workspace,
                       workspace_size, stream, nullptr, nullptr, nullptr);
}

mhcpb_status_t mhcpb_rmsnorm_backward_with_events(
    int64_t T, int32_t H, const uint16_t *g, const uint16_t *x, const void *w,
    mhcpb_dtype_t w_dtype, const float *rstd, const uint16_t *g_residual, uint16_t *dx,
    float *dw, void *workspace, size_t workspace_size, hipStream_t stream,
    hipEvent_t before_k1, hipEvent_t after_k1, hipEvent_t after_k2) {
    return run_rmsnorm(T, H, g, x, w, w_dtype, rstd, g_residual, dx, dw, workspace,
                       workspace_size, stream, before_k1, after_k1, after_k2);
}

const char *mhcpb_status_string(mhcpb_status_t status) {
    switch (status) {
    case MHCPB_SUCCESS: return "success";
    case MHCPB_ERROR_INVALID_ARGUMENT: return "invalid argument";
    case MHCPB_ERROR_UNSUPPORTED: return "unsupported shape";
    case MHCPB_ERROR_MISALIGNED: return "pointer not 16-byte aligned";
    case MHCPB_ERROR_OVERLAP: return "operand byte ranges overlap";
    case MHCPB_ERROR_WORKSPACE: return "workspace too small";
    case MHCPB_ERROR_LAUNCH: return "kernel launch failed";
    }
    return "unknown status";
}

}  // extern "C"
