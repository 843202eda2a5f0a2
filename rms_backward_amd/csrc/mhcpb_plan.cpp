// Plan creation, argument validation and the C-ABI entry points.
//
// Follows the "Prepared class API" and "Requirements and tensor contract"
// sections of the "DSv4.1 mHC projection/RMS backward" page: a plan is host
// metadata; execute() checks the operands (alignment, disjointness), then
// enqueues exactly two kernels and allocates nothing.
#include <algorithm>
#include <cstdint>
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

mhcpb_status_t validate(const mhcpb::Plan &p, const float *x, const float *w,
                        const float *grad_proj, const float *grad_r, const float *r,
                        const uint16_t *dx, const float *dw, const uint16_t *addend,
                        const void *ws, size_t ws_size) {
    if (!x || !w || !grad_proj || !grad_r || !r || !dx || !dw || !ws)
        return MHCPB_ERROR_INVALID_ARGUMENT;
    if (ws_size < p.ws_bytes)
        return MHCPB_ERROR_WORKSPACE;
    const void *ptrs[] = {x, w, grad_proj, grad_r, r, dx, dw, ws, addend};
    for (const void *q : ptrs)
        if (q && !aligned(q))
            return MHCPB_ERROR_MISALIGNED;
    const uint64_t T = static_cast<uint64_t>(p.T), K = static_cast<uint64_t>(p.K);
    auto range = [](const void *q, uint64_t bytes) {
        uintptr_t lo = reinterpret_cast<uintptr_t>(q);
        return Range{lo, lo + static_cast<uintptr_t>(bytes)};
    };
    Range rs[9];
    int n = 0;
    rs[n++] = range(x, T * K * 4);
    rs[n++] = range(w, 24 * K * 4);
    rs[n++] = range(grad_proj, T * 32 * 4);
    rs[n++] = range(grad_r, T * 4);
    rs[n++] = range(r, T * 4);
    rs[n++] = range(dx, T * K * 2);
    rs[n++] = range(dw, 24 * K * 4);
    rs[n++] = range(ws, p.ws_bytes);
    if (addend)
        rs[n++] = range(addend, T * K * 2);
    for (int i = 0; i < n; ++i) {
        if (rs[i].hi < rs[i].lo)  // address wrap-around
            return MHCPB_ERROR_INVALID_ARGUMENT;
        for (int j = i + 1; j < n; ++j)
            if (overlap(rs[i], rs[j]))
                return MHCPB_ERROR_OVERLAP;
    }
    return MHCPB_SUCCESS;
}

mhcpb_status_t run(mhcpb_plan_t plan, const float *x, const float *w,
                   const float *grad_proj, const float *grad_r, const float *r,
                   uint16_t *dx, float *dw, const uint16_t *addend, void *ws,
                   size_t ws_size, hipStream_t stream, hipEvent_t ev0, hipEvent_t ev1,
                   hipEvent_t ev2) {
    if (!plan)
        return MHCPB_ERROR_INVALID_ARGUMENT;
    const mhcpb::Plan &p = plan->plan;
    mhcpb_status_t st = validate(p, x, w, grad_proj, grad_r, r, dx, dw, addend, ws, ws_size);
    if (st != MHCPB_SUCCESS)
        return st;
    mhcpb::Args a{x, w, grad_proj, grad_r, r, dx, dw, addend, static_cast<float *>(ws)};
    if (mhcpb::launch_projection(p, a, stream, ev0, ev1) != hipSuccess)
        return MHCPB_ERROR_LAUNCH;
    if (mhcpb::launch_reduce(p, a, stream, ev2) != hipSuccess)
        return MHCPB_ERROR_LAUNCH;
    return MHCPB_SUCCESS;
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

mhcpb_status_t mhcpb_execute(mhcpb_plan_t plan, const float *x, const float *w,
                             const float *grad_proj, const float *grad_r, const float *r,
                             uint16_t *dx, float *dw, const uint16_t *grad_x_addend,
                             void *workspace, size_t workspace_size, hipStream_t stream) {
    return run(plan, x, w, grad_proj, grad_r, r, dx, dw, grad_x_addend, workspace,
               workspace_size, stream, nullptr, nullptr, nullptr);
}

mhcpb_status_t mhcpb_execute_with_events(mhcpb_plan_t plan, const float *x, const float *w,
                                         const float *grad_proj, const float *grad_r,
                                         const float *r, uint16_t *dx, float *dw,
                                         const uint16_t *grad_x_addend, void *workspace,
                                         size_t workspace_size, hipStream_t stream,
                                         hipEvent_t before_k1, hipEvent_t after_k1,
                                         hipEvent_t after_k2) {
    return run(plan, x, w, grad_proj, grad_r, r, dx, dw, grad_x_addend, workspace,
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
