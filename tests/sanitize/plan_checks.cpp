// Host-only build of the library's plan and argument validation with the
// kernel launches replaced by counters, run under AddressSanitizer and
// UndefinedBehaviorSanitizer on the CPU (tests/test_sanitizers.py).  Device
// addresses are plain integers here: nothing dereferences them once the
// launches are stubbed.  Exits non-zero on the first failed check.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "../../include/mhcpb.h"
#include "../../rms_backward_amd/csrc/mhcpb_internal.h"

namespace mhcpb {
static int g_launches = 0;
static Plan g_plan;
hipError_t launch_projection(const Plan &p, const Args &, Outputs, hipStream_t, hipEvent_t,
                             hipEvent_t) {
    ++g_launches;
    g_plan = p;
    return hipSuccess;
}
hipError_t launch_reduce(const Plan &, const Args &, hipStream_t, hipEvent_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t launch_forward(const Plan &p, const float *, const float *, float *, float *, float,
                          float *, hipStream_t, hipEvent_t, hipEvent_t, hipEvent_t) {
    ++g_launches;
    g_plan = p;
    return hipSuccess;
}
hipError_t launch_rmsnorm_backward(const RmsPlan &, const uint16_t *, const uint16_t *,
                                   const void *, bool, const float *, const uint16_t *,
                                   uint16_t *, float *, float *, hipStream_t, hipEvent_t,
                                   hipEvent_t, hipEvent_t) {
    ++g_launches;
    return hipSuccess;
}
hipError_t static_workspace(void **ptr) {
    *ptr = reinterpret_cast<void *>(uintptr_t{0x7f0000000000});
    return hipSuccess;
}
}  // namespace mhcpb

static int g_fail = 0;
#define CHECK(cond)                                                       \
    do {                                                                  \
        if (!(cond)) {                                                    \
            std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond); \
            g_fail = 1;                                                   \
        }                                                                 \
    } while (0)

template <typename T>
static T *at(uint64_t a) { return reinterpret_cast<T *>(static_cast<uintptr_t>(a)); }

int main() {
    // plans over the domain and beyond it
    for (int64_t T : {int64_t{1}, int64_t{15}, int64_t{512}, int64_t{4095}, int64_t{4096},
                      int64_t{65536}, (int64_t{1} << 31) - 1}) {
        for (int32_t hidden : {2, 130, 5120, 1 << 20}) {
            mhcpb_plan_t p = nullptr;
            CHECK(mhcpb_plan_create(&p, T, 4, hidden) == MHCPB_SUCCESS && p != nullptr);
            size_t ws = 0;
            int32_t S = 0;
            CHECK(mhcpb_workspace_bytes(p, &ws) == MHCPB_SUCCESS);
            CHECK(mhcpb_plan_split_count(p, &S) == MHCPB_SUCCESS);
            CHECK(S >= 1 && S <= 32 && ws == static_cast<size_t>(S) * 24 * 4 * hidden * 4);
            size_t fws = 0;
            CHECK(mhcpb_forward_workspace_bytes(p, &fws) == MHCPB_SUCCESS);
            CHECK(mhcpb_plan_destroy(p) == MHCPB_SUCCESS);
        }
    }
    mhcpb_plan_t bad = at<mhcpb_plan_s>(1);
    CHECK(mhcpb_plan_create(&bad, 0, 4, 64) == MHCPB_ERROR_INVALID_ARGUMENT && bad == nullptr);
    CHECK(mhcpb_plan_create(&bad, 16, 3, 64) == MHCPB_ERROR_UNSUPPORTED);
    CHECK(mhcpb_plan_create(&bad, 16, 4, 63) == MHCPB_ERROR_UNSUPPORTED);
    CHECK(mhcpb_plan_create(&bad, int64_t{1} << 31, 4, 64) == MHCPB_ERROR_UNSUPPORTED);
    CHECK(mhcpb_plan_create(nullptr, 16, 4, 64) == MHCPB_ERROR_INVALID_ARGUMENT);
    CHECK(mhcpb_plan_destroy(nullptr) == MHCPB_SUCCESS);

    // execute: a valid layout of disjoint, aligned buffers (T = 300, K = 256)
    const int64_t T = 300, K = 256;
    mhcpb_plan_t p = nullptr;
    CHECK(mhcpb_plan_create(&p, T, 4, 64) == MHCPB_SUCCESS);
    size_t wsb = 0;
    mhcpb_workspace_bytes(p, &wsb);
    uint64_t base = 0x100000000ull, off = 0;
    auto take = [&](uint64_t bytes) { uint64_t a = base + off; off += (bytes + 255) / 256 * 256; return a; };
    const uint64_t x = take(T * K * 4), w = take(24 * K * 4), gp = take(T * 32 * 4),
                   gr = take(T * 4), r = take(T * 4), dx = take(T * K * 2), dw = take(24 * K * 4),
                   ad = take(T * K * 2), ws = take(wsb);
    mhcpb::g_launches = 0;
    CHECK(mhcpb_execute(p, at<float>(x), at<float>(w), at<float>(gp), at<float>(gr), at<float>(r),
                        at<uint16_t>(dx), at<float>(dw), at<uint16_t>(ad), at<void>(ws), wsb,
                        nullptr) == MHCPB_SUCCESS);
    CHECK(mhcpb::g_launches == 2);
    CHECK(mhcpb_execute(p, nullptr, at<float>(w), at<float>(gp), at<float>(gr), at<float>(r),
                        at<uint16_t>(dx), at<float>(dw), nullptr, at<void>(ws), wsb,
                        nullptr) == MHCPB_ERROR_INVALID_ARGUMENT);
    CHECK(mhcpb_execute(p, at<float>(x + 4), at<float>(w), at<float>(gp), at<float>(gr),
                        at<float>(r), at<uint16_t>(dx), at<float>(dw), nullptr, at<void>(ws), wsb,
                        nullptr) == MHCPB_ERROR_MISALIGNED);
    CHECK(mhcpb_execute(p, at<float>(x), at<float>(w), at<float>(gp), at<float>(gr), at<float>(r),
                        at<uint16_t>(x + 16), at<float>(dw), nullptr, at<void>(ws), wsb,
                        nullptr) == MHCPB_ERROR_OVERLAP);
    CHECK(mhcpb_execute(p, at<float>(x), at<float>(w), at<float>(gp), at<float>(gr), at<float>(r),
                        at<uint16_t>(dx), at<float>(dw), nullptr, at<void>(ws), wsb - 16,
                        nullptr) == MHCPB_ERROR_WORKSPACE);
    CHECK(mhcpb_execute(p, at<float>(0xFFFFFFFFFFFFFF00ull), at<float>(w), at<float>(gp),
                        at<float>(gr), at<float>(r), at<uint16_t>(dx), at<float>(dw), nullptr,
                        at<void>(ws), wsb, nullptr) == MHCPB_ERROR_INVALID_ARGUMENT);
    CHECK(mhcpb_execute(nullptr, at<float>(x), at<float>(w), at<float>(gp), at<float>(gr),
                        at<float>(r), at<uint16_t>(dx), at<float>(dw), nullptr, at<void>(ws), wsb,
                        nullptr) == MHCPB_ERROR_INVALID_ARGUMENT);
    mhcpb::g_launches = 0;
    CHECK(mhcpb_execute_dx(p, at<float>(x), at<float>(w), at<float>(gp), at<float>(gr),
                           at<float>(r), at<uint16_t>(dx), nullptr, nullptr) == MHCPB_SUCCESS);
    CHECK(mhcpb::g_launches == 1);
    CHECK(mhcpb_execute_dw(p, at<float>(x), at<float>(gp), at<float>(dw), at<void>(ws), wsb,
                           nullptr) == MHCPB_SUCCESS);
    CHECK(mhcpb::g_launches == 3);
    CHECK(mhcpb_execute_noalloc(p, at<float>(x), at<float>(w), at<float>(gp), at<float>(gr),
                                at<float>(r), at<uint16_t>(dx), at<float>(dw), nullptr,
                                nullptr) == MHCPB_SUCCESS);
    // forward
    const uint64_t proj = take(T * 32 * 4), rr = take(T * 4);
    size_t fwsb = 0;
    mhcpb_forward_workspace_bytes(p, &fwsb);
    const uint64_t fws = take(fwsb);
    CHECK(mhcpb_forward(p, at<float>(x), at<float>(w), 1e-6f, at<float>(proj), at<float>(rr),
                        at<void>(fws), fwsb, nullptr) == MHCPB_SUCCESS);
    CHECK(mhcpb_forward(p, at<float>(x), at<float>(w), std::nanf(""), at<float>(proj),
                        at<float>(rr), at<void>(fws), fwsb, nullptr) ==
          MHCPB_ERROR_INVALID_ARGUMENT);
    CHECK(mhcpb_forward(p, at<float>(x), at<float>(w), 1e-6f, at<float>(proj), at<float>(rr),
                        at<void>(fws), fwsb - 1, nullptr) == MHCPB_ERROR_WORKSPACE);
    CHECK(mhcpb_plan_destroy(p) == MHCPB_SUCCESS);
    // a plan whose workspace exceeds the static one
    CHECK(mhcpb_plan_create(&p, 16384, 4, 6144) == MHCPB_SUCCESS);
    CHECK(mhcpb_execute_noalloc(p, at<float>(x), at<float>(w), at<float>(gp), at<float>(gr),
                                at<float>(r), at<uint16_t>(dx), at<float>(dw), nullptr,
                                nullptr) == MHCPB_ERROR_WORKSPACE);
    CHECK(mhcpb_plan_destroy(p) == MHCPB_SUCCESS);
    // the wait bound from the environment
    const char *vals[] = {"0", "1048576", "1048577", "-5", "abc", "12x", ""};
    const int32_t expect[] = {0, 1048576, 1 << 16, 1 << 16, 1 << 16, 1 << 16, 1 << 16};
    for (int i = 0; i < 7; ++i) {
        setenv("MHCPB_WAIT_POLLS", vals[i], 1);
        CHECK(mhcpb_plan_create(&p, 64, 4, 16) == MHCPB_SUCCESS);
        CHECK(p->plan.wait_polls == expect[i]);
        mhcpb_plan_destroy(p);
    }
    unsetenv("MHCPB_WAIT_POLLS");
    // RMSNorm backward
    size_t rws = 0;
    CHECK(mhcpb_rmsnorm_backward_workspace_bytes(4096, 5120, &rws) == MHCPB_SUCCESS && rws > 0);
    CHECK(mhcpb_rmsnorm_backward_workspace_bytes(16, 7, &rws) == MHCPB_ERROR_UNSUPPORTED);
    CHECK(mhcpb_rmsnorm_backward_workspace_bytes(-1, 64, &rws) == MHCPB_ERROR_INVALID_ARGUMENT);
    CHECK(mhcpb_rmsnorm_backward_workspace_bytes(0, 64, &rws) == MHCPB_SUCCESS && rws == 0);
    mhcpb_rmsnorm_backward_workspace_bytes(300, 64, &rws);
    const uint64_t g = take(300 * 64 * 2), xr = take(300 * 64 * 2), wr = take(64 * 4),
                   rs = take(300 * 4), dxr = take(300 * 64 * 2), dwr = take(64 * 4), wsr = take(rws);
    CHECK(mhcpb_rmsnorm_backward(300, 64, at<uint16_t>(g), at<uint16_t>(xr), at<void>(wr),
                                 MHCPB_DTYPE_F32, at<float>(rs), nullptr, at<uint16_t>(dxr),
                                 at<float>(dwr), at<void>(wsr), rws, nullptr) == MHCPB_SUCCESS);
    CHECK(mhcpb_rmsnorm_backward(0, 64, nullptr, nullptr, at<void>(wr), MHCPB_DTYPE_BF16, nullptr,
                                 nullptr, nullptr, at<float>(dwr), nullptr, 0, nullptr) ==
          MHCPB_SUCCESS);
    CHECK(mhcpb_rmsnorm_backward(300, 64, at<uint16_t>(g), at<uint16_t>(xr), at<void>(wr),
                                 static_cast<mhcpb_dtype_t>(7), at<float>(rs), nullptr,
                                 at<uint16_t>(dxr), at<float>(dwr), at<void>(wsr), rws,
                                 nullptr) == MHCPB_ERROR_INVALID_ARGUMENT);
    for (int s = -1; s < 9; ++s)
        CHECK(std::strlen(mhcpb_status_string(static_cast<mhcpb_status_t>(s))) > 0);
    std::printf(g_fail ? "plan checks FAILED\n" : "plan checks passed\n");
    return g_fail;
}
