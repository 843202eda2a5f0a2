// Internal declarations shared by the plan/validation code and the kernels.
#pragma once

#include <cstddef>
#include <cstdint>

#include <hip/hip_runtime_api.h>

namespace mhcpb {

constexpr int kProjCols = 24;    // columns of grad_proj that take part
constexpr int kProjStride = 32;  // row length of grad_proj (8 ignored columns)
constexpr int kMaxSplits = 32;
constexpr int64_t kRowsPerSplit = 512;
constexpr int kSmallSplits = 8;
constexpr int64_t kSmallSplitRows = 64;

// Split count as a function of T only: one partial dW slab per 512 tokens,
// at most 32, and below T = 4096 one slab per 64 tokens, up to eight (a slab
// is walked in order by one wave per column group, so a short T in few slabs
// would leave the GPU nearly idle).  At T = 4096 this gives the 8 slabs whose
// FP32 [24, K] partials make the 15,728,640-byte workspace of the page's
// supported profile.
inline int32_t split_count(int64_t T) {
    const int64_t big = (T + kRowsPerSplit - 1) / kRowsPerSplit;
    const int64_t by_rows = (T + kSmallSplitRows - 1) / kSmallSplitRows;
    const int64_t small = by_rows < kSmallSplits ? by_rows : kSmallSplits;
    const int64_t s = big > small ? big : small;
    return static_cast<int32_t>(s > kMaxSplits ? kMaxSplits : s);
}

// Launch shape of kernel 1, a performance choice only (each column's dW is
// summed over the same rows in the same order whatever the shape, so no bit
// depends on it): compute waves per workgroup (64 columns each), column
// tiles, slab groups (workgroups per tile, each walking a run of consecutive
// slabs), and the slab in which slab group 0 leaves the sum of its slabs,
// where kernel 2 starts.
struct ProjShape {
    int32_t nw;
    int32_t tiles;
    int32_t groups;
    int32_t first_slab;
};

// Workgroups kernel 1 aims at: one per CU of a 256-CU GPU.
constexpr int32_t kTargetWorkgroups = 256;

// Five compute waves per workgroup (320-column tiles, one workgroup per CU)
// unless that leaves more than half of the 256 CUs without a workgroup; then
// one compute wave (64-column tiles, up to three workgroups per CU), provided
// every workgroup still walks a single slab.  Measured on MI355X over shapes
// from T = 64 to 16384 and K = 1200 to 16384: one-wave workgroups are 17-30 %
// faster where five-wave ones fill at most 104 CUs, and up to twice as slow
// where they fill 128 or more, or where a one-wave workgroup would walk two
// slabs.  Slab groups: as many as keep the grid within 256 workgroups (five
// waves), at least one and at most S.
inline ProjShape projection_shape(int64_t K, int32_t S) {
    ProjShape sh{};
    const int64_t tiles5 = (K + 319) / 320;
    const int64_t tiles1 = (K + 63) / 64;
    if (tiles5 * S < kTargetWorkgroups / 2 && tiles1 * S <= 3 * kTargetWorkgroups) {
        sh.nw = 1;
        sh.tiles = static_cast<int32_t>(tiles1);
        sh.groups = S;
    } else {
        sh.nw = 5;
        sh.tiles = static_cast<int32_t>(tiles5);
        const int64_t g = kTargetWorkgroups / tiles5;
        sh.groups = static_cast<int32_t>(g < 1 ? 1 : (g > S ? S : g));
    }
    // Group 0 walks slabs [0, S / groups).
    sh.first_slab = S / sh.groups - 1;
    return sh;
}

struct Plan {
    int64_t T;
    int32_t streams;
    int32_t hidden;
    int64_t K;
    int32_t S;        // splits (partial dW slabs)
    int64_t L;        // rows per slab, ceil(T / S); the last slab may be shorter
    size_t ws_bytes;  // S * 24 * K * 4
    int32_t wait_polls;  // bound of the kernels' LDS counter waits
    ProjShape shape;  // launch shape of kernel 1
};

// Default bound of the kernels' LDS counter waits (polls of a few dozen
// cycles each), and the environment variable that overrides it for a plan
// created while it is set: a decimal in [0, 2^20].  0 makes every wait give
// up at once, so that the tests can reach the path on which the kernels turn
// the results they write into NaN.
constexpr int32_t kDefaultWaitPolls = 1 << 16;
constexpr const char *kWaitPollsEnv = "MHCPB_WAIT_POLLS";

struct Args {
    const float *x;
    const float *w;
    const float *grad_proj;
    const float *grad_r;
    const float *r;
    uint16_t *dx;
    float *dw;
    const uint16_t *addend;  // may be null
    float *ws;
};

// Which outputs kernel 1 produces: dX and the partial dW slabs (the fused
// stage), dX only, or the partial slabs only.
enum class Outputs { kBoth, kDxOnly, kDwOnly };

// Kernel 1: one pass over X; writes dX and/or the S partial dW slabs.  The
// optional events take the start and end times of the dispatch.
hipError_t launch_projection(const Plan &p, const Args &a, Outputs out, hipStream_t stream,
                             hipEvent_t start, hipEvent_t stop);
// Kernel 2: dW = sum of the S slabs in ascending order (from the slab in
// which kernel 1's slab group 0 left the sum of its slabs); the optional
// event takes the end time of the dispatch.
hipError_t launch_reduce(const Plan &p, const Args &a, hipStream_t stream, hipEvent_t stop);

// The static workspace of mhcpb_execute_noalloc: kStaticWorkspaceBytes of
// device memory per GPU in a file-scope array of the kernel library.
// static_workspace() gives its address on the current device (looked up once
// per device, then cached); it allocates nothing.
constexpr size_t kStaticWorkspaceBytes = size_t{64} << 20;
hipError_t static_workspace(void **ptr);

// Forward: the K columns are cut into tiles of kFwdTileCols; kernel 1
// writes one partial (24 logits and a sum of squares) per tile and token into
// the workspace, kernel 2 adds them in tile order.
constexpr int kFwdTileCols = 1024;
inline int forward_tile_count(int64_t K) {
    return static_cast<int>((K + kFwdTileCols - 1) / kFwdTileCols);
}
// Workspace of the forward: per tile and 16-token step, 8 blocks of 64 FP32
// (two tokens of 32 floats each: 24 logits, the squares, padding).
inline uint64_t forward_workspace_bytes(int64_t T, int64_t K) {
    return static_cast<uint64_t>(forward_tile_count(K)) * static_cast<uint64_t>((T + 15) / 16) *
           8 * 64 * 4;
}
// Units of work of forward kernel 1: tiles x ceil(T / 16); must stay below
// 2^31.
inline int64_t forward_units(int64_t T, int64_t K) {
    return static_cast<int64_t>(forward_tile_count(K)) * ((T + 15) / 16);
}

// Forward: kernel 1 (per tile partials into ws) and kernel 2 (proj [T, 32]
// with the logits in columns 0..23 and zeros in 24..31, r [T]).  The optional
// events take the start and end times of kernel 1 and the end time of
// kernel 2.
hipError_t launch_forward(const Plan &p, const float *x, const float *w, float *proj, float *r,
                          float eps, float *ws, hipStream_t stream, hipEvent_t start,
                          hipEvent_t mid, hipEvent_t stop);

// BF16 RMSNorm backward (second workload).  A row is cut into chunks of
// 512 columns, one wave each; a block has one wave per chunk.  Rows are
// dealt to S blocks round-robin (block b takes rows b, b + S, ...), with
// S = min(ceil(T / 16), 256 * P) and P = max(1, 12 / chunks) blocks per CU's
// worth of waves: a function of (T, H) only, never of the device.  The
// workspace holds one FP32 partial dw [H] per block.
constexpr int64_t kRmsBlockUnit = 256;
constexpr int64_t kRmsMinRowsPerBlock = 16;
constexpr int kRmsChunkCols = 512;
constexpr int kRmsWavesPerUnit = 12;
constexpr int32_t kRmsMaxH = 6144;  // 12 chunks of 512 columns

inline int rmsnorm_chunks(int32_t H) { return (H + kRmsChunkCols - 1) / kRmsChunkCols; }

struct RmsPlan {
    int64_t T;
    int32_t H;
    int64_t S;  // blocks (and partials)
};

inline RmsPlan rmsnorm_plan(int64_t T, int32_t H) {
    RmsPlan p{T, H, 0};
    if (T > 0) {
        const int nc = rmsnorm_chunks(H);
        const int64_t per_unit = nc >= kRmsWavesPerUnit ? 1 : kRmsWavesPerUnit / nc;
        int64_t s = (T + kRmsMinRowsPerBlock - 1) / kRmsMinRowsPerBlock;
        if (s > kRmsBlockUnit * per_unit) s = kRmsBlockUnit * per_unit;
        p.S = s;
    }
    return p;
}

inline uint64_t rmsnorm_workspace_bytes(const RmsPlan &p) {
    return static_cast<uint64_t>(p.S) * static_cast<uint64_t>(p.H) * 4;
}

// Kernel 1 (dx and the block partials; skipped when T = 0) and kernel 2 (dw
// from the partials).  The optional events take the start and end times of
// kernel 1 and the end time of kernel 2.
hipError_t launch_rmsnorm_backward(const RmsPlan &p, const uint16_t *g, const uint16_t *x,
                                   const void *w, bool w_f32, const float *rstd,
                                   const uint16_t *res, uint16_t *dx, float *dw, float *ws,
                                   hipStream_t stream, hipEvent_t start, hipEvent_t mid,
                                   hipEvent_t stop);

}  // namespace mhcpb

struct mhcpb_plan_s {
    mhcpb::Plan plan;
};
