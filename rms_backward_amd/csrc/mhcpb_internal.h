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

// Split count as a function of T only: one partial dW slab per 512 tokens,
// at most 32.  At T = 4096 this gives the 8 slabs whose FP32 [24, K] partials
// make the 15,728,640-byte workspace of the page's supported profile.
inline int32_t split_count(int64_t T) {
    int64_t s = (T + kRowsPerSplit - 1) / kRowsPerSplit;
    return static_cast<int32_t>(s > kMaxSplits ? kMaxSplits : s);
}

struct Plan {
    int64_t T;
    int32_t streams;
    int32_t hidden;
    int64_t K;
    int32_t S;        // splits (partial dW slabs)
    int64_t L;        // rows per slab, ceil(T / S); the last slab may be shorter
    size_t ws_bytes;  // S * 24 * K * 4
};

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
// Kernel 2: dW = sum of the S slabs in ascending order; the optional event
// takes the end time of the dispatch.
hipError_t launch_reduce(const Plan &p, const Args &a, hipStream_t stream, hipEvent_t stop);

// Columns of a row of the forward's weight planes: K rounded up to whole
// 64-column chunks (the padding is zero).
inline int64_t forward_padded_cols(int64_t K) { return (K + 63) / 64 * 64; }

// Forward, kernel 0: W [24, K] FP32 -> its TF32 split (BF16 high and low
// parts of 24 x forward_padded_cols(K) values, zero past K) in wsplit, in the
// order the pass over X loads it.
hipError_t launch_split_weight(const Plan &p, const float *w, uint16_t *wsplit, hipStream_t stream,
                               hipEvent_t start, hipEvent_t stop);
// Forward, kernel 1: proj [T, 32] (logits in columns 0..23, zeros in 24..31)
// and r [T] from X and the split W, in one pass over X.
hipError_t launch_forward(const Plan &p, const float *x, const uint16_t *wsplit, float *proj,
                          float *r, float eps, hipStream_t stream, hipEvent_t start,
                          hipEvent_t stop);

}  // namespace mhcpb

struct mhcpb_plan_s {
    mhcpb::Plan plan;
};
