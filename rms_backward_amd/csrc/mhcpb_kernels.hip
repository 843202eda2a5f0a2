// Kernels of the DSv4.1 mHC projection/RMS backward for gfx950.
//
// Kernel 1 ("projection"): the grid is (column tiles) x (S slabs of T).  Each
// workgroup owns one slab of rows and one tile of columns, reads its rows of X
// exactly once, writes the matching dX, and keeps its dW[24, tile] partial in
// registers; the partial goes to workspace slab s (one writer per element).
// Kernel 2 ("reduce"): dW = ((slab 0 + slab 1) + slab 2) + ... in FP32.
// This follows the page's structure (token reduction split over independent
// blocks, partial weight gradients, a second reduction kernel: "Source
// attribution" section) with a split count that depends on T only.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "mhcpb_internal.h"

namespace mhcpb {
namespace {

// TF32 value of an FP32 number: round the fraction to nearest-even at 10
// bits on the bit pattern, the carry running into the exponent.  NaN stays a
// (quiet) NaN and infinities stay infinite.
__device__ __forceinline__ float tf32_rne(float v) {
    uint32_t u = __float_as_uint(v);
    uint32_t rounded = (u + 0xFFFu + ((u >> 13) & 1u)) & 0xFFFFE000u;
    bool special = (u & 0x7F800000u) == 0x7F800000u;
    uint32_t keep = u | ((u & 0x007FFFFFu) ? 0x00400000u : 0u);
    return __uint_as_float(special ? keep : rounded);
}

// Two FP32 values to two BF16 (round to nearest even) packed low-first.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    __bf16 a = static_cast<__bf16>(lo);
    __bf16 b = static_cast<__bf16>(hi);
    uint16_t ua = __builtin_bit_cast(uint16_t, a);
    uint16_t ub = __builtin_bit_cast(uint16_t, b);
    return static_cast<uint32_t>(ua) | (static_cast<uint32_t>(ub) << 16);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

constexpr int kWave = 64;
constexpr int kColsPerLane = 4;
constexpr int kTileCols = kWave * kColsPerLane;  // 256 columns per workgroup
constexpr int kChunkRows = 64;                   // rows of P staged in LDS at once

// One wave per workgroup; lane l owns columns [tile0 + 4 l, tile0 + 4 l + 4).
template <bool kAddend>
__global__ __launch_bounds__(kWave) void projection_valu(
    const float *__restrict__ x, const float *__restrict__ w,
    const float *__restrict__ grad_proj, const float *__restrict__ grad_r,
    const float *__restrict__ r, uint16_t *__restrict__ dx, float *__restrict__ ws,
    const uint16_t *__restrict__ addend, int64_t T, int64_t K, int64_t L) {
    __shared__ float sP[kChunkRows][kProjCols];
    __shared__ float sC[kChunkRows];

    const int lane = threadIdx.x;
    const int64_t col = static_cast<int64_t>(blockIdx.x) * kTileCols + lane * kColsPerLane;
    const bool active = col < K;  // K is a multiple of 4: all 4 columns or none
    const int s = blockIdx.y;
    const int64_t row0 = static_cast<int64_t>(s) * L;
    const int64_t row1 = (row0 + L < T) ? row0 + L : T;
    const float kf = static_cast<float>(K);

    float wt[kProjCols][kColsPerLane];
    float acc[kProjCols][kColsPerLane];
#pragma unroll
    for (int j = 0; j < kProjCols; ++j) {
        float4 v = active ? *reinterpret_cast<const float4 *>(w + j * K + col)
                          : make_float4(0.f, 0.f, 0.f, 0.f);
        wt[j][0] = tf32_rne(v.x);
        wt[j][1] = tf32_rne(v.y);
        wt[j][2] = tf32_rne(v.z);
        wt[j][3] = tf32_rne(v.w);
#pragma unroll
        for (int q = 0; q < kColsPerLane; ++q) acc[j][q] = 0.f;
    }

    for (int64_t c0 = row0; c0 < row1; c0 += kChunkRows) {
        const int nrows = static_cast<int>((row1 - c0) < kChunkRows ? (row1 - c0) : kChunkRows);
        __syncthreads();
        if (lane < nrows) {
            const int64_t t = c0 + lane;
            const float *pr = grad_proj + t * kProjStride;
#pragma unroll
            for (int j = 0; j < kProjCols; j += 4) {
                float4 v = *reinterpret_cast<const float4 *>(pr + j);
                sP[lane][j + 0] = tf32_rne(v.x);
                sP[lane][j + 1] = tf32_rne(v.y);
                sP[lane][j + 2] = tf32_rne(v.z);
                sP[lane][j + 3] = tf32_rne(v.w);
            }
            sC[lane] = grad_r[t] / (r[t] * kf);
        }
        __syncthreads();
        if (!active) continue;
        for (int i = 0; i < nrows; ++i) {
            const int64_t t = c0 + i;
            const float4 xv = *reinterpret_cast<const float4 *>(x + t * K + col);
            const float xs[4] = {xv.x, xv.y, xv.z, xv.w};
            const float c = sC[i];
            float d[4];
            float xt[4];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                d[q] = 0.f;
                xt[q] = tf32_rne(xs[q]);
            }
#pragma unroll
            for (int j = 0; j < kProjCols; ++j) {
                const float p = sP[i][j];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    d[q] = fmaf(p, wt[j][q], d[q]);
                    acc[j][q] = fmaf(p, xt[q], acc[j][q]);
                }
            }
#pragma unroll
            for (int q = 0; q < 4; ++q) d[q] = fmaf(c, xs[q], d[q]);
            if constexpr (kAddend) {
                const uint2 a = *reinterpret_cast<const uint2 *>(addend + t * K + col);
                d[0] += bf16_to_f32(a.x & 0xFFFFu);
                d[1] += bf16_to_f32(a.x >> 16);
                d[2] += bf16_to_f32(a.y & 0xFFFFu);
                d[3] += bf16_to_f32(a.y >> 16);
            }
            uint2 o;
            o.x = pack_bf16x2(d[0], d[1]);
            o.y = pack_bf16x2(d[2], d[3]);
            *reinterpret_cast<uint2 *>(dx + t * K + col) = o;
        }
    }
    if (!active) return;
    float *slab = ws + static_cast<int64_t>(s) * kProjCols * K;
#pragma unroll
    for (int j = 0; j < kProjCols; ++j)
        *reinterpret_cast<float4 *>(slab + j * K + col) =
            make_float4(acc[j][0], acc[j][1], acc[j][2], acc[j][3]);
}

// dW[i] = (((ws[0][i] + ws[1][i]) + ws[2][i]) + ...), four elements per thread.
__global__ __launch_bounds__(256) void reduce_slabs(const float *__restrict__ ws,
                                                    float *__restrict__ dw, int S,
                                                    int64_t n4) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= n4) return;
    const float4 *src = reinterpret_cast<const float4 *>(ws);
    float4 a = src[i];
    for (int s = 1; s < S; ++s) {
        const float4 b = src[static_cast<int64_t>(s) * n4 + i];
        a.x += b.x;
        a.y += b.y;
        a.z += b.z;
        a.w += b.w;
    }
    reinterpret_cast<float4 *>(dw)[i] = a;
}

}  // namespace

hipError_t launch_projection(const Plan &p, const Args &a, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>((p.K + kTileCols - 1) / kTileCols),
                    static_cast<unsigned>(p.S));
    if (a.addend)
        hipLaunchKernelGGL(projection_valu<true>, grid, dim3(kWave), 0, stream, a.x, a.w,
                           a.grad_proj, a.grad_r, a.r, a.dx, a.ws, a.addend, p.T, p.K, p.L);
    else
        hipLaunchKernelGGL(projection_valu<false>, grid, dim3(kWave), 0, stream, a.x, a.w,
                           a.grad_proj, a.grad_r, a.r, a.dx, a.ws, a.addend, p.T, p.K, p.L);
    return hipGetLastError();
}

hipError_t launch_reduce(const Plan &p, const Args &a, hipStream_t stream) {
    const int64_t n4 = kProjCols * p.K / 4;
    const unsigned blocks = static_cast<unsigned>((n4 + 255) / 256);
    hipLaunchKernelGGL(reduce_slabs, dim3(blocks), dim3(256), 0, stream, a.ws, a.dw, p.S, n4);
    return hipGetLastError();
}

}  // namespace mhcpb
