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

// Two FP32 values to two BF16 (round to nearest even) packed low-first; one
// v_cvt_pk_bf16_f32 on gfx950.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Upper halves of two 32-bit words: (a >> 16) | (b & 0xFFFF0000).
__device__ __forceinline__ uint32_t hi_halves(uint32_t a, uint32_t b) {
    return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// TF32 rounding on the bits, then the exact split of the TF32 value into a
// BF16 high part (its upper 16 bits) and a BF16 low part (the remaining 3
// significant bits, exact in BF16).  hi + lo == TF32(v).
__device__ __forceinline__ void tf32_split(float v, uint32_t &hi_bits, float &lo) {
    uint32_t u = __float_as_uint(v);
    uint32_t t = (u + 0xFFFu + ((u >> 13) & 1u)) & 0xFFFFE000u;
    uint32_t h = t & 0xFFFF0000u;
    hi_bits = h;
    lo = __uint_as_float(t) - __uint_as_float(h);
}

// The same split for the small operands (P, W), with non-finite inputs kept
// non-finite in the high part and a zero low part.
__device__ __forceinline__ uint32_t tf32_split_packed(float v) {
    uint32_t u = __float_as_uint(v);
    if ((u & 0x7F800000u) == 0x7F800000u) {
        uint32_t q = (u & 0x007FFFFFu) ? (u | 0x00400000u) : u;
        return q >> 16;  // high part only; low part zero
    }
    uint32_t hb;
    float lo;
    tf32_split(v, hb, lo);
    return (hb >> 16) | (__float_as_uint(lo) & 0xFFFF0000u);
}

// Rows of P staged per chunk, and LDS strides (padded against bank conflicts).
constexpr int kChunk = 64;
constexpr int kSteps = kChunk / 16;
constexpr int kPsStride = 26;          // uint32 per row of packed (hi | lo << 16) P
constexpr int kPtStride = kChunk + 4;  // uint16 per (j, part) slot row of transposed P
constexpr int kSlots = 2 * kProjCols;  // (j, part) pairs: 48

struct ChunkLds {
    uint32_t ps[kChunk * kPsStride];     // [row][j]: hi | lo << 16
    uint16_t pt[kSlots * kPtStride];     // [slot][row]: one BF16 part
    float c[kChunk];                     // grad_r / (r K)
};

// (j, part) -> slot of the transposed P array; slot = 16 b + n is what lane
// n of the dW product reads for its block b.
__device__ __forceinline__ int pt_slot(int j, int part) {
    return j < 16 ? j + 16 * part : j + 16 + 8 * part;
}

// Kernel 1, MFMA form.  A workgroup of NW waves owns NW * 64 columns of one
// slab.  Per step a wave handles 16 rows x 64 columns: lane l (c = l % 16,
// g = l / 16) holds x[t0 + 4g + r][kw + 4c + i] for r, i in 0..3.
//  dX: C_i[e] = dX[t0 + 4g + e][kw + 4c + i] = c_t x + sum over 96 slots of
//      (P hi|lo of token t0 + l%16) x (W hi|lo of column kw + 4c + i), 3 MFMAs.
//  dW: acc[i][b][e] = sum over tokens of x(hi|lo) of column kw + 4(4g+e) + i
//      times the P part of slot 16 b + l%16, one MFMA per (i, b) per step.
template <int NW, bool kAddend>
__global__ __launch_bounds__(NW * kWave) void projection_mfma(
    const float *__restrict__ x, const float *__restrict__ w,
    const float *__restrict__ grad_proj, const float *__restrict__ grad_r,
    const float *__restrict__ r, uint16_t *__restrict__ dx, float *__restrict__ ws,
    const uint16_t *__restrict__ addend, int64_t T, int64_t K, int64_t L) {
    __shared__ ChunkLds lds[2];
    constexpr int kThreads = NW * kWave;
    constexpr int kItems = kChunk * (kProjCols / 4);               // float4 of P per chunk
    constexpr int kItemsPerThread = (kItems + kThreads - 1) / kThreads;

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = tid / kWave;
    const int c16 = lane % 16;
    const int g = lane / 16;
    const int s = blockIdx.y;
    const int64_t kw = static_cast<int64_t>(blockIdx.x) * (NW * 64) + wave * 64;
    const int64_t col = kw + 4 * c16;                 // first of this lane's 4 columns
    const bool active = col < K;
    const int64_t row0 = static_cast<int64_t>(s) * L;
    const int64_t row1 = (row0 + L < T) ? row0 + L : T;
    const float kf = static_cast<float>(K);

    // W side of the dX product: for column variant i and MFMA u the lane
    // holds [Wh_j Wh_j Wh_j1 Wh_j1 Wl_j Wl_j Wl_j1 Wl_j1], j = 8u + 2g.
    u32x4 bw[4][3];
#pragma unroll
    for (int u = 0; u < 3; ++u) {
        const int j = 8 * u + 2 * g;
        float4 w0 = make_float4(0.f, 0.f, 0.f, 0.f), w1 = w0;
        if (active) {
            w0 = *reinterpret_cast<const float4 *>(w + j * K + col);
            w1 = *reinterpret_cast<const float4 *>(w + (j + 1) * K + col);
        }
        const float a0[4] = {w0.x, w0.y, w0.z, w0.w};
        const float a1[4] = {w1.x, w1.y, w1.z, w1.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t p0 = tf32_split_packed(a0[i]);
            const uint32_t p1 = tf32_split_packed(a1[i]);
            const uint32_t h0 = p0 & 0xFFFFu, l0 = p0 >> 16;
            const uint32_t h1 = p1 & 0xFFFFu, l1 = p1 >> 16;
            bw[i][u] = u32x4{h0 | (h0 << 16), h1 | (h1 << 16), l0 | (l0 << 16), l1 | (l1 << 16)};
        }
    }

    f32x4 accw[4][3];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int b = 0; b < 3; ++b) accw[i][b] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Stage the P rows [c0, c0 + kChunk) of this slab: load to registers ...
    float4 pv[kItemsPerThread];
    float cv = 0.f;
    auto stage_load = [&](int64_t c0) {
#pragma unroll
        for (int it = 0; it < kItemsPerThread; ++it) {
            const int item = tid + it * kThreads;
            const int rr = item / (kProjCols / 4);
            const int q = item % (kProjCols / 4);
            const int64_t t = c0 + rr;
            pv[it] = (item < kItems && t < row1)
                         ? *reinterpret_cast<const float4 *>(grad_proj + t * kProjStride + 4 * q)
                         : make_float4(0.f, 0.f, 0.f, 0.f);
        }
        if (tid < kChunk) {
            const int64_t t = c0 + tid;
            cv = (t < row1) ? grad_r[t] / (r[t] * kf) : 0.f;
        }
    };
    // ... then split and write both LDS layouts.
    auto stage_store = [&](ChunkLds &d) {
#pragma unroll
        for (int it = 0; it < kItemsPerThread; ++it) {
            const int item = tid + it * kThreads;
            if (item < kItems) {
                const int rr = item / (kProjCols / 4);
                const int q = item % (kProjCols / 4);
                const float vv[4] = {pv[it].x, pv[it].y, pv[it].z, pv[it].w};
                uint32_t pk[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    pk[e] = tf32_split_packed(vv[e]);
                    const int j = 4 * q + e;
                    d.pt[pt_slot(j, 0) * kPtStride + rr] = static_cast<uint16_t>(pk[e] & 0xFFFFu);
                    d.pt[pt_slot(j, 1) * kPtStride + rr] = static_cast<uint16_t>(pk[e] >> 16);
                }
                uint32_t *dst = d.ps + rr * kPsStride + 4 * q;
                *reinterpret_cast<u32x2 *>(dst) = u32x2{pk[0], pk[1]};
                *reinterpret_cast<u32x2 *>(dst + 2) = u32x2{pk[2], pk[3]};
            }
        }
        if (tid < kChunk) d.c[tid] = cv;
    };

    const int64_t nchunks = (row1 - row0 + kChunk - 1) / kChunk;
    if (nchunks > 0) {
        stage_load(row0);
        stage_store(lds[0]);
    }
    __syncthreads();

    float4 xv[4];
    auto load_x = [&](int64_t t0) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const int64_t t = t0 + 4 * g + rr;
            xv[rr] = (active && t < row1) ? *reinterpret_cast<const float4 *>(x + t * K + col)
                                          : make_float4(0.f, 0.f, 0.f, 0.f);
        }
    };
    if (nchunks > 0) load_x(row0);

    for (int64_t ch = 0; ch < nchunks; ++ch) {
        const int64_t c0 = row0 + ch * kChunk;
        ChunkLds &cur = lds[ch & 1];
        const bool more = ch + 1 < nchunks;
        if (more) stage_load(c0 + kChunk);
#pragma unroll 1
        for (int st = 0; st < kSteps; ++st) {
            const int64_t t0 = c0 + 16 * st;
            if (t0 >= row1) break;
            const float4 xc[4] = {xv[0], xv[1], xv[2], xv[3]};
            const int64_t tn = t0 + 16;
            if (tn < row1) load_x(tn);

            // dX: start from the RMS term c_t * x in FP32.
            const float4 cc = *reinterpret_cast<const float4 *>(cur.c + 16 * st + 4 * g);
            const float ce[4] = {cc.x, cc.y, cc.z, cc.w};
            f32x4 accx[4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                accx[0][rr] = ce[rr] * xc[rr].x;
                accx[1][rr] = ce[rr] * xc[rr].y;
                accx[2][rr] = ce[rr] * xc[rr].z;
                accx[3][rr] = ce[rr] * xc[rr].w;
            }
#pragma unroll
            for (int u = 0; u < 3; ++u) {
                const u32x2 pa = *reinterpret_cast<const u32x2 *>(
                    cur.ps + (16 * st + c16) * kPsStride + 8 * u + 2 * g);
                const u32x4 a = u32x4{pa.x, pa.y, pa.x, pa.y};
#pragma unroll
                for (int i = 0; i < 4; ++i) accx[i] = mfma(a, bw[i][u], accx[i]);
            }

            // dW: x split into BF16 hi/lo, packed [hi r0..r3 | lo r0..r3].
            u32x4 ax[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                uint32_t hb[4];
                float lo[4];
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const float v = i == 0 ? xc[rr].x : i == 1 ? xc[rr].y : i == 2 ? xc[rr].z : xc[rr].w;
                    tf32_split(v, hb[rr], lo[rr]);
                }
                ax[i] = u32x4{hi_halves(hb[0], hb[1]), hi_halves(hb[2], hb[3]),
                              hi_halves(__float_as_uint(lo[0]), __float_as_uint(lo[1])),
                              hi_halves(__float_as_uint(lo[2]), __float_as_uint(lo[3]))};
            }
#pragma unroll
            for (int b = 0; b < 3; ++b) {
                const u32x2 pb = *reinterpret_cast<const u32x2 *>(
                    cur.pt + (16 * b + c16) * kPtStride + 16 * st + 4 * g);
                const u32x4 bb = u32x4{pb.x, pb.y, pb.x, pb.y};
#pragma unroll
                for (int i = 0; i < 4; ++i) accw[i][b] = mfma(ax[i], bb, accw[i][b]);
            }

            // dX epilogue: optional addend, one rounding to BF16, 8-byte stores.
            if (active) {
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int64_t t = t0 + 4 * g + rr;
                    if (t < row1) {
                        float d0 = accx[0][rr], d1 = accx[1][rr], d2 = accx[2][rr], d3 = accx[3][rr];
                        if constexpr (kAddend) {
                            const uint2 av = *reinterpret_cast<const uint2 *>(addend + t * K + col);
                            d0 += bf16_to_f32(av.x & 0xFFFFu);
                            d1 += bf16_to_f32(av.x >> 16);
                            d2 += bf16_to_f32(av.y & 0xFFFFu);
                            d3 += bf16_to_f32(av.y >> 16);
                        }
                        uint2 o;
                        o.x = pack_bf16x2(d0, d1);
                        o.y = pack_bf16x2(d2, d3);
                        *reinterpret_cast<uint2 *>(dx + t * K + col) = o;
                    }
                }
            }
        }
        if (more) stage_store(lds[(ch + 1) & 1]);
        __syncthreads();
    }

    // Partial dW of this slab: the Ph and Pl halves of each j are added, then
    // written once to workspace slab s.  Lane (c16, g), element e of block b
    // is column kw + 16 g + 4 e + i of slot 16 b + c16.
    float *slab = ws + static_cast<int64_t>(s) * kProjCols * K;
    const int64_t cbase = kw + 16 * g;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        float lo01[4], hi2[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            lo01[i] = accw[i][0][e] + accw[i][1][e];               // j = c16
            const float other = __shfl_xor(accw[i][2][e], 8, 16);   // slot 16 b + (c16 ^ 8)
            hi2[i] = accw[i][2][e] + other;                        // j = 16 + c16 for c16 < 8
        }
        const int64_t cc = cbase + 4 * e;
        if (cc < K) {
            *reinterpret_cast<float4 *>(slab + c16 * K + cc) =
                make_float4(lo01[0], lo01[1], lo01[2], lo01[3]);
            if (c16 < 8)
                *reinterpret_cast<float4 *>(slab + (16 + c16) * K + cc) =
                    make_float4(hi2[0], hi2[1], hi2[2], hi2[3]);
        }
    }
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

constexpr int kWavesPerGroup = 4;

hipError_t launch_projection(const Plan &p, const Args &a, hipStream_t stream) {
    constexpr int cols = kWavesPerGroup * 64;
    const dim3 grid(static_cast<unsigned>((p.K + cols - 1) / cols), static_cast<unsigned>(p.S));
    const dim3 block(kWavesPerGroup * kWave);
    if (a.addend)
        hipLaunchKernelGGL((projection_mfma<kWavesPerGroup, true>), grid, block, 0, stream, a.x,
                           a.w, a.grad_proj, a.grad_r, a.r, a.dx, a.ws, a.addend, p.T, p.K, p.L);
    else
        hipLaunchKernelGGL((projection_mfma<kWavesPerGroup, false>), grid, block, 0, stream, a.x,
                           a.w, a.grad_proj, a.grad_r, a.r, a.dx, a.ws, a.addend, p.T, p.K, p.L);
    return hipGetLastError();
}

hipError_t launch_reduce(const Plan &p, const Args &a, hipStream_t stream) {
    const int64_t n4 = kProjCols * p.K / 4;
    const unsigned blocks = static_cast<unsigned>((n4 + 255) / 256);
    hipLaunchKernelGGL(reduce_slabs, dim3(blocks), dim3(256), 0, stream, a.ws, a.dw, p.S, n4);
    return hipGetLastError();
}

}  // namespace mhcpb
