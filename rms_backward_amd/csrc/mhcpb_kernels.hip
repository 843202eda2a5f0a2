// Kernels of the DSv4.1 mHC projection/RMS backward for gfx950.
//
// Kernel 1 ("projection"): the grid is (column tiles) x (S slabs of T).  Each
// workgroup owns one slab of rows and one tile of columns, reads its rows of X
// exactly once, writes the matching dX, and keeps its dW[24, tile] partial in
// MFMA accumulators; the partial goes to workspace slab s (one writer per
// element).  Kernel 2 ("reduce"): dW = ((slab 0 + slab 1) + slab 2) + ... in
// FP32.  This follows the page's structure (the token reduction split over
// independent blocks, partial weight gradients, then a second reduction
// kernel: "Source attribution" section) with a split count that depends on T
// only.
//
// Both products run on v_mfma_f32_16x16x32_bf16.  A TF32 operand has 11
// significant bits; it splits exactly into a BF16 high part (its upper 16
// bits) and a BF16 low part (the remaining 3 bits), so the four BF16 partial
// products hi*hi, hi*lo, lo*hi, lo*lo are exact and their FP32 sum is the
// TF32 product accumulated in FP32.  96 such products per dX element (24 j x
// 4) fill exactly three 32-deep MFMAs; for dW the 48 (j, part) products of
// the P side fill three 16-wide MFMA column blocks.
//
// X is streamed from HBM straight into LDS with buffer_load_dwordx4 ... lds,
// a ring of D steps per wave, so prefetching costs no registers; rows past
// the slab end fall outside the buffer range and arrive as zeros.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "mhcpb_internal.h"

namespace mhcpb {
namespace {

#define MHCPB_LDS __attribute__((address_space(3)))

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
// Fourth word of a raw buffer resource on gfx9-class GPUs (32-bit data format).
constexpr int kRsrcWord3 = 0x00020000;
// Offsets at or above this are outside every buffer range used here.
constexpr uint32_t kOutOfRange = 0x80000000u;
constexpr int64_t kMaxRecords = 0x7FFFFFF0;
// Cache policy of the X stream (read once): non-temporal ("nt" on gfx950).
#ifndef MHCPB_X_AUX
#define MHCPB_X_AUX 2
#endif
// Cache policy of the dX stores (written once, read by a later stage):
// non-temporal as well.
#ifndef MHCPB_DX_AUX
#define MHCPB_DX_AUX 2
#endif

// Two FP32 values to two BF16 (round to nearest even) packed low-first; one
// v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

__device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                   __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// TF32 rounding on the bits (nearest even at 10 fraction bits, the carry
// running into the exponent), then the exact split of the TF32 value into a
// BF16 high part (its upper 16 bits) and a low part whose upper 16 bits are
// its exact BF16 value.  hi + lo == TF32(v).
__device__ __forceinline__ void tf32_split(float v, uint32_t &hi_bits, float &lo) {
    uint32_t u = __float_as_uint(v);
    uint32_t t = (u + 0xFFFu + ((u >> 13) & 1u)) & 0xFFFFE000u;
    uint32_t h = t & 0xFFFF0000u;
    hi_bits = h;
    lo = __uint_as_float(t) - __uint_as_float(h);
}

// The same split for the small operands (P, W) packed as hi | lo << 16, with
// non-finite inputs kept non-finite in the high part and a zero low part.
__device__ __forceinline__ uint32_t tf32_split_packed(float v) {
    const uint32_t u = __float_as_uint(v);
    uint32_t hb;
    float lo;
    tf32_split(v, hb, lo);
    const uint32_t finite = (hb >> 16) | (__float_as_uint(lo) & 0xFFFF0000u);
    const uint32_t quiet = ((u & 0x007FFFFFu) ? (u | 0x00400000u) : u) >> 16;
    return ((u & 0x7F800000u) == 0x7F800000u) ? quiet : finite;
}

// v_perm_b32 that stays where it is written: the W operands are rebuilt
// inside the loop on purpose, and a plain builtin would be hoisted out of it
// (keeping all expanded operands live and spilling).
__device__ __forceinline__ uint32_t perm_in_place(uint32_t v, uint32_t sel) {
    uint32_t r;
    asm volatile("v_perm_b32 %0, %1, %1, %2" : "=v"(r) : "v"(v), "s"(sel));
    return r;
}

// [lo0 lo0 lo1 lo1 hi0 hi0 hi1 hi1] from (lo0 | hi0 << 16, lo1 | hi1 << 16).
__device__ __forceinline__ u32x4 dup_halves(u32x2 p) {
    return u32x4{perm_in_place(p.x, 0x01000100u), perm_in_place(p.y, 0x01000100u),
                 perm_in_place(p.x, 0x03020302u), perm_in_place(p.y, 0x03020302u)};
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes) {
    const int64_t n = bytes <= 0 ? 0 : (bytes > kMaxRecords ? kMaxRecords : bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, static_cast<int>(n),
                                             kRsrcWord3);
}

// LDS reads the compiler does not track.  X in LDS was written by LDS DMA,
// whose completion the caller establishes with an explicit vmcnt wait; the
// compiler cannot see that, and would otherwise wait for every outstanding
// global load before any LDS read it cannot prove independent of the DMA.
// All hot-loop LDS reads therefore go through these, followed by one
// explicit lgkmcnt wait.
__device__ __forceinline__ f32x4 lds_read_b128(uint32_t addr) {
    f32x4 v;
    asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr));
    return v;
}

__device__ __forceinline__ u32x4 lds_read_u128(uint32_t addr) {
    u32x4 v;
    asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(addr));
    return v;
}

__device__ __forceinline__ u32x2 lds_read_u64(uint32_t addr) {
    u32x2 v;
    asm volatile("ds_read_b64 %0, %1" : "=v"(v) : "v"(addr));
    return v;
}

// LDS writes of the P staging, equally hidden from the compiler's LDS-DMA
// ordering (they never touch the X ring); completed by lds_barrier().
__device__ __forceinline__ void lds_write_u32(uint32_t addr, uint32_t v) {
    asm volatile("ds_write_b32 %0, %1" ::"v"(addr), "v"(v) : "memory");
}

__device__ __forceinline__ void lds_write_u64(uint32_t addr, u32x2 v) {
    asm volatile("ds_write_b64 %0, %1" ::"v"(addr), "v"(v) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const void *p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Keeps the compiler from moving memory instructions across this point, so
// the per-step VMEM order that the vmcnt waits count on is the program order.
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

// Barrier for LDS data only (no wait on outstanding global traffic).
__device__ __forceinline__ void lds_barrier() {
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// P rows staged per chunk, and LDS strides (padded against bank conflicts).
constexpr int kChunk = 32;
constexpr int kStepsPerChunk = kChunk / 16;
constexpr int kPsStride = 26;          // uint32 per row of packed (hi | lo << 16) P
constexpr int kPtStride = kChunk + 4;  // uint32 per j row of transposed packed P

struct ChunkLds {
    uint32_t ps[kChunk * kPsStride];  // [row][j]: hi | lo << 16
    uint32_t pt[32 * kPtStride];  // [j][row]: hi | lo << 16; rows 24..31 stay zero
    float c[kChunk];                  // grad_r / (r K)
};

// Kernel 1.  A workgroup of NW waves owns NW * 64 columns of one slab.  Per
// step a wave handles 16 rows x 64 columns: lane l (c = l % 16, g = l / 16)
// holds x[t0 + 4g + r][kw + 4c + i] for r, i in 0..3.
//  dX: C_i[e] = dX[t0 + 4g + e][kw + 4c + i] = c_t x + sum over 96 slots of
//      (P hi|lo of token t0 + l%16) x (W hi|lo of column kw + 4c + i).
//  dW: acc[i][jb][e] = sum over tokens of TF32(x) of column kw + 4(4g+e) + i
//      times TF32(P[j]), j = 16 jb + l%16: per MFMA, each lane group g holds
//      two tokens x (x hi, x lo) x (P hi, P lo) = 8 exact partial products.
// D is the depth of the per-wave LDS ring of X steps.
// Minimum waves per SIMD the register allocation must allow.  With 4-wave
// workgroups and a 3-deep ring the LDS (81 KB per workgroup) already limits a
// CU to 2 workgroups, i.e. 2 waves per SIMD.
// Minimum waves per SIMD the register allocation must allow: two 5-wave
// workgroups per CU need 3 (at most 168 VGPRs); with 4-wave workgroups the
// LDS already limits a CU to two workgroups, i.e. 2 waves per SIMD.
constexpr int waves_per_eu(int nw) { return nw == 5 ? 3 : 2; }

template <int NW, int D, bool kAddend>
__global__ __launch_bounds__(NW * kWave)
__attribute__((amdgpu_waves_per_eu(waves_per_eu(NW)))) void projection_kernel(
    const float *__restrict__ x, const float *__restrict__ w,
    const float *__restrict__ grad_proj, const float *__restrict__ grad_r,
    const float *__restrict__ r, uint16_t *__restrict__ dx, float *__restrict__ ws,
    const uint16_t *__restrict__ addend, int64_t T, int64_t K, int64_t L) {
    static_assert(D >= 2 && D <= 4, "ring depth");
    __shared__ f32x4 xring[NW][D][4][kWave];
    __shared__ ChunkLds chunk[2];
    constexpr int kThreads = NW * kWave;
    constexpr int kItems = kChunk * (kProjCols / 4);  // float4 of P per chunk
    constexpr int kItemsPerThread = (kItems + kThreads - 1) / kThreads;
    // VMEM instructions issued after the X DMA of step j and before the wait
    // for it, in steady state.  Each step issues, in this order: [4 addend
    // loads] 4 DMA loads (for step + D - 1), 4 dX stores.  The DMA of step j
    // is issued in step j - D + 1; after it come that step's 4 stores and the
    // D - 2 full steps in between.  Other VMEM instructions (P staging) only
    // add to the count, which makes the wait stricter, never looser.
    constexpr int kAfter = 4 + (D - 2) * (8 + (kAddend ? 4 : 0));
    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int c16 = lane % 16;
    const int g = lane / 16;
    const int s = blockIdx.y;
    const int64_t kw = static_cast<int64_t>(blockIdx.x) * (NW * 64) + wave * 64;
    const int64_t col = kw + 4 * c16;  // first of this lane's 4 columns
    const bool active = col < K;
    const int64_t row0 = static_cast<int64_t>(s) * L;
    const int64_t row1 = (row0 + L < T) ? row0 + L : T;
    const float kf = static_cast<float>(K);

    // Per-lane byte offsets inside one step (rows 4g + r, columns 4c..4c+3);
    // inactive columns get an offset outside every range, so their loads read
    // zeros and their stores are dropped.
    const uint32_t xoff = active ? static_cast<uint32_t>((4 * g * K + 4 * c16) * 4) : kOutOfRange;
    const uint32_t doff = active ? static_cast<uint32_t>((4 * g * K + 4 * c16) * 2) : kOutOfRange;
    // Byte offsets of rows r = 0..3 of a step.  They go into the per-lane
    // (VGPR) offset, which the hardware range check covers; the scalar offset
    // is not range-checked and stays zero.
    uint32_t xoffr[4], doffr[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
        xoffr[rr] = xoff + static_cast<uint32_t>(rr * K * 4);
        doffr[rr] = doff + static_cast<uint32_t>(rr * K * 2);
    }

    // W side of the dX product, kept as unique halves: for column variant i
    // and MFMA u the lane holds (Wh_j | Wl_j << 16, Wh_j1 | Wl_j1 << 16),
    // j = 8u + 2g; the MFMA operand [Wh_j Wh_j Wh_j1 Wh_j1 Wl_j Wl_j Wl_j1
    // Wl_j1] is rebuilt from them with v_perm right before use.
    u32x2 bwu[4][3];
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
        for (int i = 0; i < 4; ++i) bwu[i][u] = u32x2{tf32_split_packed(a0[i]), tf32_split_packed(a1[i])};
    }

    f32x4 accw[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) accw[i][jb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // ---- P staging: rows [c0, c0 + kChunk) of the slab, loaded to registers
    // with range-checked buffer loads (rows past the slab read zeros) ...
    float4 pv[kItemsPerThread];
    float grv = 0.f, rv = 0.f;
    auto stage_load = [&](int64_t c0) {
        const int64_t rows_left = row1 - c0;
        const __amdgpu_buffer_rsrc_t prs =
            make_rsrc(grad_proj + c0 * kProjStride, rows_left * kProjStride * 4);
        // Every thread issues every load (threads past the item count read an
        // out-of-range offset, i.e. zeros): no divergent loads here.
#pragma unroll
        for (int it = 0; it < kItemsPerThread; ++it) {
            const int item = tid + it * kThreads;
            const int rr = item / (kProjCols / 4);
            const int q = item % (kProjCols / 4);
            const uint32_t off = item < kItems
                                     ? static_cast<uint32_t>((rr * kProjStride + 4 * q) * 4)
                                     : kOutOfRange;
            pv[it] = __builtin_bit_cast(float4, __builtin_amdgcn_raw_buffer_load_b128(prs, off, 0, 0));
        }
        const __amdgpu_buffer_rsrc_t grs = make_rsrc(grad_r + c0, rows_left * 4);
        const __amdgpu_buffer_rsrc_t rrs = make_rsrc(r + c0, rows_left * 4);
        const uint32_t toff = tid < kChunk ? static_cast<uint32_t>(tid * 4) : kOutOfRange;
        grv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(grs, toff, 0, 0));
        rv = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rrs, toff, 0, 0));
    };
    // ... then split and written in both LDS layouts, with the RMS
    // coefficient grad_r / (r K) in FP32 (zero for rows past the slab).
    auto stage_store = [&](const ChunkLds &d, int64_t c0) {
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
                    lds_write_u32(lds_addr(d.pt + (4 * q + e) * kPtStride + rr), pk[e]);
                }
                const uint32_t dst = lds_addr(d.ps + rr * kPsStride + 4 * q);
                lds_write_u64(dst, u32x2{pk[0], pk[1]});
                lds_write_u64(dst + 8, u32x2{pk[2], pk[3]});
            }
        }
        if (tid < kChunk)
            lds_write_u32(lds_addr(d.c + tid),
                          __float_as_uint((c0 + tid < row1) ? grv / (rv * kf) : 0.f));
    };

    // ---- X ring: step j's 16 rows go to stage j % D of this wave's ring.
    const uint32_t ring_base =
        static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&xring[wave][0][0][0]));
    auto issue_x = [&](int64_t t0, int stage) {
        const __amdgpu_buffer_rsrc_t xrs = make_rsrc(x + t0 * K + kw, ((row1 - t0) * K - kw) * 4);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                xrs, (MHCPB_LDS void *)(&xring[wave][stage][rr][0]), 16, xoffr[rr],
                0, 0, MHCPB_X_AUX);
    };

    // The dW operand rows j = 24..31 of both P buffers are zero padding.
    for (int i = tid; i < 2 * (32 - kProjCols) * kPtStride; i += kThreads) {
        const int buf = i / ((32 - kProjCols) * kPtStride);
        lds_write_u32(lds_addr(chunk[buf].pt + kProjCols * kPtStride +
                               i % ((32 - kProjCols) * kPtStride)),
                      0u);
    }

    const int64_t nchunks = (row1 - row0 + kChunk - 1) / kChunk;
    if (nchunks > 0) {
        stage_load(row0);
        stage_store(chunk[0], row0);
#pragma unroll
        for (int j = 0; j < D - 1; ++j) issue_x(row0 + 16 * j, j);
    }
    lds_barrier();

    int j = 0;  // step index within the slab
    for (int64_t ch = 0; ch < nchunks; ++ch) {
        const int64_t c0 = row0 + ch * kChunk;
        const ChunkLds &cur = chunk[ch & 1];
        // The next chunk's P rows (past the slab end they read as zeros and
        // are never used), loaded now and staged after this chunk's steps.
        stage_load(c0 + kChunk);
#pragma unroll
        for (int stl = 0; stl < kStepsPerChunk; ++stl, ++j) {
            // Steps are never skipped: in a ragged last chunk a step past the
            // slab reads zeros and its stores fall outside the range, which
            // keeps every step's VMEM count identical.
            const int64_t t0 = c0 + 16 * stl;
            // Wait for this step's X, read it, then reuse the stage of the
            // previous step for the step D - 1 ahead (always issued, so the
            // count of later VMEM instructions is the same every step).
            if (j < D - 1)
                wait_vmcnt<0>();
            else
                wait_vmcnt<kAfter>();
            const int stage = j % D;
            const uint32_t xa = ring_base + static_cast<uint32_t>(((stage * 4) * kWave + lane) * 16);
            // Every LDS operand of this step in one batch: X (4 rows), the RMS
            // coefficients of rows 4g..4g+3, the dX P operands (token c16,
            // j = 8u + 2g, j + 1) and the dW P operands (j = 16 jb + c16,
            // tokens 4g..4g+3; rows j >= 24 are zero).
            f32x4 xc[4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) xc[rr] = lds_read_b128(xa + rr * kWave * 16);
            f32x4 cc = lds_read_b128(lds_addr(cur.c + 16 * stl + 4 * g));
            u32x2 pav[3];
#pragma unroll
            for (int u = 0; u < 3; ++u)
                pav[u] = lds_read_u64(lds_addr(cur.ps + (16 * stl + c16) * kPsStride + 8 * u + 2 * g));
            u32x4 pbv[2];
#pragma unroll
            for (int jb = 0; jb < 2; ++jb)
                pbv[jb] = lds_read_u128(lds_addr(cur.pt + (16 * jb + c16) * kPtStride + 16 * stl + 4 * g));
            // The wait names every register the reads above return, so no use
            // of them can be scheduled before the data has arrived.
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(xc[0]), "+v"(xc[1]), "+v"(xc[2]), "+v"(xc[3]), "+v"(cc), "+v"(pav[0]),
                           "+v"(pav[1]), "+v"(pav[2]), "+v"(pbv[0]), "+v"(pbv[1])::"memory");
            uint2 av[4];
            const __amdgpu_buffer_rsrc_t drs = make_rsrc(dx + t0 * K + kw, ((row1 - t0) * K - kw) * 2);
            if constexpr (kAddend) {
                const __amdgpu_buffer_rsrc_t ars =
                    make_rsrc(addend + t0 * K + kw, ((row1 - t0) * K - kw) * 2);
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(ars, doffr[rr], 0, 0);
                    av[rr] = make_uint2(v.x, v.y);
                }
            }
            compiler_fence();
            issue_x(t0 + 16 * (D - 1), (j + D - 1) % D);
            compiler_fence();

            const float ce[4] = {cc[0], cc[1], cc[2], cc[3]};
            u32x4 pa[3], pb[2][2];
#pragma unroll
            for (int u = 0; u < 3; ++u) pa[u] = u32x4{pav[u].x, pav[u].y, pav[u].x, pav[u].y};
#pragma unroll
            for (int jb = 0; jb < 2; ++jb) {
                pb[jb][0] = u32x4{pbv[jb].x, pbv[jb].x, pbv[jb].y, pbv[jb].y};
                pb[jb][1] = u32x4{pbv[jb].z, pbv[jb].z, pbv[jb].w, pbv[jb].w};
            }

            uint32_t packed[4][2];  // dX of row 4g + r, columns (0,1) and (2,3)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                // dX for column variant i: the RMS term c_t * x in FP32, then
                // the 96 exact partial products.
                f32x4 acc = f32x4{ce[0] * xc[0][i], ce[1] * xc[1][i], ce[2] * xc[2][i],
                                  ce[3] * xc[3][i]};
#pragma unroll
                for (int u = 0; u < 3; ++u) acc = mfma(pa[u], dup_halves(bwu[i][u]), acc);

                // dW: x of column variant i split into BF16 hi/lo; for token
                // pair h the operand is [xh_a xh_a xl_a xl_a xh_b xh_b xl_b xl_b].
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    uint32_t ha, hb2;
                    float la, lb;
                    tf32_split(xc[2 * h][i], ha, la);
                    tf32_split(xc[2 * h + 1][i], hb2, lb);
                    const u32x4 ax = u32x4{
                        __builtin_amdgcn_perm(ha, ha, 0x07060706u),
                        __builtin_amdgcn_perm(__float_as_uint(la), __float_as_uint(la), 0x07060706u),
                        __builtin_amdgcn_perm(hb2, hb2, 0x07060706u),
                        __builtin_amdgcn_perm(__float_as_uint(lb), __float_as_uint(lb), 0x07060706u)};
#pragma unroll
                    for (int jb = 0; jb < 2; ++jb) accw[i][jb] = mfma(ax, pb[jb][h], accw[i][jb]);
                }

#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    float d = acc[rr];
                    if constexpr (kAddend) {
                        const uint32_t word = (i < 2) ? av[rr].x : av[rr].y;
                        d += bf16_to_f32((i & 1) ? (word >> 16) : (word & 0xFFFFu));
                    }
                    if (i & 1)
                        packed[rr][i >> 1] = pack_bf16x2(__uint_as_float(packed[rr][i >> 1]), d);
                    else
                        packed[rr][i >> 1] = __float_as_uint(d);
                }
            }
            // One rounding to BF16 per element (above), then 8-byte
            // range-checked stores: rows past the slab end are dropped.
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                __builtin_amdgcn_raw_buffer_store_b64(u32x2{packed[rr][0], packed[rr][1]}, drs,
                                                      doffr[rr], 0, MHCPB_DX_AUX);
        }
        stage_store(chunk[(ch + 1) & 1], c0 + kChunk);
        lds_barrier();
    }
    // Drain the X DMA still in flight (steps past the slab end) before the
    // workgroup's LDS can be released.
    wait_vmcnt<0>();

    // Partial dW of this slab, written once to workspace slab s.  Lane
    // (c16, g), element e of block jb is column kw + 16 g + 4 e + i of
    // j = 16 jb + c16.
    float *slab = ws + static_cast<int64_t>(s) * kProjCols * K;
    const int64_t cbase = kw + 16 * g;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int64_t cc = cbase + 4 * e;
        if (cc < K) {
            *reinterpret_cast<float4 *>(slab + c16 * K + cc) =
                make_float4(accw[0][0][e], accw[1][0][e], accw[2][0][e], accw[3][0][e]);
            if (c16 < kProjCols - 16)
                *reinterpret_cast<float4 *>(slab + (16 + c16) * K + cc) =
                    make_float4(accw[0][1][e], accw[1][1][e], accw[2][1][e], accw[3][1][e]);
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

template <int NW, int D>
hipError_t launch_projection_t(const Plan &p, const Args &a, hipStream_t stream) {
    constexpr int cols = NW * 64;
    const dim3 grid(static_cast<unsigned>((p.K + cols - 1) / cols), static_cast<unsigned>(p.S));
    const dim3 block(NW * kWave);
    if (a.addend)
        hipLaunchKernelGGL((projection_kernel<NW, D, true>), grid, block, 0, stream, a.x, a.w,
                           a.grad_proj, a.grad_r, a.r, a.dx, a.ws, a.addend, p.T, p.K, p.L);
    else
        hipLaunchKernelGGL((projection_kernel<NW, D, false>), grid, block, 0, stream, a.x, a.w,
                           a.grad_proj, a.grad_r, a.r, a.dx, a.ws, a.addend, p.T, p.K, p.L);
    return hipGetLastError();
}

}  // namespace

// Launch shape, a performance choice only: each column's dW is summed in the
// same order whatever the workgroup width, so every shape gives the same bits.
// With 8 or fewer splits a 5-wave workgroup (320 columns) makes the grid one
// full round of two workgroups per CU at K = 20480 on 256 CUs; with more
// splits the grid is several rounds anyway and 4-wave workgroups stream
// better.
hipError_t launch_projection(const Plan &p, const Args &a, hipStream_t stream) {
    if (p.S <= 8) return launch_projection_t<5, 3>(p, a, stream);
    return launch_projection_t<4, 3>(p, a, stream);
}

hipError_t launch_reduce(const Plan &p, const Args &a, hipStream_t stream) {
    const int64_t n4 = kProjCols * p.K / 4;
    const unsigned blocks = static_cast<unsigned>((n4 + 255) / 256);
    hipLaunchKernelGGL(reduce_slabs, dim3(blocks), dim3(256), 0, stream, a.ws, a.dw, p.S, n4);
    return hipGetLastError();
}

}  // namespace mhcpb
