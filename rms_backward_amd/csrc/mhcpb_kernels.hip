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
// TF32 product accumulated in FP32.  Each MFMA k slot pairs one part of one
// operand with one part of the other: for dX the W side is held in registers
// as packed (hi, lo) pairs and the P side is staged in LDS with each part
// repeated, 4 MFMAs per 16x16 output block (24 j padded to 32); for dW the X
// side is split in registers and the P side is staged per part, 4 MFMAs per
// column group.  No operand needs a per-step shuffle.
//
// X is streamed from HBM straight into LDS with buffer_load_dwordx4 ... lds,
// a ring of D steps per wave, so prefetching costs no registers; rows past
// the slab end fall outside the buffer range and arrive as zeros.  The P rows
// of each step arrive the same way a few steps ahead.
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

// Upper halves of two 32-bit words: (a >> 16) | (b & 0xFFFF0000).
__device__ __forceinline__ uint32_t hi_halves(uint32_t a, uint32_t b) {
    return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// Buffer resource over [base, base + bytes) with bytes in [0, 2^31).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc32(const void *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, kRsrcWord3);
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

__device__ __forceinline__ float lds_read_f32(uint32_t addr) {
    float v;
    asm volatile("ds_read_b32 %0, %1" : "=v"(v) : "v"(addr));
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

__device__ __forceinline__ void lds_write_u128(uint32_t addr, u32x4 v) {
    asm volatile("ds_write_b128 %0, %1" ::"v"(addr), "v"(v) : "memory");
}

__device__ __forceinline__ void lds_write_u16(uint32_t addr, uint32_t v) {
    asm volatile("ds_write_b16 %0, %1" ::"v"(addr), "v"(v) : "memory");
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

// Rows per step (one MFMA row block) and the LDS layouts of P.
constexpr int kStepRows = 16;
constexpr int kJPad = 32;                 // j slots per part, 24..31 zero
constexpr int kPaStride = 2 * kJPad + 4;  // uint32 per row of the dX P operand
constexpr int kPbStride = kStepRows + 4;  // uint16 per (part, j) row of the dW P operand

// The P of one step as it is stored in HBM, copied by LDS DMA: 16 rows of
// grad_proj (32 floats each; the last 8 are never read from here), and one
// grad_r and r entry per DMA lane (only the first 16 are used).
struct RawStep {
    f32x4 p[kStepRows * kProjStride / 4];
    float gr[kWave];
    float r[kWave];
};

// The P of one step in operand form (TF32 split into BF16 high and low parts):
//  pa[row][part * 32 + j]: the part, duplicated in both halves of the word, as
//      the dX product reads it (4 consecutive j per lane group);
//  pb[part][j][row]: the part, as the dW product reads it (4 consecutive rows);
//  c[row]: grad_r / (r K).
// Entries with j >= 24 are zero and never written after the first clear.
struct StepP {
    uint32_t pa[kStepRows * kPaStride];
    uint16_t pb[2 * kJPad * kPbStride];
    float c[kStepRows];
};

// Kernel 1.  A workgroup of NW waves owns NW * 64 columns of one slab.  Per
// step a wave handles 16 rows x 64 columns: lane l (c = l % 16, g = l / 16)
// holds x[t0 + 4g + r][kw + 4c + i] for r, i in 0..3.
//  dX: C_i[e] = dX[t0 + 4g + e][kw + 4c + i] = c_t x + the products of the P
//      parts (token t0 + l%16) with the W parts (column kw + 4c + i): per
//      MFMA (P part p, j block b) lane group g covers j = 16b + 4g .. +3 times
//      (W hi, W lo); 4 MFMAs cover the 96 products of 24 j (8 padded).
//  dW: acc[i][b][e] = sum over tokens of TF32(x) of column kw + 4(4g+e) + i
//      times TF32(P[j]), j = 16 b + l%16: per MFMA (P part p), lane group g
//      covers rows 4g .. 4g+3 times (x hi, x lo).
//
// Memory pipeline.  Each wave streams its X through a ring of D steps in LDS
// (the DMA for step j + D - 1 is issued as soon as step j has arrived).  The
// P of step k is copied raw into LDS by waves 0..3 (one DMA instruction each)
// during step k - D - 1, converted to operand form by waves 0 and 1 at the
// end of step k - 1, and published by the workgroup barrier that ends that
// step.  Nothing waits for a load issued in the same step.
//
// Minimum waves per SIMD the register allocation must allow: two 5-wave
// workgroups per CU need 3 (at most 168 VGPRs); with 4-wave workgroups two
// per CU need 2.
constexpr int waves_per_eu(int nw) { return nw == 5 ? 3 : 2; }

template <int NW, int D, bool kAddend>
__global__ __launch_bounds__(NW * kWave)
__attribute__((amdgpu_waves_per_eu(waves_per_eu(NW)))) void projection_kernel(
    const float *__restrict__ x, const float *__restrict__ w,
    const float *__restrict__ grad_proj, const float *__restrict__ grad_r,
    const float *__restrict__ r, uint16_t *__restrict__ dx, float *__restrict__ ws,
    const uint16_t *__restrict__ addend, int64_t T, int64_t K, int64_t L) {
    static_assert(NW >= 4, "waves 0..3 copy P");
    static_assert(D >= 2 && D <= 3, "ring depth");
    constexpr int R = D + 1;  // raw P buffers; the P of step k is requested in step k - R
    __shared__ f32x4 xring[NW][D][4][kWave];
    __shared__ RawStep praw[R];
    __shared__ StepP pop[2];
    constexpr int kThreads = NW * kWave;
    constexpr int kConvItems = kStepRows * (kProjCols / 4);  // float4 of P per step
    static_assert(kConvItems + kStepRows <= kThreads, "one conversion item per thread");
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
    const int slab_rows = static_cast<int>(row1 - row0);  // <= L < 2^31
    const int nsteps = (slab_rows + kStepRows - 1) / kStepRows;
    const float kf = static_cast<float>(K);
    const int ki = static_cast<int>(K);    // K <= 2^22
    const int kwi = static_cast<int>(kw);  // kw < K + NW * 64

    // VMEM instructions issued after the X DMA of step j and before the wait
    // for it, in steady state.  Each step issues, in this order: [4 addend
    // loads] [1 P DMA, waves 0..3] 4 X DMA (for step j + D - 1), 4 dX stores.
    // The DMA of step j is issued in step j - D + 1; after it come that
    // step's 4 stores and the D - 2 full steps in between.
    const bool copies_p = wave < 4;
    auto wait_x = [&](int j) {
        if (j < D - 1) {
            wait_vmcnt<0>();
        } else if constexpr (D == 2) {
            wait_vmcnt<4>();
        } else {
            constexpr int kBase = 4 + (D - 2) * (8 + (kAddend ? 4 : 0));
            if (copies_p)
                wait_vmcnt<kBase + (D - 2)>();
            else
                wait_vmcnt<kBase>();
        }
    };

    // Per-lane byte offsets inside one row group of a step (row 4g, columns
    // 4c..4c+3); inactive columns get an offset outside every range, so their
    // loads read zeros and their stores are dropped.  Row r = 0..3 of the
    // group is addressed through a buffer resource of its own, based at row
    // t0 + r and column kw, whose range ends at the slab end or 16 rows on
    // (whichever comes first): every access of the step lies within 13 rows,
    // and a row past the slab end lies outside the range.  The per-lane
    // offset is the same for all four rows; the hardware range check covers
    // it (the scalar offset, which is not checked, stays zero).
    const uint32_t xoff = active ? static_cast<uint32_t>((4 * g * K + 4 * c16) * 4) : kOutOfRange;
    const uint32_t doff = active ? static_cast<uint32_t>((4 * g * K + 4 * c16) * 2) : kOutOfRange;
    // Byte range of a row resource: rows_left rows of the slab remain from
    // its base row on.  Scalar arithmetic only (readfirstlane marks the
    // result uniform).
    auto range_bytes = [&](int rows_left, int elem_bytes) {
        const int rl = rows_left < 0 ? 0 : (rows_left > kStepRows ? kStepRows : rows_left);
        const int n = rl * ki - kwi;
        return __builtin_amdgcn_readfirstlane(n > 0 ? n * elem_bytes : 0);
    };
    auto step_rows = [&](int rows_left) {
        return __builtin_amdgcn_readfirstlane(
            rows_left < 0 ? 0 : (rows_left > kStepRows ? kStepRows : rows_left));
    };
    const int64_t row_bytes_x = K * 4;   // one row of X
    const int64_t row_bytes_d = K * 2;   // one row of dX or the addend

    // ---- X ring: step j's 16 rows go to stage j % D of this wave's ring.
    // xs points at row 0, column kw of the step; rows_left counts the slab
    // rows from there on.
    const uint32_t ring_base =
        static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&xring[wave][0][0][0]));
    auto issue_x = [&](const char *xs, int rows_left, int stage) {
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const __amdgpu_buffer_rsrc_t xrs =
                make_rsrc32(xs + rr * row_bytes_x, range_bytes(rows_left - rr, 4));
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                xrs, (MHCPB_LDS void *)(&xring[wave][stage][rr][0]), 16, xoff, 0, 0, MHCPB_X_AUX);
        }
    };

    // ---- raw P of step k into praw[k % R]: waves 0 and 1 copy rows 0..7 and
    // 8..15 of grad_proj (16 bytes per lane), waves 2 and 3 grad_r and r (4
    // bytes per lane).  Rows past the slab end read as zeros.  src is this
    // wave's source at row 0 of the step (grad_proj, grad_r or r).
    const int64_t p_step_bytes = (wave < 2) ? kStepRows * kProjStride * 4 : kStepRows * 4;
    const char *p_src = (wave < 2) ? reinterpret_cast<const char *>(grad_proj + row0 * kProjStride)
                                   : reinterpret_cast<const char *>((wave == 2 ? grad_r : r) + row0);
    auto issue_p = [&](const char *src, int rows_left, int k) {
        const int rl = step_rows(rows_left);
        RawStep &dst = praw[k % R];
        if (wave < 2) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                make_rsrc32(src, rl * kProjStride * 4), (MHCPB_LDS void *)(&dst.p[wave * kWave]), 16,
                static_cast<uint32_t>((wave * kWave + lane) * 16), 0, 0, 0);
        } else if (wave < 4) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                make_rsrc32(src, rl * 4), (MHCPB_LDS void *)(wave == 2 ? dst.gr : dst.r), 4,
                static_cast<uint32_t>(lane * 4), 0, 0, 0);
        }
    };

    // ---- operand form of the P of step k, from praw[k % R] into pop[k & 1]:
    // threads 0..95 split one float4 of P each, threads 96..111 compute the
    // RMS coefficient grad_r / (r K) of one row in FP32 (zero past the slab).
    auto convert = [&](int k) {
        const RawStep &src = praw[k % R];
        const StepP &d = pop[k & 1];
        if (tid < kConvItems) {
            const int rr = tid / (kProjCols / 4);
            const int q = tid % (kProjCols / 4);
            f32x4 v = lds_read_b128(lds_addr(&src.p[rr * (kProjStride / 4) + q]));
            asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(v)::"memory");
            uint32_t hi[4], lo[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const uint32_t pk = tf32_split_packed(v[e]);
                hi[e] = pk & 0xFFFFu;
                lo[e] = pk >> 16;
                const int j = 4 * q + e;
                lds_write_u16(lds_addr(d.pb + (0 * kJPad + j) * kPbStride + rr), hi[e]);
                lds_write_u16(lds_addr(d.pb + (1 * kJPad + j) * kPbStride + rr), lo[e]);
            }
            const uint32_t dst = lds_addr(d.pa + rr * kPaStride + 4 * q);
            lds_write_u128(dst, u32x4{hi[0] * 0x10001u, hi[1] * 0x10001u, hi[2] * 0x10001u,
                                      hi[3] * 0x10001u});
            lds_write_u128(dst + kJPad * 4, u32x4{lo[0] * 0x10001u, lo[1] * 0x10001u,
                                                  lo[2] * 0x10001u, lo[3] * 0x10001u});
        } else if (tid < kConvItems + kStepRows) {
            const int rr = tid - kConvItems;
            float grv = lds_read_f32(lds_addr(&src.gr[rr]));
            float rv = lds_read_f32(lds_addr(&src.r[rr]));
            asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(grv), "+v"(rv)::"memory");
            const bool in_slab = kStepRows * k + rr < slab_rows;
            lds_write_u32(lds_addr(d.c + rr), __float_as_uint(in_slab ? grv / (rv * kf) : 0.f));
        }
    };

    // The X of the first D - 1 steps and the P of the first R steps are
    // requested before anything else, so that their latency overlaps the W
    // loads below.
    const char *x_next = reinterpret_cast<const char *>(x + row0 * K + kw);
#pragma unroll
    for (int j = 0; j < D - 1; ++j) {
        issue_x(x_next, slab_rows - kStepRows * j, j);
        x_next += kStepRows * row_bytes_x;
    }
    const char *p_next = p_src;
#pragma unroll
    for (int k = 0; k < R; ++k) {
        issue_p(p_next, slab_rows - kStepRows * k, k);
        p_next += p_step_bytes;
    }

    // W side of the dX product: for column variant i and j block b the lane
    // holds the packed (hi | lo << 16) TF32 split of W[j][col + i] for
    // j = 16b + 4g .. 16b + 4g + 3 (zero for j >= 24).
    u32x4 bw[4][2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        float wv[4][4];  // [e][i]
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int j = 16 * b + 4 * g + e;
            float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
            if (active && j < kProjCols) v = *reinterpret_cast<const float4 *>(w + j * K + col);
            wv[e][0] = v.x;
            wv[e][1] = v.y;
            wv[e][2] = v.z;
            wv[e][3] = v.w;
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
            bw[i][b] = u32x4{tf32_split_packed(wv[0][i]), tf32_split_packed(wv[1][i]),
                             tf32_split_packed(wv[2][i]), tf32_split_packed(wv[3][i])};
    }

    f32x4 accw[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) accw[i][jb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // The j = 24..31 entries of both operand buffers are zero padding.
    constexpr int kPadJ = kJPad - kProjCols;
    for (int i = tid; i < 2 * kStepRows * 2 * kPadJ; i += kThreads) {
        const int buf = i / (kStepRows * 2 * kPadJ);
        const int k = i % (kStepRows * 2 * kPadJ);
        const int row = k / (2 * kPadJ), rest = k % (2 * kPadJ);
        const int part = rest / kPadJ, jj = kProjCols + rest % kPadJ;
        lds_write_u32(lds_addr(pop[buf].pa + row * kPaStride + part * kJPad + jj), 0u);
    }
    for (int i = tid; i < 2 * 2 * kPadJ * kPbStride; i += kThreads) {
        const int buf = i / (2 * kPadJ * kPbStride);
        const int k = i % (2 * kPadJ * kPbStride);
        const int part = k / (kPadJ * kPbStride);
        const int off = k % (kPadJ * kPbStride);
        lds_write_u16(lds_addr(pop[buf].pb + (part * kJPad + kProjCols) * kPbStride + off), 0u);
    }

    // Raw P of the first R steps in place and visible, then step 0 in
    // operand form.
    wait_vmcnt<0>();
    lds_barrier();
    convert(0);
    lds_barrier();

    char *d_cur = reinterpret_cast<char *>(dx + row0 * K + kw);
    const char *a_cur = reinterpret_cast<const char *>(addend + row0 * K + kw);
    for (int j = 0; j < nsteps; ++j) {
        const int rows_left = slab_rows - kStepRows * j;
        // Wait for this step's X, read it, then reuse the stage of the
        // previous step for the step D - 1 ahead.  Steps past the slab end
        // are still requested (they read zeros; their stores fall outside the
        // range), which keeps every step's VMEM count identical.
        wait_x(j);
        const StepP &cur = pop[j & 1];
        const uint32_t xa = ring_base + static_cast<uint32_t>((((j % D) * 4) * kWave + lane) * 16);
        // Every LDS operand of this step in one batch: X (4 rows), the RMS
        // coefficients of rows 4g..4g+3, the dX P operands (token c16, part
        // p, j = 16b + 4g .. +3) and the dW P operands (part p, j = 16b +
        // c16, rows 4g .. 4g+3; entries j >= 24 are zero).
        f32x4 xc[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) xc[rr] = lds_read_b128(xa + rr * kWave * 16);
        f32x4 cc = lds_read_b128(lds_addr(cur.c + 4 * g));
        u32x4 pa[2][2];  // [part][block]
        u32x2 pbv[2][2];
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                pa[p][b] = lds_read_u128(
                    lds_addr(cur.pa + c16 * kPaStride + p * kJPad + 16 * b + 4 * g));
                pbv[p][b] = lds_read_u64(
                    lds_addr(cur.pb + (p * kJPad + 16 * b + c16) * kPbStride + 4 * g));
            }
        // The wait names every register the reads above return, so no use
        // of them can be scheduled before the data has arrived.
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(xc[0]), "+v"(xc[1]), "+v"(xc[2]), "+v"(xc[3]), "+v"(cc),
                       "+v"(pa[0][0]), "+v"(pa[0][1]), "+v"(pa[1][0]), "+v"(pa[1][1]),
                       "+v"(pbv[0][0]), "+v"(pbv[0][1]), "+v"(pbv[1][0]), "+v"(pbv[1][1])::"memory");
        uint2 av[4];
        if constexpr (kAddend) {
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const __amdgpu_buffer_rsrc_t ars =
                    make_rsrc32(a_cur + rr * row_bytes_d, range_bytes(rows_left - rr, 2));
                const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(ars, doff, 0, 0);
                av[rr] = make_uint2(v.x, v.y);
            }
            a_cur += kStepRows * row_bytes_d;
        }
        compiler_fence();
        issue_p(p_next, rows_left - kStepRows * R, j + R);
        issue_x(x_next, rows_left - kStepRows * (D - 1), (j + D - 1) % D);
        p_next += p_step_bytes;
        x_next += kStepRows * row_bytes_x;
        compiler_fence();

        const float ce[4] = {cc[0], cc[1], cc[2], cc[3]};
        u32x4 pb[2][2];
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
            for (int b = 0; b < 2; ++b)
                pb[p][b] = u32x4{pbv[p][b].x, pbv[p][b].y, pbv[p][b].x, pbv[p][b].y};

        uint32_t packed[4][2];  // dX of row 4g + r, columns (0,1) and (2,3)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // dX for column variant i: the RMS term c_t * x in FP32, then
            // the 96 exact partial products.
            f32x4 acc = f32x4{ce[0] * xc[0][i], ce[1] * xc[1][i], ce[2] * xc[2][i],
                              ce[3] * xc[3][i]};
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int p = 0; p < 2; ++p) acc = mfma(pa[p][b], bw[i][b], acc);

            // dW: x of column variant i split into BF16 hi/lo, packed
            // [hi r0..r3 | lo r0..r3], against each P part.
            uint32_t hb[4];
            float lo[4];
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) tf32_split(xc[rr][i], hb[rr], lo[rr]);
            const u32x4 ax = u32x4{hi_halves(hb[0], hb[1]), hi_halves(hb[2], hb[3]),
                                   hi_halves(__float_as_uint(lo[0]), __float_as_uint(lo[1])),
                                   hi_halves(__float_as_uint(lo[2]), __float_as_uint(lo[3]))};
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int p = 0; p < 2; ++p) accw[i][b] = mfma(ax, pb[p][b], accw[i][b]);

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
        // One rounding to BF16 per element (above), then 8-byte range-checked
        // stores: rows past the slab end are dropped.
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) {
            const __amdgpu_buffer_rsrc_t drs =
                make_rsrc32(d_cur + rr * row_bytes_d, range_bytes(rows_left - rr, 2));
            __builtin_amdgcn_raw_buffer_store_b64(u32x2{packed[rr][0], packed[rr][1]}, drs, doff,
                                                  0, MHCPB_DX_AUX);
        }
        d_cur += kStepRows * row_bytes_d;
        convert(j + 1);
        lds_barrier();
    }
    // Drain the DMA still in flight (steps past the slab end) before the
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
// splits the grid is several rounds anyway and 4-wave workgroups (two per CU,
// two waves per SIMD) stream better.
hipError_t launch_projection(const Plan &p, const Args &a, hipStream_t stream) {
    if (p.S <= 8) return launch_projection_t<5, 2>(p, a, stream);
    return launch_projection_t<4, 2>(p, a, stream);
}

hipError_t launch_reduce(const Plan &p, const Args &a, hipStream_t stream) {
    const int64_t n4 = kProjCols * p.K / 4;
    const unsigned blocks = static_cast<unsigned>((n4 + 255) / 256);
    hipLaunchKernelGGL(reduce_slabs, dim3(blocks), dim3(256), 0, stream, a.ws, a.dw, p.S, n4);
    return hipGetLastError();
}

}  // namespace mhcpb
