// Kernels of the mHC projection forward for gfx950: the 24 gate logits
// proj[t, j] = sum_k TF32(X[t, k]) TF32(W[j, k]) (FP32 accumulation) and the
// row RMS r[t] = sqrt(sum_k X[t, k]^2 / K + eps) in FP32, in one read of X.
// This is the map whose gradient the backward kernels compute (the backward
// page, "DSv4.1 mHC projection/RMS backward", takes r "from forward"; the
// prime-kernels pull request 15 page lists the RMS and the gate logits of the
// streams as one pass, "mhc_projection").
//
// Kernel "split_weight": W [24, K] FP32 -> the high part of TF32(W) (its
// upper 16 bits) and the exact low part as BF16, laid out in the order the
// main kernel's lanes load them, so that it spends no arithmetic on W and
// reads it in whole cache lines.  It takes the caller's workspace, zero past
// K up to a whole number of 64-column chunks.
//
// Kernel "forward_kernel": one workgroup per 16 tokens.  Its NW waves split
// the K columns into 64-column chunks (wave w takes chunks w, w + NW, ...),
// so each wave walks the whole row block once and keeps the 16 x 24 logits
// of its columns in MFMA accumulators; at the end the waves' partial sums are
// added in wave order through LDS.  The order of every sum depends on K and
// NW only, so a row's result does not depend on T or on the other rows.
//
// Products.  TF32(x) = xh + xl exactly, with xh the upper 16 bits of the TF32
// value and xl the (at most 3-bit) remainder, both BF16; likewise for W.  On
// v_mfma_f32_16x16x32_bf16 (A = 16 tokens x 32 columns, B = 32 columns x 16
// gates) lane l supplies token / gate l % 16 and columns 8 (l / 16) .. +7 of a
// 32-column group.  Gates 0..15 take four MFMAs per group (xh wh, xh wl, xl
// wh, xl wl); gates 16..23 take two, with B lanes 0..7 holding wh and lanes
// 8..15 wl of the same gates, so their logits are the sum of two accumulator
// columns at the end.  Every BF16 product is exact and the MFMA adds in FP32.
//
// Memory.  X streams from HBM into a three-stage LDS ring per wave by LDS DMA
// (buffer_load_dwordx4 ... lds, non-temporal), two chunks ahead of the one
// being computed, at no register cost.  One DMA instruction moves 8 rows x 128
// contiguous bytes; the 16-byte segments of a row are XOR-swizzled so that the
// A-operand reads (16 tokens at one segment) hit 16 different bank groups.
// W (read by every workgroup, L2-resident) is stored by split_weight in the
// order of the MFMA operands, so each W load of a wave is 1 KB of
// consecutive bytes, and is loaded into registers one chunk ahead.  Rows past T
// fall outside the X buffer range, the columns past K of a ragged last chunk
// take offsets outside it, and both read as zeros.
#include "mhcpb_device.h"
#include "mhcpb_internal.h"

namespace mhcpb {
namespace {

constexpr int kFwdRows = 16;    // tokens per workgroup
constexpr int kFwdChunk = 64;   // columns per step
constexpr int kFwdDma = 4;      // LDS DMA instructions per step (16 rows x 256 bytes)
constexpr int kFwdWLoads = 6;   // 16-byte W loads per lane per step

// Cache policy of the X stream (read once): non-temporal.
#ifndef MHCPB_FWD_X_AUX
#define MHCPB_FWD_X_AUX 2
#endif

// TF32 value of v as bits: nearest even at 10 fraction bits, the carry
// running into the exponent.  A NaN whose top fraction bits are all ones can
// carry out of the exponent here; the caller repairs such rows afterwards
// (their RMS is NaN).
__device__ __forceinline__ uint32_t tf32_bits(float v) {
    const uint32_t u = __float_as_uint(v);
    return (u + 0xFFFu + ((u >> 13) & 1u)) & 0xFFFFE000u;
}

// The four words of a raw buffer resource over [base, base + bytes).
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 rsrc_words(const void *base, int bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    return i32x4{__builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(a))),
                 __builtin_amdgcn_readfirstlane(static_cast<int>((a >> 32) & 0xFFFFu)),
                 __builtin_amdgcn_readfirstlane(bytes), kRsrcWord3};
}

// A 16-byte buffer load that the compiler does not track.  Its caller waits
// for it with an asm wait that names the destination register, in the same
// basic block: between the two the register holds no value the compiler
// knows of, and nothing may copy it.  (A tracked load would make the compiler
// insert its own waits, which do not count the X DMA at the loop head and so
// would drain the X stream.)
__device__ __forceinline__ u32x4 load_b128_untracked(i32x4 rs, uint32_t off) {
    u32x4 v;
    asm volatile("buffer_load_dwordx4 %0, %1, %2, 0 offen" : "=v"(v) : "v"(off), "s"(rs));
    return v;
}

// Waits until at most N vector memory requests are outstanding; names the
// six W registers of a step, so their values count as produced here.
template <int N>
__device__ __forceinline__ void wait_vmcnt_w(const u32x4 (&wv)[6]) {
    asm volatile("s_waitcnt vmcnt(%6)"
                 : "+v"(const_cast<u32x4 &>(wv[0])), "+v"(const_cast<u32x4 &>(wv[1])),
                   "+v"(const_cast<u32x4 &>(wv[2])), "+v"(const_cast<u32x4 &>(wv[3])),
                   "+v"(const_cast<u32x4 &>(wv[4])), "+v"(const_cast<u32x4 &>(wv[5]))
                 : "n"(N)
                 : "memory");
}

// Lower halves of two 32-bit words: (a & 0xFFFF) | (b << 16).
__device__ __forceinline__ uint32_t lo_halves(uint32_t a, uint32_t b) {
    return __builtin_amdgcn_perm(b, a, 0x05040100u);
}

// W [24, K] -> its TF32 split in the order the MFMA B operands are loaded:
// for chunk c (64 columns), operand e = 3G + kind (G: column group of 32,
// kind 0 = high parts of gates 0..15, 1 = low parts of gates 0..15, 2 = high
// parts of gates 16..23 in lanes n < 8 and low parts in lanes n >= 8) and
// lane l = 16q + n, the 16 bytes wtile[c][e][l] hold the eight BF16 parts of
// that gate at columns 64c + 32G + 8q .. +7.  One W load of a wave is then
// 1 KB of consecutive bytes.  Columns past K are zero, so a partial last
// chunk needs no mask on the W side.  One 16-byte fragment per thread (K is
// a multiple of 8, so its eight columns are all inside or all padding).
// Non-finite W keeps its class in the high part (NaN as the quiet NaN) with
// a zero low part.
__global__ __launch_bounds__(256) void split_weight(const float *__restrict__ w,
                                                    u32x4 *__restrict__ wtile, int64_t K,
                                                    int64_t nfrag) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= nfrag) return;
    const int lane = static_cast<int>(i % kWave);
    const int e = static_cast<int>((i / kWave) % kFwdWLoads);
    const int64_t c = i / (kWave * kFwdWLoads);
    const int q = lane / 16, n = lane % 16;
    const int G = e / 3, kind = e % 3;
    const int gate = kind < 2 ? n : 16 + (n & 7);
    const bool low = kind == 1 || (kind == 2 && n >= 8);
    const int64_t col = kFwdChunk * c + 32 * G + 8 * q;
    u32x4 out = {0u, 0u, 0u, 0u};
    if (col < K) {
        const f32x4 a = *reinterpret_cast<const f32x4 *>(w + gate * K + col);
        const f32x4 b = *reinterpret_cast<const f32x4 *>(w + gate * K + col + 4);
        const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        uint32_t pk[8];  // hi | lo << 16
#pragma unroll
        for (int k = 0; k < 8; ++k) pk[k] = tf32_split_packed(v[k]);
        out = low ? u32x4{hi_halves(pk[0], pk[1]), hi_halves(pk[2], pk[3]),
                          hi_halves(pk[4], pk[5]), hi_halves(pk[6], pk[7])}
                  : u32x4{lo_halves(pk[0], pk[1]), lo_halves(pk[2], pk[3]),
                          lo_halves(pk[4], pk[5]), lo_halves(pk[6], pk[7])};
    }
    wtile[i] = out;
}

template <int NW, int NS>
__global__ __launch_bounds__(NW * kWave) void forward_kernel(
    const float *__restrict__ x, const uint16_t *__restrict__ wsplit, float *__restrict__ proj,
    float *__restrict__ rout, int64_t T, int64_t K, float eps) {
    static_assert(NS >= 3, "X is requested at least two chunks ahead");
    constexpr int DX = NS - 1;  // chunks of X requested ahead of the one computed
    __shared__ f32x4 xring[NW][NS][kFwdDma][kWave];
    static_assert(sizeof(xring) >= NW * kWave * (2 * 16 + 4), "reduction area fits the ring");
    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    const int q = lane / 16;
    const int n16 = lane % 16;
    const int64_t row0 = static_cast<int64_t>(blockIdx.x) * kFwdRows;
    const int rows = static_cast<int>((T - row0) < kFwdRows ? (T - row0) : kFwdRows);
    const int ki = static_cast<int>(K);  // K <= 2^22
    const int nchunks = (ki + kFwdChunk - 1) / kFwdChunk;
    const int nsteps = wave < nchunks ? (nchunks - wave + NW - 1) / NW : 0;

    // LDS DMA: instruction rr = 2a + b of a step moves rows 8a .. 8a+7 and
    // segments 8b .. 8b+7 (16 bytes = 4 columns each) of the chunk; lane L
    // fetches row 8a + L/8, segment 8b + ((L % 8) ^ (L/8) ^ a), which lands at
    // LDS position 64 rr + L (16-byte units) of the stage.
    // The last chunk of a ragged K masks the columns past K (their offsets
    // move outside every range); chunks past the end get an empty range.
    const int tail0 = kFwdChunk * (nchunks - 1);
    uint32_t xoff[kFwdDma], xoff_tail[kFwdDma];
#pragma unroll
    for (int rr = 0; rr < kFwdDma; ++rr) {
        const int a = rr >> 1, b = rr & 1, mi = lane >> 3;
        const int seg = 8 * b + ((lane & 7) ^ mi ^ a);
        xoff[rr] = static_cast<uint32_t>(((8 * a + mi) * ki + 4 * seg) * 4);
        xoff_tail[rr] = tail0 + 4 * seg < ki ? xoff[rr] : kOutOfRange;
    }
    // A-operand reads: lane (q, token m) reads segments 8G + 2q + h (h = 0, 1)
    // of column group G; their positions in a stage follow from the DMA map.
    uint32_t rd[2][2];
    {
        const int a = n16 >> 3, mi = n16 & 7;
#pragma unroll
        for (int G = 0; G < 2; ++G)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int si = 2 * q + h;
                rd[G][h] = static_cast<uint32_t>((64 * (2 * a + G) + 8 * mi + (si ^ mi ^ a)) * 16);
            }
    }
    // W: B operand e of chunk c for this lane is the 16 bytes at
    // ((6c + e) 64 + lane) 16 of the tiled split (see split_weight).
    uint32_t woff[kFwdWLoads];
#pragma unroll
    for (int e = 0; e < kFwdWLoads; ++e) woff[e] = static_cast<uint32_t>((e * kWave + lane) * 16);

    const uint32_t ring = lds_addr(&xring[wave][0][0][0]);
    constexpr uint32_t kStageBytes = kFwdDma * kWave * 16;
    // Chunk c of X into ring stage `stage` (4 LDS DMA), and the W of chunk c
    // (6 loads).  Neither branches: the step's request count stays fixed.
    auto issue_x = [&](int c, int stage) {
        const int c0 = kFwdChunk * c;
        const int n = c < nchunks ? rows * ki - c0 : 0;
        const __amdgpu_buffer_rsrc_t rs =
            make_rsrc32(x + row0 * K + c0, __builtin_amdgcn_readfirstlane(n) * 4);
        const bool tail = c == nchunks - 1;
#pragma unroll
        for (int rr = 0; rr < kFwdDma; ++rr)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs, (MHCPB_LDS void *)(&xring[wave][stage][rr][0]), 16,
                tail ? xoff_tail[rr] : xoff[rr], 0, 0, MHCPB_FWD_X_AUX);
    };
    auto load_w = [&](int c, u32x4 (&wv)[kFwdWLoads]) {
        const int n = c < nchunks ? kFwdWLoads * kWave * 16 : 0;
        const i32x4 rs = rsrc_words(wsplit + static_cast<int64_t>(c) * (kFwdWLoads * kWave * 8), n);
#pragma unroll
        for (int e = 0; e < kFwdWLoads; ++e) wv[e] = load_b128_untracked(rs, woff[e]);
    };

    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f};  // gates 0..15
    f32x4 acc1 = {0.f, 0.f, 0.f, 0.f};  // gates 16..23: high part | low part
    float ss = 0.f;                     // sum of x^2 of token n16, this lane's columns

    // One step: chunk wave + NW j from ring stage j % NS with the W of wcur.
    // Order of the vector memory requests: W(0), W(1), X(0) .. X(DX - 1)
    // before the loop, then W(j + 2) (into wload), X(j + DX) in step j.  The
    // wait at the end of step j must leave X(j + 1) in LDS and W(j + 1) (in
    // wnext) in registers.  With DX = 2, X(j + 1) is the last request of step
    // j - 1, so the 10 requests of step j stay in flight; with DX >= 3 W(j + 1)
    // is the first request of step j - 1, so its 4 X requests and the 10 of
    // step j stay in flight.  Steps past the last chunk still request (an
    // empty range: zeros), which keeps every step's count the same.
    constexpr int kStepWait = DX == 2 ? kFwdWLoads + kFwdDma : kFwdWLoads + 2 * kFwdDma;
    // The last one or two steps of a wave (after the drain below) request
    // nothing: their X and W were requested by the steps before them.
    auto step = [&](int j, const u32x4 (&wcur)[kFwdWLoads], u32x4 (&wload)[kFwdWLoads],
                    u32x4 (&wnext)[kFwdWLoads], bool prefetch) {
        const int c = wave + NW * j;
        const uint32_t sb = ring + static_cast<uint32_t>(j % NS) * kStageBytes;
        f32x4 xv[2][2];
#pragma unroll
        for (int G = 0; G < 2; ++G)
#pragma unroll
            for (int h = 0; h < 2; ++h) xv[G][h] = lds_read_b128(sb + rd[G][h]);
        asm volatile("s_waitcnt lgkmcnt(0)"
                     : "+v"(xv[0][0]), "+v"(xv[0][1]), "+v"(xv[1][0]), "+v"(xv[1][1])::"memory");
        if (prefetch) {
            compiler_fence();
            load_w(c + 2 * NW, wload);
            issue_x(c + DX * NW, (j + DX) % NS);
            compiler_fence();
        }
#pragma unroll
        for (int G = 0; G < 2; ++G) {
            const float v[8] = {xv[G][0].x, xv[G][0].y, xv[G][0].z, xv[G][0].w,
                                xv[G][1].x, xv[G][1].y, xv[G][1].z, xv[G][1].w};
            uint32_t t[8], lo[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                t[e] = tf32_bits(v[e]);
                lo[e] = __float_as_uint(__uint_as_float(t[e]) - __uint_as_float(t[e] & 0xFFFF0000u));
            }
            const u32x4 ahi = {hi_halves(t[0], t[1]), hi_halves(t[2], t[3]),
                               hi_halves(t[4], t[5]), hi_halves(t[6], t[7])};
            const u32x4 alo = {hi_halves(lo[0], lo[1]), hi_halves(lo[2], lo[3]),
                               hi_halves(lo[4], lo[5]), hi_halves(lo[6], lo[7])};
            acc0 = mfma(ahi, wcur[3 * G + 0], acc0);
            acc0 = mfma(ahi, wcur[3 * G + 1], acc0);
            acc0 = mfma(alo, wcur[3 * G + 0], acc0);
            acc0 = mfma(alo, wcur[3 * G + 1], acc0);
            acc1 = mfma(ahi, wcur[3 * G + 2], acc1);
            acc1 = mfma(alo, wcur[3 * G + 2], acc1);
#pragma unroll
            for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(v[e], v[e], ss);
        }
        if (prefetch) wait_vmcnt_w<kStepWait>(wnext);
    };

    // Three W register sets in rotation: step j computes with W(j), while
    // W(j + 1) may still be arriving and W(j + 2) is requested.
    u32x4 wa[kFwdWLoads], wb[kFwdWLoads], wc[kFwdWLoads];
    load_w(wave, wa);
    load_w(wave + NW, wb);
    compiler_fence();
#pragma unroll
    for (int k = 0; k < DX; ++k) issue_x(wave + k * NW, k);
    wait_vmcnt_w<kFwdDma * (DX - 1)>(wa);
    int j = 0;
    for (; j + 2 < nsteps; j += 3) {
        step(j, wa, wc, wb, true);
        step(j + 1, wb, wa, wc, true);
        step(j + 2, wc, wb, wa, true);
    }
    // Every request of this wave lands here, before the last steps and
    // before the ring is reused below.  The wait names every W register set:
    // none may be reused before its last load has landed, and after it no
    // load is in flight, so the branches below cannot meet one.
    asm volatile("s_waitcnt vmcnt(0)"
                 : "+v"(wa[0]), "+v"(wa[1]), "+v"(wa[2]), "+v"(wa[3]), "+v"(wa[4]), "+v"(wa[5]),
                   "+v"(wb[0]), "+v"(wb[1]), "+v"(wb[2]), "+v"(wb[3]), "+v"(wb[4]), "+v"(wb[5]),
                   "+v"(wc[0]), "+v"(wc[1]), "+v"(wc[2]), "+v"(wc[3]), "+v"(wc[4]), "+v"(wc[5])
                 :
                 : "memory");
    if (j < nsteps) step(j, wa, wc, wb, false);
    if (j + 1 < nsteps) step(j + 1, wb, wa, wc, false);
    __syncthreads();

    // Partial sums of each wave, then their sum in wave order by wave 0.
    f32x4 *red0 = &xring[0][0][0][0];
    f32x4 *red1 = red0 + NW * kWave;
    float *red2 = reinterpret_cast<float *>(red1 + NW * kWave);
    red0[wave * kWave + lane] = acc0;
    red1[wave * kWave + lane] = acc1;
    red2[wave * kWave + lane] = ss;
    __syncthreads();
    if (wave != 0) return;
    f32x4 s0 = red0[lane], s1 = red1[lane];
#pragma unroll
    for (int w = 1; w < NW; ++w) {
        s0 += red0[w * kWave + lane];
        s1 += red1[w * kWave + lane];
    }
    // Lanes 0..15: RMS of token `lane` (waves in order, the four column
    // quarters of each in order).
    float st = 0.f;
    if (lane < kFwdRows) {
        for (int w = 0; w < NW; ++w)
#pragma unroll
            for (int qq = 0; qq < 4; ++qq) st += red2[w * kWave + 16 * qq + lane];
    }
    const float rv = __builtin_sqrtf(st / static_cast<float>(ki) + eps);
    // Accumulator lane l holds gate l % 16 of tokens 4 (l / 16) + i.  Gates
    // 16..23 add the high-part column (this lane) and the low-part column
    // (lane + 8).  A row whose RMS is NaN has a NaN in X: its logits are NaN.
    const float qnan = __builtin_nanf("");
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = 4 * q + i;
        const float rm = __shfl(rv, m);
        const float other = __shfl_xor(s1[i], 8);
        if (m < rows) {
            float *row = proj + (row0 + m) * kProjStride;
            const bool nan_row = rm != rm;
            row[n16] = nan_row ? qnan : s0[i];
            row[16 + n16] = n16 < 8 ? (nan_row ? qnan : s1[i] + other) : 0.f;
        }
    }
    if (lane < rows) rout[row0 + lane] = rv;
}

}  // namespace

hipError_t launch_split_weight(const Plan &p, const float *w, uint16_t *wsplit, hipStream_t stream,
                               hipEvent_t start, hipEvent_t stop) {
    const int64_t nfrag = forward_padded_cols(p.K) / kFwdChunk * kFwdWLoads * kWave;
    const unsigned blocks = static_cast<unsigned>((nfrag + 255) / 256);
    launch(split_weight, dim3(blocks), dim3(256), stream, start, stop, w,
           reinterpret_cast<u32x4 *>(wsplit), p.K, nfrag);
    return hipGetLastError();
}

// Eight waves per workgroup: 96 KB of ring, one workgroup per CU; at
// T = 4096 the grid is one workgroup per CU on 256 CUs.
hipError_t launch_forward(const Plan &p, const float *x, const uint16_t *wsplit, float *proj,
                          float *r, float eps, hipStream_t stream, hipEvent_t start,
                          hipEvent_t stop) {
    constexpr int NW = 8;
    constexpr int NS = 3;
    const dim3 grid(static_cast<unsigned>((p.T + kFwdRows - 1) / kFwdRows));
    launch(forward_kernel<NW, NS>, grid, dim3(NW * kWave), stream, start, stop, x, wsplit, proj, r,
           p.T, p.K, eps);
    return hipGetLastError();
}

}  // namespace mhcpb
