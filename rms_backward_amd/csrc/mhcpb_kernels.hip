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
// a two-step ring per wave, so prefetching costs no registers; rows past the
// slab end fall outside the buffer range and arrive as zeros.  The P rows of
// each step arrive the same way a few steps ahead.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>

#include "mhcpb_device.h"
#include "mhcpb_internal.h"

namespace mhcpb {
namespace {

// Cache policy of the X stream (read once): non-temporal ("nt" on gfx950).
#ifndef MHCPB_X_AUX
#define MHCPB_X_AUX 2
#endif
// Cache policy of the dX stores (written once, read by a later stage):
// non-temporal as well.
#ifndef MHCPB_DX_AUX
#define MHCPB_DX_AUX 2
#endif

// Rows per step (one MFMA row block) and the LDS layouts of P.
constexpr int kStepRows = 16;
constexpr int kJPad = 32;                 // j slots per part, 24..31 zero
constexpr int kPaStride = 2 * kJPad + 4;  // uint32 per row of the dX P operand
constexpr int kPbJStride = 40;            // uint16 per j of the dW P operand (32 + 8 padding)

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
//  pb[j][g][part][r]: the part of row 4g + r, as the dW product reads it (both
//      parts of 4 consecutive rows in 16 bytes);
//  c[row]: grad_r / (r K).
// Entries with j >= 24 are zero and never written after the first clear.
struct alignas(16) StepP {
    uint32_t pa[kStepRows * kPaStride];
    uint16_t pb[kJPad * kPbJStride];
    float c[kStepRows];
};

// Operand slots in rotation, and how many steps ahead of its conversion the
// producer requests the raw P of a step.
constexpr int kSlots = 4;
constexpr int kRawAhead = 2;
constexpr int kRawBufs = kRawAhead + 1;

// Kernel 1.  A workgroup has NW compute waves, which own NW * 64 columns of
// one slab, and one producer wave.  Per step a compute wave handles 16 rows x
// 64 columns: lane l (c = l % 16, g = l / 16) holds x[t0 + 4g + r][kw + 4c + i]
// for r, i in 0..3.
//  dX: C_i[e] = dX[t0 + 4g + e][kw + 4c + i] = c_t x + the products of the P
//      parts (token t0 + l%16) with the W parts (column kw + 4c + i): per
//      MFMA (P part p, j block b) lane group g covers j = 16b + 4g .. +3 times
//      (W hi, W lo); 4 MFMAs cover the 96 products of 24 j (8 padded).
//  dW: acc[i][b][e] = sum over tokens of TF32(x) of column kw + 4(4g+e) + i
//      times TF32(P[j]), j = 16 b + l%16: per MFMA (P part p), lane group g
//      covers rows 4g .. 4g+3 times (x hi, x lo).
//
// Memory pipeline.  Each compute wave streams its X through a two-step ring
// in LDS: the DMA for step j + 1 is issued as soon as step j has arrived, so
// one step per wave is in flight.  The producer wave copies the raw P of step
// k into LDS (DMA) two steps ahead, converts it into operand slot k % 4 and
// publishes it; it never touches X.
//
// Synchronisation.  Each slot has two monotonic LDS counters: "ready" (one
// count per use, from the producer) and "consumed" (one count per compute
// wave per use, once its reads of the slot have completed).  A compute wave
// reads step k once ready[k % 4] reaches k / 4 + 1; the producer writes step
// k once consumed[k % 4] reaches NW (k / 4), i.e. once every compute wave has
// read step k - 4 from the slot.  A slot's next use needs the previous one
// consumed by every wave, so the counts identify the use exactly, and every
// wait refers to an event of an earlier step, so none can deadlock.  The
// waits are also bounded, so a broken invariant cannot hang the GPU.  Compute
// waves never wait for each other.
//
// kDX and kDW select the outputs: both (the fused stage), dX only or dW only
// (the split forms); the arithmetic of each output is the same in every form.
//
// Two workgroups per CU make 12 waves (NW = 5), three per SIMD: the register
// allocation must stay within 168 VGPRs.
// A pointer the compiler may have kept in vector registers, as the uniform
// value it is (from the first lane).  The deferred dX stores take their
// buffer resource from values carried across loop iterations; without this
// the compiler wrapped each such store in a loop over distinct resources.
__device__ __forceinline__ char *uniform_ptr(char *p) {
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
    return reinterpret_cast<char *>((static_cast<uint64_t>(hi) << 32) | lo);
}

template <int NW, bool kAddend, bool kDX, bool kDW>
__global__ __launch_bounds__((NW + 1) * kWave)
__attribute__((amdgpu_waves_per_eu(3))) void projection_kernel(
    const float *__restrict__ x, const float *__restrict__ w,
    const float *__restrict__ grad_proj, const float *__restrict__ grad_r,
    const float *__restrict__ r, uint16_t *__restrict__ dx, float *__restrict__ ws,
    const uint16_t *__restrict__ addend, int64_t T, int64_t K, int64_t L) {
    __shared__ f32x4 xring[NW][2][4][kWave];
    __shared__ RawStep praw[kRawBufs];
    __shared__ StepP pop[kSlots];
    __shared__ uint32_t ready[kSlots], consumed[kSlots];
    constexpr int kThreads = (NW + 1) * kWave;
    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int c16 = lane % 16;
    const int g = lane / 16;
    const int s = blockIdx.y;
    const int64_t row0 = static_cast<int64_t>(s) * L;
    const int64_t row1 = (row0 + L < T) ? row0 + L : T;
    const int slab_rows = static_cast<int>(row1 - row0);  // <= L < 2^31
    const int nsteps = (slab_rows + kStepRows - 1) / kStepRows;
    const float kf = static_cast<float>(K);
    const int ki = static_cast<int>(K);  // K <= 2^22
    const uint32_t ready_addr = lds_addr(&ready[0]);
    const uint32_t consumed_addr = lds_addr(&consumed[0]);
    // Rows of the slab from row 16 k on, clamped to one step.
    auto step_rows = [&](int rows_left) {
        return __builtin_amdgcn_readfirstlane(
            rows_left < 0 ? 0 : (rows_left > kStepRows ? kStepRows : rows_left));
    };

    // ---- producer: raw P of step k into praw[k % kRawBufs], two 64-lane DMA
    // of 16 bytes for the 16 rows of grad_proj and, when dX is produced, one
    // of 4 bytes each for grad_r and r (the dW-only form is given neither).
    // Rows past the slab end read as zeros.
    const bool producer = wave == NW;
    constexpr int kRawDma = kDX ? 4 : 2;  // DMA instructions per step
    auto issue_raw = [&](int k) {
        const int rl = step_rows(slab_rows - kStepRows * k);
        RawStep &d = praw[k % kRawBufs];
        const int64_t r0 = row0 + static_cast<int64_t>(kStepRows) * k;
        const __amdgpu_buffer_rsrc_t prs = make_rsrc32(grad_proj + r0 * kProjStride, rl * kProjStride * 4);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(prs, (MHCPB_LDS void *)(&d.p[0]), 16,
                                                 static_cast<uint32_t>(lane * 16), 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(prs, (MHCPB_LDS void *)(&d.p[kWave]), 16,
                                                 static_cast<uint32_t>((kWave + lane) * 16), 0, 0, 0);
        if constexpr (kDX) {
            __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc32(grad_r + r0, rl * 4),
                                                     (MHCPB_LDS void *)d.gr, 4,
                                                     static_cast<uint32_t>(lane * 4), 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(make_rsrc32(r + r0, rl * 4),
                                                     (MHCPB_LDS void *)d.r, 4,
                                                     static_cast<uint32_t>(lane * 4), 0, 0, 0);
        }
    };

    // The j = 24..31 entries of every operand slot are zero padding; the
    // counters start at zero.
    constexpr int kPadJ = kJPad - kProjCols;
    for (int i = tid; i < kSlots * kStepRows * 2 * kPadJ; i += kThreads) {
        const int buf = i / (kStepRows * 2 * kPadJ);
        const int k = i % (kStepRows * 2 * kPadJ);
        const int row = k / (2 * kPadJ), rest = k % (2 * kPadJ);
        const int part = rest / kPadJ, jj = kProjCols + rest % kPadJ;
        lds_write_u32(lds_addr(pop[buf].pa + row * kPaStride + part * kJPad + jj), 0u);
    }
    for (int i = tid; i < kSlots * kPadJ * kPbJStride; i += kThreads) {
        const int buf = i / (kPadJ * kPbJStride);
        const int off = i % (kPadJ * kPbJStride);
        lds_write_u16(lds_addr(pop[buf].pb + kProjCols * kPbJStride + off), 0u);
    }
    if (tid < kSlots) {
        lds_write_u32(ready_addr + 4 * tid, 0u);
        lds_write_u32(consumed_addr + 4 * tid, 0u);
    }

    if (producer) {
#pragma unroll
        for (int k = 0; k < kRawAhead; ++k) issue_raw(k);
        lds_barrier();
        // Lane = row * 4 + q converts j = 6q .. 6q + 5 of one row of P into
        // both operand layouts; lanes 0..15 also compute the RMS coefficient
        // grad_r / (r K) of row lane in FP32 (zero past the slab end).
        const int prow = lane / 4;
        const int pj0 = 6 * (lane % 4);
        for (int k = 0; k < nsteps; ++k) {
            issue_raw(k + kRawAhead);
            // The raw P of step k was requested before that of the kRawAhead
            // steps after it, kRawDma DMA instructions each.
            wait_vmcnt<kRawDma * kRawAhead>();
            const int slot = k % kSlots;
            lds_wait_at_least(consumed_addr + 4 * slot, NW * static_cast<uint32_t>(k / kSlots));
            const RawStep &src = praw[k % kRawBufs];
            const StepP &d = pop[slot];
            const uint32_t ra = lds_addr(&src.p[0]) + static_cast<uint32_t>((prow * kProjStride + pj0) * 4);
            u32x2 v0 = lds_read_u64(ra), v1 = lds_read_u64(ra + 8), v2 = lds_read_u64(ra + 16);
            float grv = 0.f, rv = 1.f;
            if constexpr (kDX) {
                grv = lds_read_f32(lds_addr(&src.gr[lane]));
                rv = lds_read_f32(lds_addr(&src.r[lane]));
            }
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(v0), "+v"(v1), "+v"(v2), "+v"(grv), "+v"(rv)::"memory");
            const uint32_t vv[6] = {v0.x, v0.y, v1.x, v1.y, v2.x, v2.y};
            uint32_t pk[6];  // hi | lo << 16
#pragma unroll
            for (int e = 0; e < 6; ++e) pk[e] = tf32_split_packed_p(__uint_as_float(vv[e]));
            const uint32_t pa_hi = lds_addr(d.pa + prow * kPaStride + pj0);
            const uint32_t pa_lo = pa_hi + kJPad * 4;
#pragma unroll
            for (int e = 0; e < 6; e += 2) {
                lds_write_u64(pa_hi + 4 * e, u32x2{dup_low_half(pk[e]), dup_low_half(pk[e + 1])});
                lds_write_u64(pa_lo + 4 * e, u32x2{dup_high_half(pk[e]), dup_high_half(pk[e + 1])});
            }
            const uint32_t pb0 = lds_addr(d.pb + pj0 * kPbJStride + (prow / 4) * 8 + prow % 4);
            const uint32_t pb1 = pb0 + 4 * 2;
#pragma unroll
            for (int e = 0; e < 6; ++e) {
                lds_write_u16(pb0 + e * kPbJStride * 2, pk[e]);
                lds_write_u16_hi(pb1 + e * kPbJStride * 2, pk[e]);
            }
            if (kDX && lane < kStepRows) {
                const bool in_slab = kStepRows * k + lane < slab_rows;
                lds_write_u32(lds_addr(d.c + lane), __float_as_uint(in_slab ? grv / (rv * kf) : 0.f));
            }
            lds_signal(ready_addr + 4 * slot, lane);
        }
        // Drain the copies still in flight before the workgroup's LDS can be
        // released.
        wait_vmcnt<0>();
        return;
    }

    // ---- compute waves: X ring, W in registers.
    const int64_t kw = static_cast<int64_t>(blockIdx.x) * (NW * 64) + wave * 64;
    const int kwi = static_cast<int>(kw);  // kw < K + NW * 64
    const int64_t col = kw + 4 * c16;      // first of this lane's 4 columns
    const bool active = col < K;
    // A step is addressed through one buffer resource per tensor, based at
    // row t0 and column kw, whose range ends at the slab end or 16 rows on,
    // whichever comes first; lane offsets (row 4g + r, columns 4c..4c+3) go
    // in the per-lane offset, which the hardware range check covers (the
    // scalar offset, which is not checked, stays zero).  An element of a
    // slab row lies in the range because K and the lane's column are
    // multiples of 4; a row past the slab end lies outside it.  Inactive
    // columns get an offset outside every range, so their loads read zeros
    // and their stores are dropped.
    uint32_t xoff[4], doff[4];
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
        xoff[rr] = active ? static_cast<uint32_t>(((4 * g + rr) * K + 4 * c16) * 4) : kOutOfRange;
        doff[rr] = active ? static_cast<uint32_t>(((4 * g + rr) * K + 4 * c16) * 2) : kOutOfRange;
    }
    // Elements of the range of a step resource (times the element size).
    auto range_elems = [&](int rows_left) {
        const int rl = rows_left < 0 ? 0 : (rows_left > kStepRows ? kStepRows : rows_left);
        const int n = rl * ki - kwi;
        return __builtin_amdgcn_readfirstlane(n > 0 ? n : 0);
    };
    const int64_t row_bytes_x = K * 4;  // one row of X
    const int64_t row_bytes_d = K * 2;  // one row of dX or the addend
    const uint32_t ring_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&xring[wave][0][0][0]));
    // xs points at row 0, column kw of a step; rows_left counts the slab rows
    // from there on.
    auto issue_x = [&](const char *xs, int rows_left, int stage) {
        const __amdgpu_buffer_rsrc_t xrs = make_rsrc32(xs, range_elems(rows_left) * 4);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                xrs, (MHCPB_LDS void *)(&xring[wave][stage][rr][0]), 16, xoff[rr], 0, 0, MHCPB_X_AUX);
    };
    // W of this lane's columns (for the dX product): loaded first, then the X
    // of steps 0 and 1 (both ring stages are free at the start), so that the
    // wait for W below does not wait for X, and two steps stream in while the
    // prologue runs.
    float4 wraw[2][4] = {};  // [j block][e]: W[16 b + 4 g + e][col .. col + 3]
    if constexpr (kDX) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int jj = 16 * b + 4 * g + e;
                wraw[b][e] = (active && jj < kProjCols)
                                 ? *reinterpret_cast<const float4 *>(w + jj * K + col)
                                 : make_float4(0.f, 0.f, 0.f, 0.f);
            }
    }
    compiler_fence();
    const char *x_next = reinterpret_cast<const char *>(x + row0 * K + kw);
    issue_x(x_next, slab_rows, 0);
    issue_x(x_next + kStepRows * row_bytes_x, slab_rows - kStepRows, 1);
    x_next += 2 * kStepRows * row_bytes_x;
    compiler_fence();
    // Padding and counters visible (the producer passes the same barrier).
    lds_barrier();

    // W side of the dX product: for column variant i and j block b the lane
    // holds the packed (hi | lo << 16) TF32 split of W[j][col + i] for
    // j = 16b + 4g .. 16b + 4g + 3 (zero for j >= 24).
    u32x4 bw[4][2] = {};
#pragma unroll
    for (int b = 0; b < 2 && kDX; ++b) {
        const float wv[4][4] = {{wraw[b][0].x, wraw[b][0].y, wraw[b][0].z, wraw[b][0].w},
                                {wraw[b][1].x, wraw[b][1].y, wraw[b][1].z, wraw[b][1].w},
                                {wraw[b][2].x, wraw[b][2].y, wraw[b][2].z, wraw[b][2].w},
                                {wraw[b][3].x, wraw[b][3].y, wraw[b][3].z, wraw[b][3].w}};  // [e][i]
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

    char *d_cur = reinterpret_cast<char *>(dx + row0 * K + kw);
    const char *a_cur = reinterpret_cast<const char *>(addend + row0 * K + kw);
    // The ready count of a step's slot is read one step early, so that its
    // round trip is off the step's critical path.
    uint32_t ready_seen = lds_read_u32(ready_addr);
    // With the addend, the dX stores of a step are issued one step late,
    // right after the next X request (same bits; at T = 16384 with the
    // addend 466 against 475 us, while without it they cost about 2 us at
    // T = 4096, so only this form defers them).
    constexpr bool kDefer = kAddend && kDX;
    uint32_t pend[4][2] = {};
    char *d_prev = d_cur;
    int d_range_prev = 0;
    for (int j = 0; j < nsteps; ++j) {
        const int rows_left = slab_rows - kStepRows * j;
        // From the top of the step until the next X is requested the wave
        // runs at raised priority: once its X has arrived, the LDS reads and
        // the next request go ahead of the other waves' arithmetic on the
        // SIMD (about 1 % faster at T = 4096, K = 20480; the bits are those
        // of the same kernel without it).
        __builtin_amdgcn_s_setprio(1);
        const int slot = j % kSlots;
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(ready_seen)::"memory");
        const uint32_t want = static_cast<uint32_t>(j / kSlots + 1);
        if (__builtin_amdgcn_readfirstlane(ready_seen) < want)
            lds_wait_at_least(ready_addr + 4 * slot, want);
        const StepP &cur = pop[slot];
        // The P operands of this step are requested first: the RMS
        // coefficients of rows 4g..4g+3, the dX P operands (token c16, part
        // p, j = 16b + 4g .. +3) and the dW P operands (part p, j = 16b +
        // c16, rows 4g .. 4g+3; entries j >= 24 are zero).
        f32x4 cc = {};
        u32x4 pa[2][2] = {};  // [part][block]
        u32x4 pbv[2] = {};    // [block]: part 0 in .xy, part 1 in .zw
        if constexpr (kDX) cc = lds_read_b128(lds_addr(cur.c + 4 * g));
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            if constexpr (kDX) {
#pragma unroll
                for (int p = 0; p < 2; ++p)
                    pa[p][b] = lds_read_u128(
                        lds_addr(cur.pa + c16 * kPaStride + p * kJPad + 16 * b + 4 * g));
            }
            if constexpr (kDW)
                pbv[b] = lds_read_u128(lds_addr(cur.pb + (16 * b + c16) * kPbJStride + 8 * g));
        }
        // Then wait for this step's X and read it (4 rows).  Step j >= 1
        // issues, in this order: [4 addend loads] 4 X DMA (for step j + 1),
        // [4 dX stores of step j - 1 when deferred], [4 dX stores of step j
        // otherwise]; step 0 issues no X (the prologue requested steps 0 and
        // 1, after the W loads).  So after the X of step j come at most 4
        // stores (of step j - 1, or of step j - 2 when deferred; none without
        // dX), and after the X of step 0 the X of step 1: vmcnt(4), or
        // vmcnt(0) for the later steps of the dW-only form, covers it.  With
        // deferred stores step 0 stores nothing, so step 1 waits for
        // vmcnt(0).  For step 1 with the addend, step 0's addend loads come
        // after the X of step 1 as well, and the wait is only stricter.
        // Steps past the slab end are still requested (they read zeros;
        // their stores fall outside the range), which keeps every step's
        // count identical.
        if (j == 0 || (kDX && !(kDefer && j == 1)))
            wait_vmcnt<4>();
        else
            wait_vmcnt<0>();
        const uint32_t xa = ring_base + static_cast<uint32_t>((((j & 1) * 4) * kWave + lane) * 16);
        f32x4 xc[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) xc[rr] = lds_read_b128(xa + rr * kWave * 16);
        // The wait names every register the reads above return, so no use
        // of them can be scheduled before the data has arrived.
        if constexpr (kDX && kDW)
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(xc[0]), "+v"(xc[1]), "+v"(xc[2]), "+v"(xc[3]), "+v"(cc),
                           "+v"(pa[0][0]), "+v"(pa[0][1]), "+v"(pa[1][0]), "+v"(pa[1][1]),
                           "+v"(pbv[0]), "+v"(pbv[1])::"memory");
        else if constexpr (kDX)
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(xc[0]), "+v"(xc[1]), "+v"(xc[2]), "+v"(xc[3]), "+v"(cc),
                           "+v"(pa[0][0]), "+v"(pa[0][1]), "+v"(pa[1][0]),
                           "+v"(pa[1][1])::"memory");
        else
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(xc[0]), "+v"(xc[1]), "+v"(xc[2]), "+v"(xc[3]), "+v"(pbv[0]),
                           "+v"(pbv[1])::"memory");
        lds_signal(consumed_addr + 4 * slot, lane);
        uint2 av[4] = {};
        const int d_range = range_elems(rows_left) * 2;
        if constexpr (kAddend) {
            const __amdgpu_buffer_rsrc_t ars = make_rsrc32(a_cur, d_range);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(ars, doff[rr], 0, 0);
                av[rr] = make_uint2(v.x, v.y);
            }
            a_cur += kStepRows * row_bytes_d;
        }
        compiler_fence();
        if (j > 0) {
            issue_x(x_next, rows_left - kStepRows, (j + 1) & 1);
            x_next += kStepRows * row_bytes_x;
        }
        compiler_fence();
        __builtin_amdgcn_s_setprio(0);
        if (kDefer && j > 0) {
            const __amdgpu_buffer_rsrc_t prs =
                make_rsrc32(uniform_ptr(d_prev), __builtin_amdgcn_readfirstlane(d_range_prev));
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                __builtin_amdgcn_raw_buffer_store_b64(u32x2{pend[rr][0], pend[rr][1]}, prs,
                                                      doff[rr], 0, MHCPB_DX_AUX);
        }
        compiler_fence();

        const float ce[4] = {cc[0], cc[1], cc[2], cc[3]};
        u32x4 pb[2][2];
#pragma unroll
        for (int p = 0; p < 2; ++p)
#pragma unroll
            for (int b = 0; b < 2; ++b)
                pb[p][b] = p == 0 ? u32x4{pbv[b].x, pbv[b].y, pbv[b].x, pbv[b].y}
                                  : u32x4{pbv[b].z, pbv[b].w, pbv[b].z, pbv[b].w};

        uint32_t packed[4][2];  // dX of row 4g + r, columns (0,1) and (2,3)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // dX for column variant i: the RMS term c_t * x in FP32, then
            // the 96 exact partial products.
            f32x4 acc = {};
            if constexpr (kDX) {
                acc = f32x4{ce[0] * xc[0][i], ce[1] * xc[1][i], ce[2] * xc[2][i], ce[3] * xc[3][i]};
#pragma unroll
                for (int b = 0; b < 2; ++b)
#pragma unroll
                    for (int p = 0; p < 2; ++p) acc = mfma(pa[p][b], bw[i][b], acc);
            }

            // dW: x of column variant i split into BF16 hi/lo, packed
            // [hi r0..r3 | lo r0..r3], against each P part.
            if constexpr (kDW) {
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
        // One rounding to BF16 per element (above), then 8-byte range-checked
        // stores: rows past the slab end are dropped.
        if constexpr (kDefer) {
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) {
                pend[rr][0] = packed[rr][0];
                pend[rr][1] = packed[rr][1];
            }
            d_prev = d_cur;
            d_range_prev = d_range;
        } else if constexpr (kDX) {
            const __amdgpu_buffer_rsrc_t drs = make_rsrc32(d_cur, d_range);
#pragma unroll
            for (int rr = 0; rr < 4; ++rr)
                __builtin_amdgcn_raw_buffer_store_b64(u32x2{packed[rr][0], packed[rr][1]}, drs,
                                                      doff[rr], 0, MHCPB_DX_AUX);
        }
        d_cur += kStepRows * row_bytes_d;
        ready_seen = lds_read_u32(ready_addr + 4 * ((j + 1) % kSlots));
    }
    if (kDefer && nsteps > 0) {  // the last step's stores
        const __amdgpu_buffer_rsrc_t prs =
            make_rsrc32(uniform_ptr(d_prev), __builtin_amdgcn_readfirstlane(d_range_prev));
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
            __builtin_amdgcn_raw_buffer_store_b64(u32x2{pend[rr][0], pend[rr][1]}, prs, doff[rr],
                                                  0, MHCPB_DX_AUX);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(ready_seen)::"memory");
    // Drain the X DMA still in flight (the step past the slab end) before
    // the workgroup's LDS can be released.
    wait_vmcnt<0>();

    // Partial dW of this slab, written once to workspace slab s.  Lane
    // (c16, g), element e of block jb holds column kw + 16 g + 4 e + i of
    // j = 16 jb + c16.  The wave's 32 x 64 block goes through its own X ring
    // (8 KB, idle after the drain above) so that each store instruction
    // writes four whole 256-byte rows: j = 4 q + g, columns kw + 4 c16 ..
    // + 3.  With whole lines the stores can be non-temporal (with the
    // 64-byte pieces of the register layout they cost about 10 us more).
    if constexpr (!kDW) return;
    float *slab = ws + static_cast<int64_t>(s) * kProjCols * K;
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e)
            lds_write_u128(ring_base + static_cast<uint32_t>(((16 * b + c16) * 64 + 16 * g + 4 * e) * 4),
                           u32x4{__float_as_uint(accw[0][b][e]), __float_as_uint(accw[1][b][e]),
                                 __float_as_uint(accw[2][b][e]), __float_as_uint(accw[3][b][e])});
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    static_assert(kProjCols / 4 == 6, "the wait below names the six rows of four");
    u32x4 tv[kProjCols / 4];
#pragma unroll
    for (int q = 0; q < kProjCols / 4; ++q)
        tv[q] = lds_read_u128(ring_base + static_cast<uint32_t>(((4 * q + g) * 64 + 4 * c16) * 4));
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(tv[0]), "+v"(tv[1]), "+v"(tv[2]), "+v"(tv[3]), "+v"(tv[4]), "+v"(tv[5])::"memory");
    if (active) {
#pragma unroll
        for (int q = 0; q < kProjCols / 4; ++q)
            __builtin_nontemporal_store(__builtin_bit_cast(f32x4, tv[q]),
                                        reinterpret_cast<f32x4 *>(slab + (4 * q + g) * K + col));
    }
}

// dW[i] = (((ws[0][i] + ws[1][i]) + ws[2][i]) + ...), four elements per thread.
// The slabs are loaded eight at a time before they are added (in order), so
// the loads overlap.
constexpr int kReduceBatch = 8;
__global__ __launch_bounds__(256) void reduce_slabs(const float *__restrict__ ws,
                                                    float *__restrict__ dw, int S,
                                                    int64_t n4) {
    const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= n4) return;
    const f32x4 *src = reinterpret_cast<const f32x4 *>(ws) + i;
    f32x4 a = __builtin_nontemporal_load(src);
    for (int s0 = 1; s0 < S; s0 += kReduceBatch) {
        f32x4 b[kReduceBatch];
        // Past the last slab the addend is -0, which leaves every sum as it
        // is (x + -0 == x, signed zeros included).
#pragma unroll
        for (int u = 0; u < kReduceBatch; ++u)
            b[u] = (s0 + u < S) ? __builtin_nontemporal_load(src + static_cast<int64_t>(s0 + u) * n4)
                                : f32x4{-0.f, -0.f, -0.f, -0.f};
#pragma unroll
        for (int u = 0; u < kReduceBatch; ++u) a += b[u];
    }
    reinterpret_cast<f32x4 *>(dw)[i] = a;
}

template <int NW>
hipError_t launch_projection_t(const Plan &p, const Args &a, Outputs out, hipStream_t stream,
                               hipEvent_t start, hipEvent_t stop) {
    constexpr int cols = NW * 64;
    const dim3 grid(static_cast<unsigned>((p.K + cols - 1) / cols), static_cast<unsigned>(p.S));
    const dim3 block((NW + 1) * kWave);
#define MHCPB_LAUNCH(ADD, DX, DW)                                                               \
    launch(projection_kernel<NW, ADD, DX, DW>, grid, block, stream, start, stop, a.x, a.w,      \
           a.grad_proj, a.grad_r, a.r, a.dx, a.ws, a.addend, p.T, p.K, p.L)
    switch (out) {
    case Outputs::kBoth:
        if (a.addend)
            MHCPB_LAUNCH(true, true, true);
        else
            MHCPB_LAUNCH(false, true, true);
        break;
    case Outputs::kDxOnly:
        if (a.addend)
            MHCPB_LAUNCH(true, true, false);
        else
            MHCPB_LAUNCH(false, true, false);
        break;
    case Outputs::kDwOnly:
        MHCPB_LAUNCH(false, false, true);
        break;
    }
#undef MHCPB_LAUNCH
    return hipGetLastError();
}

}  // namespace

// Launch shape, a performance choice only: each column's dW is summed in the
// same order whatever the workgroup width, so every shape gives the same bits.
// Five compute waves and the producer make two workgroups per CU exactly
// three waves per SIMD; at K = 20480 with 8 splits the grid is one full round
// of two workgroups per CU on 256 CUs.
hipError_t launch_projection(const Plan &p, const Args &a, Outputs out, hipStream_t stream,
                             hipEvent_t start, hipEvent_t stop) {
    return launch_projection_t<5>(p, a, out, stream, start, stop);
}

hipError_t launch_reduce(const Plan &p, const Args &a, hipStream_t stream, hipEvent_t stop) {
    const int64_t n4 = kProjCols * p.K / 4;
    const unsigned blocks = static_cast<unsigned>((n4 + 255) / 256);
    launch(reduce_slabs, dim3(blocks), dim3(256), stream, nullptr, stop, a.ws, a.dw, p.S, n4);
    return hipGetLastError();
}

}  // namespace mhcpb
