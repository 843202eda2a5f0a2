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
#include <mutex>

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

// Kernel 1.  A workgroup has NW compute waves, which own the NW * 64 columns
// of one column tile, and one producer wave.  The workgroup walks, one after
// the other, the slabs s = sg, sg + G, sg + 2G, ... < S of its tile (sg = its
// slab group): one unit of work per slab, each unit's rows in ascending
// 16-row steps, and the steps of all its units form one continuous sequence
// (global step k).  Per step a compute wave handles 16 rows x 64 columns:
// lane l (c = l % 16, g = l / 16) holds x[t0 + 4g + r][kw + 4c + i] for r, i
// in 0..3.
//  dX: C_i[e] = dX[t0 + 4g + e][kw + 4c + i] = c_t x + the products of the P
//      parts (token t0 + l%16) with the W parts (column kw + 4c + i): per
//      MFMA (P part p, j block b) lane group g covers j = 16b + 4g .. +3 times
//      (W hi, W lo); 4 MFMAs cover the 96 products of 24 j (8 padded).
//  dW: acc[i][b][e] = sum over the slab's tokens of TF32(x) of column
//      kw + 4(4g+e) + i times TF32(P[j]), j = 16 b + l%16: per MFMA (P part
//      p), lane group g covers rows 4g .. 4g+3 times (x hi, x lo).  At the
//      end of each unit the 24 x 64 partial goes to workspace slab s and the
//      accumulators restart from zero.
//
// Why one workgroup walks several slabs: a workgroup needs 6 waves and
// 75 KB of LDS, so a CU holds one at a time; with one workgroup per (tile,
// slab) the supported profile (64 tiles x 8 slabs) ran as two rounds of 256
// workgroups, each with its own start-up (the first X and W requests) and
// drain.  With G = 4 slab groups the 256 workgroups each stream two slabs
// back to back: the X of the next unit is requested while the last step of
// the current one is computed and its partial is stored.  A column's dW sums
// the same rows in the same order whatever the grouping, so the grouping
// changes no bit of the result.
//
// Memory pipeline.  Each compute wave streams its X through a two-step ring
// in LDS: the DMA for step k + 1 is issued as soon as step k has arrived, so
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
// waits are also bounded, so a broken invariant cannot hang the GPU; a wave
// whose wait gives up raises the workgroup's poison word, and from then on
// every dX value and dW partial the workgroup writes is NaN (the results
// computed after a give-up could come from stale or overwritten operands).
// Compute waves never wait for each other.
//
// kDX and kDW select the outputs: both (the fused stage), dX only or dW only
// (the split forms); the arithmetic of each output is the same in every form.
//
// A CU holds one workgroup (six waves, at most two per SIMD), so a wave may
// use up to 256 VGPRs.
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

// Position in a workgroup's sequence of steps: unit u (slab sg + u G), step j
// of that slab, the slab's first row and row count, and its step count.  Past
// the last unit the slab has no rows, so every request of such a step falls
// outside its buffer range.
struct StepCursor {
    int u;
    int j;
    int nst;        // steps of the current slab
    int slab_rows;  // rows of the current slab (0 past the last unit)
    int64_t row0;   // first row of the current slab
};

__device__ __forceinline__ int slab_rows_at(int64_t row0, int64_t L, int64_t T) {
    const int64_t n = T - row0 < L ? T - row0 : L;
    return static_cast<int>(n > 0 ? n : 0);
}

__device__ __forceinline__ StepCursor cursor_start(int sg, int64_t L, int64_t T) {
    StepCursor c;
    c.u = 0;
    c.j = 0;
    c.row0 = static_cast<int64_t>(sg) * L;
    c.slab_rows = slab_rows_at(c.row0, L, T);
    c.nst = (c.slab_rows + 15) / 16;
    return c;
}

// Advances by one step; returns true when the step left was the last of its
// unit.
__device__ __forceinline__ bool cursor_next(StepCursor &c, int G, int64_t L, int64_t T) {
    if (++c.j < c.nst) return false;
    c.j = 0;
    ++c.u;
    c.row0 += static_cast<int64_t>(G) * L;
    c.slab_rows = slab_rows_at(c.row0, L, T);
    c.nst = (c.slab_rows + 15) / 16;
    return true;
}

// Number of store instructions of one partial dW write (per compute wave).
constexpr int kPartialStores = 6;

template <int NW, bool kAddend, bool kDX, bool kDW>
__global__ __launch_bounds__((NW + 1) * kWave)
__attribute__((amdgpu_waves_per_eu(2))) void projection_kernel(
    const float *__restrict__ x, const float *__restrict__ w,
    const float *__restrict__ grad_proj, const float *__restrict__ grad_r,
    const float *__restrict__ r, uint16_t *__restrict__ dx, float *__restrict__ ws,
    const uint16_t *__restrict__ addend, int64_t T, int64_t K, int64_t L, int S, int tiles,
    int G, int max_polls) {
    __shared__ f32x4 xring[NW][2][4][kWave];
    __shared__ RawStep praw[kRawBufs];
    __shared__ StepP pop[kSlots];
    __shared__ uint32_t ready[kSlots], consumed[kSlots], poison[1];
    constexpr int kThreads = (NW + 1) * kWave;
    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int c16 = lane % 16;
    const int g = lane / 16;
    const int tile = static_cast<int>(blockIdx.x) % tiles;
    const int sg = static_cast<int>(blockIdx.x) / tiles;  // slab group, < G <= S
    const float kf = static_cast<float>(K);
    const int ki = static_cast<int>(K);  // K <= 2^22
    const uint32_t ready_addr = lds_addr(&ready[0]);
    const uint32_t consumed_addr = lds_addr(&consumed[0]);
    const uint32_t poison_addr = lds_addr(&poison[0]);
    // Rows of a slab from row 16 j on, clamped to one step.
    auto step_rows = [&](int rows_left) {
        return __builtin_amdgcn_readfirstlane(
            rows_left < 0 ? 0 : (rows_left > kStepRows ? kStepRows : rows_left));
    };

    // ---- producer: raw P of a step into praw[k % kRawBufs], two 64-lane DMA
    // of 16 bytes for the 16 rows of grad_proj and, when dX is produced, one
    // of 4 bytes each for grad_r and r (the dW-only form is given neither).
    // Rows past the slab end read as zeros.
    const bool producer = wave == NW;
    constexpr int kRawDma = kDX ? 4 : 2;  // DMA instructions per step
    auto issue_raw = [&](int k, const StepCursor &at) {
        const int rl = step_rows(at.slab_rows - kStepRows * at.j);
        RawStep &d = praw[k % kRawBufs];
        const int64_t r0 = at.row0 + static_cast<int64_t>(kStepRows) * at.j;
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
    // counters and the poison word start at zero.
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
    if (tid == 0) lds_write_u32(poison_addr, 0u);

    if (producer) {
        StepCursor ahead = cursor_start(sg, L, T);
#pragma unroll
        for (int k = 0; k < kRawAhead; ++k) {
            issue_raw(k, ahead);
            cursor_next(ahead, G, L, T);
        }
        lds_barrier();
        // Lane = row * 4 + q converts j = 6q .. 6q + 5 of one row of P into
        // both operand layouts; lanes 0..15 also compute the RMS coefficient
        // grad_r / (r K) of row lane in FP32 (zero past the slab end).
        const int prow = lane / 4;
        const int pj0 = 6 * (lane % 4);
        StepCursor cur = cursor_start(sg, L, T);
        for (int k = 0; cur.slab_rows > 0; ++k) {
            issue_raw(k + kRawAhead, ahead);
            cursor_next(ahead, G, L, T);
            // The raw P of step k was requested before that of the kRawAhead
            // steps after it, kRawDma DMA instructions each.
            wait_vmcnt<kRawDma * kRawAhead>();
            const int slot = k % kSlots;
            if (!lds_wait_at_least(consumed_addr + 4 * slot, NW * static_cast<uint32_t>(k / kSlots), max_polls))
                lds_raise_poison(poison_addr, lane);
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
                const bool in_slab = kStepRows * cur.j + lane < cur.slab_rows;
                lds_write_u32(lds_addr(d.c + lane), __float_as_uint(in_slab ? grv / (rv * kf) : 0.f));
            }
            lds_signal(ready_addr + 4 * slot, lane);
            cursor_next(cur, G, L, T);
        }
        // Drain the copies still in flight before the workgroup's LDS can be
        // released.
        wait_vmcnt<0>();
        return;
    }

    // ---- compute waves: X ring, W in registers.
    const int64_t kw = static_cast<int64_t>(tile) * (NW * 64) + wave * 64;
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
    const int64_t row_bytes_d = K * 2;  // one row of dX or the addend
    const uint32_t ring_base = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(&xring[wave][0][0][0]));
    // The X request of the step `at` points to, into ring stage `stage`.
    auto issue_x = [&](const StepCursor &at, int stage) {
        const char *xs = reinterpret_cast<const char *>(x + (at.row0 + kStepRows * at.j) * K + kw);
        const __amdgpu_buffer_rsrc_t xrs =
            make_rsrc32(xs, range_elems(at.slab_rows - kStepRows * at.j) * 4);
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                xrs, (MHCPB_LDS void *)(&xring[wave][stage][rr][0]), 16, xoff[rr], 0, 0, MHCPB_X_AUX);
    };
    // Partial dW stores: after the transpose through LDS (store_partial
    // below) lane (c16, g) holds columns kw + 4 c16 .. + 3 of row j = 4 q + g
    // for q = 0..5; a lane past K gets an offset outside the slab's range, so
    // every partial write issues the same kPartialStores instructions.
    uint32_t poff[kPartialStores];
#pragma unroll
    for (int q = 0; q < kPartialStores; ++q)
        poff[q] = active ? static_cast<uint32_t>(((4 * q + g) * K + 4 * c16 + kw) * 4) : kOutOfRange;
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
    StepCursor nxt = cursor_start(sg, L, T);  // the next step whose X is requested
    issue_x(nxt, 0);
    cursor_next(nxt, G, L, T);
    issue_x(nxt, 1);
    cursor_next(nxt, G, L, T);
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
    // Writes the partial dW of slab `slab_s` (or NaN when `poisoned`) to the
    // workspace as whole 256-byte rows: the 32 x 64 block of accumulators
    // (lane (c16, g), element e of block b: column kw + 16 g + 4 e + i of
    // j = 16 b + c16) is transposed through `buf`, 4 KB of this wave's X ring
    // that no request is writing, in two halves (rows 0..15, then 16..23), so
    // that each store writes rows j = 4 q + g, columns kw + 4 c16 .. + 3.
    // Whole lines need no fill in the L2; the stores use the default policy,
    // so kernel 2 finds the slabs in the Infinity Cache.
    auto store_partial = [&](int slab_s, uint32_t buf, bool poisoned) {
        const __amdgpu_buffer_rsrc_t wrs =
            make_rsrc32(ws + static_cast<int64_t>(slab_s) * kProjCols * K, kProjCols * ki * 4);
        u32x4 tv[4];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            if (h == 0 || c16 < kProjCols - 16) {
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    lds_write_u128(buf + static_cast<uint32_t>((c16 * 64 + 16 * g + 4 * e) * 4),
                                   u32x4{__float_as_uint(accw[0][h][e]), __float_as_uint(accw[1][h][e]),
                                         __float_as_uint(accw[2][h][e]), __float_as_uint(accw[3][h][e])});
            }
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            constexpr int kQ = 4;
            const int nq = h == 0 ? 4 : 2;
#pragma unroll
            for (int q = 0; q < kQ; ++q)
                if (q < nq) tv[q] = lds_read_u128(buf + static_cast<uint32_t>(((4 * q + g) * 64 + 4 * c16) * 4));
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(tv[0]), "+v"(tv[1]), "+v"(tv[2]), "+v"(tv[3])::"memory");
            if (poisoned) {
#pragma unroll
                for (int q = 0; q < kQ; ++q) tv[q] = u32x4{0x7FC00000u, 0x7FC00000u, 0x7FC00000u, 0x7FC00000u};
            }
            compiler_fence();
#pragma unroll
            for (int q = 0; q < kQ; ++q)
                if (q < nq) __builtin_amdgcn_raw_buffer_store_b128(tv[q], wrs, poff[4 * h + q], 0, 0);
            compiler_fence();
        }
    };

    StepCursor cur = cursor_start(sg, L, T);  // the step being computed
    char *d_cur = reinterpret_cast<char *>(dx + cur.row0 * K + kw);
    const char *a_cur = reinterpret_cast<const char *>(addend + cur.row0 * K + kw);
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
    bool bad = false;           // this workgroup's results can no longer be trusted
    bool after_unit = false;    // the previous step ended a unit (its partial was stored)
    int last_unit_s = sg;       // slab of the unit whose partial is still to be stored
    for (int k = 0; cur.slab_rows > 0; ++k) {
        const int rows_left = cur.slab_rows - kStepRows * cur.j;
        // From the top of the step until the next X is requested the wave
        // runs at raised priority: once its X has arrived, the LDS reads and
        // the next request go ahead of the other waves' arithmetic on the
        // SIMD (about 1 % faster at T = 4096, K = 20480; the bits are those
        // of the same kernel without it).
        __builtin_amdgcn_s_setprio(1);
        const int slot = k % kSlots;
        asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(ready_seen)::"memory");
        const uint32_t want = static_cast<uint32_t>(k / kSlots + 1);
        if (__builtin_amdgcn_readfirstlane(ready_seen) < want &&
            !lds_wait_at_least(ready_addr + 4 * slot, want, max_polls)) {
            bad = true;
            lds_raise_poison(poison_addr, lane);
        }
        const StepP &cur_p = pop[slot];
        // The P operands of this step are requested first: the RMS
        // coefficients of rows 4g..4g+3, the dX P operands (token c16, part
        // p, j = 16b + 4g .. +3) and the dW P operands (part p, j = 16b +
        // c16, rows 4g .. 4g+3; entries j >= 24 are zero).
        f32x4 cc = {};
        u32x4 pa[2][2] = {};  // [part][block]
        u32x4 pbv[2] = {};    // [block]: part 0 in .xy, part 1 in .zw
        if constexpr (kDX) cc = lds_read_b128(lds_addr(cur_p.c + 4 * g));
#pragma unroll
        for (int b = 0; b < 2; ++b) {
            if constexpr (kDX) {
#pragma unroll
                for (int p = 0; p < 2; ++p)
                    pa[p][b] = lds_read_u128(
                        lds_addr(cur_p.pa + c16 * kPaStride + p * kJPad + 16 * b + 4 * g));
            }
            if constexpr (kDW)
                pbv[b] = lds_read_u128(lds_addr(cur_p.pb + (16 * b + c16) * kPbJStride + 8 * g));
        }
        // Then wait for this step's X and read it (4 rows).  Step k >= 1
        // issues, in this order: [4 addend loads] 4 X DMA (for step k + 1),
        // [4 dX stores of step k - 1 when deferred], [4 dX stores of step k
        // otherwise], [the kPartialStores partial stores when step k ends a
        // unit]; step 0 issues no X (the prologue requested steps 0 and 1,
        // after the W loads).  So after the X of step k come at most 4 dX
        // stores (of step k - 1, or of step k - 2 when deferred; none without
        // dX) and, when step k - 1 ended a unit, that unit's partial stores;
        // after the X of step 0 the X of step 1: vmcnt(4), or vmcnt(0) for
        // the later steps of the dW-only form, plus kPartialStores after a
        // unit's end, covers it.  With deferred stores step 0 stores nothing,
        // so step 1 waits for vmcnt(0) (or the partial stores alone).  For
        // step 1 with the addend, step 0's addend loads come after the X of
        // step 1 as well, and the wait is only stricter.  Steps past the slab
        // end are still requested (they read zeros; their stores fall outside
        // the range), which keeps every step's count identical.
        const bool four = k == 0 || (kDX && !(kDefer && k == 1));
        if (!after_unit || !kDW) {
            if (four)
                wait_vmcnt<4>();
            else
                wait_vmcnt<0>();
        } else {
            if (four)
                wait_vmcnt<4 + kPartialStores>();
            else
                wait_vmcnt<kPartialStores>();
        }
        const uint32_t xa = ring_base + static_cast<uint32_t>((((k & 1) * 4) * kWave + lane) * 16);
        f32x4 xc[4];
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) xc[rr] = lds_read_b128(xa + rr * kWave * 16);
        // The poison word is read after the slot: a producer that gave up
        // raised it before it overwrote a slot.
        uint32_t pois = lds_read_u32(poison_addr);
        // The wait names every register the reads above return, so no use
        // of them can be scheduled before the data has arrived.
        if constexpr (kDX && kDW)
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(xc[0]), "+v"(xc[1]), "+v"(xc[2]), "+v"(xc[3]), "+v"(cc),
                           "+v"(pa[0][0]), "+v"(pa[0][1]), "+v"(pa[1][0]), "+v"(pa[1][1]),
                           "+v"(pbv[0]), "+v"(pbv[1]), "+v"(pois)::"memory");
        else if constexpr (kDX)
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(xc[0]), "+v"(xc[1]), "+v"(xc[2]), "+v"(xc[3]), "+v"(cc),
                           "+v"(pa[0][0]), "+v"(pa[0][1]), "+v"(pa[1][0]),
                           "+v"(pa[1][1]), "+v"(pois)::"memory");
        else
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(xc[0]), "+v"(xc[1]), "+v"(xc[2]), "+v"(xc[3]), "+v"(pbv[0]),
                           "+v"(pbv[1]), "+v"(pois)::"memory");
        bad = bad || __builtin_amdgcn_readfirstlane(pois) != 0;
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
        }
        compiler_fence();
        if (k > 0) {
            issue_x(nxt, (k + 1) & 1);
            cursor_next(nxt, G, L, T);
        }
        compiler_fence();
        __builtin_amdgcn_s_setprio(0);
        if (kDefer && k > 0) {
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
        if (bad) {  // results past a give-up are not trusted: two BF16 NaNs per word
#pragma unroll
            for (int rr = 0; rr < 4; ++rr) packed[rr][0] = packed[rr][1] = 0x7FC07FC0u;
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
        if constexpr (kAddend) a_cur += kStepRows * row_bytes_d;
        ready_seen = lds_read_u32(ready_addr + 4 * ((k + 1) % kSlots));
        const int s_done = sg + cur.u * G;
        after_unit = cursor_next(cur, G, L, T);
        if (after_unit) {
            d_cur = reinterpret_cast<char *>(dx + cur.row0 * K + kw);
            if constexpr (kAddend) a_cur = reinterpret_cast<const char *>(addend + cur.row0 * K + kw);
        }
        // At the end of a unit that is not the last, its partial dW goes to
        // workspace slab s_done while the X of the next unit is already in
        // flight (through ring stage k & 1, which holds no request until the
        // next step); the accumulators restart from zero.  The last unit's
        // partial is stored after the drain below.
        if (kDW && after_unit) {
            if (cur.slab_rows > 0) {
                store_partial(s_done, ring_base + static_cast<uint32_t>((k & 1) * 4 * kWave * 16), bad);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int jb = 0; jb < 2; ++jb) accw[i][jb] = f32x4{0.f, 0.f, 0.f, 0.f};
            } else {
                last_unit_s = s_done;
            }
        }
    }
    if constexpr (kDefer) {  // the last step's stores
        const __amdgpu_buffer_rsrc_t prs =
            make_rsrc32(uniform_ptr(d_prev), __builtin_amdgcn_readfirstlane(d_range_prev));
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
            __builtin_amdgcn_raw_buffer_store_b64(u32x2{pend[rr][0], pend[rr][1]}, prs, doff[rr],
                                                  0, MHCPB_DX_AUX);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(ready_seen)::"memory");
    // Drain the X DMA still in flight (the steps past the last unit) before
    // the workgroup's LDS can be released.
    wait_vmcnt<0>();

    // Partial dW of the last unit, written once to workspace slab
    // last_unit_s (the ring is idle after the drain).
    if constexpr (kDW) store_partial(last_unit_s, ring_base, bad);
}

// dW[i] = (((ws[0][i] + ws[1][i]) + ws[2][i]) + ...), four elements (one
// quad) per column group; a thread takes kReduceQuads quads spaced by the
// grid's thread count, and requests eight slabs of each of them before it
// adds them in order, so that 8 x kReduceQuads loads are in flight.
#ifndef MHCPB_K2_QPT
#define MHCPB_K2_QPT 1
#endif
constexpr int kReduceBatch = 8;
constexpr int kReduceQuads = MHCPB_K2_QPT;
__global__ __launch_bounds__(256) void reduce_slabs(const float *__restrict__ ws,
                                                    float *__restrict__ dw, int S,
                                                    int64_t n4) {
    const int64_t nthreads = static_cast<int64_t>(gridDim.x) * blockDim.x;
    const int64_t i0 = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const f32x4 *src = reinterpret_cast<const f32x4 *>(ws);
    f32x4 a[kReduceQuads];
#pragma unroll
    for (int q = 0; q < kReduceQuads; ++q) {
        const int64_t i = i0 + q * nthreads;
        a[q] = i < n4 ? __builtin_nontemporal_load(src + i) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    for (int s0 = 1; s0 < S; s0 += kReduceBatch) {
        f32x4 b[kReduceQuads][kReduceBatch];
        // Past the last slab the addend is -0, which leaves every sum as it
        // is (x + -0 == x, signed zeros included).
#pragma unroll
        for (int q = 0; q < kReduceQuads; ++q)
#pragma unroll
            for (int u = 0; u < kReduceBatch; ++u) {
                const int64_t i = i0 + q * nthreads;
                b[q][u] = (s0 + u < S && i < n4)
                              ? __builtin_nontemporal_load(src + static_cast<int64_t>(s0 + u) * n4 + i)
                              : f32x4{-0.f, -0.f, -0.f, -0.f};
            }
#pragma unroll
        for (int q = 0; q < kReduceQuads; ++q)
#pragma unroll
            for (int u = 0; u < kReduceBatch; ++u) a[q] += b[q][u];
    }
#pragma unroll
    for (int q = 0; q < kReduceQuads; ++q) {
        const int64_t i = i0 + q * nthreads;
        if (i < n4) reinterpret_cast<f32x4 *>(dw)[i] = a[q];
    }
}

// Slab groups G of kernel 1: enough workgroups (tiles x G) for one per CU of
// a 256-CU GPU where the tiles allow it, never more groups than slabs.  A
// performance choice only: no bit of the result depends on it.
constexpr int kTargetWorkgroups = 256;
inline int slab_groups(int tiles, int S) {
    int G = kTargetWorkgroups / (tiles > 0 ? tiles : 1);
    if (G > S) G = S;
    return G < 1 ? 1 : G;
}

template <int NW>
hipError_t launch_projection_t(const Plan &p, const Args &a, Outputs out, hipStream_t stream,
                               hipEvent_t start, hipEvent_t stop) {
    constexpr int cols = NW * 64;
    const int tiles = static_cast<int>((p.K + cols - 1) / cols);
    const int G = slab_groups(tiles, p.S);
    const dim3 grid(static_cast<unsigned>(tiles) * static_cast<unsigned>(G));
    const dim3 block((NW + 1) * kWave);
#define MHCPB_LAUNCH(ADD, DX, DW)                                                               \
    return launch(projection_kernel<NW, ADD, DX, DW>, grid, block, stream, start, stop, a.x, a.w, \
           a.grad_proj, a.grad_r, a.r, a.dx, a.ws, a.addend, p.T, p.K, p.L, p.S, tiles, G,     \
           p.wait_polls)
    switch (out) {
    case Outputs::kBoth:
        if (a.addend)
            MHCPB_LAUNCH(true, true, true);
        else
            MHCPB_LAUNCH(false, true, true);
    case Outputs::kDxOnly:
        if (a.addend)
            MHCPB_LAUNCH(true, true, false);
        else
            MHCPB_LAUNCH(false, true, false);
    case Outputs::kDwOnly:
        MHCPB_LAUNCH(false, false, true);
    }
#undef MHCPB_LAUNCH
    return hipErrorInvalidValue;
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
    const unsigned blocks = static_cast<unsigned>((n4 + 256 * kReduceQuads - 1) / (256 * kReduceQuads));
    return launch(reduce_slabs, dim3(blocks), dim3(256), stream, nullptr, stop, a.ws, a.dw, p.S, n4);
}

// Static workspace for callers that cannot allocate (mhcpb_execute_noalloc).
// One copy per GPU, held from the library's load until the process ends; the
// kernels take the address hipGetSymbolAddress gives for the current device,
// never the host-side name of the array.
namespace {
static __device__ __align__(256) unsigned char scratch[kStaticWorkspaceBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t static_workspace(void **ptr) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        if (!p) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return hipSuccess;
}

}  // namespace mhcpb
