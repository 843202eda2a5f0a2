// Kernels of the DSv4.1 mHC projection/RMS backward for gfx950.
//
// Kernel 1 ("projection"): T is cut into S slabs (S a function of T only)
// and K into column tiles; the grid is (column tiles) x (slab groups), each
// workgroup walking a run of consecutive slabs of its tile.  For each slab it
// reads the slab's rows of X exactly once, writes the matching dX, and keeps
// the slab's dW[24, tile] partial in MFMA accumulators; the partial goes to
// workspace slab s (one writer per element), except that the workgroups
// holding slabs 0, 1, ... add theirs up first, in that order, and store the
// sum.  Kernel 2 ("reduce"): dW = ((slab 0 + slab 1) + slab 2) + ... in FP32,
// starting from that sum.  This follows the page's structure (the token
// reduction split over independent blocks, partial weight gradients, then a
// second reduction kernel: "Source attribution" section).
//
// Both products run on v_mfma_f32_16x16x32_bf16.  A TF32 operand has 11
// significant bits; it splits exactly into a BF16 high part (its upper 16
// bits) and a BF16 low part (the remaining 3 bits), so the four BF16 partial
// products hi*hi, hi*lo, lo*hi, lo*lo are exact and their FP32 sum is the
// TF32 product accumulated in FP32.  Each MFMA k slot pairs one part of one
// operand with one part of the other: for dX the W side is held in registers
// as packed (hi, lo) pairs and the P side is staged in LDS with each part
// repeated, 3 MFMAs per 16x16 output block (the 96 products of 24 j); for dW
// the X side is split in registers and the P side is staged per part, twice
// over, 4 MFMAs per column group (24 j padded to 32).  No operand needs a
// per-step shuffle.
//
// X is streamed from HBM straight into LDS with buffer_load_dwordx4 ... lds,
// a two-step ring per wave, so prefetching costs no registers; rows past the
// slab end fall outside the buffer range and arrive as zeros.  The P rows of
// each step arrive the same way a few steps ahead.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstddef>
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
// non-temporal as well.  Write-through stores (sc1) are faster only while the
// whole dX fits the 256 MB Infinity Cache and the next call rewrites the same
// buffer (T = 4096, one buffer: 87 against 92 us per call); with the buffers
// rotated, or at T = 16384, they are 2-5 % slower.
#ifndef MHCPB_DX_AUX
#define MHCPB_DX_AUX 2
#endif

// Rows per step (one MFMA row block) and the LDS layouts of P.
constexpr int kStepRows = 16;
constexpr int kPaStride = 2 * kProjCols + 4;  // uint32 per row of the dX P operand (4 padding)
constexpr int kPbEntries = kProjCols + 1;     // j entries of the dW P operand, the last one zero
constexpr int kPbJStride = 72;                // uint16 per j entry (64 + 8 padding)

// The P of one step as it is stored in HBM, copied by LDS DMA: 16 rows of
// grad_proj (32 floats each; the last 8 are never read from here), and one
// grad_r and r entry per DMA lane (only the first 16 are used).
struct RawStep {
    f32x4 p[kStepRows * kProjStride / 4];
    float gr[kWave];
    float r[kWave];
};

// The P of one step in operand form (TF32 split into BF16 high and low parts):
//  pa[row][part * 24 + j]: the part, duplicated in both halves of the word, as
//      the dX product reads it (4 consecutive j per lane group);
//  pb[j][g][part][h][r]: the part of row 4g + r, twice (h = 0, 1), as the dW
//      product reads it: 16 bytes hold one part of 4 consecutive rows, once
//      against the high and once against the low part of x.  Entry j = 24 is
//      zero (cleared once) and stands for every padded j of that product;
//  c[row]: grad_r / (r K).
struct alignas(16) StepP {
    uint32_t pa[kStepRows * kPaStride];
    uint16_t pb[kPbEntries * kPbJStride];
    float c[kStepRows];
};

// Operand slots in rotation, and how many steps ahead of its conversion the
// producer requests the raw P of a step.
constexpr int kSlots = 4;
constexpr int kRawAhead = 2;
constexpr int kRawBufs = kRawAhead + 1;

// Kernel 1.  A workgroup has NW compute waves, which own the NW * 64 columns
// of one column tile, and one producer wave.  The workgroup walks, one after
// the other, the consecutive slabs [sg S / G, (sg + 1) S / G) of its tile (sg
// = its slab group, G <= S groups): one unit of work per slab, each unit's
// rows in ascending 16-row steps, and the steps of all its units form one
// continuous sequence (global step k).  Per step a compute wave handles 16 rows x 64 columns:
// lane l (c = l % 16, g = l / 16) holds x[t0 + 4g + r][kw + 4c + i] for r, i
// in 0..3.
//  dX: C_i[e] = dX[t0 + 4g + e][kw + 4c + i] = c_t x + the products of the P
//      parts (token t0 + l%16) with the W parts (column kw + 4c + i): in
//      the MFMAs of P part p = 0, 1 lane group g covers j = 4g .. 4g + 3
//      times (W hi, W lo); in the third, j = 16 + 4 (g % 2) .. +3 of P part
//      g / 2, so 3 MFMAs cover the 96 products of 24 j.
//  dW: acc[i][b][e] = sum over the slab's tokens of TF32(x) of column
//      kw + 4(4g+e) + i times TF32(P[j]), j = 16 b + l%16: per MFMA (P part
//      p), lane group g covers rows 4g .. 4g+3 times (x hi, x lo).  At the
//      end of each unit the 24 x 64 partial goes to workspace slab s and the
//      accumulators restart from zero.
//
// Why one workgroup walks several slabs: a workgroup needs 6 waves and
// more than 64 KB of LDS, so a CU holds one at a time; with one workgroup per (tile,
// slab) the supported profile (64 tiles x 8 slabs) ran as two rounds of 256
// workgroups, each with its own start-up (the first X and W requests) and
// drain.  With G = 4 slab groups the 256 workgroups each stream two slabs
// back to back: the X of the next unit is requested while the last step of
// the current one is computed and its partial is stored.  Group 0 holds the
// first slabs, so it can also add their partials up in the order kernel 2
// would (one slab fewer to write and to read back at that profile).  A
// column's dW sums the same rows in the same order whatever the grouping, so
// the grouping changes no bit of the result.
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
    int s;          // slab of the current unit
    int s_end;      // one past the workgroup's last slab
    int j;
    int nst;        // steps of the current slab
    int slab_rows;  // rows of the current slab (0 past the last unit)
    int64_t row0;   // first row of the current slab
};

// First slab of slab group sg: the G groups split the S slabs into runs of
// consecutive slabs, as even as they can be (G <= S, so none is empty).
__device__ __forceinline__ int group_first_slab(int sg, int S, int G) {
    return static_cast<int>((static_cast<int64_t>(sg) * S) / G);
}

__device__ __forceinline__ int slab_rows_at(int64_t row0, int64_t L, int64_t T) {
    const int64_t n = T - row0 < L ? T - row0 : L;
    return static_cast<int>(n > 0 ? n : 0);
}

__device__ __forceinline__ StepCursor cursor_start(int sg, int S, int G, int64_t L, int64_t T) {
    StepCursor c;
    c.s = group_first_slab(sg, S, G);
    c.s_end = group_first_slab(sg + 1, S, G);
    c.j = 0;
    c.row0 = static_cast<int64_t>(c.s) * L;
    c.slab_rows = slab_rows_at(c.row0, L, T);
    c.nst = (c.slab_rows + 15) / 16;
    return c;
}

// Advances by one step; returns true when the step left was the last of its
// unit.
__device__ __forceinline__ bool cursor_next(StepCursor &c, int64_t L, int64_t T) {
    if (++c.j < c.nst) return false;
    c.j = 0;
    ++c.s;
    c.row0 += L;
    c.slab_rows = c.s < c.s_end ? slab_rows_at(c.row0, L, T) : 0;
    c.nst = (c.slab_rows + 15) / 16;
    return true;
}

// Number of store instructions of one partial dW write (per compute wave).
constexpr int kPartialStores = 6;

// The producer's writes of j = pj0 + E and pj0 + E + 1 (E even) of one row
// into the dX operand: pa_hi points at the row's part 0 entry of j = pj0.
template <int E>
__device__ __forceinline__ void put_pa(uint32_t pa_hi, uint32_t a, uint32_t b) {
    lds_write_u64<4 * E>(pa_hi, u32x2{dup_low_half(a), dup_low_half(b)});
    lds_write_u64<4 * E + 4 * kProjCols>(pa_hi, u32x2{dup_high_half(a), dup_high_half(b)});
}

// The producer's writes of j = pj0 + E of one row into the dW operand:
// pb0 points at pb[pj0][g][0][0][r]; 8 bytes lie between the two copies, 16
// between the parts.
template <int E>
__device__ __forceinline__ void put_pb(uint32_t pb0, uint32_t v) {
    constexpr int o = E * kPbJStride * 2;
    lds_write_u16<o>(pb0, v);
    lds_write_u16<o + 8>(pb0, v);
    lds_write_u16_hi<o + 16>(pb0, v);
    lds_write_u16_hi<o + 24>(pb0, v);
}

// What a compute wave reads from LDS at the top of a step.
struct StepRead {
    f32x4 cc;          // RMS coefficients of rows 4g .. 4g + 3
    u32x4 pa[3];       // dX P operands: parts 0 and 1 of j = 4g .. 4g + 3, then block 1
    u32x4 pb[2][2];    // dW P operands [part][block]
    f32x4 xc[4];       // the step's X, 4 rows
    uint32_t pois;     // the workgroup's poison word
    uint32_t ready;    // ready count of the next step's slot
    uint32_t mate;     // steps begun by the compute wave that shares this one's SIMD
};

// The LDS reads of one step as a single asm statement that ends with the
// wait for all of them (the destination of an asm load holds no value the
// compiler may use until a wait in the same statement has passed): the P
// operands of the step's slot (a_c, a_pa, a_pa3, a_pb[2]; the forms without
// dX or without dW skip theirs), then the wait for this step's X
// (vmcnt(kVm), chosen by the caller), the four X rows at xa (64 lanes x 16
// bytes apart), the poison word and the next slot's ready count.
template <int kVm, bool kDX, bool kDW>
__device__ __forceinline__ void read_step(StepRead &r, uint32_t a_c, uint32_t a_pa, uint32_t a_pa3,
                                          uint32_t a_pb0, uint32_t a_pb1, uint32_t xa,
                                          uint32_t a_pois, uint32_t a_ready, uint32_t a_mate) {
    static_assert(kVm >= 0 && kVm < 64, "vmcnt range");
    if constexpr (kDX && kDW) {
        asm volatile(
            "ds_read_b128 %0, %15\n\t"
            "ds_read_b128 %1, %16\n\t"
            "ds_read_b128 %2, %16 offset:%24\n\t"
            "ds_read_b128 %3, %17\n\t"
            "ds_read_b128 %4, %18\n\t"
            "ds_read_b128 %5, %19\n\t"
            "ds_read_b128 %6, %18 offset:16\n\t"
            "ds_read_b128 %7, %19 offset:16\n\t"
            "s_waitcnt vmcnt(%25)\n\t"
            "ds_read_b128 %8, %20\n\t"
            "ds_read_b128 %9, %20 offset:1024\n\t"
            "ds_read_b128 %10, %20 offset:2048\n\t"
            "ds_read_b128 %11, %20 offset:3072\n\t"
            "ds_read_b32 %12, %21\n\t"
            "ds_read_b32 %13, %22\n\t"
            "ds_read_b32 %14, %23\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(r.cc), "=&v"(r.pa[0]), "=&v"(r.pa[1]), "=&v"(r.pa[2]), "=&v"(r.pb[0][0]),
              "=&v"(r.pb[0][1]), "=&v"(r.pb[1][0]), "=&v"(r.pb[1][1]), "=&v"(r.xc[0]),
              "=&v"(r.xc[1]), "=&v"(r.xc[2]), "=&v"(r.xc[3]), "=&v"(r.pois), "=&v"(r.ready),
              "=&v"(r.mate)
            : "v"(a_c), "v"(a_pa), "v"(a_pa3), "v"(a_pb0), "v"(a_pb1), "v"(xa), "v"(a_pois),
              "v"(a_ready), "v"(a_mate), "n"(4 * kProjCols), "n"(kVm)
            : "memory");
    } else if constexpr (kDX) {
        asm volatile(
            "ds_read_b128 %0, %11\n\t"
            "ds_read_b128 %1, %12\n\t"
            "ds_read_b128 %2, %12 offset:%18\n\t"
            "ds_read_b128 %3, %13\n\t"
            "s_waitcnt vmcnt(%19)\n\t"
            "ds_read_b128 %4, %14\n\t"
            "ds_read_b128 %5, %14 offset:1024\n\t"
            "ds_read_b128 %6, %14 offset:2048\n\t"
            "ds_read_b128 %7, %14 offset:3072\n\t"
            "ds_read_b32 %8, %15\n\t"
            "ds_read_b32 %9, %16\n\t"
            "ds_read_b32 %10, %17\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(r.cc), "=&v"(r.pa[0]), "=&v"(r.pa[1]), "=&v"(r.pa[2]), "=&v"(r.xc[0]),
              "=&v"(r.xc[1]), "=&v"(r.xc[2]), "=&v"(r.xc[3]), "=&v"(r.pois), "=&v"(r.ready),
              "=&v"(r.mate)
            : "v"(a_c), "v"(a_pa), "v"(a_pa3), "v"(xa), "v"(a_pois), "v"(a_ready), "v"(a_mate),
              "n"(4 * kProjCols), "n"(kVm)
            : "memory");
    } else {
        asm volatile(
            "ds_read_b128 %0, %11\n\t"
            "ds_read_b128 %1, %12\n\t"
            "ds_read_b128 %2, %11 offset:16\n\t"
            "ds_read_b128 %3, %12 offset:16\n\t"
            "s_waitcnt vmcnt(%17)\n\t"
            "ds_read_b128 %4, %13\n\t"
            "ds_read_b128 %5, %13 offset:1024\n\t"
            "ds_read_b128 %6, %13 offset:2048\n\t"
            "ds_read_b128 %7, %13 offset:3072\n\t"
            "ds_read_b32 %8, %14\n\t"
            "ds_read_b32 %9, %15\n\t"
            "ds_read_b32 %10, %16\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(r.pb[0][0]), "=&v"(r.pb[0][1]), "=&v"(r.pb[1][0]), "=&v"(r.pb[1][1]),
              "=&v"(r.xc[0]), "=&v"(r.xc[1]), "=&v"(r.xc[2]), "=&v"(r.xc[3]), "=&v"(r.pois),
              "=&v"(r.ready), "=&v"(r.mate)
            : "v"(a_pb0), "v"(a_pb1), "v"(xa), "v"(a_pois), "v"(a_ready), "v"(a_mate), "n"(kVm)
            : "memory");
    }
}

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
    __shared__ uint32_t ready[kSlots], consumed[kSlots], poison[1], prog[NW];
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

    // The zero entry of the dW P operand of every slot; the counters and the
    // poison word start at zero.
    constexpr int kPbWords = kPbJStride / 2;  // uint32 per entry
    for (int i = tid; i < kSlots * kPbWords; i += kThreads)
        lds_write_u32(lds_addr(pop[i / kPbWords].pb + kProjCols * kPbJStride) + 4 * (i % kPbWords), 0u);
    if (tid < kSlots) {
        lds_write_u32(ready_addr + 4 * tid, 0u);
        lds_write_u32(consumed_addr + 4 * tid, 0u);
    }
    if (tid == 0) lds_write_u32(poison_addr, 0u);
    if (tid < NW) lds_write_u32(lds_addr(&prog[tid]), 0u);

    if (producer) {
        StepCursor ahead = cursor_start(sg, S, G, L, T);
#pragma unroll
        for (int k = 0; k < kRawAhead; ++k) {
            issue_raw(k, ahead);
            cursor_next(ahead, L, T);
        }
        lds_barrier();
        // Lane = row * 4 + q converts j = 6q .. 6q + 5 of one row of P into
        // both operand layouts; lanes 0..15 also compute the RMS coefficient
        // grad_r / (r K) of row lane in FP32 (zero past the slab end).
        const int prow = lane / 4;
        const int pj0 = 6 * (lane % 4);
        StepCursor cur = cursor_start(sg, S, G, L, T);
        for (int k = 0; cur.slab_rows > 0; ++k) {
            issue_raw(k + kRawAhead, ahead);
            cursor_next(ahead, L, T);
            // The raw P of step k was requested before that of the kRawAhead
            // steps after it, kRawDma DMA instructions each.
            wait_vmcnt<kRawDma * kRawAhead>();
            const int slot = k % kSlots;
            if (!lds_wait_at_least(consumed_addr + 4 * slot, NW * static_cast<uint32_t>(k / kSlots), max_polls))
                lds_raise_poison(poison_addr, lane);
            const RawStep &src = praw[k % kRawBufs];
            const StepP &d = pop[slot];
            const uint32_t ra = lds_addr(&src.p[0]) + static_cast<uint32_t>((prow * kProjStride + pj0) * 4);
            u32x2 v0, v1, v2;
            float grv = 0.f, rv = 1.f;
            if constexpr (kDX) {
                const uint32_t rl = lds_addr(&src) + 4 * lane;
                asm volatile(
                    "ds_read_b64 %0, %5\n\t"
                    "ds_read_b64 %1, %5 offset:8\n\t"
                    "ds_read_b64 %2, %5 offset:16\n\t"
                    "ds_read_b32 %3, %6 offset:%7\n\t"
                    "ds_read_b32 %4, %6 offset:%8\n\t"
                    "s_waitcnt lgkmcnt(0)"
                    : "=&v"(v0), "=&v"(v1), "=&v"(v2), "=&v"(grv), "=&v"(rv)
                    : "v"(ra), "v"(rl), "n"(offsetof(RawStep, gr)), "n"(offsetof(RawStep, r))
                    : "memory");
            } else {
                asm volatile(
                    "ds_read_b64 %0, %3\n\t"
                    "ds_read_b64 %1, %3 offset:8\n\t"
                    "ds_read_b64 %2, %3 offset:16\n\t"
                    "s_waitcnt lgkmcnt(0)"
                    : "=&v"(v0), "=&v"(v1), "=&v"(v2)
                    : "v"(ra)
                    : "memory");
            }
            const uint32_t vv[6] = {v0.x, v0.y, v1.x, v1.y, v2.x, v2.y};
            uint32_t pk[6];  // hi | lo << 16
#pragma unroll
            for (int e = 0; e < 6; ++e) pk[e] = tf32_split_packed_p(__uint_as_float(vv[e]));
            const uint32_t pa_hi = lds_addr(d.pa + prow * kPaStride + pj0);
            put_pa<0>(pa_hi, pk[0], pk[1]);
            put_pa<2>(pa_hi, pk[2], pk[3]);
            put_pa<4>(pa_hi, pk[4], pk[5]);
            // pb[j][g][part][h][r] with g = prow / 4, r = prow % 4.
            const uint32_t pb0 = lds_addr(d.pb + pj0 * kPbJStride + (prow / 4) * 16 + prow % 4);
            put_pb<0>(pb0, pk[0]);
            put_pb<1>(pb0, pk[1]);
            put_pb<2>(pb0, pk[2]);
            put_pb<3>(pb0, pk[3]);
            put_pb<4>(pb0, pk[4]);
            put_pb<5>(pb0, pk[5]);
            if (kDX && lane < kStepRows) {
                const bool in_slab = kStepRows * cur.j + lane < cur.slab_rows;
                lds_write_u32(lds_addr(d.c + lane), __float_as_uint(in_slab ? grv / (rv * kf) : 0.f));
            }
            lds_signal(ready_addr + 4 * slot, lane);
            cursor_next(cur, L, T);
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
    // Byte offsets, within an operand slot, of this lane's P operands: the
    // RMS coefficients of rows 4g .. 4g + 3; the dX P operands of token c16
    // (part 0 of j = 4g .. 4g + 3, part 1 4 kProjCols bytes on, and the
    // third MFMA's j = 16 + 4 (g % 2) .. +3 of part g / 2); the dW P operands
    // of j = c16 and of j = 16 + c16 or, past j = 23, the zero entry (part 1
    // 16 bytes on).
    const uint32_t off_c = static_cast<uint32_t>(offsetof(StepP, c) + 16 * g);
    const uint32_t off_pa = static_cast<uint32_t>((c16 * kPaStride + 4 * g) * 4);
    const uint32_t off_pa3 =
        static_cast<uint32_t>((c16 * kPaStride + (g >> 1) * kProjCols + 16 + 4 * (g & 1)) * 4);
    const uint32_t off_pb[2] = {
        static_cast<uint32_t>(offsetof(StepP, pb) + (c16 * kPbJStride + 16 * g) * 2),
        static_cast<uint32_t>(offsetof(StepP, pb) +
                              ((c16 < kProjCols - 16 ? 16 + c16 : kProjCols) * kPbJStride + 16 * g) * 2)};
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
    // [j block][e]: W[jb + e][col .. col + 3] with jb = 4 g in block 0 and
    // 16 + 4 (g % 2) in block 1 (j = 16..23 twice, once per P part).
    float4 wraw[2][4] = {};
    if constexpr (kDX) {
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int jj = (b == 0 ? 4 * g : 16 + 4 * (g & 1)) + e;
                wraw[b][e] = active ? *reinterpret_cast<const float4 *>(w + jj * K + col)
                                    : make_float4(0.f, 0.f, 0.f, 0.f);
            }
    }
    compiler_fence();
    StepCursor nxt = cursor_start(sg, S, G, L, T);  // the next step whose X is requested
    issue_x(nxt, 0);
    cursor_next(nxt, L, T);
    issue_x(nxt, 1);
    cursor_next(nxt, L, T);
    compiler_fence();
    // Padding and counters visible (the producer passes the same barrier).
    lds_barrier();

    // W side of the dX product: for column variant i and j block b the lane
    // holds the packed (hi | lo << 16) TF32 split of W[j][col + i] for the
    // four j of wraw[b].
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
            // Rows 4 q + g, q < nq, 1 KB apart.
            const uint32_t tb = buf + static_cast<uint32_t>((g * 64 + 4 * c16) * 4);
            if (h == 0) {
                asm volatile(
                    "ds_read_b128 %0, %4\n\t"
                    "ds_read_b128 %1, %4 offset:1024\n\t"
                    "ds_read_b128 %2, %4 offset:2048\n\t"
                    "ds_read_b128 %3, %4 offset:3072\n\t"
                    "s_waitcnt lgkmcnt(0)"
                    : "=&v"(tv[0]), "=&v"(tv[1]), "=&v"(tv[2]), "=&v"(tv[3])
                    : "v"(tb)
                    : "memory");
            } else {
                asm volatile(
                    "ds_read_b128 %0, %2\n\t"
                    "ds_read_b128 %1, %2 offset:1024\n\t"
                    "s_waitcnt lgkmcnt(0)"
                    : "=&v"(tv[0]), "=&v"(tv[1])
                    : "v"(tb)
                    : "memory");
            }
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

    StepCursor cur = cursor_start(sg, S, G, L, T);  // the step being computed
    // Waves go to the four SIMDs in turn, so of five compute waves and the
    // producer, waves 0 and 4 share a SIMD (and wave 1 the producer's).
    const int mate = (NW == 5 && (wave == 0 || wave == 4)) ? 4 - wave : wave;
    const uint32_t mate_addr = lds_addr(&prog[mate]);
    const uint32_t my_prog_addr = lds_addr(&prog[wave]);
    char *d_cur = reinterpret_cast<char *>(dx + cur.row0 * K + kw);
    const char *a_cur = reinterpret_cast<const char *>(addend + cur.row0 * K + kw);
    // The ready count of a step's slot is read one step early (with the
    // previous step's LDS reads), so that its round trip is off the step's
    // critical path.
    uint32_t ready_seen = lds_load_u32(ready_addr);
    // With the addend, the dX stores of a step are issued one step late,
    // right after the next X request (same bits; at T = 16384 with the
    // addend 466 against 475 us, while without it they cost about 2 us at
    // T = 4096, so only this form defers them).
    constexpr bool kDefer = kAddend && kDX;
    uint32_t pend[4][2] = {};
    char *d_prev = d_cur;
    int d_range_prev = 0;
    bool bad = false;           // this workgroup's results can no longer be trusted
    bool stored = false;        // the previous step ended a unit and stored its partial
    int last_unit_s = cur.s;    // slab of the unit whose partial is still to be stored
    // Slab group 0 adds the partials of its slabs (0, 1, ...) up in
    // registers, in that order, and stores only the sum, into its last slab:
    // the first adds of kernel 2's ascending order, the same FP32 operations
    // in the same order, done before the partials leave the CU (-0 is the
    // identity of x + y, signed zeros included).
    const bool fold = sg == 0;
    f32x4 pref[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) pref[i][jb] = f32x4{-0.f, -0.f, -0.f, -0.f};
    for (int k = 0; cur.slab_rows > 0; ++k) {
        const int rows_left = cur.slab_rows - kStepRows * cur.j;
        // From the top of the step until the next X is requested the wave
        // runs at raised priority: once its X has arrived, the LDS reads and
        // the next request go ahead of the other waves' arithmetic on the
        // SIMD (about 1 % faster at T = 4096, K = 20480; the bits are those
        // of the same kernel without it).
        __builtin_amdgcn_s_setprio(1);
        const int slot = k % kSlots;
        const uint32_t want = static_cast<uint32_t>(k / kSlots + 1);
        if (__builtin_amdgcn_readfirstlane(ready_seen) < want &&
            !lds_wait_at_least(ready_addr + 4 * slot, want, max_polls)) {
            bad = true;
            lds_raise_poison(poison_addr, lane);
        }
        // The P operands of this step are requested first: the RMS
        // coefficients of rows 4g..4g+3, the dX P operands (token c16, part
        // p, j = 16b + 4g .. +3) and the dW P operands (part p, j = 16b +
        // c16, rows 4g .. 4g+3; entries j >= 24 are zero).  Then the wait for
        // this step's X, and its 4 rows.  Step k >= 1 issues, in this order:
        // [4 addend loads] 4 X DMA (for step k + 1), [4 dX stores of step
        // k - 1 when deferred], [4 dX stores of step k otherwise], [the
        // kPartialStores partial stores when step k ends a unit]; step 0
        // issues no X (the prologue requested steps 0 and 1, after the W
        // loads).  So after the X of step k come at most 4 dX stores (of step
        // k - 1, or of step k - 2 when deferred; none without dX) and, when
        // step k - 1 ended a unit and stored its partial, those stores;
        // after the X of step 0 the X of step 1: vmcnt(4), or vmcnt(0) for
        // the later steps of the dW-only form, plus kPartialStores after a
        // unit's end, covers it.  With deferred stores step 0 stores nothing,
        // so step 1 waits for vmcnt(0) (or the partial stores alone).  For
        // step 1 with the addend, step 0's addend loads come after the X of
        // step 1 as well, and the wait is only stricter.  Steps past the slab
        // end are still requested (they read zeros; their stores fall outside
        // the range), which keeps every step's count identical.  The poison
        // word is read after the slot: a producer that gave up raised it
        // before it overwrote a slot.
        const uint32_t slot_base = lds_addr(&pop[slot]);
        const uint32_t xa = ring_base + static_cast<uint32_t>((((k & 1) * 4) * kWave + lane) * 16);
        const uint32_t a_ready = ready_addr + 4 * ((k + 1) % kSlots);
        StepRead rd;
        const bool four = k == 0 || (kDX && !(kDefer && k == 1));
#define MHCPB_READ_STEP(VM)                                                                     \
    read_step<VM, kDX, kDW>(rd, slot_base + off_c, slot_base + off_pa, slot_base + off_pa3,    \
                            slot_base + off_pb[0], slot_base + off_pb[1], xa, poison_addr,    \
                            a_ready, mate_addr)
        if (!stored || !kDW) {
            if (four)
                MHCPB_READ_STEP(4);
            else
                MHCPB_READ_STEP(0);
        } else {
            if (four)
                MHCPB_READ_STEP(4 + kPartialStores);
            else
                MHCPB_READ_STEP(kPartialStores);
        }
#undef MHCPB_READ_STEP
        const f32x4 cc = rd.cc;
        const u32x4(&pa)[3] = rd.pa;
        const u32x4(&pb)[2][2] = rd.pb;
        const f32x4(&xc)[4] = rd.xc;
        const uint32_t pois = rd.pois;
        ready_seen = rd.ready;
        // Of the two compute waves that share a SIMD (0 and 4 of five), the
        // one that is not ahead of the other runs this step one priority
        // level up, so that the older wave no longer wins every tie and the
        // younger one no longer ends the workgroup 2 us after the others
        // (0.4 us less per call at T = 4096, 1.6 at T = 16384; same bits).
        // With five compute waves every wave publishes the steps it has
        // begun; a wave without a mate reads its own count, which is never
        // ahead of it (one-wave workgroups skip all of this).
        constexpr bool kMates = NW == 5;
        const bool behind = kMates && static_cast<int>(__builtin_amdgcn_readfirstlane(rd.mate)) > k;
        if (behind) __builtin_amdgcn_s_setprio(2);
        if (kMates) lds_publish(my_prog_addr, static_cast<uint32_t>(k + 1), lane);
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
            cursor_next(nxt, L, T);
        }
        compiler_fence();
        if (behind)
            __builtin_amdgcn_s_setprio(1);
        else
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

        uint32_t packed[4][2];  // dX of row 4g + r, columns (0,1) and (2,3)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            // dX for column variant i: the RMS term c_t * x in FP32, then
            // the 96 exact partial products.
            f32x4 acc = {};
            if constexpr (kDX) {
                acc = f32x4{ce[0] * xc[0][i], ce[1] * xc[1][i], ce[2] * xc[2][i], ce[3] * xc[3][i]};
                acc = mfma(pa[0], bw[i][0], acc);
                acc = mfma(pa[1], bw[i][0], acc);
                acc = mfma(pa[2], bw[i][1], acc);
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
        const int s_done = cur.s;
        const bool after_unit = cursor_next(cur, L, T);
        if (after_unit) {
            d_cur = reinterpret_cast<char *>(dx + cur.row0 * K + kw);
            if constexpr (kAddend) a_cur = reinterpret_cast<const char *>(addend + cur.row0 * K + kw);
        }
        // At the end of a unit that is not the last, its partial dW goes to
        // workspace slab s_done while the X of the next unit is already in
        // flight (through ring stage k & 1, which holds no request until the
        // next step), or, in group 0, into the running sum; the accumulators
        // restart from zero.  The last unit's partial (group 0: the sum) is
        // stored after the drain below.
        stored = false;
        if (kDW && after_unit) {
            const bool last = cur.slab_rows == 0;
            if (fold) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int jb = 0; jb < 2; ++jb) pref[i][jb] += accw[i][jb];
            } else if (!last) {
                store_partial(s_done, ring_base + static_cast<uint32_t>((k & 1) * 4 * kWave * 16), bad);
                stored = true;
            }
            if (last) {
                last_unit_s = s_done;
                if (fold) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
#pragma unroll
                        for (int jb = 0; jb < 2; ++jb) accw[i][jb] = pref[i][jb];
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int jb = 0; jb < 2; ++jb) accw[i][jb] = f32x4{0.f, 0.f, 0.f, 0.f};
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
    // Drain the X DMA still in flight (the steps past the last unit) before
    // the workgroup's LDS can be released.
    wait_vmcnt<0>();

    // Partial dW of the last unit, written once to workspace slab
    // last_unit_s (the ring is idle after the drain).
    if constexpr (kDW) store_partial(last_unit_s, ring_base, bad);
}

// dW[i] = (((ws[f][i] + ws[f + 1][i]) + ws[f + 2][i]) + ...) + ws[S - 1][i]:
// slab f holds the sum of slabs 0 .. f, added in that order by kernel 1's
// slab group 0, so this is the ascending sum over every slab.  Four
// elements (one quad) per thread; a thread requests eight slabs of its quad
// before it adds them in order, so that eight loads are in flight.
//
// The quads are dealt to blocks by kernel 1's column tiles: block b takes the
// tiles t with t % 8 == b % 8, which are the tiles whose partials kernel 1's
// workgroups on the same XCD wrote when workgroups go to the 8 XCDs
// round-robin by index and the tile count is a multiple of 8 (the supported
// profile), so that the slabs stored last are still in that XCD's L2.  Any
// other placement gives the same sums, only slower.
constexpr int kReduceBatch = 8;
constexpr int kXcds = 8;
constexpr int kReduceThreads = 256;
__device__ __forceinline__ f32x4 load_slab_quad(const f32x4 *p) {
    return __builtin_nontemporal_load(p);
}
__global__ __launch_bounds__(kReduceThreads) void reduce_slabs(const float *__restrict__ ws,
                                                               float *__restrict__ dw, int first,
                                                               int S, int64_t K, int tile_quads,
                                                               int tiles) {
    const int xcd = static_cast<int>(blockIdx.x) % kXcds;
    // Quad q of this XCD's share: tile xcd + 8 (q / per_tile), row j, column
    // quad c4 of the tile.
    const int q = (static_cast<int>(blockIdx.x) / kXcds) * kReduceThreads + static_cast<int>(threadIdx.x);
    const int per_tile = kProjCols * tile_quads;
    const int t = xcd + kXcds * (q / per_tile);
    const int qt = q % per_tile;
    const int j = qt / tile_quads;
    const int64_t k4 = K / 4;
    const int64_t c4 = static_cast<int64_t>(t) * tile_quads + qt % tile_quads;
    if (t >= tiles || c4 >= k4) return;
    const int64_t n4 = kProjCols * k4;  // quads per slab
    const int64_t i = j * k4 + c4;
    const f32x4 *src = reinterpret_cast<const f32x4 *>(ws) + i;
    f32x4 a = load_slab_quad(src + first * n4);
    for (int s0 = first + 1; s0 < S; s0 += kReduceBatch) {
        f32x4 b[kReduceBatch];
        // Past the last slab the addend is -0, which leaves every sum as it
        // is (x + -0 == x, signed zeros included).
#pragma unroll
        for (int u = 0; u < kReduceBatch; ++u)
            b[u] = s0 + u < S ? load_slab_quad(src + static_cast<int64_t>(s0 + u) * n4)
                              : f32x4{-0.f, -0.f, -0.f, -0.f};
#pragma unroll
        for (int u = 0; u < kReduceBatch; ++u) a += b[u];
    }
    reinterpret_cast<f32x4 *>(dw)[i] = a;
}

template <int NW>
hipError_t launch_projection_t(const Plan &p, const Args &a, Outputs out, hipStream_t stream,
                               hipEvent_t start, hipEvent_t stop) {
    const int tiles = p.shape.tiles;
    const int G = p.shape.groups;
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

// Launch shape (the plan's, a performance choice only): five compute waves
// and the producer per workgroup, one workgroup per CU (at K = 20480 with 8
// splits, 64 column tiles x 4 slab groups fill 256 CUs once); one compute
// wave per workgroup for narrow problems, which would otherwise leave most
// CUs idle.
hipError_t launch_projection(const Plan &p, const Args &a, Outputs out, hipStream_t stream,
                             hipEvent_t start, hipEvent_t stop) {
    switch (p.shape.nw) {
    case 5:
        return launch_projection_t<5>(p, a, out, stream, start, stop);
    case 1:
        return launch_projection_t<1>(p, a, out, stream, start, stop);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_reduce(const Plan &p, const Args &a, hipStream_t stream, hipEvent_t stop) {
    // The column tiles of kernel 1 (nw * 64 columns each).
    const int tile_quads = p.shape.nw * kWave / 4;
    const int tiles = p.shape.tiles;
    const int64_t per_xcd = static_cast<int64_t>((tiles + kXcds - 1) / kXcds) * kProjCols * tile_quads;
    const unsigned blocks =
        static_cast<unsigned>(kXcds * ((per_xcd + kReduceThreads - 1) / kReduceThreads));
    return launch(reduce_slabs, dim3(blocks), dim3(kReduceThreads), stream, nullptr, stop, a.ws,
                  a.dw, p.shape.first_slab, p.S, p.K, tile_quads, tiles);
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
