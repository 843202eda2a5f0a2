// Kernels of the mHC projection forward for gfx950: the 24 gate logits
// proj[t, j] = sum_k TF32(X[t, k]) TF32(W[j, k]) (FP32 accumulation) and the
// row RMS r[t] = sqrt(sum_k X[t, k]^2 / K + eps) in FP32, in one read of X.
// This is the map whose gradient the backward kernels compute (the backward
// page, "DSv4.1 mHC projection/RMS backward", takes r "from forward"; the
// prime-kernels pull request 15 page lists the RMS and the gate logits of the
// streams as one pass, "mhc_projection").
//
// Kernel 1 ("forward_tiles").  The K columns are cut into tiles of 1024 and
// the tokens into steps of 16; a unit of work is (tile, step).  Workgroup b
// takes a contiguous run of units, tile-major, so one round of workgroups
// covers any T.  Each of its 8 waves owns 128 columns of the tile and keeps
// their W, split into BF16 high and low parts, in registers for as long as
// the tile lasts: W is read once per workgroup and tile instead of once per
// token block.  A wave streams its 16 x 128 block of each unit from HBM into
// a three-stage LDS ring by LDS DMA, 64 columns a step, two steps ahead (one
// DMA instruction moves 8 rows x 128 contiguous bytes; the 16-byte segments
// of a row are XOR-swizzled so that the A-operand reads, 16 tokens at one
// segment, hit 16 different bank groups).  It forms the 16 x 24 logits of its
// columns on the MFMA and the sums of squares of its x; the 8 waves' results
// are added in wave order through LDS slots, each wave reducing two of the
// 16 tokens, and the tile's partial logits and sums of squares go to the
// workspace.  Kernel 2 ("forward_reduce") adds the tiles' partials of each
// token in tile order and computes r.  Every sum has an order fixed by K
// alone, so a row's result does not depend on T, on the other rows or on the
// launch shape.
//
// Products.  TF32(x) = xh + xl exactly, with xh the upper 16 bits of the TF32
// value and xl the (at most 3-bit) remainder, both BF16; likewise for W.  On
// v_mfma_f32_16x16x32_bf16 (A = 16 tokens x 32 columns, B = 32 columns x 16
// gates) lane l supplies token / gate l % 16 and eight columns of a 32-column
// group: 8q .. 8q + 7 (q = l / 16; A and B agree).
// Gates 0..15 take four MFMAs per group (xh wh, xh wl, xl wh, xl wl); gates
// 16..23 take two, with B lanes 0..7 holding wh and lanes 8..15 wl of the
// same gates, so their logits are the sum of two accumulator columns.  Every
// BF16 product is exact and the MFMA adds in FP32.
#include <cstddef>

#include "mhcpb_device.h"
#include "mhcpb_internal.h"

namespace mhcpb {
namespace {

constexpr int kFwdRows = 16;                 // tokens per unit
constexpr int kFwdPairs = kFwdRows / 2;      // partial blocks (two tokens each) per unit
constexpr int kFwdStepCols = 64;             // columns per step (2 MFMA groups)
constexpr int kFwdDma = 4;                   // LDS DMA instructions per step
constexpr int kFwdStages = 3;                // LDS ring stages per wave
constexpr int kFwdSlots = 3;                 // LDS reduction slots in rotation

// Cache policy of the X stream (read once): non-temporal.
#ifndef MHCPB_FWD_X_AUX
#define MHCPB_FWD_X_AUX 2
#endif

// TF32 value of v as bits: nearest even at 10 fraction bits, the carry
// running into the exponent.  A NaN whose top fraction bits are all ones can
// carry out of the exponent here; kernel 2 repairs such rows (their RMS is
// NaN).
__device__ __forceinline__ uint32_t tf32_bits(float v) {
    const uint32_t u = __float_as_uint(v);
    return (u + 0xFFFu + ((u >> 13) & 1u)) & 0xFFFFE000u;
}

// A buffer offset, moved outside every range unless `in` holds.
__device__ __forceinline__ uint32_t offset_if(bool in, uint32_t off) {
    return in ? off : kOutOfRange;
}

// Lower halves of two 32-bit words: (a & 0xFFFF) | (b << 16).
__device__ __forceinline__ uint32_t lo_halves(uint32_t a, uint32_t b) {
    return __builtin_amdgcn_perm(b, a, 0x05040100u);
}

// One reduction slot: each wave's 16 x 32 accumulator block in MFMA output
// layout (acc[w][b][lane] holds rows 4 (lane / 16) + i, column 16 b + lane %
// 16, i = 0..3) and the sums of squares of its 16 tokens.
template <int NW>
struct FwdSlot {
    f32x4 acc[NW][2][kWave];
    float ss[NW][kFwdRows];
};

// Untracked vector memory: the kernel counts its own requests (LDS DMA of
// X, W loads, partial stores) in explicit vmcnt waits, so none of them may
// make the compiler insert a wait of its own, which would not count the DMA
// and would drain the X stream.  Loads are issued in an asm statement that
// ends with their wait (an asm load's destination holds no value the
// compiler may use before that).
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x4 rsrc_words(const void *base, int bytes) {
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    return i32x4{__builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint32_t>(a))),
                 __builtin_amdgcn_readfirstlane(static_cast<int>((a >> 32) & 0xFFFFu)),
                 __builtin_amdgcn_readfirstlane(bytes), kRsrcWord3};
}
// Sixteen 16-byte loads at offsets o[0..15] of the buffer rs, then a wait for
// every request of the wave (vmcnt(0)).
__device__ __forceinline__ void load16_b128_wait_all(i32x4 rs, const uint32_t (&o)[16],
                                                     f32x4 (&v)[16]) {
    asm volatile(
        "buffer_load_dwordx4 %0, %16, %32, 0 offen\n\t"
        "buffer_load_dwordx4 %1, %17, %32, 0 offen\n\t"
        "buffer_load_dwordx4 %2, %18, %32, 0 offen\n\t"
        "buffer_load_dwordx4 %3, %19, %32, 0 offen\n\t"
        "buffer_load_dwordx4 %4, %20, %32, 0 offen\n\t"
        "buffer_load_dwordx4 %5, %21, %32, 0 offen\n\t"
        "buffer_load_dwordx4 %6, %22, %32, 0 offen\n\t"
        "buffer_load_dwordx4 %7, %23, %32, 0 offen\n\t"
        "buffer_load_dwordx4 %8, %24, %32, 0 offen\n\t"
        "buffer_load_dwordx4 %9, %25, %32, 0 offen\n\t"
        "buffer_load_dwordx4 %10, %26, %32, 0 offen\n\t"
        "buffer_load_dwordx4 %11, %27, %32, 0 offen\n\t"
        "buffer_load_dwordx4 %12, %28, %32, 0 offen\n\t"
        "buffer_load_dwordx4 %13, %29, %32, 0 offen\n\t"
        "buffer_load_dwordx4 %14, %30, %32, 0 offen\n\t"
        "buffer_load_dwordx4 %15, %31, %32, 0 offen\n\t"
        "s_waitcnt vmcnt(0)"
        : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]),
          "=&v"(v[6]), "=&v"(v[7]), "=&v"(v[8]), "=&v"(v[9]), "=&v"(v[10]), "=&v"(v[11]),
          "=&v"(v[12]), "=&v"(v[13]), "=&v"(v[14]), "=&v"(v[15])
        : "v"(o[0]), "v"(o[1]), "v"(o[2]), "v"(o[3]), "v"(o[4]), "v"(o[5]), "v"(o[6]),
          "v"(o[7]), "v"(o[8]), "v"(o[9]), "v"(o[10]), "v"(o[11]), "v"(o[12]), "v"(o[13]),
          "v"(o[14]), "v"(o[15]), "s"(rs)
        : "memory");
}
__device__ __forceinline__ void store_b32_untracked(i32x4 rs, uint32_t off, float v) {
    asm volatile("buffer_store_dword %0, %1, %2, 0 offen" ::"v"(v), "v"(off), "s"(rs) : "memory");
}

// What one wave of forward_tiles knows of its work (all uniform but the
// lane fields).
struct FwdCtx {
    const float *x;
    const float *w;
    float *part;
    int64_t T;
    int ki;       // K (<= 2^22)
    int nsteps;   // 16-token steps of T
    int u_begin;
    int nu;       // units of this workgroup
    int wcols;    // columns per wave
    int wave;
    int lane, q, n16;
    uint32_t ring;   // LDS address of this wave's X ring
    uint32_t slots;  // LDS address of the reduction slots
    uint32_t ready, consumed;
    uint32_t poison;  // LDS word raised by a wave whose bounded wait gave up
    int max_polls;    // bound of the counter waits
};

// A unit of the workgroup's run: tile kt, 16-token step s (first token
// 16 s), its rows (16, or fewer at the end of T), and whether it lies in the
// run.  Uniform; advanced one unit at a time without divisions.
struct FwdUnit {
    int kt;
    int s;
    int rows;
    bool valid;
};
__device__ __forceinline__ FwdUnit fwd_unit_at(const FwdCtx &c, int s, int kt, int i) {
    FwdUnit r;
    r.kt = kt;
    r.s = s;
    const int64_t left = c.T - static_cast<int64_t>(s) * kFwdRows;
    r.rows = static_cast<int>(left < kFwdRows ? left : kFwdRows);
    r.valid = i < c.nu;
    return r;
}
__device__ __forceinline__ FwdUnit fwd_first(const FwdCtx &c) {
    return fwd_unit_at(c, c.u_begin % c.nsteps, c.u_begin / c.nsteps, 0);
}
// The unit after un, which is unit i of the run.
__device__ __forceinline__ FwdUnit fwd_next(const FwdCtx &c, const FwdUnit &un, int i) {
    const bool wrap = un.s + 1 == c.nsteps;
    return fwd_unit_at(c, wrap ? 0 : un.s + 1, wrap ? un.kt + 1 : un.kt, i);
}
__device__ __forceinline__ int fwd_colbase(const FwdCtx &c, int kt) {
    return __builtin_amdgcn_readfirstlane(kt * kFwdTileCols + c.wave * c.wcols);
}

// Step h of unit un (64 columns) into the ring stage at LDS address `stage`
// by 4 LDS DMA: instruction rr = 2a + b moves rows 8a .. 8a+7 and 16-byte
// segments 8b .. 8b+7 of the 64 columns; lane L fetches row 8a + L/8,
// segment 8b + ((L % 8) ^ (L/8) ^ a), which lands at LDS position 64 rr + L
// (16-byte units) of the stage.  Units past the workgroup's run get an empty
// range, rows past T fall outside the range, and columns past K take
// out-of-range offsets; all of them read zeros.
__device__ __forceinline__ void fwd_issue_x(const FwdCtx &c, const FwdUnit &un, int h,
                                            uint32_t stage, const uint32_t (&xoff)[kFwdDma],
                                            const int (&xcol)[kFwdDma]) {
    const int col0 = fwd_colbase(c, un.kt) + kFwdStepCols * h;
    const int n = un.valid ? un.rows * c.ki - col0 : 0;
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc32(c.x + static_cast<int64_t>(un.s) * kFwdRows * c.ki + col0,
                    __builtin_amdgcn_readfirstlane(n > 0 ? n : 0) * 4);
    const int lim = c.ki - col0;
#pragma unroll
    for (int rr = 0; rr < kFwdDma; ++rr)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rs, (MHCPB_LDS void *)(static_cast<uintptr_t>(stage + rr * kWave * 16)), 16,
            offset_if(xcol[rr] < lim, xoff[rr]), 0, 0, MHCPB_FWD_X_AUX);
}

// The B operands of tile kt for this wave: per group G, [0] high parts of
// gate n16, [1] its low parts, [2] the high (n16 < 8) or low (n16 >= 8)
// parts of gate 16 + n16 % 8, at columns 32G + 8q .. + 7 of the wave's
// columns; columns past K are zero.  Waits for every request of the wave (a
// tile change is rare).
template <int NG>
__device__ __forceinline__ void fwd_load_w(const FwdCtx &c, int kt, u32x4 (&bw)[NG][3]) {
    const int colbase = fwd_colbase(c, kt);
    const i32x4 rs = rsrc_words(c.w, kProjCols * c.ki * 4);
    const int g1 = 16 + (c.n16 & 7);
#pragma unroll
    for (int G0 = 0; G0 < NG; G0 += 4) {  // four groups (16 loads) per wait
        // Load n = 4 (2 G + h) + i: i = 0 gate n16, i = 1 gate g1, at column
        // group G0 + G, half h.
        uint32_t off[16];
#pragma unroll
        for (int G = 0; G < 4; ++G)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int col = colbase + 32 * (G0 + G) + 8 * c.q + 4 * h;
                const bool in = col < c.ki;
                off[4 * G + 2 * h] = offset_if(in, static_cast<uint32_t>((c.n16 * c.ki + col) * 4));
                off[4 * G + 2 * h + 1] = offset_if(in, static_cast<uint32_t>((g1 * c.ki + col) * 4));
            }
        f32x4 lv[16];
        load16_b128_wait_all(rs, off, lv);
        f32x4 v0[4][2], v1[4][2];
#pragma unroll
        for (int G = 0; G < 4; ++G)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                v0[G][h] = lv[4 * G + 2 * h];
                v1[G][h] = lv[4 * G + 2 * h + 1];
            }
#pragma unroll
        for (int G = 0; G < 4; ++G) {
            uint32_t p0[8], p1[8];  // hi | lo << 16
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                p0[e] = tf32_split_packed(v0[G][e / 4][e % 4]);
                p1[e] = tf32_split_packed(v1[G][e / 4][e % 4]);
            }
            bw[G0 + G][0] = u32x4{lo_halves(p0[0], p0[1]), lo_halves(p0[2], p0[3]),
                                  lo_halves(p0[4], p0[5]), lo_halves(p0[6], p0[7])};
            bw[G0 + G][1] = u32x4{hi_halves(p0[0], p0[1]), hi_halves(p0[2], p0[3]),
                                  hi_halves(p0[4], p0[5]), hi_halves(p0[6], p0[7])};
            bw[G0 + G][2] = c.n16 < 8 ? u32x4{lo_halves(p1[0], p1[1]), lo_halves(p1[2], p1[3]),
                                              lo_halves(p1[4], p1[5]), lo_halves(p1[6], p1[7])}
                                      : u32x4{hi_halves(p1[0], p1[1]), hi_halves(p1[2], p1[3]),
                                              hi_halves(p1[4], p1[5]), hi_halves(p1[6], p1[7])};
        }
    }
}

// LDS addresses within a slot (FwdSlot<NW> layout).
template <int NW>
__device__ __forceinline__ uint32_t fwd_slot_acc(const FwdCtx &c, int slot, int w, int b, int l) {
    return c.slots + static_cast<uint32_t>(slot * sizeof(FwdSlot<NW>) +
                                           ((w * 2 + b) * kWave + l) * sizeof(f32x4));
}
template <int NW>
__device__ __forceinline__ uint32_t fwd_slot_ss(const FwdCtx &c, int slot, int w, int m) {
    return c.slots + static_cast<uint32_t>(slot * sizeof(FwdSlot<NW>) +
                                           offsetof(FwdSlot<NW>, ss) + (w * kFwdRows + m) * 4);
}

// Reduction of unit i by this wave: token pairs p = wave (8 / NW) + j, one
// pair per pass; lane L takes token 2p + L / 32, column L % 32 of the
// 32-wide rows (0..15 gates 0..15, 16..23 high parts and 24..31 low parts of
// gates 16..23), and the lanes of column 24 also sum the squares.  Waits
// until every wave has written unit i, adds the NW waves in order, frees the
// slot and writes block (tile, step, p) of the workspace: 64 floats in lane
// order, token 2p + h at floats 32 h .. 32 h + 31 (logits 0..23, the squares
// at 24, zeros after), one store per pair.  For i < 0 the stores go to an
// empty range: every unit issues the same requests.
template <int NW>
__device__ __forceinline__ void fwd_reduce(const FwdCtx &c, int i, const FwdUnit &un) {
    constexpr int kPairsPerWave = kFwdPairs / NW;
    const int col = c.lane % 32;
    float sum[kPairsPerWave], ssum[kPairsPerWave];
    bool poisoned = false;
#pragma unroll
    for (int j = 0; j < kPairsPerWave; ++j) sum[j] = ssum[j] = 0.f;
    if (i >= 0) {
        const int slot = i % kFwdSlots;
        if (!lds_wait_at_least(c.ready + 4 * slot, NW * static_cast<uint32_t>(i / kFwdSlots + 1),
                                c.max_polls))
            lds_raise_poison(c.poison, c.lane);
        const int b = col / 16, nn = col % 16;
        float v[kPairsPerWave][NW], sv[kPairsPerWave][NW];
        // The NW waves' values of this lane's element, 2 KB apart (pairs
        // of them 256-byte strides 0 and 8 apart), their sums of squares 64
        // bytes apart (dword offsets 0 and 16), then the poison word (read
        // after the slot: a wave that gave up raised it before it
        // overwrote a slot), in one asm statement with its wait.
        static_assert(kPairsPerWave == 1 && NW == 8, "reduction reads laid out for 8 waves");
        const int m = 2 * c.wave + c.lane / 32;
        const uint32_t src = fwd_slot_acc<NW>(c, slot, 0, b, 16 * (m / 4) + nn) + 4 * (m % 4);
        const uint32_t ssrc = fwd_slot_ss<NW>(c, slot, 0, m);
        static_assert(2 * kWave * 16 == 8 * 256 && kFwdRows * 4 == 16 * 4, "read2 strides");
        u32x2 p[4], q[4];
        uint32_t pois;
        asm volatile(
            "ds_read2st64_b32 %0, %9 offset1:8\n\t"
            "ds_read2st64_b32 %1, %9 offset0:16 offset1:24\n\t"
            "ds_read2st64_b32 %2, %9 offset0:32 offset1:40\n\t"
            "ds_read2st64_b32 %3, %9 offset0:48 offset1:56\n\t"
            "ds_read2_b32 %4, %10 offset1:16\n\t"
            "ds_read2_b32 %5, %10 offset0:32 offset1:48\n\t"
            "ds_read2_b32 %6, %10 offset0:64 offset1:80\n\t"
            "ds_read2_b32 %7, %10 offset0:96 offset1:112\n\t"
            "ds_read_b32 %8, %11\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(p[0]), "=&v"(p[1]), "=&v"(p[2]), "=&v"(p[3]), "=&v"(q[0]), "=&v"(q[1]),
              "=&v"(q[2]), "=&v"(q[3]), "=&v"(pois)
            : "v"(src), "v"(ssrc), "v"(c.poison)
            : "memory");
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) {
            v[0][ww] = __uint_as_float(ww % 2 ? p[ww / 2].y : p[ww / 2].x);
            sv[0][ww] = __uint_as_float(ww % 2 ? q[ww / 2].y : q[ww / 2].x);
        }
        poisoned = __builtin_amdgcn_readfirstlane(pois) != 0;
        lds_signal(c.consumed + 4 * slot, c.lane);
#pragma unroll
        for (int j = 0; j < kPairsPerWave; ++j) {
            sum[j] = v[j][0];
            ssum[j] = sv[j][0];
#pragma unroll
            for (int ww = 1; ww < NW; ++ww) {
                sum[j] += v[j][ww];
                ssum[j] += sv[j][ww];
            }
        }
    }
#pragma unroll
    for (int j = 0; j < kPairsPerWave; ++j) {
        const float low = __shfl_xor(sum[j], 8);  // column + 8: the low part
        if (col >= 16 && col < 24) sum[j] += low;
        // After a give-up the sums of squares become NaN, which makes the
        // token's r and all its logits NaN in kernel 2.
        const float ssv = poisoned ? __builtin_nanf("") : ssum[j];
        const float out = col < kProjCols ? sum[j] : (col == kProjCols ? ssv : 0.f);
        const int p = c.wave * kPairsPerWave + j;
        const int64_t blk = (static_cast<int64_t>(un.kt) * c.nsteps + un.s) * kFwdPairs + p;
        const i32x4 brs = rsrc_words(c.part + blk * kWave, i >= 0 ? kWave * 4 : 0);
        store_b32_untracked(brs, static_cast<uint32_t>(c.lane * 4), out);
    }
}

// Step h of unit i (groups 2h, 2h + 1 of the wave's W), read from ring stage
// sb; requests step (h + 2) of the same unit or step h + 2 - SPU of the next
// (two steps ahead) into stage sb_next.  Requests: 4 DMA per step, and at the
// end of each unit the NW-dependent partial stores (kStores) of the
// reduction of the previous unit.  At the top of step h the requests after
// its X are the next step's 4 DMA, plus the stores when a unit's end lies
// between (h < 2): the wait leaves exactly those in flight.  `first` marks
// the first unit, before which no stores were issued.
template <int NW, int NG, int H>
__device__ __forceinline__ void fwd_step(const FwdCtx &c, bool first, uint32_t sb, uint32_t sb_next,
                                         const FwdUnit &pre, const uint32_t (&xoff)[kFwdDma],
                                         const int (&xcol)[kFwdDma], const uint32_t (&rd)[2][2],
                                         const u32x4 (&bw)[NG][3], f32x4 &acc0, f32x4 &acc1,
                                         float &ss) {
    constexpr int SPU = NG / 2;
    constexpr int kStores = kFwdPairs / NW;
    if (H >= 2 || first)
        wait_vmcnt<kFwdDma>();
    else
        wait_vmcnt<kFwdDma + kStores>();
    f32x4 xv[2][2];
    asm volatile(
        "ds_read_b128 %0, %4\n\t"
        "ds_read_b128 %1, %5\n\t"
        "ds_read_b128 %2, %6\n\t"
        "ds_read_b128 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(xv[0][0]), "=&v"(xv[0][1]), "=&v"(xv[1][0]), "=&v"(xv[1][1])
        : "v"(sb + rd[0][0]), "v"(sb + rd[0][1]), "v"(sb + rd[1][0]), "v"(sb + rd[1][1])
        : "memory");
    compiler_fence();
    fwd_issue_x(c, pre, (H + 2) % SPU, sb_next, xoff, xcol);
    compiler_fence();
#pragma unroll
    for (int G2 = 0; G2 < 2; ++G2) {
        const int G = 2 * H + G2;
        const float v[8] = {xv[G2][0].x, xv[G2][0].y, xv[G2][0].z, xv[G2][0].w,
                            xv[G2][1].x, xv[G2][1].y, xv[G2][1].z, xv[G2][1].w};
        uint32_t tv[8], lo[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            tv[e] = tf32_bits(v[e]);
            lo[e] = __float_as_uint(__uint_as_float(tv[e]) - __uint_as_float(tv[e] & 0xFFFF0000u));
        }
        const u32x4 ahi = {hi_halves(tv[0], tv[1]), hi_halves(tv[2], tv[3]),
                           hi_halves(tv[4], tv[5]), hi_halves(tv[6], tv[7])};
        const u32x4 alo = {hi_halves(lo[0], lo[1]), hi_halves(lo[2], lo[3]),
                           hi_halves(lo[4], lo[5]), hi_halves(lo[6], lo[7])};
        acc0 = mfma(ahi, bw[G][0], acc0);
        acc0 = mfma(ahi, bw[G][1], acc0);
        acc0 = mfma(alo, bw[G][0], acc0);
        acc0 = mfma(alo, bw[G][1], acc0);
        acc1 = mfma(ahi, bw[G][2], acc1);
        acc1 = mfma(alo, bw[G][2], acc1);
#pragma unroll
        for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(v[e], v[e], ss);
    }
}

// The steps of one unit, H = 0 .. SPU - 1; stage indices cycle through 3.
template <int NW, int NG, int H>
__device__ __forceinline__ void fwd_steps(const FwdCtx &c, bool first, int &stage,
                                          const FwdUnit &cur, const FwdUnit &nxt,
                                          const uint32_t (&xoff)[kFwdDma], const int (&xcol)[kFwdDma],
                                          const uint32_t (&rd)[2][2], const u32x4 (&bw)[NG][3],
                                          f32x4 &acc0, f32x4 &acc1, float &ss) {
    if constexpr (H < NG / 2) {
        constexpr uint32_t kStage = kFwdDma * kWave * 16;
        const int s1 = stage == 2 ? 0 : stage + 1;
        const int s2 = s1 == 2 ? 0 : s1 + 1;  // stage of the step two ahead
        fwd_step<NW, NG, H>(c, first, c.ring + stage * kStage, c.ring + s2 * kStage,
                            H + 2 < NG / 2 ? cur : nxt, xoff, xcol, rd, bw, acc0, acc1, ss);
        stage = s1;
        fwd_steps<NW, NG, H + 1>(c, first, stage, cur, nxt, xoff, xcol, rd, bw, acc0, acc1, ss);
    }
}

template <int NW>
__global__ __launch_bounds__(NW * kWave) void forward_tiles(
    const float *__restrict__ x, const float *__restrict__ w, float *__restrict__ part, int64_t T,
    int64_t K, int units, int upw, int nsteps, int max_polls) {
    constexpr int NG = kFwdTileCols / (32 * NW);  // 32-column groups per wave
    constexpr int SPU = NG / 2;                   // steps per unit
    static_assert(NG % 2 == 0 && SPU >= 2, "at least two steps per unit");
    __shared__ f32x4 xring[NW][kFwdStages][kFwdDma][kWave];
    __shared__ FwdSlot<NW> slots[kFwdSlots];
    __shared__ uint32_t ready[kFwdSlots], consumed[kFwdSlots], poison[1];
    FwdCtx c;
    c.x = x;
    c.w = w;
    c.part = part;
    c.T = T;
    c.ki = static_cast<int>(K);
    c.nsteps = nsteps;
    c.u_begin = static_cast<int>(blockIdx.x) * upw;
    c.nu = (c.u_begin + upw < units ? c.u_begin + upw : units) - c.u_begin;
    c.wcols = NG * 32;
    c.lane = threadIdx.x % kWave;
    c.wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
    c.q = c.lane / 16;
    c.n16 = c.lane % 16;
    c.ring = lds_addr(&xring[c.wave][0][0][0]);
    c.slots = lds_addr(&slots[0]);
    c.ready = lds_addr(&ready[0]);
    c.consumed = lds_addr(&consumed[0]);
    c.poison = lds_addr(&poison[0]);
    c.max_polls = max_polls;
    if (threadIdx.x < kFwdSlots) {
        lds_write_u32(c.ready + 4 * threadIdx.x, 0u);
        lds_write_u32(c.consumed + 4 * threadIdx.x, 0u);
    }
    if (threadIdx.x == 0) lds_write_u32(c.poison, 0u);
    lds_barrier();

    // DMA offsets of this lane (see fwd_issue_x) and the A-operand reads:
    // lane (q, token m) reads segments 8G + 2q + h (h = 0, 1) of column group
    // G of the step; their positions in a stage follow from the DMA map.
    uint32_t xoff[kFwdDma];
    int xcol[kFwdDma];
#pragma unroll
    for (int rr = 0; rr < kFwdDma; ++rr) {
        const int a = rr >> 1, b = rr & 1, mi = c.lane >> 3;
        const int seg = 8 * b + ((c.lane & 7) ^ mi ^ a);
        xcol[rr] = 4 * seg;
        xoff[rr] = static_cast<uint32_t>(((8 * a + mi) * c.ki + 4 * seg) * 4);
    }
    uint32_t rd[2][2];
    {
        const int a = c.n16 >> 3, mi = c.n16 & 7;
#pragma unroll
        for (int G = 0; G < 2; ++G)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int si = 2 * c.q + h;
                rd[G][h] = static_cast<uint32_t>((64 * (2 * a + G) + 8 * mi + (si ^ mi ^ a)) * 16);
            }
    }

    u32x4 bw[NG][3];
    FwdUnit cur = fwd_first(c);
    FwdUnit nxt = fwd_next(c, cur, 1);
    FwdUnit prev = cur;
    int kt_loaded = cur.kt;
    fwd_load_w<NG>(c, kt_loaded, bw);
    constexpr uint32_t kStage = kFwdDma * kWave * 16;
    fwd_issue_x(c, cur, 0, c.ring, xoff, xcol);
    fwd_issue_x(c, cur, 1, c.ring + kStage, xoff, xcol);

    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f};  // gates 0..15
    f32x4 acc1 = {0.f, 0.f, 0.f, 0.f};  // gates 16..23: high part | low part
    float ss = 0.f;                     // squares of token n16, this lane's columns
    int stage = 0;                      // ring stage of the unit's first step
    for (int i = 0; i < c.nu; ++i) {
        if (cur.kt != kt_loaded) {  // a new tile: reload W (its wait drains everything)
            fwd_load_w<NG>(c, cur.kt, bw);
            kt_loaded = cur.kt;
        }
        fwd_steps<NW, NG, 0>(c, i == 0, stage, cur, nxt, xoff, xcol, rd, bw, acc0, acc1, ss);
        // Squares of token n16 over the wave's columns: the four quarters in
        // order ((q0 + q1) + (q2 + q3)).
        ss += __shfl_xor(ss, 16);
        ss += __shfl_xor(ss, 32);
        const int slot = i % kFwdSlots;
        if (!lds_wait_at_least(c.consumed + 4 * slot, NW * static_cast<uint32_t>(i / kFwdSlots),
                                c.max_polls))
            lds_raise_poison(c.poison, c.lane);
        lds_write_u128(fwd_slot_acc<NW>(c, slot, c.wave, 0, c.lane), __builtin_bit_cast(u32x4, acc0));
        lds_write_u128(fwd_slot_acc<NW>(c, slot, c.wave, 1, c.lane), __builtin_bit_cast(u32x4, acc1));
        if (c.lane < kFwdRows)
            lds_write_u32(fwd_slot_ss<NW>(c, slot, c.wave, c.lane), __float_as_uint(ss));
        lds_signal(c.ready + 4 * slot, c.lane);
        fwd_reduce<NW>(c, i - 1, prev);
        acc0 = f32x4{0.f, 0.f, 0.f, 0.f};
        acc1 = f32x4{0.f, 0.f, 0.f, 0.f};
        ss = 0.f;
        prev = cur;
        cur = nxt;
        nxt = fwd_next(c, nxt, i + 2);
    }
    if (c.nu > 0) fwd_reduce<NW>(c, c.nu - 1, prev);
    // The requests past the run (zeros) and the stores land before the
    // workgroup's LDS is released.
    wait_vmcnt<0>();
}

// proj[t] = sum over tiles (in order) of the partial logits, r[t] from the
// summed squares; columns 24..31 of proj are zero.  A row whose sum of
// squares is NaN has a NaN in X: its logits are NaN.  Thread (t, e) handles
// logits 4e .. 4e + 3 of token t for e < 6, and e == 6 r and the zero
// columns; the tiles' loads are issued before they are added, in tile order.
// Token t's partial of tile kt is at floats 32 (t % 2) .. of block
// (kt, t / 16, (t % 16) / 2) (see fwd_reduce).
constexpr int kFwdReduceBatch = 24;
__global__ __launch_bounds__(256) void forward_reduce(const float *__restrict__ part,
                                                      float *__restrict__ proj,
                                                      float *__restrict__ rout, int64_t T,
                                                      int nkt, int nsteps, int64_t K, float eps) {
    constexpr int kParts = kProjCols / 4 + 1;
    const int64_t id = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const int64_t t = id / kParts;
    const int e = static_cast<int>(id % kParts);
    if (t >= T) return;
    const int64_t s = t / kFwdRows;
    const int m = static_cast<int>(t % kFwdRows);
    // floats of token t in tile 0; tile kt adds kt * tile_stride
    const int64_t base = (s * kFwdPairs + m / 2) * kWave + 32 * (m % 2);
    const int64_t tile_stride = static_cast<int64_t>(nsteps) * kFwdPairs * kWave;
    // The squares and the logits of all tiles are requested together (one
    // round trip), then added in tile order.  The thread of r (e == 6) reads
    // floats 24..27 of the block as its "logits" and ignores them.
    float ss = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < nkt; k0 += kFwdReduceBatch) {
        float vs[kFwdReduceBatch];
        f32x4 v[kFwdReduceBatch];
#pragma unroll
        for (int k = 0; k < kFwdReduceBatch; ++k) {
            const bool in = k0 + k < nkt;
            const float *blk = part + base + (k0 + k) * tile_stride;
            vs[k] = in ? __builtin_nontemporal_load(blk + kProjCols) : 0.f;
            v[k] = in ? __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(blk) + e)
                      : f32x4{0.f, 0.f, 0.f, 0.f};
        }
#pragma unroll
        for (int k = 0; k < kFwdReduceBatch; ++k)
            if (k0 + k < nkt) {
                ss = (k0 + k == 0) ? vs[k] : ss + vs[k];
                acc = (k0 + k == 0) ? v[k] : acc + v[k];
            }
    }
    const float rv = __builtin_sqrtf(ss / static_cast<float>(K) + eps);
    const bool nan_row = rv != rv;
    f32x4 *out = reinterpret_cast<f32x4 *>(proj + t * kProjStride);
    if (e == kParts - 1) {
        out[kProjCols / 4] = f32x4{0.f, 0.f, 0.f, 0.f};
        out[kProjCols / 4 + 1] = f32x4{0.f, 0.f, 0.f, 0.f};
        rout[t] = rv;
        return;
    }
    const float qnan = __builtin_nanf("");
    out[e] = nan_row ? f32x4{qnan, qnan, qnan, qnan} : acc;
}

}  // namespace

// Launch shape, a performance choice only: the partials' sums run in an
// order fixed by the 1024-column tiles, so every shape gives the same bits.
#ifndef MHCPB_FWD_WAVES
#define MHCPB_FWD_WAVES 8
#endif
hipError_t launch_forward(const Plan &p, const float *x, const float *w, float *proj, float *r,
                          float eps, float *ws, hipStream_t stream, hipEvent_t start,
                          hipEvent_t mid, hipEvent_t stop) {
    constexpr int NW = MHCPB_FWD_WAVES;
    // workgroups resident per CU (LDS) times 256 CUs: one round
    constexpr int kGrid = NW == 8 ? 256 : 512;
    const int nkt = forward_tile_count(p.K);
    const int nsteps = static_cast<int>((p.T + kFwdRows - 1) / kFwdRows);
    const int64_t units64 = static_cast<int64_t>(nkt) * nsteps;
    const int units = static_cast<int>(units64);  // < 2^31: checked before the launch
    const int upw = (units + kGrid - 1) / kGrid;
    const int grid = (units + upw - 1) / upw;
    const hipError_t e = launch(forward_tiles<NW>, dim3(grid), dim3(NW * kWave), stream, start,
                                mid, x, w, ws, p.T, p.K, units, upw, nsteps, p.wait_polls);
    if (e != hipSuccess) return e;
    // Kernel 2: 256 threads per block, or 128 where 256 would give fewer
    // blocks than CUs (below about 9400 tokens): the reduce is bound by the
    // latency of its loads, and at 4096 tokens the smaller blocks spread it
    // over twice the CUs (5.6 -> 4.5 us; the same bits).
    const int64_t threads = p.T * (kProjCols / 4 + 1);
    const int64_t bs = (threads + 255) / 256 < 256 ? 128 : 256;
    const unsigned blocks = static_cast<unsigned>((threads + bs - 1) / bs);
    return launch(forward_reduce, dim3(blocks), dim3(static_cast<unsigned>(bs)), stream, nullptr,
                  stop, ws, proj, r, p.T, nkt, nsteps, p.K, eps);
}

}  // namespace mhcpb
