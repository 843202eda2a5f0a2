// Deterministic BF16 RMSNorm backward for gfx950 (the second workload).
//
// The operation follows the signature and parameter list of the
// "flashinfer.cake_rmsnorm_det_train.cake_rmsnorm_det_train_backward" page:
// BF16 g and x of shape [T, H], a BF16 or FP32 weight w [H], the forward's
// FP32 rstd [T], an optional BF16 g_residual added once, BF16 dx and FP32 dw.
// The page prints no formula; this is the gradient of y = x * rstd * w per
// row with rstd = (mean(x^2) + eps)^(-1/2) taken as the forward returned it:
//
//   c1[t]   = sum_h w[h] g[t,h] x[t,h] / H
//   dx[t,h] = rstd[t] w[h] g[t,h] - rstd[t]^3 c1[t] x[t,h]  (+ g_residual[t,h])
//   dw[h]   = sum_t g[t,h] x[t,h] rstd[t]
//
// dx is computed in FP32 and rounded to BF16 once (the residual added before
// that rounding).  The same page's notes on reproducibility set the design
// of dw: its rows are split into blocks whose number depends on (T, H) alone
// (never on the CU count), and the block partials are added in a fixed
// order, so dw is bitwise reproducible on any MI355X for a given (T, H), and
// dx of a row depends on that row alone.
//
// Kernel 1 ("rows"): a block has one wave per 512-column chunk of a row
// (every lane 8 columns, loaded as 16-byte vectors) and owns the rows b,
// b + S, b + 2S, ... (S blocks; neighbouring blocks take neighbouring rows,
// so the whole GPU sweeps the tensors front to back).  It takes its rows in
// groups of R = 4: each wave sums w g x over its chunk of each row (one wave
// reduction per row) and puts the R sums into LDS; after a barrier every
// wave adds the chunks' sums of a row in chunk order, which gives the same
// c1 in every wave, then writes its chunk of dx.  The wave's 8 weights and
// 8 dw accumulators per lane stay in registers; at the end each wave writes
// its columns of the block's FP32 partial dw [H] into the workspace.  While a
// group is finished, the wave's registers of each row are reloaded with the
// row R places later, so a wave keeps R rows of loads in flight.  The row
// loads are non-temporal when g, x (and g_residual) reach 4 MB, and the dx
// stores always are: with the calls' buffers rotated, so that no call finds
// an earlier call's data in the 256 MB Infinity Cache, that is 3-10 % faster
// at every size from 8 MB of inputs up (rms_train 30.9 -> 28.8 us); below 4
// MB non-temporal loads are slower (300 x 1536: 11.0 -> 12.0 us).
// Kernel 2 ("reduce") adds the S block partials in a fixed order: 16 groups
// of consecutive blocks, each summed in ascending order, then the group sums
// in group order.
//
// Bound: HBM.  Per row 4 H bytes are read (g, x; 6 H with g_residual) and
// 2 H written (dx); the partials add 8 S H bytes per call.
#include "mhcpb_device.h"
#include "mhcpb_internal.h"

namespace mhcpb {
namespace {

#define MHCPB_CONST __attribute__((address_space(4)))

constexpr int kRmsChunk = 512;  // columns per chunk: 64 lanes x 8 BF16
constexpr int kRmsGroup = 4;  // rows a block takes at a time
constexpr uint64_t kRmsStreamBytes = uint64_t{4} << 20;
// Cache policy of the dx stores: non-temporal.
constexpr int kRmsDxAux = 2;
constexpr int kReduceGroups = 16;  // kernel 2: block groups per column (one wave each)
constexpr int kReduceBatch = 32;   // kernel 2: partials a lane requests before adding them

struct RmsArgs {
    const uint16_t *g;
    const uint16_t *x;
    const void *w;
    const float *rstd;
    const uint16_t *res;  // may be null
    uint16_t *dx;
    float *ws;  // [S, H] block partials
    int64_t T;
    int H;
};

__device__ __forceinline__ float lo_bf16(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float hi_bf16(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }

// Sum over the 64 lanes in a fixed order, the same value in every lane:
// within each row of 16 lanes, pairs (lane ^ 1), then quads (lane ^ 2), then
// the two quads of each half-row (mirrored), then the two half-rows
// (mirrored), all by DPP moves, so every lane of a row holds the same row sum;
// then (row 0 + row 1) + (row 2 + row 3).
template <int kCtrl>
__device__ __forceinline__ float dpp_step(float v) {
    const int moved = __builtin_amdgcn_mov_dpp(__float_as_int(v), kCtrl, 0xF, 0xF, true);
    return v + __int_as_float(moved);
}

__device__ __forceinline__ float wave_sum(float v) {
    v = dpp_step<0xB1>(v);   // quad_perm [1, 0, 3, 2]
    v = dpp_step<0x4E>(v);   // quad_perm [2, 3, 0, 1]
    v = dpp_step<0x141>(v);  // row_half_mirror
    v = dpp_step<0x140>(v);  // row_mirror
    const int b = __float_as_int(v);
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(b, 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(b, 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(b, 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(b, 48));
    return (r0 + r1) + (r2 + r3);
}

// A wave-uniform 64-bit value, held in scalar registers.
__device__ __forceinline__ int64_t uniform64(int64_t v) {
    const uint64_t u = static_cast<uint64_t>(v);
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(u >> 32));
    return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

template <int NC, bool WF32, bool RES, bool NT>
__global__ __launch_bounds__(NC * kWave) void rmsnorm_bwd_rows(RmsArgs a) {
    // Cache policy of the row loads: non-temporal (nt) when the rows are
    // streamed through once at sizes beyond the Infinity Cache.
    constexpr int kLoadAux = NT ? 2 : 0;
    constexpr int R = kRmsGroup;
    // Per group: each chunk's sum of every row, double-buffered so that one
    // barrier per group suffices.
    __shared__ float part[2][NC][R];

    const int lane = threadIdx.x & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);  // = chunk
    const int H = a.H;
    const int col0 = wave * kRmsChunk + lane * 8;  // this lane's first column
    const bool cols_ok = col0 < H;                 // H % 8 == 0: all 8 or none
    const uint32_t off = static_cast<uint32_t>(col0) * 2u;  // byte offset in a row

    // The lane's 8 weights as FP32 (zero past H).
    float wv[8];
    if (cols_ok) {
        if constexpr (WF32) {
            const f32x4 w0 = *reinterpret_cast<const f32x4 *>(static_cast<const float *>(a.w) + col0);
            const f32x4 w1 =
                *reinterpret_cast<const f32x4 *>(static_cast<const float *>(a.w) + col0 + 4);
#pragma unroll
            for (int j = 0; j < 4; ++j) wv[j] = w0[j], wv[j + 4] = w1[j];
        } else {
            const u32x4 wb =
                *reinterpret_cast<const u32x4 *>(static_cast<const uint16_t *>(a.w) + col0);
#pragma unroll
            for (int j = 0; j < 8; ++j) wv[j] = (j & 1) ? hi_bf16(wb[j >> 1]) : lo_bf16(wb[j >> 1]);
        }
    } else {
#pragma unroll
        for (int j = 0; j < 8; ++j) wv[j] = 0.0f;
    }
    float dw[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) dw[j] = 0.0f;

    // rstd is read-only for the whole kernel: read through the constant
    // address space it is fetched by scalar loads (one per row and wave),
    // which do not count against the vector-memory waits of the row data.
    const MHCPB_CONST float *rstd_c = (const MHCPB_CONST float *)(a.rstd);
    const int64_t S = gridDim.x;
    const int64_t blk = blockIdx.x;
    // Rows of this block: blk + k S for k < nrows (at least one: S <= T).
    const int64_t nrows = uniform64((a.T - blk + S - 1) / S);
    const int row_bytes = H * 2;

    // Row slot r holds row index k0 + r of the current group.  A row past the
    // block's last reads as zeros (an empty buffer range), its stores are
    // dropped and its rstd is 0, so it adds nothing to dw.
    u32x4 gv[R], xv[R], rv[RES ? R : 1];
    float rs[R];
    __amdgpu_buffer_rsrc_t drs[R];
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const bool ok = r < nrows;
        const int64_t t = blk + (ok ? r : 0) * S;
        const int nbytes = ok ? row_bytes : 0;
        gv[r] = __builtin_amdgcn_raw_buffer_load_b128(make_rsrc32(a.g + t * H, nbytes), off, 0, kLoadAux);
        xv[r] = __builtin_amdgcn_raw_buffer_load_b128(make_rsrc32(a.x + t * H, nbytes), off, 0, kLoadAux);
        if constexpr (RES)
            rv[r] = __builtin_amdgcn_raw_buffer_load_b128(make_rsrc32(a.res + t * H, nbytes), off,
                                                          0, kLoadAux);
        drs[r] = make_rsrc32(a.dx + t * H, nbytes);
        rs[r] = ok ? rstd_c[t] : 0.0f;
        // Issued in the order of the reloads below (row by row: g, x,
        // residual), so the compiler's counter waits stay exact where the two
        // paths meet at the loop head.
        __builtin_amdgcn_sched_barrier(0);
    }

    for (int64_t k0 = 0; k0 < nrows; k0 += R) {
        const int buf = static_cast<int>((k0 / R) & 1);
        // Pass 1: the chunk's sum of w g x for every row, and dw += (g x)
        // rstd (g x is exact in FP32: two 8-bit significands).
        float psum[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            float s = 0.0f;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t gw = gv[r][j >> 1], xw = xv[r][j >> 1];
                const float gj = (j & 1) ? hi_bf16(gw) : lo_bf16(gw);
                const float xj = (j & 1) ? hi_bf16(xw) : lo_bf16(xw);
                const float p = gj * xj;
                s = __builtin_fmaf(wv[j], p, s);
                dw[j] = __builtin_fmaf(p, rs[r], dw[j]);
            }
            // The accumulations happen here, not sunk below the group (which
            // would keep every product of the group alive).
#pragma unroll
            for (int j = 0; j < 8; ++j) asm volatile("" : "+v"(dw[j]));
            psum[r] = wave_sum(s);
        }
        // Lane r publishes row r's sum of this chunk.
        float mine = 0.0f;
#pragma unroll
        for (int r = 0; r < R; ++r) mine = (lane == r) ? psum[r] : mine;
        if (lane < R) part[buf][wave][lane] = mine;
        __syncthreads();
        // Lane r: c1 of row r from the chunks' sums in chunk order, then
        // k = c1 rstd^3.
        float kv = 0.0f;
        if (lane < R) {
            float tot = part[buf][0][lane];
#pragma unroll
            for (int c = 1; c < NC; ++c) tot += part[buf][c][lane];
            float rsl = 0.0f;
#pragma unroll
            for (int r = 0; r < R; ++r) rsl = (lane == r) ? rs[r] : rsl;
            const float c1 = tot / static_cast<float>(H);
            kv = c1 * rsl * rsl * rsl;
        }
        // Pass 2 unpacks g and x again rather than keeping pass 1's unpacked
        // values alive: the packed words pass through an empty asm, so
        // nothing is reused across.
#pragma unroll
        for (int r = 0; r < R; ++r) asm volatile("" : "+v"(gv[r]), "+v"(xv[r]));
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const float k = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(kv), r));
            const float rsr = rs[r];
            float v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint32_t gw = gv[r][j >> 1], xw = xv[r][j >> 1];
                const float gj = (j & 1) ? hi_bf16(gw) : lo_bf16(gw);
                const float xj = (j & 1) ? hi_bf16(xw) : lo_bf16(xw);
                v[j] = __builtin_fmaf(rsr * wv[j], gj, -(k * xj));
                if constexpr (RES) {
                    const uint32_t rw = rv[r][j >> 1];
                    v[j] += (j & 1) ? hi_bf16(rw) : lo_bf16(rw);
                }
            }
            const u32x4 out{pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                            pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7])};
            __builtin_amdgcn_raw_buffer_store_b128(out, drs[r], off, 0, kRmsDxAux);
            // The slot's next row (R places later); the reloads stay below
            // this row's use of the registers.
            compiler_fence();
            const int64_t kn = k0 + R + r;
            const bool ok = kn < nrows;
            const int64_t t = blk + (ok ? kn : 0) * S;
            const int nbytes = ok ? row_bytes : 0;
            gv[r] = __builtin_amdgcn_raw_buffer_load_b128(make_rsrc32(a.g + t * H, nbytes), off, 0,
                                                          kLoadAux);
            xv[r] = __builtin_amdgcn_raw_buffer_load_b128(make_rsrc32(a.x + t * H, nbytes), off, 0,
                                                          kLoadAux);
            if constexpr (RES)
                rv[r] = __builtin_amdgcn_raw_buffer_load_b128(make_rsrc32(a.res + t * H, nbytes),
                                                              off, 0, kLoadAux);
            drs[r] = make_rsrc32(a.dx + t * H, nbytes);
            rs[r] = ok ? rstd_c[t] : 0.0f;
            __builtin_amdgcn_sched_barrier(0);
        }
    }

    // This wave's columns of the block partial.
    if (cols_ok) {
        float *dst = a.ws + blk * H + col0;
        *reinterpret_cast<f32x4 *>(dst) = f32x4{dw[0], dw[1], dw[2], dw[3]};
        *reinterpret_cast<f32x4 *>(dst + 4) = f32x4{dw[4], dw[5], dw[6], dw[7]};
    }
}

// dw[h] = sum over the S block partials: group q (one wave) adds blocks
// [q P, min(S, (q + 1) P)) in ascending order, P = ceil(S / 16), starting
// from +0; the 16 group sums are then added in group order.  64 columns per
// workgroup; a lane requests up to 32 partials before adding them, so a group
// of up to 32 blocks costs one round trip to memory.
__global__ __launch_bounds__(kReduceGroups * kWave) void rmsnorm_dw_reduce(
    const float *__restrict__ ws, float *__restrict__ dw, int S, int H) {
    __shared__ float sums[kReduceGroups][kWave];
    const int lane = threadIdx.x & (kWave - 1);
    const int q = threadIdx.x / kWave;
    const int h = blockIdx.x * kWave + lane;
    const int per = (S + kReduceGroups - 1) / kReduceGroups;
    const int b0 = q * per;
    const int b1 = (S < b0 + per) ? S : b0 + per;
    float acc = 0.0f;
    if (h < H) {
        for (int b = b0; b < b1; b += kReduceBatch) {
            float v[kReduceBatch];
#pragma unroll
            for (int u = 0; u < kReduceBatch; ++u)
                v[u] = (b + u < b1) ? __builtin_nontemporal_load(
                                          ws + static_cast<int64_t>(b + u) * H + h)
                                    : -0.0f;
#pragma unroll
            for (int u = 0; u < kReduceBatch; ++u) acc += v[u];
        }
    }
    sums[q][lane] = acc;
    __syncthreads();
    if (q == 0 && h < H) {
        float t = sums[0][lane];
#pragma unroll
        for (int g = 1; g < kReduceGroups; ++g) t += sums[g][lane];
        dw[h] = t;
    }
}

using RowsKernel = void (*)(RmsArgs);

template <int NC, bool NT>
RowsKernel pick_nt(bool wf32, bool res) {
    if (wf32)
        return res ? rmsnorm_bwd_rows<NC, true, true, NT> : rmsnorm_bwd_rows<NC, true, false, NT>;
    return res ? rmsnorm_bwd_rows<NC, false, true, NT> : rmsnorm_bwd_rows<NC, false, false, NT>;
}

template <int NC>
RowsKernel pick_rows(bool wf32, bool res, bool nt) {
    return nt ? pick_nt<NC, true>(wf32, res) : pick_nt<NC, false>(wf32, res);
}

RowsKernel rows_kernel(int nc, bool wf32, bool res, bool nt) {
    switch (nc) {
    case 1: return pick_rows<1>(wf32, res, nt);
    case 2: return pick_rows<2>(wf32, res, nt);
    case 3: return pick_rows<3>(wf32, res, nt);
    case 4: return pick_rows<4>(wf32, res, nt);
    case 5: return pick_rows<5>(wf32, res, nt);
    case 6: return pick_rows<6>(wf32, res, nt);
    case 7: return pick_rows<7>(wf32, res, nt);
    case 8: return pick_rows<8>(wf32, res, nt);
    case 9: return pick_rows<9>(wf32, res, nt);
    case 10: return pick_rows<10>(wf32, res, nt);
    case 11: return pick_rows<11>(wf32, res, nt);
    case 12: return pick_rows<12>(wf32, res, nt);
    }
    return nullptr;
}

}  // namespace

hipError_t launch_rmsnorm_backward(const RmsPlan &p, const uint16_t *g, const uint16_t *x,
                                   const void *w, bool w_f32, const float *rstd,
                                   const uint16_t *res, uint16_t *dx, float *dw, float *ws,
                                   hipStream_t stream, hipEvent_t start, hipEvent_t mid,
                                   hipEvent_t stop) {
    if (p.T > 0) {
        const int nc = rmsnorm_chunks(p.H);
        // Rows streamed through once: non-temporal loads once g, x (and
        // g_residual) exceed about three quarters of the 256 MB Infinity
        // Cache, which they would only thrash; smaller inputs may stay in it.
        const uint64_t in_bytes = static_cast<uint64_t>(p.T) * static_cast<uint64_t>(p.H) * 2 *
                                  (res != nullptr ? 3 : 2);
        RowsKernel k = rows_kernel(nc, w_f32, res != nullptr, in_bytes >= kRmsStreamBytes);
        if (!k) return hipErrorInvalidValue;
        RmsArgs a{g, x, w, rstd, res, dx, ws, p.T, p.H};
        const hipError_t e = launch(k, dim3(static_cast<unsigned>(p.S)), dim3(nc * kWave), stream,
                                    start, mid, a);
        if (e != hipSuccess) return e;
    }
    else if (start || mid) {
        // No rows: kernel 1 is not launched and its events mark this point.
        if (start && hipEventRecord(start, stream) != hipSuccess) return hipErrorLaunchFailure;
        if (mid && hipEventRecord(mid, stream) != hipSuccess) return hipErrorLaunchFailure;
    }
    const unsigned blocks = static_cast<unsigned>((p.H + kWave - 1) / kWave);
    return launch(rmsnorm_dw_reduce, dim3(blocks), dim3(kReduceGroups * kWave), stream, nullptr,
                  stop, static_cast<const float *>(ws), dw, static_cast<int>(p.S), p.H);
}

}  // namespace mhcpb
