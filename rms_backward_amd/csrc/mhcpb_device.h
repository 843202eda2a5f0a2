// Device helpers shared by the kernels of the library (gfx950): vector
// types, the BF16 MFMA, TF32 splitting, buffer resources, LDS accesses the
// compiler does not track, counter waits, and the launch wrapper.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>
#include <tuple>

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

// The same split for W, packed as hi | lo << 16, with non-finite inputs kept
// non-finite in the high part and a zero low part.
__device__ __forceinline__ uint32_t tf32_split_packed(float v) {
    const uint32_t u = __float_as_uint(v);
    uint32_t hb;
    float lo;
    tf32_split(v, hb, lo);
    const uint32_t finite = (hb >> 16) | (__float_as_uint(lo) & 0xFFFF0000u);
    const uint32_t quiet = ((u & 0x007FFFFFu) ? (u | 0x00400000u) : u) >> 16;
    return ((u & 0x7F800000u) == 0x7F800000u) ? quiet : finite;
}

// The split of a P value for the producer wave: like tf32_split_packed for
// finite values; a NaN is first replaced by the canonical quiet NaN (so the
// rounding cannot carry it out of the exponent), and an infinity keeps an
// infinite high part (its low part is then NaN).  Either way every product
// with the value is non-finite, as IEEE arithmetic on the TF32 value gives.
__device__ __forceinline__ uint32_t tf32_split_packed_p(float v) {
    const float q = (v != v) ? __uint_as_float(0x7FC00000u) : v;
    uint32_t hb;
    float lo;
    tf32_split(q, hb, lo);
    return __builtin_amdgcn_perm(__float_as_uint(lo), hb, 0x07060302u);
}

// Both 16-bit halves equal to the low (sel = 0x05040504) or the high
// (sel = 0x07060706) half of a.
__device__ __forceinline__ uint32_t dup_low_half(uint32_t a) {
    return __builtin_amdgcn_perm(a, a, 0x05040504u);
}
__device__ __forceinline__ uint32_t dup_high_half(uint32_t a) {
    return __builtin_amdgcn_perm(a, a, 0x07060706u);
}

// Upper halves of two 32-bit words: (a >> 16) | (b & 0xFFFF0000).
__device__ __forceinline__ uint32_t hi_halves(uint32_t a, uint32_t b) {
    return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// Buffer resource over [base, base + bytes) with bytes in [0, 2^31).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc32(const void *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, bytes, kRsrcWord3);
}

// LDS accesses the compiler does not track.  X in LDS was written by LDS
// DMA, whose completion the caller establishes with an explicit vmcnt wait;
// the compiler cannot see that, and would otherwise wait for every
// outstanding global load before any LDS read it cannot prove independent of
// the DMA.  The hot loops therefore read LDS in asm statements of their own,
// each of which ends with the wait for its reads (the destination of an asm
// load holds no value the compiler may use until a wait in the same
// statement has passed), and write it through the helpers below.  The
// template argument is a constant byte offset that goes into the
// instruction's offset field (no address arithmetic).
#define MHCPB_LDS_OFFSET_CHECK static_assert(kOff >= 0 && kOff < 65536, "LDS offset field")

// LDS writes of the operand staging and the counters, equally hidden from the
// compiler's LDS-DMA ordering (they never touch the X ring); a wave waits for
// them (lgkmcnt) before it passes a barrier or signals a counter.
template <int kOff = 0>
__device__ __forceinline__ void lds_write_u32(uint32_t addr, uint32_t v) {
    MHCPB_LDS_OFFSET_CHECK;
    asm volatile("ds_write_b32 %0, %1 offset:%2" ::"v"(addr), "v"(v), "n"(kOff) : "memory");
}

template <int kOff = 0>
__device__ __forceinline__ void lds_write_u128(uint32_t addr, u32x4 v) {
    MHCPB_LDS_OFFSET_CHECK;
    asm volatile("ds_write_b128 %0, %1 offset:%2" ::"v"(addr), "v"(v), "n"(kOff) : "memory");
}

template <int kOff = 0>
__device__ __forceinline__ void lds_write_u16(uint32_t addr, uint32_t v) {
    MHCPB_LDS_OFFSET_CHECK;
    asm volatile("ds_write_b16 %0, %1 offset:%2" ::"v"(addr), "v"(v), "n"(kOff) : "memory");
}

// Writes the high 16 bits of v.
template <int kOff = 0>
__device__ __forceinline__ void lds_write_u16_hi(uint32_t addr, uint32_t v) {
    MHCPB_LDS_OFFSET_CHECK;
    asm volatile("ds_write_b16_d16_hi %0, %1 offset:%2" ::"v"(addr), "v"(v), "n"(kOff) : "memory");
}

template <int kOff = 0>
__device__ __forceinline__ void lds_write_u64(uint32_t addr, u32x2 v) {
    MHCPB_LDS_OFFSET_CHECK;
    asm volatile("ds_write_b64 %0, %1 offset:%2" ::"v"(addr), "v"(v), "n"(kOff) : "memory");
}
#undef MHCPB_LDS_OFFSET_CHECK

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

// One LDS word, read and waited for in the same asm statement.
__device__ __forceinline__ uint32_t lds_load_u32(uint32_t addr) {
    uint32_t v;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
    return v;
}

// Adds one to the LDS counter at addr once this wave's earlier LDS accesses
// have completed (lane 0 does the add).
__device__ __forceinline__ void lds_signal(uint32_t addr, int lane) {
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    if (lane == 0) asm volatile("ds_add_u32 %0, %1" ::"v"(addr), "v"(1u) : "memory");
}

// Waits until the LDS counter at addr is at least target, polling at most
// max_polls times; returns false if it gave up.  The callers' counters always
// get there, within a few steps' time; the bound (2^16 polls by default, a
// few milliseconds) only keeps a broken invariant from hanging the GPU, and a
// caller whose wait gives up marks what it writes from then on as
// untrustworthy (NaN outputs).  With max_polls = 0 every wait gives up at
// once, which is how the tests reach that path.
__device__ __forceinline__ bool lds_wait_at_least(uint32_t addr, uint32_t target, int max_polls) {
    for (int poll = 0; poll < max_polls; ++poll) {
        uint32_t v;
        asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
        if (__builtin_amdgcn_readfirstlane(v) >= target) return true;
        __builtin_amdgcn_s_sleep(1);
    }
    return false;
}

// Lane 0 writes v to the LDS word at addr; no wait (a reader takes whatever
// value it finds).
__device__ __forceinline__ void lds_publish(uint32_t addr, uint32_t v, int lane) {
    if (lane == 0) asm volatile("ds_write_b32 %0, %1" ::"v"(addr), "v"(v) : "memory");
}

// Sets the workgroup's LDS poison word at addr (lane 0 writes it) and waits
// until the write has completed, so that LDS accesses issued afterwards by
// this wave come after it.
__device__ __forceinline__ void lds_raise_poison(uint32_t addr, int lane) {
    if (lane == 0) asm volatile("ds_write_b32 %0, %1" ::"v"(addr), "v"(1u) : "memory");
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

// A launch with the given events attached to the dispatch (start and end
// times), or a plain launch when both are null.  Returns the status of this
// launch alone (the runtime's return value, not the thread's last error, which
// could be left over from unrelated earlier work).
template <typename... KArgs, typename... Args>
hipError_t launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t stream,
                  hipEvent_t start, hipEvent_t stop, Args... args) {
    static_assert(sizeof...(KArgs) == sizeof...(Args), "argument count");
    std::tuple<KArgs...> values(static_cast<KArgs>(args)...);
    void *ptrs[sizeof...(KArgs)];
    std::apply([&](auto &...v) {
        int i = 0;
        ((ptrs[i++] = static_cast<void *>(&v)), ...);
    }, values);
    const void *fn = reinterpret_cast<const void *>(kernel);
    if (start || stop) return hipExtLaunchKernel(fn, grid, block, ptrs, 0, stream, start, stop, 0);
    return hipLaunchKernel(fn, grid, block, ptrs, 0, stream);
}

}  // namespace
}  // namespace mhcpb
