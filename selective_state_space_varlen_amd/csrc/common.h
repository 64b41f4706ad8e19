// Device helpers shared by the ssmpack kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

#include "ssmpack.h"

namespace ssmp {

constexpr int kWave = 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// bf16 is carried as its 16 raw bits. Widening is exact; narrowing rounds to
// nearest even (one v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ float bf16_to_f32(uint32_t bits) { return __builtin_bit_cast(float, bits << 16); }
__device__ __forceinline__ float bf16_hi_to_f32(uint32_t word) { return __builtin_bit_cast(float, word & 0xffff0000u); }
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

// A buffer resource over n bytes at p. Raw buffer stores past the n bytes are
// dropped by the hardware and loads there return zero, so lanes (and rows,
// with n = 0) that have nothing to store or read need neither a branch nor a
// clamped address. The address is a 64-bit scalar base plus a 32-bit lane
// offset, with no per-lane 64-bit arithmetic. The third word is the gfx9
// raw-buffer format (32-bit data format, no swizzle).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t bytes_rsrc(const void* p, uint32_t n) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), 0, (int)n, 0x00020000);
}
// cache-policy argument of a raw buffer access: non-temporal
constexpr int kBufNT = 2;

template <typename T>
struct Elt;

// st_rsrc<kBufNT>: a non-temporal store, for outputs that no kernel of the
// pass reads again soon (they then do not push shared inputs out of the L2).
// Only where a wave's stores cover whole 128-byte lines: partial lines stored
// this way reach memory unmerged.
// raw: the element's bits, loaded without conversion (so a load issued ahead
// of its use is not waited on at once); cvt: those bits as fp32.
template <>
struct Elt<float> {
    static __device__ __forceinline__ float ld(const float* __restrict__ p, size_t i) { return p[i]; }
    static __device__ __forceinline__ uint32_t raw(const float* __restrict__ p, size_t i) {
        return __builtin_bit_cast(uint32_t, p[i]);
    }
    static __device__ __forceinline__ float cvt(uint32_t b) { return __builtin_bit_cast(float, b); }
    // raw bits at byte offset o of a buffer resource (zero past its end)
    static __device__ __forceinline__ uint32_t raw_rsrc(__amdgpu_buffer_rsrc_t r, uint32_t o) {
        return __builtin_amdgcn_raw_buffer_load_b32(r, (int)o, 0, 0);
    }
    static __device__ __forceinline__ void st(float* __restrict__ p, size_t i, float v) { p[i] = v; }
    // store at byte offset o of a buffer resource (dropped past its end);
    // AUX 2 marks it non-temporal
    template <int AUX = 0>
    static __device__ __forceinline__ void st_rsrc(__amdgpu_buffer_rsrc_t r, uint32_t o, float v) {
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), r, (int)o, 0, AUX);
    }
};

// p advanced by a 32-bit byte offset: a wave-uniform base plus a lane offset
// that loads and stores take as they are (no 64-bit address arithmetic)
template <typename T>
__device__ __forceinline__ T* at_bytes(T* p, uint32_t o) {
    return reinterpret_cast<T*>(reinterpret_cast<char*>(p) + o);
}
template <typename T>
__device__ __forceinline__ const T* at_bytes(const T* p, uint32_t o) {
    return reinterpret_cast<const T*>(reinterpret_cast<const char*>(p) + o);
}

template <>
struct Elt<uint16_t> {
    static __device__ __forceinline__ float ld(const uint16_t* __restrict__ p, size_t i) { return bf16_to_f32(p[i]); }
    static __device__ __forceinline__ uint32_t raw(const uint16_t* __restrict__ p, size_t i) { return p[i]; }
    static __device__ __forceinline__ float cvt(uint32_t b) { return bf16_to_f32(b); }
    static __device__ __forceinline__ uint32_t raw_rsrc(__amdgpu_buffer_rsrc_t r, uint32_t o) {
        return __builtin_amdgcn_raw_buffer_load_b16(r, (int)o, 0, 0);
    }
    static __device__ __forceinline__ void st(uint16_t* __restrict__ p, size_t i, float v) { p[i] = f32_to_bf16(v); }
    template <int AUX = 0>
    static __device__ __forceinline__ void st_rsrc(__amdgpu_buffer_rsrc_t r, uint32_t o, float v) {
        __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(v), r, (int)o, 0, AUX);
    }
};

// One row of NS values of a (T, N) tensor at a wave-uniform address. bf16
// rows are read as 32-bit words (N even) so the loads stay scalar.
template <int NS>
__device__ __forceinline__ void load_row(const float* __restrict__ p, float (&v)[NS]) {
#pragma unroll
    for (int n = 0; n < NS; ++n) v[n] = p[n];
}

template <int NS>
__device__ __forceinline__ void load_row(const uint16_t* __restrict__ p, float (&v)[NS]) {
    if constexpr (NS % 2 == 0) {
        const uint32_t* __restrict__ q = reinterpret_cast<const uint32_t*>(p);
#pragma unroll
        for (int n = 0; n < NS / 2; ++n) {
            const uint32_t w = q[n];
            v[2 * n] = bf16_to_f32(w);
            v[2 * n + 1] = bf16_hi_to_f32(w);
        }
    } else {
#pragma unroll
        for (int n = 0; n < NS; ++n) v[n] = bf16_to_f32(p[n]);
    }
}

// 2^x on the transcendental unit (v_exp_f32). Results below the normal range
// flush to zero, which only ever removes a decayed contribution.
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Logistic sigmoid 1 / (1 + e^-v) from v_exp_f32 and v_rcp_f32 (about 2 ulp).
__device__ __forceinline__ float sigmoid_fast(float v) {
    return __builtin_amdgcn_rcpf(1.0f + exp2_fast(-v * kLog2e));
}

// Ordering point for LDS traffic inside a one-wave workgroup. A wave's LDS
// operations execute in issue order, so no hardware barrier is needed; this
// only stops the compiler from moving LDS accesses across it.
__device__ __forceinline__ void wave_sync() { __builtin_amdgcn_wave_barrier(); }

// Wait for every scalar load (and LDS access) in flight, as a real s_waitcnt
// that the compiler's wait pass sees, and keep later instructions after it.
// Scalar loads complete out of order, so any wait for one waits for all:
// issued before the loads of the next token's rows, it keeps the wait for
// this token's rows from landing after them, which would expose their whole
// latency on every token.
__device__ __forceinline__ void scalar_loads_done() {
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt at their maxima
    asm volatile("" ::: "memory");       // no load moves above it
    __builtin_amdgcn_sched_barrier(0);
}

// Value of the neighbouring lane (lane ^ 1) through DPP, without the LDS path.
__device__ __forceinline__ float swap_adjacent(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0xB1, 0xF, 0xF, true));
}

// Zero n floats: where an empty input still has sums to report. A kernel,
// not a memset, so that a caller may capture the call in a graph.
template <int kUnused = 0>
__global__ __launch_bounds__(256) void k_zero_f32(float* __restrict__ p, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0.0f;
}
inline int zero_f32(float* p, int64_t n, hipStream_t s) {
    if (!p || n <= 0) return SSMP_OK;
    k_zero_f32<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(p, n);
    return hipGetLastError() == hipSuccess ? SSMP_OK : SSMP_ERR_HIP;
}

// sum_{r < n} p[r * stride], added in the order r = 0, 1, ..., n-1 (so the
// result does not depend on the batch size), with kB loads in flight at a time
// instead of one.
template <int kB = 16>
__device__ __forceinline__ float ordered_sum(const float* __restrict__ p, int64_t n, size_t stride) {
    float acc = 0.0f;
    int64_t r = 0;
    for (; r + kB <= n; r += kB) {
        float v[kB];
#pragma unroll
        for (int j = 0; j < kB; ++j) v[j] = p[(size_t)(r + j) * stride];
#pragma unroll
        for (int j = 0; j < kB; ++j) acc += v[j];
    }
    for (; r < n; ++r) acc += p[(size_t)r * stride];
    return acc;
}

// f(integral_constant<0>), ..., f(integral_constant<N-1>): a loop whose index
// is a compile-time constant in each step
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}
// the same, stopping before step n (n <= N, wave-uniform)
template <typename F, int... I>
__device__ __forceinline__ void static_for_until_impl(F& f, int n, std::integer_sequence<int, I...>) {
    (void)((I < n && (f(std::integral_constant<int, I>{}), true)) && ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for_until(F&& f, int n) {
    static_for_until_impl(f, n, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

}  // namespace ssmp

// Host-side: launch check.
#define SSMP_LAUNCH_CHECK()                                   \
    do {                                                      \
        if (hipGetLastError() != hipSuccess) return SSMP_ERR_HIP; \
    } while (0)
