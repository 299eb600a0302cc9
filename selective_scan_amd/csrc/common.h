// Device-side helpers shared by the gfx950 kernels of this library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssm {

constexpr float kLog2e = 1.4426950408889634f;

// Raw buffer descriptor word 3 for gfx9-class parts (raw, untyped dword access).
constexpr int kBufferFlags = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kBufferFlags);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float(((uint32_t)v) << 16); }

// fp32 -> bf16, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// 2^x on the transcendental unit (v_exp_f32).
__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float rcp_fast(float x) { return __builtin_amdgcn_rcpf(x); }

// silu(z) = z * sigmoid(z) = z / (1 + 2^(-z log2 e))
__device__ __forceinline__ float silu(float z) {
    return z * rcp_fast(1.0f + exp2_fast(-z * kLog2e));
}

// One element of an io tensor through a buffer descriptor; byte offsets.
template <bool BF16>
__device__ __forceinline__ float load_io(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    if constexpr (BF16) {
        return bf16_to_f32(__builtin_amdgcn_raw_buffer_load_b16(r, (int)voff, (int)soff, 0));
    } else {
        return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0));
    }
}

template <bool BF16>
__device__ __forceinline__ void store_io(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff, float v) {
    if constexpr (BF16) {
        __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16(v), r, (int)voff, (int)soff, 0);
    } else {
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, (int)voff, (int)soff, 0);
    }
}

// A row of N io-dtype values that is the same for every lane of the wave
// (B_t or C_t): read with scalar loads and widened to fp32 by SALU ops.
// The constant address space tells the compiler the data is read-only for the
// kernel's lifetime, which is what lets it pick scalar (SMEM) loads.
typedef __attribute__((address_space(4))) const uint32_t cu32;
typedef __attribute__((address_space(4))) const float cf32;

template <int N, bool BF16>
__device__ __forceinline__ void load_uniform_row(const void* __restrict__ base, long row, float (&out)[N]) {
    if constexpr (BF16) {
        cu32* p = (cu32*)(base) + row * (N / 2);
#pragma unroll
        for (int k = 0; k < N / 2; ++k) {
            uint32_t w = p[k];
            out[2 * k] = bf16_lo(w);
            out[2 * k + 1] = bf16_hi(w);
        }
    } else {
        cf32* p = (cf32*)(base) + row * N;
#pragma unroll
        for (int k = 0; k < N; ++k) out[k] = p[k];
    }
}

// Uniform rows of B or C for one time step, kept packed until use.
template <int N, bool BF16>
struct Row {
    static constexpr int K = BF16 ? N / 2 : N;
    uint32_t v[K];
    // row `row` of a matrix whose rows are `rw` 32-bit words apart
    __device__ __forceinline__ void load(const void* base, long row, int rw) {
        cu32* p = (cu32*)(base) + row * rw;
#pragma unroll
        for (int k = 0; k < K; ++k) v[k] = p[k];
    }
    __device__ __forceinline__ float at(int n) const {
        if constexpr (BF16) return (n & 1) ? bf16_hi(v[n >> 1]) : bf16_lo(v[n >> 1]);
        else return __uint_as_float(v[n]);
    }
};

// Raw element of an io tensor (bf16 bits or fp32 bits); widened only at use, so a
// prefetched load is not waited for until the step that consumes it.
template <bool BF16>
__device__ __forceinline__ uint32_t load_raw(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    if constexpr (BF16) return __builtin_amdgcn_raw_buffer_load_b16(r, (int)voff, (int)soff, 0);
    else return __builtin_amdgcn_raw_buffer_load_b32(r, (int)voff, (int)soff, 0);
}

template <bool BF16>
__device__ __forceinline__ float widen(uint32_t v) {
    if constexpr (BF16) return __uint_as_float(v << 16);
    else return __uint_as_float(v);
}

}  // namespace ssm
