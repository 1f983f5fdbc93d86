// gdn_common.h -- device helpers shared by the HIP kernels of libgdn (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/gdn.h"

namespace gdn {

// ---------------------------------------------------------------- io types
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// Round to nearest even; NaN stays a quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float round_to_bf16(float f) {
    return bf16_bits_to_f32(f32_to_bf16_bits(f));
}

template <typename IO> struct io_traits;

template <> struct io_traits<float> {
    static constexpr int bytes = 4;
    __device__ static __forceinline__ float load(const void* p, int64_t i) {
        return static_cast<const float*>(p)[i];
    }
    __device__ static __forceinline__ void store(void* p, int64_t i, float v) {
        static_cast<float*>(p)[i] = v;
    }
    __device__ static __forceinline__ float round(float v) { return v; }
    __device__ static __forceinline__ void copy(void* dst, int64_t di, const void* src, int64_t si) {
        static_cast<float*>(dst)[di] = static_cast<const float*>(src)[si];
    }
};

template <> struct io_traits<bf16_t> {
    static constexpr int bytes = 2;
    __device__ static __forceinline__ float load(const void* p, int64_t i) {
        return bf16_bits_to_f32(static_cast<const uint16_t*>(p)[i]);
    }
    __device__ static __forceinline__ void store(void* p, int64_t i, float v) {
        static_cast<uint16_t*>(p)[i] = static_cast<uint16_t>(f32_to_bf16_bits(v));
    }
    __device__ static __forceinline__ float round(float v) { return round_to_bf16(v); }
    __device__ static __forceinline__ void copy(void* dst, int64_t di, const void* src, int64_t si) {
        static_cast<uint16_t*>(dst)[di] = static_cast<const uint16_t*>(src)[si];
    }
};

// ---------------------------------------------------------------- scalar math
// softplus(x) = max(x, 0) + log(1 + exp(-|x|)): no overflow, no cancellation.
__device__ __forceinline__ float softplus_f32(float x) {
    return fmaxf(x, 0.0f) + log1pf(expf(-fabsf(x)));
}

__device__ __forceinline__ float sigmoid_f32(float x) { return 1.0f / (1.0f + expf(-x)); }

__device__ __forceinline__ float silu_f32(float x) { return x / (1.0f + expf(-x)); }

// SiLU with the hardware exp2 and reciprocal (about 2 ulp of fp32), for
// results that are rounded to bf16 or scaled further right after.
__device__ __forceinline__ float silu_fast(float y) {
    return y * __builtin_amdgcn_rcpf(1.0f + __expf(-y));
}

// Wave-wide (64 lanes) butterfly sum; every lane gets the total.  The order of
// additions is fixed, so the result is deterministic.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

}  // namespace gdn
