// device_common.h -- small device helpers shared by the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ssd {

constexpr float kLog2e = 1.4426950408889634f;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Storage types.  bf16 is carried as its 16-bit pattern.
struct bf16_t {
    uint16_t bits;
};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) {
    return __uint_as_float(b16 << 16);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> one word holding (lo, hi) bf16: gfx950's v_cvt_pk_bf16_f32
// (round to nearest even in the default rounding mode; NaN stays NaN).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2 v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// fp32 -> bf16 bit pattern (same conversion).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    return pack_bf16x2(f, 0.0f) & 0xffffu;
}

template <typename T>
struct Elem;

template <>
struct Elem<float> {
    __device__ __forceinline__ static float load(const float* p, int64_t i) { return p[i]; }
    __device__ __forceinline__ static void store(float* p, int64_t i, float v) { p[i] = v; }
};

template <>
struct Elem<bf16_t> {
    __device__ __forceinline__ static float load(const bf16_t* p, int64_t i) {
        return bf16_bits_to_f32(p[i].bits);
    }
    __device__ __forceinline__ static void store(bf16_t* p, int64_t i, float v) {
        p[i].bits = (uint16_t)f32_to_bf16_bits(v);
    }
};

__device__ __forceinline__ float fast_exp2(float v) { return __builtin_amdgcn_exp2f(v); }

// silu(v) = v / (1 + e^-v), with the hardware exp2 and reciprocal (about 1
// ulp each): the gate out = y silu(z) of the block around the scan, in its own
// kernel and inside chunk_scan's store, and the convolution's activation.
__device__ __forceinline__ float silu_f(float v) {
    return v * __builtin_amdgcn_rcpf(1.0f + fast_exp2(-v * kLog2e));
}

// Exact zero-order-hold input weight (exp(dt a) - 1) / a, dt where a = 0
// (page "State Space Models (SSM)", ultralytics.com glossary, section "Come
// funzionano gli SSM": Bbar = (Abar - 1) / A B).  expm1 keeps the small-step
// case accurate: the weight tends to dt as dt a -> 0.
__device__ __forceinline__ float zoh_weight(float dt, float a) {
    return a == 0.0f ? dt : (float)(expm1((double)dt * (double)a) / (double)a);
}

// Map a linear workgroup id to a logical work item so that the 8 XCDs each
// receive one contiguous range of the logical order (workgroups are handed to
// XCDs round-robin).  Identity when the count is not a multiple of 8.
__device__ __forceinline__ uint32_t xcd_logical_id(uint32_t wg, uint32_t count) {
    if ((count & 7u) != 0u) return wg;
    return (wg & 7u) * (count >> 3) + (wg >> 3);
}

}  // namespace ssd
