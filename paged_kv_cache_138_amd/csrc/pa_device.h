// Device-side helpers shared by the libpa kernels: element decoding,
// rounding of outputs and wavefront reductions (64-lane CDNA wavefronts).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// Stored element types. A 32-bit word holds two consecutive elements, the
// lower-addressed one in the low half.
// ---------------------------------------------------------------------------

struct KvF16 {
    // a.lo*b.lo + a.hi*b.hi + acc with fp32 accumulation (v_dot2_f32_f16);
    // fp16 products are exact in fp32.
    static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
        return __builtin_amdgcn_fdot2(__builtin_bit_cast(h2_t, a), __builtin_bit_cast(h2_t, b),
                                      acc, false);
    }
    static __device__ __forceinline__ float lo(uint32_t v) {
        return (float)__builtin_bit_cast(h2_t, v).x;
    }
    static __device__ __forceinline__ float hi(uint32_t v) {
        return (float)__builtin_bit_cast(h2_t, v).y;
    }
};

struct KvBF16 {
    // bf16 products are exact in fp32 (8-bit significands).
    static __device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float acc) {
        return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2_t, a),
                                               __builtin_bit_cast(bf2_t, b), acc, false);
    }
    static __device__ __forceinline__ float lo(uint32_t v) { return __uint_as_float(v << 16); }
    static __device__ __forceinline__ float hi(uint32_t v) {
        return __uint_as_float(v & 0xffff0000u);
    }
};

// ---------------------------------------------------------------------------
// Output element types: round to nearest even from fp32.
// ---------------------------------------------------------------------------

__device__ __forceinline__ uint32_t f32_to_bf16_rne(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;  // NaN stays NaN
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t f32_to_f16_rne(float x) {
    // v_cvt_f16_f32 rounds to nearest even in the default mode
    _Float16 h = (_Float16)x;
    return (uint32_t)__builtin_bit_cast(uint16_t, h);
}

struct OutF32 {
    static constexpr int kBytes = 4;
    static __device__ __forceinline__ void store(void* base, size_t idx, float v) {
        ((float*)base)[idx] = v;
    }
    static __device__ __forceinline__ void store2(void* base, size_t idx, float a, float b) {
        float2 t;
        t.x = a;
        t.y = b;
        *(float2*)((float*)base + idx) = t;
    }
};

struct OutF16 {
    static constexpr int kBytes = 2;
    static __device__ __forceinline__ void store(void* base, size_t idx, float v) {
        ((uint16_t*)base)[idx] = (uint16_t)f32_to_f16_rne(v);
    }
    static __device__ __forceinline__ void store2(void* base, size_t idx, float a, float b) {
        *(uint32_t*)((uint16_t*)base + idx) = f32_to_f16_rne(a) | (f32_to_f16_rne(b) << 16);
    }
};

struct OutBF16 {
    static constexpr int kBytes = 2;
    static __device__ __forceinline__ void store(void* base, size_t idx, float v) {
        ((uint16_t*)base)[idx] = (uint16_t)f32_to_bf16_rne(v);
    }
    static __device__ __forceinline__ void store2(void* base, size_t idx, float a, float b) {
        *(uint32_t*)((uint16_t*)base + idx) = f32_to_bf16_rne(a) | (f32_to_bf16_rne(b) << 16);
    }
};

// ---------------------------------------------------------------------------
// Wavefront helpers
// ---------------------------------------------------------------------------

__device__ __forceinline__ float fast_exp2(float x) {
    // v_exp_f32: 2^x, exp2(-inf) = 0
    return __builtin_amdgcn_exp2f(x);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
    return v;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

}  // namespace pa
