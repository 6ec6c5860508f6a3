// Device-side helpers shared by the libpa kernels: element decoding,
// rounding of outputs and wavefront reductions (64-lane CDNA wavefronts).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace pa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
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

// DPP lane permutations inside 16-lane rows (CDNA DPP controls).
namespace dpp {
constexpr int quad_perm(int a, int b, int c, int d) { return a | (b << 2) | (c << 4) | (d << 6); }
constexpr int kXor1 = quad_perm(1, 0, 3, 2);
constexpr int kXor2 = quad_perm(2, 3, 0, 1);
constexpr int kHalfMirror = 0x141;  // lane i of 8 <- lane 7-i
constexpr int kRowRor8 = 0x128;     // lane i of 16 <- lane (i+8) mod 16
constexpr int kRowNewBcast0 = 0x150;  // all 16 lanes of a row <- its lane n (0x150 + n)
}  // namespace dpp

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
    return __int_as_float(
        __builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Value of lane `src` of this lane's group of G lanes (G = 8 or 16).
template <int G, int SRC>
__device__ __forceinline__ float group_bcast(float v) {
    static_assert(G == 8 || G == 16, "group of 8 or 16 lanes");
    if constexpr (G == 16) {
        return dpp_mov<dpp::kRowNewBcast0 + SRC>(v);
    } else {
        // ds_swizzle bitmask mode over 32 lanes: lane = (lane & 0x18) | SRC
        constexpr int pattern = 0x18 | (SRC << 5);
        return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), pattern));
    }
}

// Partner lane for the transpose-reduce step that splits on bit `HALF` of
// the lane's index inside its group. Steps run from the high bit down; any
// pairing works that flips bit HALF while keeping the higher bits (those of
// earlier steps), so row rotation by 8 and the half-row mirror serve for the
// two high bits.
template <int HALF>
__device__ __forceinline__ float tr_partner(float v) {
    if constexpr (HALF == 8) return dpp_mov<dpp::kRowRor8>(v);
    else if constexpr (HALF == 4) return dpp_mov<dpp::kHalfMirror>(v);
    else if constexpr (HALF == 2) return dpp_mov<dpp::kXor2>(v);
    else return dpp_mov<dpp::kXor1>(v);
}

// Maximum over the 64 lanes, returned in every lane: DPP inside each
// 16-lane row, then the four row results read as scalars.
__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, dpp_mov<dpp::kXor1>(v));
    v = fmaxf(v, dpp_mov<dpp::kXor2>(v));
    v = fmaxf(v, dpp_mov<dpp::kHalfMirror>(v));
    v = fmaxf(v, dpp_mov<dpp::kRowRor8>(v));
    const float r0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float r1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float r2 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float r3 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
}

// Buffer resource for a byte range starting at `base` (wavefront-uniform):
// buffer loads at offsets >= num_records return zero without touching
// memory, which masks absent rows and blocks for free.
constexpr int kBufferFlags = 0x00020000;  // raw 32-bit data format (gfx9 family)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base,
                                                            uint32_t num_records) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)num_records,
                                             kBufferFlags);
}

// Cache policy of the KV stream: every cache row is read once per step, so
// loads are marked non-temporal (the `nt` bit); on MI355X this lifts a pure
// 16-byte streaming read from about 6.2 to about 7.0 TB/s.
#ifndef PA_LOAD_AUX
#define PA_LOAD_AUX 2
#endif
// Bytes of padding after each K/V row in the LDS tiles of the matrix-core
// kernels. 32 spreads their 16-byte K reads and transposed V reads over the
// banks; other values build variants for comparison (the rocprofv3
// SQ_LDS_BANK_CONFLICT counts of both are kept with the profiles).
#ifndef PA_LDS_ROW_PAD
#define PA_LDS_ROW_PAD 32
#endif

// the policy for rows whose head slices share cache lines (see the kernels)
#ifndef PA_LOAD_AUX_SHARED_LINES
#define PA_LOAD_AUX_SHARED_LINES 0
#endif

// Added to the in-block offset of a lane whose 16-byte slice of the row
// does not exist (head_dim laid out wider than it is): past every range a
// descriptor has (at most a block, and the host requires blocks below
// 2^27 bytes), so the load reads zeros without touching memory.
constexpr uint32_t kNoSlice = 1u << 27;

template <int AUX = PA_LOAD_AUX>
__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, AUX);
}

// Compile-time loop: f(std::integral_constant<int, I>) for I in [B, E).
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

}  // namespace pa
