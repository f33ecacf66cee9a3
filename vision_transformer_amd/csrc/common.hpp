// Shared device definitions for the gfx950 kernels: storage types,
// conversions, MFMA wrappers and small reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace jepa {

// 16-bit storage types are carried as raw bits.
struct bf16_t { uint16_t v; };
struct f16_t  { uint16_t v; };

typedef __bf16   bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8  __attribute__((ext_vector_type(8)));
typedef float    f32x16 __attribute__((ext_vector_type(16)));
typedef float    f32x4  __attribute__((ext_vector_type(4)));

enum Dt { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2, DT_Q8_0 = 3, DT_Q4_0 = 4, DT_Q4_K = 5, DT_Q6_K = 6 };

// ---------------------------------------------------------------------------
// scalar conversions (round to nearest even)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float to_f32(float x) { return x; }
__device__ __forceinline__ float to_f32(bf16_t x) {
    return __builtin_bit_cast(float, (uint32_t)x.v << 16);
}
__device__ __forceinline__ float to_f32(f16_t x) {
    return (float)__builtin_bit_cast(_Float16, x.v);
}

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float x) {
    return bf16_t{__builtin_bit_cast(uint16_t, (__bf16)x)};
}
template <> __device__ __forceinline__ f16_t from_f32<f16_t>(float x) {
    return f16_t{__builtin_bit_cast(uint16_t, (_Float16)x)};
}
// two values rounded to a 16-bit type, a in the low half (one packed
// conversion instruction for bf16)
template <typename T> __device__ __forceinline__ uint32_t pack2(float a, float b);
template <> __device__ __forceinline__ uint32_t pack2<bf16_t>(float a, float b) {
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    const bf16x2 v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}
template <> __device__ __forceinline__ uint32_t pack2<f16_t>(float a, float b) {
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
    const f16x2 v = {(_Float16)a, (_Float16)b};
    return __builtin_bit_cast(uint32_t, v);
}

// ---------------------------------------------------------------------------
// MFMA 32x32 tiles.  Operand lane layout, for lane l, g = l / 32:
//   A (rows x k): row l % 32, k = g*VEC + j for slot j < VEC
//   B (k x cols): col l % 32, same k mapping
// Any consistent k mapping gives the same contraction; what matters is the
// accumulator layout: element v of lane l is C[8*(v/4) + 4*g + v%4][l%32].
// ---------------------------------------------------------------------------
template <typename T> struct Mfma;

template <> struct Mfma<bf16_t> {
    static constexpr int VEC = 8;          // elements per lane per operand
    static constexpr int KC = 16;          // k per instruction
    typedef bf16x8 vec;
    __device__ __forceinline__ static f32x16 mma(vec a, vec b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
    }
    __device__ __forceinline__ static vec load(const void *p) {
        return __builtin_bit_cast(vec, *(const uint4 *)p);
    }
};

template <> struct Mfma<f16_t> {
    static constexpr int VEC = 8;
    static constexpr int KC = 16;
    typedef f16x8 vec;
    __device__ __forceinline__ static f32x16 mma(vec a, vec b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
    }
    __device__ __forceinline__ static vec load(const void *p) {
        return __builtin_bit_cast(vec, *(const uint4 *)p);
    }
};

template <> struct Mfma<float> {
    static constexpr int VEC = 1;
    static constexpr int KC = 2;
    typedef float vec;
    __device__ __forceinline__ static f32x16 mma(vec a, vec b, f32x16 c) {
        return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
    }
    __device__ __forceinline__ static vec load(const void *p) { return *(const float *)p; }
};

// Pack VEC consecutive f32 values (already in registers) as one operand.
template <typename T> __device__ __forceinline__ typename Mfma<T>::vec pack_operand(const float *x);
template <> __device__ __forceinline__ bf16x8 pack_operand<bf16_t>(const float *x) {
    bf16x8 r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = (__bf16)x[j];
    return r;
}
template <> __device__ __forceinline__ f16x8 pack_operand<f16_t>(const float *x) {
    f16x8 r;
#pragma unroll
    for (int j = 0; j < 8; ++j) r[j] = (_Float16)x[j];
    return r;
}
template <> __device__ __forceinline__ float pack_operand<float>(const float *x) { return x[0]; }

// ---------------------------------------------------------------------------
// wavefront reductions (64 lanes)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__host__ __device__ __forceinline__ int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace jepa
