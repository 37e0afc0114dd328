// gfx950.hpp - small device helpers shared by the CDNA4 kernels of libfa.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// D(32x32, f32) += A(32x16, bf16) * B(16x32, bf16) on the matrix cores.
// Operand layout per lane l (h = l / 32): A holds row l % 32, k = 8h .. 8h+7;
// B holds column l % 32, k = 8h .. 8h+7; D register r holds row 8(r/4) + 4h + r%4,
// column l % 32.
__device__ __forceinline__ f32x16 mfma_32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Hardware base-2 exponential (v_exp_f32): exp2(-inf) = 0.
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Two floats to two bfloat16 with round-to-nearest-even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    f32x2 t = {lo, hi};
    bf16x2 r = __builtin_convertvector(t, bf16x2);
    return __builtin_bit_cast(uint32_t, r);
}

// Exchange a value with lane l ^ 32 and combine: after the swap every lane of the pair sees
// both halves, so max/sum of the two results is the pair's max/sum in both lanes.
__device__ __forceinline__ float pair32_max(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// Maximum that propagates NaN instead of quieting its inputs first (v_maximum3_f32 on
// gfx950): max/fmaxf on values the compiler cannot prove canonical (MFMA results, lane
// swaps) cost an extra instruction per input.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float pair32_vmax(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return vmax(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair32_sum(float x) {
    auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// bf16 bit patterns (low / high half of a packed word) widened to f32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

template <typename T>
__device__ __forceinline__ T min_(T a, T b) { return a < b ? a : b; }
template <typename T>
__device__ __forceinline__ T max_(T a, T b) { return a > b ? a : b; }

}  // namespace fa
