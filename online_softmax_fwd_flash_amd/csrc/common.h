// Shared device helpers for the gfx950 attention kernels: vector types, MFMA wrappers and the
// cross-lane reductions the online softmax needs.  CDNA4 only (wave64, MFMA, LDS).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "block_class.h"

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegMax = -3.402823466e+38f;  // running max starts here, never at -inf

// D(16x16) += A(16x32) * B(32x16), bf16 inputs, fp32 accumulate.  Lane l supplies A row
// (l % 16) and B column (l % 16), each with 8 consecutive k of group l / 16; D element r of
// lane l is row 4*(l/16) + r, column l % 16.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// The same MFMA shape with IEEE half inputs (same lane layout).
__device__ __forceinline__ f32x4 mfma16x16x32(f16x8 a, f16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// D(16x16) += A(16x4) * B(4x16), fp32.  Lane l supplies A[l%16][l/16] and B[l/16][l%16];
// D element r of lane l is row 4*(l/16) + r, column l % 16.
__device__ __forceinline__ f32x4 mfma16x16x4f32(float a, float b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// LDS transpose read (ds_read_b64_tr_b16), per 16-lane group: when lane j of the group reads
// 4 consecutive bf16 of row r0 + j/4 starting at column c0 + 4*(j%4), lane i receives column
// c0 + i of rows r0 .. r0+3.  `p` must point into LDS.
__device__ __forceinline__ bf16x4 lds_read_tr4(const uint16_t* p) {
    typedef __bf16 v4bf16 __attribute__((ext_vector_type(4)));
    return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
        (__attribute__((address_space(3))) v4bf16*)(p));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// max(v[l], v[l ^ 32]) for every lane l, in VALU (v_permlane32_swap_b32 exchanges lanes 32-63
// of one copy of v with lanes 0-31 of another: the two results hold v[l % 32] and
// v[32 + l % 32] in some order, and max does not care which)
__device__ __forceinline__ float halves_max(float v) {
    const unsigned u = __builtin_bit_cast(unsigned, v);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const unsigned r0 = r[0], r1 = r[1];
    return __builtin_elementwise_maximum(__builtin_bit_cast(float, r0), __builtin_bit_cast(float, r1));
}

// v[l] + v[l ^ 32] for every lane l (same exchange as halves_max; a two-term float sum is
// commutative, so both halves get the same bits)
__device__ __forceinline__ float halves_sum(float v) {
    const unsigned u = __builtin_bit_cast(unsigned, v);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const unsigned r0 = r[0], r1 = r[1];
    return __builtin_bit_cast(float, r0) + __builtin_bit_cast(float, r1);
}

// max of v over lanes l, l ^ 16, l ^ 32 and l ^ 48 (the four 16-lane rows of the wave), in
// VALU: halves_max, then v_permlane16_swap_b32 pairs each lane with lane l ^ 16.
__device__ __forceinline__ float rows4_max(float v) {
    const unsigned u = __builtin_bit_cast(unsigned, halves_max(v));
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const unsigned r0 = r[0], r1 = r[1];
    return __builtin_elementwise_maximum(__builtin_bit_cast(float, r0), __builtin_bit_cast(float, r1));
}

// v summed over lanes l, l ^ 16, l ^ 32 and l ^ 48 (the four 16-lane rows of the wave), in
// VALU: halves_sum, then v_permlane16_swap_b32 pairs each lane with lane l ^ 16.  Every step
// adds two terms, which commutes, so all four lanes get the same bits.
__device__ __forceinline__ float rows4_sum(float v) {
    const unsigned u = __builtin_bit_cast(unsigned, halves_sum(v));
    const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    const unsigned r0 = r[0], r1 = r[1];
    return __builtin_bit_cast(float, r0) + __builtin_bit_cast(float, r1);
}

__device__ __forceinline__ float xor_shfl(float v, int mask) {
    return __shfl_xor(v, mask, 64);
}

// The 16-bit element types of the MFMA kernels (the I/O type of Q, K, V, O and dO; products
// accumulate in fp32): scalar, and the 8-, 4- and 2-element vectors the kernels move.
struct Bf16 {
    typedef __bf16 s;
    typedef bf16x8 v8;
    typedef bf16x4 v4;
    typedef bf16x2 v2;
};
struct F16 {
    typedef _Float16 s;
    typedef f16x8 v8;
    typedef f16x4 v4;
    typedef f16x2 v2;
};

// Name of an element type in launch logs.
template <class E> struct ElemName;
template <> struct ElemName<Bf16> { static constexpr const char* value = "bf16"; };
template <> struct ElemName<F16> { static constexpr const char* value = "f16"; };

// Placed first in the body of a wave-uniform `if`, keeps it a branch: the compiler does not
// speculate an asm statement with side effects, so it cannot flatten the body into selects
// executed on every path (the diagonal-block masks would otherwise run on every block).
__device__ __forceinline__ void keep_branch() { asm volatile(""); }

// x unchanged, but opaque to the compiler: a float result rounded to 16 bits after this is
// rounded from its float32 value (the compiler may otherwise fold the product feeding a
// conversion into a mixed-precision multiply that rounds only once, to 16 bits).
__device__ __forceinline__ float opaque(float x) {
    asm volatile("" : "+v"(x));
    return x;
}

// Round-to-nearest-even float -> element pair, packed low element first.
template <class E>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
    typename E::v2 r;
    r[0] = (typename E::s)lo;
    r[1] = (typename E::s)hi;
    return __builtin_bit_cast(uint32_t, r);
}

// LDS transpose read of 16-bit elements (the instruction moves 16-bit lanes whatever their
// type; see lds_read_tr4).
template <class E>
__device__ __forceinline__ typename E::v4 lds_read_tr4e(const uint16_t* p) {
    return __builtin_bit_cast(typename E::v4, lds_read_tr4(p));
}

// sum_i a_i * b_i over the 8 elements packed in two 16-byte words, in fp32 (exact products,
// fp32 sums in element order).
template <class E>
__device__ __forceinline__ float dot8(const u32x4& a, const u32x4& b, float s);
template <>
__device__ __forceinline__ float dot8<Bf16>(const u32x4& a, const u32x4& b, float s) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t x = a[i], y = b[i];
        s = fmaf(__builtin_bit_cast(float, x << 16), __builtin_bit_cast(float, y << 16), s);
        s = fmaf(__builtin_bit_cast(float, x & 0xffff0000u), __builtin_bit_cast(float, y & 0xffff0000u), s);
    }
    return s;
}
template <>
__device__ __forceinline__ float dot8<F16>(const u32x4& a, const u32x4& b, float s) {
    const f16x8 x = __builtin_bit_cast(f16x8, a), y = __builtin_bit_cast(f16x8, b);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const _Float16 xi = x[i], yi = y[i];
        s = fmaf((float)xi, (float)yi, s);
    }
    return s;
}

}  // namespace fa
