// Device-side helpers shared by the gfx950 kernels of the NVFP4 MoE library.
//
// Number formats (PR #385 "What this adds": packed 4-bit codes with 16-wide
// FP8 scale blocks and per-row fp32 globals): codes are E2M1, element 2j of
// a row in the low nibble of byte j; scales are OCP E4M3FN.  gfx950 decodes
// both in hardware: v_cvt_f32_fp8 follows OCP E4M3FN (all 256 bytes checked
// exhaustively by the dequant test), and v_cvt_scalef32_pk_{f32,bf16}_fp4
// decodes two E2M1 codes exactly when the scale operand is 1.0 (the
// instruction only uses the scale's exponent, so block scales are applied
// separately).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// E4M3FN byte SEL of `word` -> f32 (exact).
template <int SEL>
__device__ __forceinline__ float e4m3_f32(uint32_t word) {
    return __builtin_amdgcn_cvt_f32_fp8(word, SEL);
}

// The two E2M1 codes in byte SEL of `word` -> (low nibble, high nibble) as f32 (exact).
template <int SEL>
__device__ __forceinline__ f32x2_t e2m1x2_f32(uint32_t word) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, SEL);
}

// The two E2M1 codes in byte SEL of `word` -> bf16x2 (exact).
template <int SEL>
__device__ __forceinline__ bf16x2_t e2m1x2_bf16(uint32_t word) {
    return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, 1.0f, SEL);
}

__device__ __forceinline__ float bf16_bits_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

// 2-element bf16 dot product accumulated in f32 (v_dot2c_f32_bf16).
__device__ __forceinline__ float dot2_bf16(bf16x2_t a, bf16x2_t b, float c) {
    return __builtin_amdgcn_fdot2_f32_bf16(a, b, c, false);
}

__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t u) { return __builtin_bit_cast(bf16x2_t, u); }

// 16 E2M1 codes (8 bytes = 2 words, one scale block) dotted with 16 bf16
// activations (8 packed words): exact products, f32 accumulation.
__device__ __forceinline__ float block16_dot_bf16(uint32_t w0, uint32_t w1, const uint32_t* xw) {
    float p = 0.0f;
    p = dot2_bf16(e2m1x2_bf16<0>(w0), as_bf16x2(xw[0]), p);
    p = dot2_bf16(e2m1x2_bf16<1>(w0), as_bf16x2(xw[1]), p);
    p = dot2_bf16(e2m1x2_bf16<2>(w0), as_bf16x2(xw[2]), p);
    p = dot2_bf16(e2m1x2_bf16<3>(w0), as_bf16x2(xw[3]), p);
    p = dot2_bf16(e2m1x2_bf16<0>(w1), as_bf16x2(xw[4]), p);
    p = dot2_bf16(e2m1x2_bf16<1>(w1), as_bf16x2(xw[5]), p);
    p = dot2_bf16(e2m1x2_bf16<2>(w1), as_bf16x2(xw[6]), p);
    p = dot2_bf16(e2m1x2_bf16<3>(w1), as_bf16x2(xw[7]), p);
    return p;
}

// Sum over groups of G consecutive lanes (G a power of two <= 64); every lane
// of a group ends with the group's total.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
    for (int off = G / 2; off > 0; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

__device__ __forceinline__ float wave_sum(float v) { return group_sum<kWave>(v); }

// Opaque to the optimiser: keeps code words from being decoded once and held
// decoded across a loop (which would multiply their register footprint).
__device__ __forceinline__ void keep_packed(u32x4_t& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void keep_packed(uint32_t& v) { asm volatile("" : "+v"(v)); }

__device__ __forceinline__ float sigmoidf_(float z) { return 1.0f / (1.0f + expf(-z)); }

}  // namespace moe
