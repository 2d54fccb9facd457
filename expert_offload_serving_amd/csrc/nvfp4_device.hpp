// Device-side helpers shared by the gfx950 kernels of the NVFP4 MoE library.
//
// Number formats (PR #385 "What this adds": packed 4-bit codes with 16-wide
// FP8 scale blocks and per-row fp32 globals): codes are E2M1, of two columns
// sharing a byte the even one in the low nibble; scales are OCP E4M3FN.
// gfx950 decodes both in hardware: v_cvt_f32_fp8 follows OCP E4M3FN (all 256
// bytes checked exhaustively by the dequant test), and
// v_cvt_scalef32_pk_{f32,f16,bf16}_fp4 decodes two E2M1 codes exactly when
// the scale operand is 1.0 (the instruction only uses the scale's exponent,
// so block scales are applied separately).
//
// Slot records (byte formulas in moe_nvfp4.h): a record is 1 KiB of codes
// and 128 bytes of scales.  Lane L = 16*g + i of a wave reads the 16 code
// bytes at 16*L (dword d = one 16x16x32 MFMA operand fragment: row i of a
// 16-row tile, columns [8g, 8g+8) of a 32-column chunk) and the scale dword
// at lane_scale_off(L) (byte d = the E4M3 scale of that fragment).  For
// gate_up the dwords d of a record are four consecutive 32-column chunks of
// one 16-row tile; for down they are four consecutive 16-row tiles of one
// 32-column chunk.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));

constexpr int kWave = 64;
constexpr int kRecBytes = 1024;     // codes per record
constexpr int kRecScaleBytes = 128; // scales per record

__device__ __forceinline__ int lane_scale_off(int lane) { return 64 * (lane >> 5) + 4 * (lane & 15); }

// Raw buffer loads (gfx9 buffer resource, stride 0): a byte offset at or past
// the resource's size returns zeros without touching memory, so optional
// loads need no branch and every load of a kernel stays in one straight
// line (exact vmcnt accounting, nothing forces an early wait).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kOob = 0x7FFFFF00;  // an offset past every resource used here (< 2 GiB each)
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4_t buf_load16(rsrc_t r, int off) {
    return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ uint32_t buf_load4(rsrc_t r, int off) {
    return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}
// A store at an offset past the resource's size is dropped.
__device__ __forceinline__ void buf_store16(rsrc_t r, int off, f32x4_t v) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, off, 0, 0);
}

// E4M3 byte SEL of a scale dword as an fp16 pair (exact: E4M3 values fit fp16).
template <int SEL>
__device__ __forceinline__ f16x2_t scale_f16x2(uint32_t sdw) {
    const _Float16 v = (_Float16)__builtin_amdgcn_cvt_f32_fp8(sdw, SEL);
    return f16x2_t{v, v};
}

// One dword of codes (8 E2M1 values, column order) times the block scale S:
// an fp16 MFMA operand fragment.  Exact: e2m1 * e4m3 has at most 6
// significant bits and lies within [2^-10, 2688].
__device__ __forceinline__ f16x8_t frag_f16(uint32_t c, f16x2_t S) {
    const f16x2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 0) * S;
    const f16x2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 1) * S;
    const f16x2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 2) * S;
    const f16x2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c, 1.0f, 3) * S;
    const u32x4_t u = {__builtin_bit_cast(uint32_t, v0), __builtin_bit_cast(uint32_t, v1),
                       __builtin_bit_cast(uint32_t, v2), __builtin_bit_cast(uint32_t, v3)};
    return __builtin_bit_cast(f16x8_t, u);
}

__device__ __forceinline__ uint32_t word_of(const u32x4_t& v, int d) {
    return d == 0 ? v.x : (d == 1 ? v.y : (d == 2 ? v.z : v.w));
}

// Power-of-two exponent that puts a row maximum amax in [2^14, 2^15) (0 for amax == 0).
__device__ __forceinline__ int fp16_shift(float amax) {
    int e = 0;
    if (amax > 0.0f) (void)frexpf(amax, &e);
    return amax > 0.0f ? 15 - e : 0;
}

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

// Wave-wide reductions by DPP moves (VALU only, no LDS round trips), in a
// fixed order: lane pairs (xor 1), pairs of pairs (xor 2), the two quads of
// each 8-lane half-row, the two halves of each 16-lane row, then row 0 into
// row 1 and row 2 into row 3, and rows 0+1 into row 3; the result is lane
// 63's, returned to every lane.  Lanes a step does not write keep their value
// (sum: plus 0; max: their own), which only rows 0-2 see.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float add_dpp(float v) {
    return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xF, false));
}
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float max_dpp(float v) {
    const int b = __float_as_int(v);
    return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(b, b, CTRL, ROW_MASK, 0xF, false)));
}

// Maximum over each aligned group of 4 lanes, returned to every lane of it.
__device__ __forceinline__ float quad_max(float v) {
    v = max_dpp<0xB1, 0xF>(v);  // quad_perm [1, 0, 3, 2]
    return max_dpp<0x4E, 0xF>(v);  // quad_perm [2, 3, 0, 1]
}

// Maximum over each 16-lane row, returned to every lane of the row.
__device__ __forceinline__ float row16_max(float v) {
    v = quad_max(v);
    v = max_dpp<0x141, 0xF>(v);  // row_half_mirror
    return max_dpp<0x140, 0xF>(v);  // row_mirror
}

__device__ __forceinline__ float wave_sum(float v) {
    v = add_dpp<0xB1, 0xF>(v);   // quad_perm [1, 0, 3, 2]
    v = add_dpp<0x4E, 0xF>(v);   // quad_perm [2, 3, 0, 1]
    v = add_dpp<0x141, 0xF>(v);  // row_half_mirror
    v = add_dpp<0x140, 0xF>(v);  // row_mirror
    v = add_dpp<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
    v = add_dpp<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ float wave_max(float v) {
    v = max_dpp<0xB1, 0xF>(v);
    v = max_dpp<0x4E, 0xF>(v);
    v = max_dpp<0x141, 0xF>(v);
    v = max_dpp<0x140, 0xF>(v);
    v = max_dpp<0x142, 0xA>(v);
    v = max_dpp<0x143, 0xC>(v);
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// Opaque to the optimiser: keeps code words from being decoded once and held
// decoded across a loop (which would multiply their register footprint).
__device__ __forceinline__ void keep_packed(u32x4_t& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void keep_packed(uint32_t& v) { asm volatile("" : "+v"(v)); }

__device__ __forceinline__ float sigmoidf_(float z) { return 1.0f / (1.0f + expf(-z)); }

// silu(g) = g / (1 + e^-g) with the hardware base-2 exponential and reciprocal
// (v_exp_f32, v_rcp_f32: about 1 ulp each, far inside the layer's tolerance).
// Large |g| saturates correctly: e^-g -> inf gives -0, e^-g -> 0 gives g.
__device__ __forceinline__ float silu_fast(float g) {
    return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-g * 1.4426950408889634f));
}

}  // namespace moe
