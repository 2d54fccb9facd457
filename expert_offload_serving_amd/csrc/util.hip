// NVFP4 dequantisation (test hook) and intermediate-axis bank slicing for gfx950.
#include "internal.hpp"
#include "nvfp4_device.hpp"

namespace moe {
namespace {

// One thread per 16-byte code chunk (32 elements, two scale blocks):
// out = f32(f32(e2m1 * e4m3) * global), the same decode as the forward kernels.
__global__ void __launch_bounds__(256) dequant_kernel(const uint8_t* __restrict__ codes,
                                                       const uint8_t* __restrict__ scales,
                                                       const float* __restrict__ globals, int rows, int K,
                                                       float* __restrict__ out) {
    const int cpr = K / 32;
    const long q = (long)blockIdx.x * 256 + threadIdx.x;
    if (q >= (long)rows * cpr) return;
    const int r = (int)(q / cpr), c = (int)(q % cpr);
    const u32x4_t cw = *reinterpret_cast<const u32x4_t*>(codes + (size_t)r * (K / 2) + (size_t)c * 16);
    const uint32_t s16 = *reinterpret_cast<const uint16_t*>(scales + (size_t)r * (K / 16) + (size_t)c * 2);
    const float s[2] = {e4m3_f32<0>(s16), e4m3_f32<1>(s16)};
    const float g = globals[r];
    const uint32_t words[4] = {cw.x, cw.y, cw.z, cw.w};
    float v[32];
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
        f32x2_t a0 = e2m1x2_f32<0>(words[qq]), a1 = e2m1x2_f32<1>(words[qq]);
        f32x2_t a2 = e2m1x2_f32<2>(words[qq]), a3 = e2m1x2_f32<3>(words[qq]);
        v[8 * qq + 0] = a0.x; v[8 * qq + 1] = a0.y; v[8 * qq + 2] = a1.x; v[8 * qq + 3] = a1.y;
        v[8 * qq + 4] = a2.x; v[8 * qq + 5] = a2.y; v[8 * qq + 6] = a3.x; v[8 * qq + 7] = a3.y;
    }
    f32x4_t* o = reinterpret_cast<f32x4_t*>(out + (size_t)r * K + (size_t)c * 32);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float sb = s[i / 4];
        f32x4_t r4;
        r4.x = (v[4 * i + 0] * sb) * g;
        r4.y = (v[4 * i + 1] * sb) * g;
        r4.z = (v[4 * i + 2] * sb) * g;
        r4.w = (v[4 * i + 3] * sb) * g;
        o[i] = r4;
    }
}

// Copy one region of every slot: dst row i (rb bytes) <- src row srow(i) at
// byte col_off of a src row of pitch src_pitch.  With split > 0, dst rows
// [0, split) come from src rows rowA + i and the rest from rowB + (i - split).
template <int W>
__global__ void __launch_bounds__(256) slice_region_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                            size_t src_slot, size_t dst_slot, size_t src_base,
                                                            size_t dst_base, int rows, int rb, int src_pitch,
                                                            int col_off, int split, int rowA, int rowB) {
    const int units_per_row = rb / W;
    const long u = (long)blockIdx.x * 256 + threadIdx.x;
    if (u >= (long)rows * units_per_row) return;
    const int i = (int)(u / units_per_row), b = (int)(u % units_per_row) * W;
    const int srow = split > 0 ? (i < split ? rowA + i : rowB + (i - split)) : i;
    const uint8_t* sp = src + blockIdx.y * src_slot + src_base + (size_t)srow * src_pitch + col_off + b;
    uint8_t* dp = dst + blockIdx.y * dst_slot + dst_base + (size_t)i * rb + b;
    if constexpr (W == 16) {
        *reinterpret_cast<u32x4_t*>(dp) = *reinterpret_cast<const u32x4_t*>(sp);
    } else if constexpr (W == 4) {
        *reinterpret_cast<uint32_t*>(dp) = *reinterpret_cast<const uint32_t*>(sp);
    } else {
        *dp = *sp;
    }
}

hipError_t copy_region(const uint8_t* src, uint8_t* dst, int num_slots, size_t src_slot, size_t dst_slot,
                       size_t src_base, size_t dst_base, int rows, int rb, int src_pitch, int col_off, int split,
                       int rowA, int rowB, hipStream_t s) {
    auto fits = [&](size_t w) {
        return rb % w == 0 && src_pitch % w == 0 && col_off % w == 0 && src_base % w == 0 && dst_base % w == 0 &&
               src_slot % w == 0 && dst_slot % w == 0;
    };
    const int W = fits(16) ? 16 : (fits(4) ? 4 : 1);
    const long units = (long)rows * (rb / W);
    dim3 grid((unsigned)((units + 255) / 256), (unsigned)num_slots);
    if (W == 16)
        hipLaunchKernelGGL(slice_region_kernel<16>, grid, dim3(256), 0, s, src, dst, src_slot, dst_slot, src_base,
                           dst_base, rows, rb, src_pitch, col_off, split, rowA, rowB);
    else if (W == 4)
        hipLaunchKernelGGL(slice_region_kernel<4>, grid, dim3(256), 0, s, src, dst, src_slot, dst_slot, src_base,
                           dst_base, rows, rb, src_pitch, col_off, split, rowA, rowB);
    else
        hipLaunchKernelGGL(slice_region_kernel<1>, grid, dim3(256), 0, s, src, dst, src_slot, dst_slot, src_base,
                           dst_base, rows, rb, src_pitch, col_off, split, rowA, rowB);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dequant(const uint8_t* codes, const uint8_t* scales, const float* globals, int rows, int K,
                          float* out, hipStream_t s) {
    const long chunks = (long)rows * (K / 32);
    hipLaunchKernelGGL(dequant_kernel, dim3((unsigned)((chunks + 255) / 256)), dim3(256), 0, s, codes, scales,
                       globals, rows, K, out);
    return hipGetLastError();
}

// Slice r of n along I (issue #62 "What it touches"): gate rows [r*Il, (r+1)*Il)
// and up rows [I + r*Il, I + (r+1)*Il) with their scales and globals; down
// columns [r*Il, (r+1)*Il) of all H rows with all H globals.
hipError_t launch_slice_bank(const uint8_t* src, int num_slots, int H, int I, int r, int n, uint8_t* dst,
                             hipStream_t s) {
    const int Il = I / n;
    const SlotGeom S = slot_geom(H, I), D = slot_geom(H, Il);
    const int ga = r * Il, ua = I + r * Il;
    hipError_t e;
    // gate_up codes / scales / globals: 2*Il rows taken from two src row ranges
    if ((e = copy_region(src, dst, num_slots, S.total, D.total, S.gu_codes, D.gu_codes, 2 * Il, H / 2, H / 2, 0, Il,
                         ga, ua, s)) != hipSuccess) return e;
    if ((e = copy_region(src, dst, num_slots, S.total, D.total, S.gu_scales, D.gu_scales, 2 * Il, H / 16, H / 16, 0,
                         Il, ga, ua, s)) != hipSuccess) return e;
    if ((e = copy_region(src, dst, num_slots, S.total, D.total, S.gu_glob, D.gu_glob, 2 * Il, 4, 4, 0, Il, ga, ua,
                         s)) != hipSuccess) return e;
    // down codes / scales: column slice of every row; globals unchanged
    if ((e = copy_region(src, dst, num_slots, S.total, D.total, S.dn_codes, D.dn_codes, H, Il / 2, I / 2,
                         r * (Il / 2), 0, 0, 0, s)) != hipSuccess) return e;
    if ((e = copy_region(src, dst, num_slots, S.total, D.total, S.dn_scales, D.dn_scales, H, Il / 16, I / 16,
                         r * (Il / 16), 0, 0, 0, s)) != hipSuccess) return e;
    return copy_region(src, dst, num_slots, S.total, D.total, S.dn_glob, D.dn_glob, 1, 4 * H, 4 * H, 0, 0, 0, 0, s);
}

}  // namespace moe
