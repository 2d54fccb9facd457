// NVFP4 dequantisation (test hook) and intermediate-axis bank slicing for gfx950.
#include "internal.hpp"
#include "nvfp4_device.hpp"

namespace moe {
namespace {

// One thread per lane record: 16 code bytes (four operand fragments) and
// their scale dword, decoded with frag_f16 exactly as the forward kernels do,
// then out = f32(e2m1 * e4m3) * global, written row-major.
template <bool DOWN>
__global__ void __launch_bounds__(256) dequant_kernel(const uint8_t* __restrict__ slot, int H, int I, size_t codes_off,
                                                      size_t scales_off, size_t glob_off, float* __restrict__ out) {
    const int N = DOWN ? H : 2 * I, K = DOWN ? I : H;
    const long n_lanes = (long)N * K / 32;  // 16 code bytes each
    const long q = (long)blockIdx.x * 256 + threadIdx.x;
    if (q >= n_lanes) return;
    const long rec = q / kWave;
    const int lane = (int)(q % kWave), i = lane & 15, g = lane >> 4;
    const u32x4_t cw = *reinterpret_cast<const u32x4_t*>(slot + codes_off + rec * kRecBytes + 16 * lane);
    const uint32_t sw =
        *reinterpret_cast<const uint32_t*>(slot + scales_off + rec * kRecScaleBytes + lane_scale_off(lane));
    const float* glob = reinterpret_cast<const float*>(slot + glob_off);
    // record -> (row tile, column chunk) of each of its four fragments
    int row[4], col[4];
    if (!DOWN) {
        const int NT = N / 16, q128 = (int)(rec / NT), t = (int)(rec % NT);
        for (int d = 0; d < 4; ++d) row[d] = 16 * t + i, col[d] = 128 * q128 + 32 * d + 8 * g;
    } else {
        const int NG = N / 64, kc = (int)(rec / NG), p = (int)(rec % NG);
        for (int d = 0; d < 4; ++d) row[d] = 64 * p + 16 * d + i, col[d] = 32 * kc + 8 * g;
    }
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        f16x2_t S;
        if (d == 0) S = scale_f16x2<0>(sw);
        else if (d == 1) S = scale_f16x2<1>(sw);
        else if (d == 2) S = scale_f16x2<2>(sw);
        else S = scale_f16x2<3>(sw);
        const f16x8_t v = frag_f16(word_of(cw, d), S);
        const float gl = glob[row[d]];
        f32x4_t lo, hi;
        for (int e = 0; e < 4; ++e) lo[e] = (float)v[e] * gl, hi[e] = (float)v[4 + e] * gl;
        f32x4_t* o = reinterpret_cast<f32x4_t*>(out + (size_t)row[d] * K + col[d]);
        o[0] = lo;
        o[1] = hi;
    }
}

// Row-major matrix: one thread per code dword (8 consecutive columns of a
// row, element 2j in the low nibble of byte j), decoded by frag_f16 with
// the scale of its 16-column block, then times the row's global.
__global__ void __launch_bounds__(256) dequant_rows_kernel(const uint8_t* __restrict__ codes,
                                                           const uint8_t* __restrict__ scales,
                                                           const float* __restrict__ globals, int rows, int K,
                                                           float* __restrict__ out) {
    const long per_row = K / 8;
    const long q = (long)blockIdx.x * 256 + threadIdx.x;
    if (q >= (long)rows * per_row) return;
    const long r = q / per_row;
    const int c0 = (int)(q % per_row) * 8;
    const uint32_t cw = *reinterpret_cast<const uint32_t*>(codes + r * (K / 2) + c0 / 2);
    const uint32_t sb = scales[r * (K / 16) + c0 / 16];
    const f16x8_t v = frag_f16(cw, scale_f16x2<0>(sb));
    const float gl = globals[r];
    f32x4_t lo, hi;
    for (int e = 0; e < 4; ++e) lo[e] = (float)v[e] * gl, hi[e] = (float)v[4 + e] * gl;
    f32x4_t* o = reinterpret_cast<f32x4_t*>(out + r * K + c0);
    o[0] = lo;
    o[1] = hi;
}

// Copy records of every slot: dst record o*per + i of a region <- src record
// o*src_per + (i < split ? a + i : b + (i - split)), rb bytes each.
__global__ void __launch_bounds__(256) copy_records_kernel(const uint8_t* __restrict__ src, uint8_t* __restrict__ dst,
                                                           size_t src_slot, size_t dst_slot, size_t src_base,
                                                           size_t dst_base, int n_outer, int per, int src_per, int rb,
                                                           int split, int ra, int rb2) {
    const int units = rb / 4;
    const long u = (long)blockIdx.x * 256 + threadIdx.x;
    if (u >= (long)n_outer * per * units) return;
    const long d = u / units;
    const int w = (int)(u % units);
    const int o = (int)(d / per), i = (int)(d % per);
    const long sr = (long)o * src_per + (i < split ? ra + i : rb2 + (i - split));
    const uint32_t* sp = reinterpret_cast<const uint32_t*>(src + blockIdx.y * src_slot + src_base + sr * rb) + w;
    uint32_t* dp = reinterpret_cast<uint32_t*>(dst + blockIdx.y * dst_slot + dst_base + d * rb) + w;
    *dp = *sp;
}

hipError_t copy_records(const uint8_t* src, uint8_t* dst, int num_slots, size_t src_slot, size_t dst_slot,
                        size_t src_base, size_t dst_base, int n_outer, int per, int src_per, int rb, int split, int ra,
                        int rb2, hipStream_t s) {
    const long units = (long)n_outer * per * (rb / 4);
    dim3 grid((unsigned)((units + 255) / 256), (unsigned)num_slots);
    hipLaunchKernelGGL(copy_records_kernel, grid, dim3(256), 0, s, src, dst, src_slot, dst_slot, src_base, dst_base,
                       n_outer, per, src_per, rb, split, ra, rb2);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dequant(const uint8_t* slot, int H, int I, int matrix, float* out, hipStream_t s) {
    const SlotGeom gm = slot_geom(H, I);
    const long lanes = (long)2 * I * H / 32;  // both matrices hold 2*I*H/2 and H*I/2 code bytes
    if (matrix == 0) {
        hipLaunchKernelGGL(dequant_kernel<false>, dim3((unsigned)((lanes + 255) / 256)), dim3(256), 0, s, slot, H, I,
                           gm.gu_codes, gm.gu_scales, gm.gu_glob, out);
    } else {
        hipLaunchKernelGGL(dequant_kernel<true>, dim3((unsigned)((lanes / 2 + 255) / 256)), dim3(256), 0, s, slot, H,
                           I, gm.dn_codes, gm.dn_scales, gm.dn_glob, out);
    }
    return hipGetLastError();
}

hipError_t launch_dequant_rows(const uint8_t* codes, const uint8_t* scales, const float* globals, int rows, int K,
                               float* out, hipStream_t s) {
    const long n = (long)rows * (K / 8);
    hipLaunchKernelGGL(dequant_rows_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, codes, scales,
                       globals, rows, K, out);
    return hipGetLastError();
}

// Slice r of n along I (issue #62 "What it touches"): gate rows [r*Il, (r+1)*Il)
// and up rows [I + r*Il, I + (r+1)*Il) with their scales and globals; down
// columns [r*Il, (r+1)*Il) of all H rows with all H globals.  In the slot's
// operand order these are whole records: gate_up records are 16-row tiles
// (per 128-column step), down records are 32-column chunks of 64-row groups.
hipError_t launch_slice_bank(const uint8_t* src, int num_slots, int H, int I, int r, int n, uint8_t* dst,
                             hipStream_t s) {
    const int Il = I / n;
    const SlotGeom S = slot_geom(H, I), D = slot_geom(H, Il);
    const int KQ = H / 128, NTs = 2 * I / 16, NTd = 2 * Il / 16, NG = H / 64;
    const int gt = r * Il / 16, ut = I / 16 + r * Il / 16;  // first gate / up tile of the slice
    hipError_t e;
    if ((e = copy_records(src, dst, num_slots, S.total, D.total, S.gu_codes, D.gu_codes, KQ, NTd, NTs, 1024,
                          Il / 16, gt, ut, s)) != hipSuccess) return e;
    if ((e = copy_records(src, dst, num_slots, S.total, D.total, S.gu_scales, D.gu_scales, KQ, NTd, NTs, 128,
                          Il / 16, gt, ut, s)) != hipSuccess) return e;
    if ((e = copy_records(src, dst, num_slots, S.total, D.total, S.gu_glob, D.gu_glob, 1, 2 * Il, 2 * I, 4, Il,
                          r * Il, I + r * Il, s)) != hipSuccess) return e;
    const int nrec = (Il / 32) * NG, first = (r * Il / 32) * NG;
    if ((e = copy_records(src, dst, num_slots, S.total, D.total, S.dn_codes, D.dn_codes, 1, nrec, 0, 1024, nrec,
                          first, 0, s)) != hipSuccess) return e;
    if ((e = copy_records(src, dst, num_slots, S.total, D.total, S.dn_scales, D.dn_scales, 1, nrec, 0, 128, nrec,
                          first, 0, s)) != hipSuccess) return e;
    return copy_records(src, dst, num_slots, S.total, D.total, S.dn_glob, D.dn_glob, 1, 1, 0, 4 * H, 1, 0, 0, s);
}

// The same slice of an MXFP4 bank.  In the checkpoints' transposed tensors
// it runs along N of gate_up (blocks_t [H/2, 2I]: two column ranges) and
// along K of down (blocks_t [I/2, H]: a row range), with the scales sliced to
// match (issue #62 "What it touches"); in the slot's operand order both are
// whole records: gate_up 16-row tiles per 128-column step (64 scale bytes
// each), down 32-column chunks of 64-row groups (64 scale bytes each).
hipError_t launch_mx_slice_bank(const uint8_t* src, int num_slots, int H, int I, int r, int n, uint8_t* dst,
                                hipStream_t s) {
    const int Il = I / n;
    const SlotGeom S = mx_slot_geom(H, I), D = mx_slot_geom(H, Il);
    const int KQ = H / 128, NTs = 2 * I / 16, NTd = 2 * Il / 16, NG = H / 64;
    const int gt = r * Il / 16, ut = I / 16 + r * Il / 16;
    hipError_t e;
    if ((e = copy_records(src, dst, num_slots, S.total, D.total, S.gu_codes, D.gu_codes, KQ, NTd, NTs, 1024,
                          Il / 16, gt, ut, s)) != hipSuccess) return e;
    if ((e = copy_records(src, dst, num_slots, S.total, D.total, S.gu_scales, D.gu_scales, KQ, NTd, NTs, 64,
                          Il / 16, gt, ut, s)) != hipSuccess) return e;
    const int nrec = (Il / 32) * NG, first = (r * Il / 32) * NG;
    if ((e = copy_records(src, dst, num_slots, S.total, D.total, S.dn_codes, D.dn_codes, 1, nrec, 0, 1024, nrec,
                          first, 0, s)) != hipSuccess) return e;
    return copy_records(src, dst, num_slots, S.total, D.total, S.dn_scales, D.dn_scales, 1, nrec, 0, 64, nrec, first,
                        0, s);
}

}  // namespace moe
