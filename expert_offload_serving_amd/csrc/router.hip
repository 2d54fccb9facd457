// Router projection for gfx950: logits[t, e] = x[t, :] . w_r[e, :] over bf16
// activations x [T, H] and bf16 router weights w_r [E, H], fp32 out.  The
// router is replicated and its logits feed the top-k of route.hip (issue #62,
// R9700 interim report: norm_topk_prob over a replicated router).
//
// The product is a dense contraction, so it runs on v_mfma_f32_16x16x32_bf16
// (bf16 x bf16 products are exact in fp32; fp32 accumulation).  A workgroup
// owns a tile of 16*MI tokens x 16*NJ experts; its 8 waves split H into 8
// equal ranges and each wave streams its range with 16-byte buffer loads
// straight into MFMA operands (lane (row i, group g) takes columns
// [8g, 8g+8) of each 32-column chunk, the same for both operands).  The 8
// partial tiles meet in LDS and are added in wave order, so the result does
// not depend on timing.  Rows past T or E read zeros and are not written.
//   decode (T <= 16): MI = NJ = 1, one workgroup per 16 experts: the weights
//                     are the traffic (E*H*2 bytes), streamed by E/16 CUs.
//   larger T:         MI = 2, NJ = 4 (32 tokens x 64 experts per workgroup),
//                     loads in two groups of five 32-column chunks.
#include "internal.hpp"
#include "nvfp4_device.hpp"

namespace moe {
namespace {

constexpr int kRW = 8;  // waves per workgroup, one contraction range each

template <int MI, int NJ>
__global__ void __launch_bounds__(kRW * kWave) router_logits_kernel(const uint16_t* __restrict__ x,
                                                                    const uint16_t* __restrict__ wr, int T, int H,
                                                                    int E, float* __restrict__ logits, int nbe) {
    __shared__ f32x4_t part[kRW][MI * NJ][kWave];
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int l16 = lane & 15, g = lane >> 4;
    const int tb = (int)blockIdx.x / nbe, eb = (int)blockIdx.x % nbe;
    const int t0 = 16 * MI * tb, e0 = 16 * NJ * eb;
    const int kw = H / kRW;          // columns of this wave's range (a multiple of 32)
    const int kbeg = wave * kw;
    const rsrc_t xres = make_rsrc(x, (uint32_t)((size_t)T * H * 2));
    const rsrc_t wres = make_rsrc(wr, (uint32_t)((size_t)E * H * 2));
    int xoff[MI], woff[NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i) {
        const int t = t0 + 16 * i + l16;
        xoff[i] = t < T ? 2 * (t * H + kbeg + 8 * g) : kOob;
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int e = e0 + 16 * j + l16;
        woff[j] = e < E ? 2 * (e * H + kbeg + 8 * g) : kOob;
    }
    f32x4_t acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    // G chunks of 32 columns per group: every load of a group is issued before its first MFMA (decode: the
    // whole range at once).  Chunks past the range, and lanes past T or E, load zeros (an offset past the
    // resource), which add nothing.
    constexpr int G = (MI + NJ <= 2) ? 10 : 5;
    for (int c0 = 0; c0 < kw; c0 += 32 * G) {
        u32x4_t a[G][MI], b[G][NJ];
#pragma unroll
        for (int q = 0; q < G; ++q) {
            const int c = c0 + 32 * q;
            const bool in = c < kw;
#pragma unroll
            for (int i = 0; i < MI; ++i) a[q][i] = buf_load16(xres, in && xoff[i] != kOob ? xoff[i] + 2 * c : kOob);
#pragma unroll
            for (int j = 0; j < NJ; ++j) b[q][j] = buf_load16(wres, in && woff[j] != kOob ? woff[j] + 2 * c : kOob);
        }
#pragma unroll
        for (int q = 0; q < G; ++q)
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[q][i]),
                                                                         __builtin_bit_cast(bf16x8_t, b[q][j]),
                                                                         acc[i][j], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) part[wave][NJ * i + j][lane] = acc[i][j];
    __syncthreads();
    // lane (l16, g) of tile (i, j) holds tokens t0 + 16 i + 4 g + [0, 4) of expert e0 + 16 j + l16
    for (int q = tid; q < MI * NJ * kWave; q += kRW * kWave) {
        const int ij = q / kWave, ln = q % kWave;
        f32x4_t s = part[0][ij][ln];
#pragma unroll
        for (int w = 1; w < kRW; ++w) s += part[w][ij][ln];
        const int i = ij / NJ, j = ij % NJ;
        const int e = e0 + 16 * j + (ln & 15);
        const int tt = t0 + 16 * i + 4 * (ln >> 4);
        if (e < E) {
#pragma unroll
            for (int r = 0; r < 4; ++r)
                if (tt + r < T) logits[(size_t)(tt + r) * E + e] = s[r];
        }
    }
}

template <int MI, int NJ>
hipError_t launch_router_cfg(const uint16_t* x, const uint16_t* wr, int T, int H, int E, float* logits,
                             hipStream_t s) {
    const int nbt = ceil_div(T, 16 * MI), nbe = ceil_div(E, 16 * NJ);
    hipLaunchKernelGGL((router_logits_kernel<MI, NJ>), dim3(nbt * nbe), dim3(kRW * kWave), 0, s, x, wr, T, H, E,
                       logits, nbe);
    return hipGetLastError();
}

}  // namespace

bool router_shape_supported(int T, int H, int E) {
    // every byte offset stays below the out-of-range offset kOob
    return H > 0 && H % (32 * kRW) == 0 && H <= 16384 && (size_t)T * H * 2 <= (size_t)kOob &&
           (size_t)E * H * 2 <= (size_t)kOob;
}

hipError_t launch_router(const uint16_t* x, const uint16_t* wr, int T, int H, int E, float* logits, hipStream_t s) {
    if (T <= 16) return launch_router_cfg<1, 1>(x, wr, T, H, E, logits, s);
    return launch_router_cfg<2, 4>(x, wr, T, H, E, logits, s);
}

}  // namespace moe
