// Router projection for gfx950: logits[t, e] = x[t, :] . w_r[e, :] over bf16
// activations x [T, H] and bf16 router weights w_r [E, H], fp32 out.  The
// router is replicated and its logits feed the top-k of route.hip (issue #62,
// R9700 interim report: norm_topk_prob over a replicated router).
//
// With more than 16 tokens the product is a dense contraction, so it runs on
// v_mfma_f32_16x16x32_bf16 (bf16 x bf16 products are exact in fp32; fp32
// accumulation).  A workgroup owns a tile of 32 tokens x 64 experts; its 8
// waves split H into 8 equal ranges.  A wave streams its range in groups of
// 64 columns: each 16-byte buffer load covers 8 rows x 128 bytes (whole
// cache lines), the group goes to the wave's own LDS area, and the MFMA
// operands (lane (row i, group g): columns [8g, 8g+8) of a 32-column chunk)
// are read from there while the next group's loads are in flight.  Loading
// the operands straight from memory in MFMA order (16 rows x 64 bytes per
// load) streams about 3x slower from L2.  The 8 partial tiles meet in LDS
// and are added in wave order, so the result does not depend on timing.
// Rows past T or E read zeros and are not written.  The tiles are dealt to
// the XCDs in contiguous ranges, so that the four expert tiles of a token
// tile share one L2.
// Decode batches (T <= 16) take the vector path below instead: the weights
// are the traffic (E*H*2 bytes), so one workgroup per expert row spreads them
// over E CUs (a 16-expert matrix tile would leave all but E/16 CUs idle).
#include "internal.hpp"
#include "nvfp4_device.hpp"

namespace moe {
namespace {

constexpr int kRW = 8;  // waves per workgroup, one contraction range each

template <int MI, int NJ>
__global__ void __launch_bounds__(kRW * kWave) router_logits_kernel(const uint16_t* __restrict__ x,
                                                                    const uint16_t* __restrict__ wr, int T, int H,
                                                                    int E, float* __restrict__ logits, int nbe) {
    constexpr int XR = 16 * MI, WR = 16 * NJ;  // token rows and expert rows of the tile
    constexpr int PITCH = 144;                 // LDS bytes per staged row: 128 + 16, conflict-free fragment reads
    constexpr int NXI = XR / 8, NWI = WR / 8;  // loads per 64-column group (8 rows x 128 bytes each)
    constexpr int STAGE = (XR + WR) * PITCH;   // one wave's staging area
    static_assert(kRW * MI * NJ * kWave * 16 <= kRW * STAGE, "the partial tiles reuse the staging areas");
    __shared__ __attribute__((aligned(16))) uint8_t lds[kRW * STAGE];
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int l16 = lane & 15, g = lane >> 4;
    // XCD-aware order: workgroups are dealt round-robin to the 8 XCDs (block b to XCD b % 8), so the blocks of
    // XCD x take one contiguous range of (token tile, expert tile) pairs: the expert tiles of a token tile then
    // run on one XCD and its activation rows come from HBM once, into that XCD's L2, instead of once per tile
    const int nblk = (int)gridDim.x, per = nblk / 8, extra = nblk % 8, xcd = (int)blockIdx.x % 8;
    const int lb = xcd * per + min(xcd, extra) + (int)blockIdx.x / 8;
    const int tb = lb / nbe, eb = lb % nbe;
    const int t0 = XR * tb, e0 = WR * eb;
    const int kw = H / kRW;          // columns of this wave's range (a multiple of 32)
    const int kbeg = wave * kw;
    const rsrc_t xres = make_rsrc(x, (uint32_t)((size_t)T * H * 2));
    const rsrc_t wres = make_rsrc(wr, (uint32_t)((size_t)E * H * 2));
    // loads: lane (r = lane / 8, c = lane % 8) takes row 8 q + r, bytes [16 c, 16 c + 16) of the group's 128 bytes;
    // a wave load is then 8 whole 128-byte lines (16 rows x 64 bytes per load, the MFMA operand order, streams
    // about 3x slower from L2)
    const int lr = lane >> 3, lc = lane & 7;
    int xoff[NXI], woff[NWI];
#pragma unroll
    for (int q = 0; q < NXI; ++q) {
        const int t = t0 + 8 * q + lr;
        xoff[q] = t < T ? 2 * (t * H + kbeg + 8 * lc) : kOob;
    }
#pragma unroll
    for (int q = 0; q < NWI; ++q) {
        const int e = e0 + 8 * q + lr;
        woff[q] = e < E ? 2 * (e * H + kbeg + 8 * lc) : kOob;
    }
    uint8_t* st = lds + wave * STAGE;  // this wave's rows: tokens 0 .. XR-1, then experts
    u32x4_t rx[NXI], rw[NWI];
    auto load = [&](int n) {  // group n: columns [64 n, 64 n + 64) of the wave's range; past the range: zeros
        const bool in = 64 * n + 8 * lc < kw;
#pragma unroll
        for (int q = 0; q < NXI; ++q) rx[q] = buf_load16(xres, in && xoff[q] != kOob ? xoff[q] + 128 * n : kOob);
#pragma unroll
        for (int q = 0; q < NWI; ++q) rw[q] = buf_load16(wres, in && woff[q] != kOob ? woff[q] + 128 * n : kOob);
    };
    f32x4_t acc[MI][NJ];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    const int ngroups = (kw + 63) / 64;
    load(0);
    for (int n = 0; n < ngroups; ++n) {
        // the wave's own staging area: its LDS operations run in order, so no barrier is needed
#pragma unroll
        for (int q = 0; q < NXI; ++q) *reinterpret_cast<u32x4_t*>(st + (8 * q + lr) * PITCH + 16 * lc) = rx[q];
#pragma unroll
        for (int q = 0; q < NWI; ++q) *reinterpret_cast<u32x4_t*>(st + (XR + 8 * q + lr) * PITCH + 16 * lc) = rw[q];
        if (n + 1 < ngroups) load(n + 1);  // in flight while this group is multiplied
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            if (64 * n + 32 * m >= kw) break;  // uniform: the half group past the range
            bf16x8_t fa[MI], fb[NJ];
#pragma unroll
            for (int i = 0; i < MI; ++i)
                fa[i] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(st + (16 * i + l16) * PITCH + 64 * m + 16 * g));
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                fb[j] = __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(st + (XR + 16 * j + l16) * PITCH + 64 * m + 16 * g));
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int j = 0; j < NJ; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
    }
    __syncthreads();  // every wave is done with its staging area: it now holds the partial tiles
    f32x4_t(*part)[MI * NJ][kWave] = reinterpret_cast<f32x4_t(*)[MI * NJ][kWave]>(lds);
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

// Decode batches: one 256-thread workgroup per expert e.  Thread j takes the
// 16-byte chunks j, j + 256, ... of row e of W_r and of each token row of x
// (those rows are few and stay in L2 for every workgroup).  bf16 pairs are
// multiplied exactly and accumulated in fp32 (v_dot2_f32_bf16) in a fixed
// order: per thread over its chunks in order, then over the wave's lanes
// (wave_sum), then the four waves in order, so repeated calls give identical bits.
// C: chunks per thread (H <= 2048 C); TG: tokens per pass.
template <int C, int TG>
__global__ void __launch_bounds__(256) router_gemv_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ wr, int T, int H, int E,
                                                          float* __restrict__ logits) {
    __shared__ float red[4][TG];
    const int e = (int)blockIdx.x, tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int nch = H / 8;  // 16-byte chunks per row
    const rsrc_t xres = make_rsrc(x, (uint32_t)((size_t)T * H * 2));
    const rsrc_t wres = make_rsrc(wr, (uint32_t)((size_t)E * H * 2));
    u32x4_t wv[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int ch = tid + 256 * c;
        wv[c] = buf_load16(wres, ch < nch ? 2 * (e * H + 8 * ch) : kOob);
    }
    // workgroup e visits the tokens of a pass starting at e mod TG, so the workgroups' first loads spread over
    // TG different rows of x instead of all asking L2 for the same lines at once
    const int rot = e % TG;
    for (int t0 = 0; t0 < T; t0 += TG) {
        u32x4_t xv[TG][C];
#pragma unroll
        for (int q = 0; q < TG; ++q)
#pragma unroll
            for (int c = 0; c < C; ++c) {
                const int t = t0 + (q + rot) % TG, ch = tid + 256 * c;
                xv[q][c] = buf_load16(xres, t < T && ch < nch ? 2 * (t * H + 8 * ch) : kOob);
            }
#pragma unroll
        for (int q = 0; q < TG; ++q) {
            float acc = 0.0f;
#pragma unroll
            for (int c = 0; c < C; ++c)
#pragma unroll
                for (int d = 0; d < 4; ++d) acc = dot2_bf16(as_bf16x2(word_of(xv[q][c], d)), as_bf16x2(word_of(wv[c], d)), acc);
            acc = wave_sum(acc);
            if (lane == 0) red[wave][(q + rot) % TG] = acc;
        }
        __syncthreads();
        if (tid < TG && t0 + tid < T)
            logits[(size_t)(t0 + tid) * E + e] = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
        __syncthreads();
    }
}

template <int C>
hipError_t launch_router_gemv(const uint16_t* x, const uint16_t* wr, int T, int H, int E, float* logits,
                              hipStream_t s) {
    // as many tokens per pass as the registers allow (TG * C 16-byte chunks per thread, at most 64), so a
    // batch of up to 16 tokens is one round trip to L2 for x
    constexpr int kMaxTG = 64 / C < 16 ? 64 / C : 16;
    if (T == 1)
        hipLaunchKernelGGL((router_gemv_kernel<C, 1>), dim3(E), dim3(256), 0, s, x, wr, T, H, E, logits);
    else if (T == 2)
        hipLaunchKernelGGL((router_gemv_kernel<C, 2>), dim3(E), dim3(256), 0, s, x, wr, T, H, E, logits);
    else if (T <= 4)
        hipLaunchKernelGGL((router_gemv_kernel<C, 4>), dim3(E), dim3(256), 0, s, x, wr, T, H, E, logits);
    else if (T <= 8 || kMaxTG < 16)
        hipLaunchKernelGGL((router_gemv_kernel<C, 8>), dim3(E), dim3(256), 0, s, x, wr, T, H, E, logits);
    else
        hipLaunchKernelGGL((router_gemv_kernel<C, kMaxTG>), dim3(E), dim3(256), 0, s, x, wr, T, H, E, logits);
    return hipGetLastError();
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
    if (T <= 16) {
        const int c = ceil_div(H / 8, 256);  // chunks per thread; H <= 16384 gives c <= 8
        if (c <= 1) return launch_router_gemv<1>(x, wr, T, H, E, logits, s);
        if (c <= 2) return launch_router_gemv<2>(x, wr, T, H, E, logits, s);
        if (c <= 4) return launch_router_gemv<4>(x, wr, T, H, E, logits, s);
        return launch_router_gemv<8>(x, wr, T, H, E, logits, s);
    }
    return launch_router_cfg<2, 4>(x, wr, T, H, E, logits, s);
}

}  // namespace moe
