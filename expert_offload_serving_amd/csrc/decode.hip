// Decode path (T <= 16) of the NVFP4 routed-MoE layer for gfx950.
//
// The expert FFN is cut along the intermediate axis, exactly as the pages cut
// it across GPUs (issue #62 "The fix that fits": a slice of I turns gate_up
// into a row range and down into a column range whose outputs are partial
// sums).  One work item is (expert, 32-row slice of I):
//   phase A  gate rows and up rows of the slice against the expert's tokens
//            (K = H), reduced across the workgroup's waves, SwiGLU;
//   phase B  the down columns of the slice against the 32 hidden values,
//            giving a partial sum over all H outputs, times the routing weight.
// Both phases stream their weights with one 16-byte load per lane per record,
// and the down records are in flight while phase A computes, so one kernel
// moves all of an item's bytes.  A second kernel adds the partial outputs of
// every (expert, slice) of a token in a fixed order and the shared expert's
// sigmoid-gated term (PR #385 "What this adds": routed + sigmoid(gate) *
// shared before one reduction).
//
// Arithmetic: v_mfma_f32_16x16x32_f16 with the weights as the 16-row operand
// and up to 16 tokens as the 16 columns.  Weights decode exactly to fp16
// (frag_f16).  Activations enter as fp16 times a power of two per (wave,
// token) that puts the wave's largest magnitude in [2^14, 2^15), so the
// bf16 -> fp16 conversion is exact in the fp16 normal range; the scale is
// undone exactly on the fp32 result.  The hidden slice is rescaled the same
// way before phase B.  Accumulation is fp32 and every sum runs in a fixed
// order, so results are bit-reproducible.
#include "internal.hpp"
#include "nvfp4_device.hpp"

namespace moe {
namespace {

constexpr int kDW = 8;              // waves per work item
constexpr int kDT = kDW * kWave;    // threads per work item
constexpr int kSl = 32;             // intermediate rows per work item
constexpr int kMaxChunks = 16;      // E <= 1024 experts, 64 per ballot

struct DecArgs {
    const uint8_t* bank;
    size_t slot_bytes;
    const int32_t* slot_of_expert;
    const uint8_t* shared;
    const uint16_t* wg;
    const uint16_t* x;
    int T, H, I, E, k;
    const float* w;
    const int32_t* offsets;
    const int32_t* sorted_assign;
    float* part;   // [(T*k + T) * nsl, H]: row (assignment or T*k + token) * nsl + slice
    float* y;
    int accumulate;
    size_t gu_codes, gu_scales, gu_glob, dn_codes, dn_scales, dn_glob;
};

struct ItemExpert {
    int e;       // expert, E for the shared expert, -1 for no work
    int begin;   // first position in sorted_assign (routed experts)
    int count;   // assignments of the expert
};

// Item u -> the u-th expert (ascending) that has assignments; u equal to the
// number of such experts is the shared expert.  All lanes agree.
__device__ ItemExpert item_expert(const DecArgs& a, int u, int lane) {
    int lo[kMaxChunks], hi[kMaxChunks];
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
        const int e = 64 * c + lane;
        lo[c] = e < a.E ? a.offsets[e] : 0;
        hi[c] = e < a.E ? a.offsets[e + 1] : 0;
    }
    ItemExpert r{-1, 0, 0};
    int base = 0;
    const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
#pragma unroll
    for (int c = 0; c < kMaxChunks; ++c) {
        const bool act = hi[c] > lo[c];
        const uint64_t m = __ballot(act);
        const int n = __popcll(m);
        if (r.e < 0 && u < base + n) {
            const uint64_t hit = __ballot(act && __popcll(m & below) == u - base);
            const int li = __ffsll((unsigned long long)hit) - 1;
            r.e = 64 * c + li;
            r.begin = __builtin_amdgcn_readlane(lo[c], li);
            r.count = __builtin_amdgcn_readlane(hi[c], li) - r.begin;
        }
        base += n;
    }
    if (r.e < 0 && u == base) r.e = a.E;
    return r;
}

// One work item per workgroup.  KQW: most 128-column steps of K = H per wave
// (steps wave, wave + 8, ...); NRGW: most 64-row down groups per wave.
template <int KQW, int NRGW>
__global__ void __launch_bounds__(kDT) fused_kernel(DecArgs a, int nsl) {
    __shared__ __attribute__((aligned(16))) f32x4_t red[kDW][4][kWave];
    __shared__ float hmax[kDW][16];
    __shared__ __attribute__((aligned(16))) _Float16 hs[16][kSl];

    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int u = blockIdx.x / nsl, s = blockIdx.x % nsl;
    const int H = a.H, I = a.I, T = a.T, k = a.k;
    const ItemExpert it = item_expert(a, u, lane);
    if (it.e < 0 || (it.e == a.E && a.shared == nullptr)) return;  // uniform

    // Column c of the MFMA is the item's c-th token.
    const int c = lane & 15, g = lane >> 4;
    int ne, tok = -1, prow = 0;
    float wc = 0.0f;
    const uint8_t* slot;
    if (it.e < a.E) {
        ne = it.count;
        if (c < ne) {
            const int as = a.sorted_assign[it.begin + c];
            tok = as / k;
            prow = as;
            wc = a.w[as];
        }
        const int sl = __builtin_amdgcn_readfirstlane(a.slot_of_expert[it.e]);
        slot = sl >= 0 ? a.bank + (size_t)sl * a.slot_bytes : nullptr;
    } else {
        ne = T;
        if (c < ne) tok = c, prow = T * k + c, wc = 1.0f;
        slot = a.shared;
    }
    float* prow_ptr = a.part + ((size_t)prow * nsl + s) * H;

    if (slot == nullptr) {  // expert left out of this call: its partial outputs are zero
        for (int cc = 0; cc < ne; ++cc) {
            const int pr = a.sorted_assign[it.begin + cc];
            f32x4_t* dst = reinterpret_cast<f32x4_t*>(a.part + ((size_t)pr * nsl + s) * H);
            for (int v = tid; v < H / 4; v += kDT) dst[v] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        }
        return;
    }

    const int KQ = H / 128, NT = 2 * I / 16, NG = H / 64;
    const rsrc_t xres = make_rsrc(a.x, (uint32_t)T * H * 2);
    const rsrc_t sres = make_rsrc(slot, (uint32_t)a.slot_bytes);
    const int gcodes = (int)a.gu_codes, gscales = (int)a.gu_scales, gglob = (int)a.gu_glob;
    const int dcodes = (int)a.dn_codes, dscales = (int)a.dn_scales, dglob = (int)a.dn_glob;
    const int tiles[4] = {2 * s, 2 * s + 1, I / 16 + 2 * s, I / 16 + 2 * s + 1};  // gate, gate, up, up
    const int soff = lane_scale_off(lane);

    // ---- issue every load of the item in one straight line: activations
    // first, then gate_up records, then down records (absent ones read as 0)
    u32x4_t xr[KQW][4];
#pragma unroll
    for (int i = 0; i < KQW; ++i) {
        const int kq = wave + kDW * i;
#pragma unroll
        for (int m = 0; m < 4; ++m)
            xr[i][m] = buf_load16(xres, (kq < KQ && tok >= 0) ? 2 * (tok * H + 128 * kq + 32 * m + 8 * g) : kOob);
    }
    u32x4_t ar[KQW][4];
    uint32_t asc[KQW][4];
#pragma unroll
    for (int i = 0; i < KQW; ++i) {
        const int kq = wave + kDW * i;
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const int rec = kq * NT + tiles[tt];
            ar[i][tt] = buf_load16(sres, kq < KQ ? gcodes + rec * kRecBytes + 16 * lane : kOob);
            asc[i][tt] = buf_load4(sres, kq < KQ ? gscales + rec * kRecScaleBytes + soff : kOob);
        }
    }
    u32x4_t br[NRGW];
    uint32_t bsc[NRGW];
#pragma unroll
    for (int i = 0; i < NRGW; ++i) {
        const int rg = wave + kDW * i;
        const int rec = s * NG + rg;
        br[i] = buf_load16(sres, rg < NG ? dcodes + rec * kRecBytes + 16 * lane : kOob);
        bsc[i] = buf_load4(sres, rg < NG ? dscales + rec * kRecScaleBytes + soff : kOob);
    }
    // SwiGLU thread (hi, ht): hidden row hi of the slice, token column ht
    const int hi = tid >> 4, ht = tid & 15;
    const float g_glob = __uint_as_float(buf_load4(sres, gglob + 4 * (kSl * s + hi)));
    const float u_glob = __uint_as_float(buf_load4(sres, gglob + 4 * (I + kSl * s + hi)));
    // keep the scheduler from sinking loads towards their uses: all of them
    // must be in flight before the first wait
    __builtin_amdgcn_sched_barrier(0);

    // ---- activations: per-(wave, token) power-of-two scale, exact fp16
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < KQW; ++i)
#pragma unroll
        for (int m = 0; m < 4; ++m)
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint32_t wv = word_of(xr[i][m], d);
                amax = fmaxf(amax, fmaxf(fabsf(__uint_as_float(wv << 16)), fabsf(__uint_as_float(wv & 0xFFFF0000u))));
            }
    amax = fmaxf(amax, __shfl_xor(amax, 16, kWave));
    amax = fmaxf(amax, __shfl_xor(amax, 32, kWave));
    const int xsh = fp16_shift(amax);
    const float xsc = ldexpf(1.0f, xsh), xinv = ldexpf(1.0f, -xsh);

    // ---- phase A: gate and up rows of the slice, this wave's share of K
    f32x4_t acc[4];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) acc[tt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < KQW; ++i) {
        if (wave + kDW * i >= KQ) break;  // uniform per wave
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            uint32_t xh[4];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint32_t wv = word_of(xr[i][m], d);
                const f16x2_t p = {(_Float16)(__uint_as_float(wv << 16) * xsc),
                                   (_Float16)(__uint_as_float(wv & 0xFFFF0000u) * xsc)};
                xh[d] = __builtin_bit_cast(uint32_t, p);
            }
            const f16x8_t X = __builtin_bit_cast(f16x8_t, u32x4_t{xh[0], xh[1], xh[2], xh[3]});
#pragma unroll
            for (int tt = 0; tt < 4; ++tt) {
                f16x2_t S;
                if (m == 0) S = scale_f16x2<0>(asc[i][tt]);
                else if (m == 1) S = scale_f16x2<1>(asc[i][tt]);
                else if (m == 2) S = scale_f16x2<2>(asc[i][tt]);
                else S = scale_f16x2<3>(asc[i][tt]);
                const f16x8_t A = frag_f16(word_of(ar[i][tt], m), S);
                acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, X, acc[tt], 0, 0, 0);
            }
        }
    }
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) red[wave][tt][lane] = acc[tt] * xinv;

    // down globals of this wave's output rows (lane rows 16j + 4g + [0, 4) of each group)
    f32x4_t dg[NRGW][4];
#pragma unroll
    for (int i = 0; i < NRGW; ++i) {
        const int rg = wave + kDW * i;
#pragma unroll
        for (int j = 0; j < 4; ++j)
            dg[i][j] = __builtin_bit_cast(f32x4_t, buf_load16(sres, rg < NG ? dglob + 4 * (64 * rg + 16 * j + 4 * g)
                                                                          : kOob));
    }
    __syncthreads();

    // ---- SwiGLU: thread (hi, ht) sums its gate and up values over the waves in order
    float hv;
    {
        const int tt = hi >> 4, r = hi & 15, L = 16 * (r >> 2) + ht, ii = r & 3;
        float gs = 0.0f, us = 0.0f;
#pragma unroll
        for (int w = 0; w < kDW; ++w) {
            gs += red[w][tt][L][ii];
            us += red[w][2 + tt][L][ii];
        }
        const float gv = gs * g_glob, uv = us * u_glob;
        hv = gv / (1.0f + expf(-gv)) * uv;
        float hm = fabsf(hv);
        hm = fmaxf(hm, __shfl_xor(hm, 16, kWave));
        hm = fmaxf(hm, __shfl_xor(hm, 32, kWave));
        if (lane < 16) hmax[wave][lane] = hm;
    }
    __syncthreads();
    float hm_t = 0.0f, hm_c = 0.0f;
#pragma unroll
    for (int w = 0; w < kDW; ++w) hm_t = fmaxf(hm_t, hmax[w][ht]), hm_c = fmaxf(hm_c, hmax[w][c]);
    hs[ht][hi] = (_Float16)(hv * ldexpf(1.0f, fp16_shift(hm_t)));
    __syncthreads();

    // ---- phase B: the slice's 32 down columns for this wave's row groups
    const f16x8_t B = __builtin_bit_cast(f16x8_t, *reinterpret_cast<const u32x4_t*>(&hs[c][8 * g]));
    const float oscale = ldexpf(1.0f, -fp16_shift(hm_c)) * wc;
#pragma unroll
    for (int i = 0; i < NRGW; ++i) {
        const int rg = wave + kDW * i;
        if (rg >= NG) break;  // uniform per wave
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f16x2_t S;
            if (j == 0) S = scale_f16x2<0>(bsc[i]);
            else if (j == 1) S = scale_f16x2<1>(bsc[i]);
            else if (j == 2) S = scale_f16x2<2>(bsc[i]);
            else S = scale_f16x2<3>(bsc[i]);
            const f16x8_t A = frag_f16(word_of(br[i], j), S);
            const f32x4_t D =
                __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B, f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
            if (c < ne) {
                const f32x4_t o = (D * oscale) * dg[i][j];
                *reinterpret_cast<f32x4_t*>(prow_ptr + 64 * rg + 16 * j + 4 * g) = o;
            }
        }
    }
}

// y_t = sum over (j, slice) of the routed partials of token t, plus
// sigmoid(x_t . w_g) times the shared expert's partials, in a fixed order.
// Workgroup: one token and 64 output columns; thread (q, cl) sums partial
// rows q, q + 16, ... of columns [4 cl, 4 cl + 4).  Each pass issues all of
// its loads before the first add (partial rows past the end read as zero).
constexpr int kCR = 16;  // partial rows per thread per pass
__global__ void __launch_bounds__(256) dcombine_kernel(DecArgs a, int nsl, int nch) {
    __shared__ f32x4_t rr[16][16], rsh[16][16];
    __shared__ float dots[4];
    const int t = blockIdx.x / nch, ch = blockIdx.x % nch;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave, cl = tid & 15, q = tid >> 4;
    const int H = a.H, k = a.k, T = a.T;
    const int col = 64 * ch + 4 * cl;
    const int nr = k * nsl;
    const rsrc_t pres = make_rsrc(a.part, (uint32_t)((size_t)(T * k + T) * nsl * H * 4));
    const int rbase = t * k * nsl, sbase = (T * k + t) * nsl;
    const bool has_shared = a.shared != nullptr;
    f32x4_t sr = {0.0f, 0.0f, 0.0f, 0.0f}, ss = {0.0f, 0.0f, 0.0f, 0.0f};
    float gd = 0.0f;
    {
        f32x4_t v[kCR], vs[2];
        u32x4_t xv[2], wv[2];
#pragma unroll
        for (int i = 0; i < kCR; ++i) {
            const int r = q + 16 * i;
            v[i] = __builtin_bit_cast(f32x4_t, buf_load16(pres, r < nr ? 4 * ((rbase + r) * H + col) : kOob));
        }
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int r = q + 16 * i;
            vs[i] = __builtin_bit_cast(f32x4_t,
                                       buf_load16(pres, has_shared && r < nsl ? 4 * ((sbase + r) * H + col) : kOob));
        }
        const rsrc_t xres = make_rsrc(a.x + (size_t)t * H, (uint32_t)H * 2);
        const rsrc_t gres = make_rsrc(a.wg, has_shared ? (uint32_t)H * 2 : 0u);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            const int vv = tid + 256 * i;
            xv[i] = buf_load16(xres, has_shared && vv < H / 8 ? 16 * vv : kOob);
            wv[i] = buf_load16(gres, has_shared && vv < H / 8 ? 16 * vv : kOob);
        }
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int i = 0; i < kCR; ++i) sr += v[i];
        ss = vs[0] + vs[1];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            gd = dot2_bf16(as_bf16x2(xv[i].x), as_bf16x2(wv[i].x), gd);
            gd = dot2_bf16(as_bf16x2(xv[i].y), as_bf16x2(wv[i].y), gd);
            gd = dot2_bf16(as_bf16x2(xv[i].z), as_bf16x2(wv[i].z), gd);
            gd = dot2_bf16(as_bf16x2(xv[i].w), as_bf16x2(wv[i].w), gd);
        }
    }
    // rare shapes: more partial rows, or more of the shared expert / H, than one pass covers
    for (int r0 = 16 * kCR; r0 < nr; r0 += 16 * kCR)
        for (int r = r0 + q; r < nr && r < r0 + 16 * kCR; r += 16)
            sr += __builtin_bit_cast(f32x4_t, buf_load16(pres, 4 * ((rbase + r) * H + col)));
    if (has_shared) {
        for (int r = q + 32; r < nsl; r += 16)
            ss += __builtin_bit_cast(f32x4_t, buf_load16(pres, 4 * ((sbase + r) * H + col)));
        const u32x4_t* xp = reinterpret_cast<const u32x4_t*>(a.x + (size_t)t * H);
        const u32x4_t* wp = reinterpret_cast<const u32x4_t*>(a.wg);
        for (int vv = tid + 512; vv < H / 8; vv += 256) {
            const u32x4_t xx = xp[vv], ww = wp[vv];
            gd = dot2_bf16(as_bf16x2(xx.x), as_bf16x2(ww.x), gd);
            gd = dot2_bf16(as_bf16x2(xx.y), as_bf16x2(ww.y), gd);
            gd = dot2_bf16(as_bf16x2(xx.z), as_bf16x2(ww.z), gd);
            gd = dot2_bf16(as_bf16x2(xx.w), as_bf16x2(ww.w), gd);
        }
        gd = wave_sum(gd);
    }
    rr[q][cl] = sr;
    rsh[q][cl] = ss;
    if (lane == 0) dots[wave] = gd;
    __syncthreads();
    if (tid >= 16) return;
    f32x4_t tr = {0.0f, 0.0f, 0.0f, 0.0f}, ts = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < 16; ++i) tr += rr[i][tid], ts += rsh[i][tid];
    f32x4_t out = tr;
    if (has_shared) out += sigmoidf_(((dots[0] + dots[1]) + dots[2]) + dots[3]) * ts;
    f32x4_t* yp = reinterpret_cast<f32x4_t*>(a.y + (size_t)t * H + 64 * ch + 4 * tid);
    if (a.accumulate) out += *yp;
    *yp = out;
}

template <int KQW, int NRGW>
hipError_t launch_fused(const DecArgs& a, int items, int nsl, hipStream_t s) {
    hipLaunchKernelGGL((fused_kernel<KQW, NRGW>), dim3(items * nsl), dim3(kDT), 0, s, a, nsl);
    return hipGetLastError();
}

}  // namespace

// Per-wave register budget: the kernel keeps all of an item's loads in
// flight at once, sized for H up to 3072 (larger H runs the prefill path).
bool decode_shape_supported(int H, int I) { return H % 128 == 0 && I % kSl == 0 && H <= 3072; }

size_t decode_part_bytes(int T, int H, int I, int k) { return (size_t)(T * k + T) * (I / kSl) * H * 4; }

hipError_t launch_decode(const Layer& L, const uint16_t* x, int T, const float* w, const int32_t* ids,
                         const int32_t* offsets, const int32_t* sorted_assign, const int32_t* assign_pos, float* y,
                         int accumulate, void* ws, hipStream_t s) {
    (void)ids;
    (void)assign_pos;
    const int H = L.H, I = L.I, E = L.E, k = L.k;
    const WsLayout wl = ws_layout(T, H, I, E, k);
    DecArgs a;
    a.bank = L.bank; a.slot_bytes = L.slot_bytes; a.slot_of_expert = L.slot_of_expert;
    a.shared = L.shared; a.wg = L.wg; a.x = x;
    a.T = T; a.H = H; a.I = I; a.E = E; a.k = k;
    a.w = w; a.offsets = offsets; a.sorted_assign = sorted_assign;
    a.part = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + wl.part);
    a.y = y; a.accumulate = accumulate;
    const SlotGeom gm = slot_geom(H, I);
    a.gu_codes = gm.gu_codes; a.gu_scales = gm.gu_scales; a.gu_glob = gm.gu_glob;
    a.dn_codes = gm.dn_codes; a.dn_scales = gm.dn_scales; a.dn_glob = gm.dn_glob;

    const int nsl = I / kSl;
    const int items = (T * k < E ? T * k : E) + 1;
    hipError_t e;
    if (H <= 2560) e = launch_fused<3, 5>(a, items, nsl, s);
    else e = launch_fused<3, 6>(a, items, nsl, s);
    if (e != hipSuccess) return e;
    const int nch = H / 64;
    hipLaunchKernelGGL(dcombine_kernel, dim3(T * nch), dim3(256), 0, s, a, nsl, nch);
    return hipGetLastError();
}

}  // namespace moe
