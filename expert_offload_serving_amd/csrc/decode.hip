// Decode path (T <= 16) of the NVFP4 routed-MoE layer for gfx950.
//
// The layer (PR #385 "What this adds"; issue #62 "What it touches"):
//   h = silu(W_gate x) * (W_up x)   with gate rows [0, I) and up rows [I, 2I) of gate_up [2I, H]
//   o = W_dn h                      with down [H, I]
//   y_t = sum_j w_tj o_{e_tj}(x_t) + sigmoid(x_t . w_g) o_shared(x_t)
// At decode batch sizes this is a set of GEMVs over the distinct routed
// experts, bound by the HBM bytes of their NVFP4 weights.  Three kernels:
//
// gate_up: one workgroup per (active expert, block of gate rows).  Each wave
//   owns RW gate rows and the RW matching up rows; LPR lanes share a row and
//   each owns CPL 16-byte code chunks (32 elements, two scale blocks), so
//   every load instruction reads whole row segments with 128-bit loads and a
//   lane's activation chunks serve the gate pass and the up pass.  Codes are
//   decoded to bf16 (exact) and dotted with the bf16 activations by v_dot2c
//   (exact products, f32 sums); each 16-block's sum is scaled by its E4M3
//   scale, the lanes of a row are reduced with cross-lane shuffles, the row
//   globals are applied, and silu(gate) * up is written as the fp32 hidden
//   state of that (token, expert) assignment.  The shared expert's first
//   block also computes the shared gate sigmoid(x_t . w_g).
//
// down: one workgroup per (active expert, block of output rows).  CPR = I/32
//   lanes share a row (one 16-byte chunk each) and keep their 32-element
//   slice of the fp32 hidden state in registers across the rows they
//   process; the row sum is a segmented shuffle reduction.  Outputs go to a
//   per-assignment buffer.
//
// combine: y_t = sum_j w_tj o_tj + s_t o_shared, summed in a fixed order, so
//   results are bit-reproducible.  Each kernel's inputs were completed by the
//   previous launch, so no workgroup ever waits on another.
#include "internal.hpp"
#include "nvfp4_device.hpp"

namespace moe {
namespace {

struct DecodeArgs {
    const uint8_t* bank;
    size_t slot_bytes;
    const int32_t* slot_of_expert;
    const uint8_t* shared;
    const uint16_t* wg;
    const uint16_t* x;
    int T, H, I, E, k;
    const float* w;
    const int32_t* ids;
    const int32_t* offsets;
    const int32_t* sorted_assign;
    const int32_t* assign_pos;
    float* hbuf;    // f32 [(T*k + T), I]: row p = sorted assignment p; row T*k + t = shared expert, token t
    float* obuf;    // f32 [(T*k + T), H]: expert outputs, same row order
    float* sbuf;    // f32 [T]: shared gate sigmoid(x_t . w_g)
    float* y;
    int accumulate;
    size_t gu_codes, gu_scales, gu_glob, dn_codes, dn_scales, dn_glob;
};

__device__ __forceinline__ uint64_t lanes_below(int lane) { return lane == 0 ? 0ull : (~0ull >> (64 - lane)); }

// The workgroup's expert: the ai-th active routed expert in ascending order
// (count > 0 and a slot), then the shared expert (returned as E).  One pass of
// parallel loads of the offsets and the slot map; the winner publishes
// (expert, slot, first sorted row, token count) through LDS.
struct ExpertInfo {
    int e, slot, p0, ne, n_total;
};

template <int NT>
__device__ ExpertInfo find_expert(const DecodeArgs& a, int ai, int* sh /* LDS, >= NT/64 + 5 ints */) {
    constexpr int NW = NT / kWave;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    if (tid == 0) sh[NW] = -1;
    int base = 0;
    for (int e0 = 0; e0 < a.E; e0 += NT) {
        const int e = e0 + tid;
        int o0 = 0, o1 = 0, sl = -1;
        if (e < a.E) {
            o0 = a.offsets[e];
            o1 = a.offsets[e + 1];
            sl = a.slot_of_expert[e];
        }
        const bool act = e < a.E && o1 > o0 && sl >= 0;
        const uint64_t m = __ballot(act);
        if (lane == 0) sh[wave] = __popcll(m);
        __syncthreads();
        int before = 0, tot = 0;
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            const int c = sh[i];
            before += i < wave ? c : 0;
            tot += c;
        }
        if (act && base + before + __popcll(m & lanes_below(lane)) == ai) {
            sh[NW] = e;
            sh[NW + 1] = sl;
            sh[NW + 2] = o0;
            sh[NW + 3] = o1 - o0;
        }
        base += tot;
        __syncthreads();
    }
    ExpertInfo r;
    const bool has_shared = a.shared != nullptr;
    r.n_total = __builtin_amdgcn_readfirstlane(base) + (has_shared ? 1 : 0);
    r.e = __builtin_amdgcn_readfirstlane(sh[NW]);
    if (r.e >= 0) {
        r.slot = __builtin_amdgcn_readfirstlane(sh[NW + 1]);
        r.p0 = __builtin_amdgcn_readfirstlane(sh[NW + 2]);
        r.ne = __builtin_amdgcn_readfirstlane(sh[NW + 3]);
    } else if (has_shared && ai == r.n_total - 1) {
        r.e = a.E;
        r.slot = -1;
        r.p0 = a.T * a.k;
        r.ne = a.T;
    } else {
        r.slot = -1;
        r.p0 = 0;
        r.ne = 0;
    }
    return r;
}

__device__ __forceinline__ const uint8_t* slot_ptr(const DecodeArgs& a, const ExpertInfo& x) {
    return x.e == a.E ? a.shared : a.bank + (size_t)x.slot * a.slot_bytes;
}

// ------------------------------------------------------------------ gate_up + SwiGLU
// Dynamic LDS: two activation rows of H bf16 (double-buffered over tokens).
template <int CPL, int LPR>
__global__ void __launch_bounds__(256) decode_gateup_kernel(DecodeArgs a, int NB) {
    constexpr int RW = kWave / LPR;  // gate rows (and up rows) per wave
    constexpr int RG = 4 * RW;       // gate rows per workgroup
    __shared__ int sh[16];
    __shared__ int tok[kDecodeMaxT];
    __shared__ float red[4];
    extern __shared__ __attribute__((aligned(16))) uint8_t xlds[];

    const int ai = blockIdx.x / NB, nb = blockIdx.x % NB;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int H = a.H, I = a.I, T = a.T, k = a.k;
    const int nvec = H / 8;  // 16-byte vectors per activation row
    auto stage_x = [&](int t, int buf) {
        const u32x4_t* src = reinterpret_cast<const u32x4_t*>(a.x + (size_t)t * H);
        u32x4_t* dst = reinterpret_cast<u32x4_t*>(xlds + (size_t)buf * H * 2);
        for (int v = tid; v < nvec; v += 256) dst[v] = src[v];
    };
        if (T == 1) stage_x(0, 0);  // the only token: no need to wait for the plan
    const ExpertInfo ex = find_expert<256>(a, ai, sh);
    if (ex.e < 0) return;
    const uint8_t* slot = slot_ptr(a, ex);
    const bool is_shared = ex.e == a.E;
    // A token routes to an expert at most once, so ne <= T <= 16; the clamp
    // only guards the LDS arrays against routing not made by moe_route_topk.
    const int ne = min(ex.ne, kDecodeMaxT), p0 = ex.p0;

    const int lir = lane % LPR, rsub = lane / LPR;
    const int i = nb * RG + wave * RW + rsub;  // gate row; its up row is I + i
    const bool valid = i < I;
    const int ig = valid ? i : 0;
    const uint8_t* gcodes = slot + a.gu_codes + (size_t)ig * (H / 2);
    const uint8_t* ucodes = slot + a.gu_codes + (size_t)(I + ig) * (H / 2);
    const uint8_t* gsc = slot + a.gu_scales + (size_t)ig * (H / 16);
    const uint8_t* usc = slot + a.gu_scales + (size_t)(I + ig) * (H / 16);
    const float* glob = reinterpret_cast<const float*>(slot + a.gu_glob);

    u32x4_t cg[CPL], cu[CPL];
    uint32_t sg[CPL], su[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int c = lir + LPR * j;
        cg[j] = *reinterpret_cast<const u32x4_t*>(gcodes + c * 16);
        cu[j] = *reinterpret_cast<const u32x4_t*>(ucodes + c * 16);
        sg[j] = *reinterpret_cast<const uint16_t*>(gsc + c * 2);
        su[j] = *reinterpret_cast<const uint16_t*>(usc + c * 2);
    }
    const float g_gate = glob[ig], g_up = glob[I + ig];
    if (tid < ne) tok[tid] = (is_shared || T == 1) ? tid : a.sorted_assign[p0 + tid] / k;

    // Shared gate s_t = sigmoid(x_t . w_g): the first block of the shared expert
    // dots each staged activation row with w_g (16-byte vectors, block reduction).
    const bool do_gate = is_shared && nb == 0;
    u32x4_t wgv[4];
    const int nvec_wg = H / 8;  // <= 1024 for H <= 8192
    if (do_gate) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int v = tid + 256 * q;
            wgv[q] = v < nvec_wg ? reinterpret_cast<const u32x4_t*>(a.wg)[v] : u32x4_t{0, 0, 0, 0};
        }
    }
    __syncthreads();
    if (T > 1) stage_x(tok[0], 0);
    for (int ti = 0; ti < ne; ++ti) {
        __syncthreads();
        if (ti + 1 < ne) stage_x(tok[ti + 1], (ti + 1) & 1);
        const uint8_t* xb = xlds + (size_t)(ti & 1) * H * 2;
        if (do_gate) {
            float d = 0.0f;
            #pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int v = tid + 256 * q;
                if (v < nvec_wg) {
                    const u32x4_t xv = reinterpret_cast<const u32x4_t*>(xb)[v];
                    const uint32_t xs[4] = {xv.x, xv.y, xv.z, xv.w};
                    const uint32_t ws[4] = {wgv[q].x, wgv[q].y, wgv[q].z, wgv[q].w};
#pragma unroll
                    for (int m = 0; m < 4; ++m) d = dot2_bf16(as_bf16x2(xs[m]), as_bf16x2(ws[m]), d);
                }
            }
            d = wave_sum(d);
            if (lane == 0) red[wave] = d;
        }
        float accg = 0.0f, accu = 0.0f;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int c = lir + LPR * j;
            const u32x4_t* xp = reinterpret_cast<const u32x4_t*>(xb + c * 64);
            uint32_t xw[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const u32x4_t v = xp[q];
                xw[4 * q + 0] = v.x; xw[4 * q + 1] = v.y; xw[4 * q + 2] = v.z; xw[4 * q + 3] = v.w;
            }
            accg += e4m3_f32<0>(sg[j]) * block16_dot_bf16(cg[j].x, cg[j].y, xw) +
                    e4m3_f32<1>(sg[j]) * block16_dot_bf16(cg[j].z, cg[j].w, xw + 8);
            accu += e4m3_f32<0>(su[j]) * block16_dot_bf16(cu[j].x, cu[j].y, xw) +
                    e4m3_f32<1>(su[j]) * block16_dot_bf16(cu[j].z, cu[j].w, xw + 8);
        }
        accg = group_sum<LPR>(accg);
        accu = group_sum<LPR>(accu);
        if (lir == 0 && valid) {
            const float gate = accg * g_gate, up = accu * g_up;
            a.hbuf[(size_t)(p0 + ti) * I + i] = gate * sigmoidf_(gate) * up;
        }
        if (do_gate) {
            __syncthreads();
            if (tid == 0) a.sbuf[ti] = sigmoidf_(red[0] + red[1] + red[2] + red[3]);
        }
    }
}

// ------------------------------------------------------------------ down + combine
constexpr int kDownPW = 4;  // row passes per wave

// Segmented sum over the LEN consecutive lanes of a segment (c = lane index
// inside the segment, segments start at multiples of LEN); the total ends in
// the lane with c == 0.  Lanes only add values from their own segment.
template <int LEN>
__device__ __forceinline__ float segment_sum(float v, int c) {
    int len = LEN;
#pragma unroll
    for (int it = 0; it < 7; ++it) {
        if (len <= 1) break;
        const int half = (len + 1) / 2;
        const float other = __shfl_down(v, half, kWave);
        if (c + half < len) v += other;
        len = half;
    }
    return v;
}

// One workgroup = one active expert x RBD output rows.  CPR = I/32 lanes per
// row, RPP = 64/CPR rows per pass, kDownPW passes per wave, 4 waves.
template <int CPR>
__global__ void __launch_bounds__(256) decode_down_kernel(DecodeArgs a, int NB) {
    constexpr int RPP = kWave / CPR;
    constexpr int RBD = RPP * kDownPW * 4;
    __shared__ int sh[16];
    const int ai = blockIdx.x / NB, rb = blockIdx.x % NB;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int H = a.H, I = a.I;
    const int r0 = rb * RBD;
    const int g = lane / CPR, c = lane % CPR;
    const bool lane_on = g < RPP;
    const ExpertInfo ex = find_expert<256>(a, ai, sh);

    if (ex.e >= 0) {
        const uint8_t* slot = slot_ptr(a, ex);
        const float* dglob = reinterpret_cast<const float*>(slot + a.dn_glob);
        u32x4_t cw[kDownPW];
        uint32_t sc[kDownPW];
        float grow[kDownPW];
        int rows[kDownPW];
#pragma unroll
        for (int q = 0; q < kDownPW; ++q) {
            const int row = r0 + (q * 4 + wave) * RPP + g;
            rows[q] = (lane_on && row < H) ? row : -1;
            const int rr = rows[q] < 0 ? 0 : rows[q];
            cw[q] = *reinterpret_cast<const u32x4_t*>(slot + a.dn_codes + (size_t)rr * (I / 2) + c * 16);
            sc[q] = *reinterpret_cast<const uint16_t*>(slot + a.dn_scales + (size_t)rr * (I / 16) + c * 2);
            grow[q] = dglob[rr];
        }
        for (int ti = 0; ti < ex.ne; ++ti) {
            const int p = ex.p0 + ti;
            const f32x4_t* hp = reinterpret_cast<const f32x4_t*>(a.hbuf + (size_t)p * I + c * 32);
            f32x4_t h[8];
#pragma unroll
            for (int q = 0; q < 8; ++q) h[q] = hp[q];
#pragma unroll
            for (int q = 0; q < kDownPW; ++q) {
                const uint32_t words[4] = {cw[q].x, cw[q].y, cw[q].z, cw[q].w};
                float lo = 0.0f, hi = 0.0f;
#pragma unroll
                for (int wd = 0; wd < 4; ++wd) {
                    const f32x2_t v0 = e2m1x2_f32<0>(words[wd]), v1 = e2m1x2_f32<1>(words[wd]);
                    const f32x2_t v2 = e2m1x2_f32<2>(words[wd]), v3 = e2m1x2_f32<3>(words[wd]);
                    const f32x4_t ha = h[2 * wd], hb = h[2 * wd + 1];
                    float s = v0.x * ha.x;
                    s += v0.y * ha.y;
                    s += v1.x * ha.z;
                    s += v1.y * ha.w;
                    s += v2.x * hb.x;
                    s += v2.y * hb.y;
                    s += v3.x * hb.z;
                    s += v3.y * hb.w;
                    if (wd < 2) lo += s; else hi += s;
                }
                const float part = e4m3_f32<0>(sc[q]) * lo + e4m3_f32<1>(sc[q]) * hi;
                const float sum = segment_sum<CPR>(part, c);
                if (c == 0 && rows[q] >= 0) a.obuf[(size_t)p * H + rows[q]] = sum * grow[q];
            }
        }
    }
}

// y_t (=|+=) sum_j w_tj o[pos(t,j)] + s_t o[shared row t], summed in a fixed
// order (j ascending, then the shared expert).  One workgroup per (token,
// 256 output rows); the token's routing and the slot map are staged in LDS.
constexpr int kCombineMaxK = 1024;

__global__ void __launch_bounds__(256) decode_combine_kernel(DecodeArgs a, int nchunk) {
    __shared__ int pos_s[kCombineMaxK];
    __shared__ float w_s[kCombineMaxK];
    const int t = blockIdx.x / nchunk, chunk = blockIdx.x % nchunk;
    const int tid = threadIdx.x;
    const int H = a.H, T = a.T, k = a.k;
    for (int j = tid; j < k; j += 256) {
        const int aidx = t * k + j;
        const bool ok = a.slot_of_expert[a.ids[aidx]] >= 0;
        pos_s[j] = ok ? a.assign_pos[aidx] : -1;
        w_s[j] = a.w[aidx];
    }
    const float st = a.shared != nullptr ? a.sbuf[t] : 0.0f;
    __syncthreads();
    const int row = chunk * 256 + tid;
    if (row >= H) return;
    float acc = 0.0f;
    for (int j = 0; j < k; ++j) {
        const int p = pos_s[j];
        if (p >= 0) acc += w_s[j] * a.obuf[(size_t)p * H + row];
    }
    if (a.shared != nullptr) acc += st * a.obuf[(size_t)(T * k + t) * H + row];
    float* yp = a.y + (size_t)t * H + row;
    *yp = a.accumulate ? *yp + acc : acc;
}

struct GateupCfg {
    int cpl, lpr;
};

GateupCfg gateup_cfg(int H) {
    const int cpr = H / 32;
    int lpr = 1;
    while (lpr < 64 && cpr % (lpr * 2) == 0) lpr *= 2;
    return {cpr / lpr, lpr};
}

template <int CPL>
hipError_t launch_gateup_cpl(int lpr, const DecodeArgs& a, int nb, int grid, hipStream_t s) {
    const size_t lds = (size_t)2 * a.H * 2;
    switch (lpr) {
#define CASE(L)                                                                                      \
    case L:                                                                                          \
        hipLaunchKernelGGL((decode_gateup_kernel<CPL, L>), dim3(grid), dim3(256), lds, s, a, nb);    \
        return hipGetLastError();
        CASE(1) CASE(2) CASE(4) CASE(8) CASE(16) CASE(32) CASE(64)
#undef CASE
    }
    return hipErrorInvalidValue;
}

template <int CPR>
hipError_t launch_down_cpr(const DecodeArgs& a, int na_max, hipStream_t s) {
    constexpr int RBD = (kWave / CPR) * kDownPW * 4;
    const int nb = ceil_div(a.H, RBD);
    hipLaunchKernelGGL((decode_down_kernel<CPR>), dim3(max(1, na_max) * nb), dim3(256), 0, s, a, nb);
    return hipGetLastError();
}

hipError_t launch_down(const DecodeArgs& a, int na_max, hipStream_t s) {
    switch (a.I / 32) {
#define CASE(C) \
    case C: return launch_down_cpr<C>(a, na_max, s);
        CASE(1) CASE(2) CASE(3) CASE(4) CASE(5) CASE(6) CASE(7) CASE(8) CASE(9) CASE(10) CASE(11) CASE(12)
        CASE(13) CASE(14) CASE(15) CASE(16) CASE(17) CASE(18) CASE(19) CASE(20) CASE(21) CASE(22) CASE(23) CASE(24)
        CASE(25) CASE(26) CASE(27) CASE(28) CASE(29) CASE(30) CASE(31) CASE(32) CASE(40) CASE(48) CASE(64)
#undef CASE
    }
    return hipErrorInvalidValue;
}

bool down_supported(int I) {
    const int c = I / 32;
    return (c >= 1 && c <= 32) || c == 40 || c == 48 || c == 64;
}

}  // namespace

bool decode_shape_supported(int H, int I) {
    GateupCfg c = gateup_cfg(H);
    return c.cpl >= 1 && c.cpl <= 8 && down_supported(I) && H <= 8192;
}

hipError_t launch_decode(const Layer& L, const uint16_t* x, int T, const float* w, const int32_t* ids,
                         const int32_t* offsets, const int32_t* sorted_assign, const int32_t* assign_pos, float* y,
                         int accumulate, void* ws, hipStream_t s) {
    const int H = L.H, I = L.I, E = L.E, k = L.k;
    uint8_t* p = static_cast<uint8_t*>(ws);
    const WsLayout wl = ws_layout(T, H, I, E, k);
    DecodeArgs a;
    a.bank = L.bank;
    a.slot_bytes = L.slot_bytes;
    a.slot_of_expert = L.slot_of_expert;
    a.shared = L.shared;
    a.wg = L.wg;
    a.x = x;
    a.T = T; a.H = H; a.I = I; a.E = E; a.k = k;
    a.w = w; a.ids = ids; a.offsets = offsets; a.sorted_assign = sorted_assign; a.assign_pos = assign_pos;
    a.hbuf = reinterpret_cast<float*>(p + wl.h);
    a.obuf = reinterpret_cast<float*>(p + wl.o);
    a.sbuf = reinterpret_cast<float*>(p + wl.s);
    a.y = y;
    a.accumulate = accumulate;
    SlotGeom gm = slot_geom(H, I);
    a.gu_codes = gm.gu_codes; a.gu_scales = gm.gu_scales; a.gu_glob = gm.gu_glob;
    a.dn_codes = gm.dn_codes; a.dn_scales = gm.dn_scales; a.dn_glob = gm.dn_glob;

    const int na_max = min(E, T * k) + (L.shared ? 1 : 0);
    GateupCfg c = gateup_cfg(H);
    const int rg = 4 * (64 / c.lpr);
    const int nb_gu = ceil_div(I, rg);
    hipError_t err = hipSuccess;
    const int grid = max(1, na_max) * nb_gu;
    switch (c.cpl) {
        case 1: err = launch_gateup_cpl<1>(c.lpr, a, nb_gu, grid, s); break;
        case 2: err = launch_gateup_cpl<2>(c.lpr, a, nb_gu, grid, s); break;
        case 3: err = launch_gateup_cpl<3>(c.lpr, a, nb_gu, grid, s); break;
        case 4: err = launch_gateup_cpl<4>(c.lpr, a, nb_gu, grid, s); break;
        case 5: err = launch_gateup_cpl<5>(c.lpr, a, nb_gu, grid, s); break;
        case 6: err = launch_gateup_cpl<6>(c.lpr, a, nb_gu, grid, s); break;
        case 7: err = launch_gateup_cpl<7>(c.lpr, a, nb_gu, grid, s); break;
        case 8: err = launch_gateup_cpl<8>(c.lpr, a, nb_gu, grid, s); break;
        default: return hipErrorInvalidValue;
    }
    if (err != hipSuccess) return err;
    if ((err = launch_down(a, na_max, s)) != hipSuccess) return err;
    const int nchunk = ceil_div(H, 256);
    hipLaunchKernelGGL(decode_combine_kernel, dim3(T * nchunk), dim3(256), 0, s, a, nchunk);
    return hipGetLastError();
}

}  // namespace moe
