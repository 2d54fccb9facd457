// Decode path (T <= 16) of the NVFP4 routed-MoE layer for gfx950.
//
// The layer (PR #385 "What this adds"; issue #62 "What it touches"):
//   h = silu(W_gate x) * (W_up x)   with gate rows [0, I) and up rows [I, 2I) of gate_up [2I, H]
//   o = W_dn h                      with down [H, I]
//   y_t = sum_j w_tj o_{e_tj}(x_t) + sigmoid(x_t . w_g) o_shared(x_t)
// At decode batch sizes this is a set of GEMVs over the distinct routed
// experts, bound by the HBM bytes of their NVFP4 weights.  Two kernels:
//
// gate_up: one workgroup per (active expert, block of gate rows and the
//   matching up rows).  LPR lanes share a row and each owns CPL 16-byte code
//   chunks (32 elements, two scale blocks) of it, so every wave reads whole
//   coalesced row segments with 128-bit loads.  Codes are decoded to bf16 in
//   registers (exact) and dotted with the bf16 activations by v_dot2c (exact
//   products, f32 sums); each 16-block's sum is scaled by its E4M3 scale, the
//   lanes of a row are reduced with cross-lane shuffles, the row global is
//   applied, and silu(gate) * up is written as the fp32 hidden state.
//
// down: one single-wave workgroup per (active expert, 64 output rows).  The
//   64 rows' codes and scales are staged through LDS with coalesced 128-bit
//   loads, then each lane owns one row and walks it, while the fp32 hidden
//   state (the same for all lanes) is read with wave-uniform loads.  Each
//   workgroup writes its expert's outputs o, and the last workgroup to finish
//   a 64-row block (an atomic arrival counter) combines that block for all
//   tokens in a fixed order: y = sum_j w_tj o_{tj} + s_t o_shared.  No atomic
//   ever adds a value, so results are bit-reproducible.
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
    float* hbuf;    // f32 [(T*k + T), I]: row p = sorted assignment p, row T*k + t = shared expert, token t
    float* obuf;    // f32 [(T*k + T), H]: expert outputs, same row order
    float* sbuf;    // f32 [T]: shared gate sigmoid(x_t . w_g)
    int* counters;  // i32 [ceil(H/64)]: arrivals per 64-row block of the down kernel
    float* y;
    int accumulate;
    size_t gu_codes, gu_scales, gu_glob, dn_codes, dn_scales, dn_glob;
};

__device__ __forceinline__ bool expert_active(const DecodeArgs& a, int e) {
    return a.offsets[e + 1] > a.offsets[e] && a.slot_of_expert[e] >= 0;
}

// Which expert the workgroup's active index `ai` names: the ai-th active
// routed expert in ascending order, then the shared expert (returned as E).
// Returns -1 past the end.  *n_total = active routed experts + shared.
// NT = threads in the workgroup; `scratch` holds >= NT/64 + 2 ints of LDS.
template <int NT>
__device__ int find_active(const DecodeArgs& a, int ai, int* n_total, int* scratch) {
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    constexpr int NW = NT / kWave;
    const int per = (a.E + NT - 1) / NT;
    const int e0 = tid * per, e1 = min(a.E, e0 + per);
    int cnt = 0;
    for (int e = e0; e < e1; ++e) cnt += expert_active(a, e) ? 1 : 0;
    int incl = cnt;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        int o = __shfl_up(incl, off, kWave);
        if (lane >= off) incl += o;
    }
    if (NW > 1) {
        if (lane == kWave - 1) scratch[2 + wave] = incl;
        __syncthreads();
    }
    int before = 0, total = 0;
    if (NW > 1) {
#pragma unroll
        for (int i = 0; i < NW; ++i) {
            int s = scratch[2 + i];
            if (i < wave) before += s;
            total += s;
        }
    } else {
        total = __shfl(incl, kWave - 1, kWave);
    }
    const int excl = before + incl - cnt;
    if (tid == 0) scratch[0] = -1;
    __syncthreads();
    if (ai >= excl && ai < excl + cnt) {
        int want = ai - excl;
        for (int e = e0; e < e1; ++e)
            if (expert_active(a, e)) {
                if (want == 0) { scratch[0] = e; break; }
                --want;
            }
    }
    __syncthreads();
    int e = __builtin_amdgcn_readfirstlane(scratch[0]);
    total = __builtin_amdgcn_readfirstlane(total);
    const bool has_shared = a.shared != nullptr;
    if (e < 0 && has_shared && ai == total) e = a.E;
    *n_total = total + (has_shared ? 1 : 0);
    __syncthreads();
    return e;
}

__device__ __forceinline__ const uint8_t* slot_ptr(const DecodeArgs& a, int e) {
    return e == a.E ? a.shared : a.bank + (size_t)a.slot_of_expert[e] * a.slot_bytes;
}

// ------------------------------------------------------------------ gate_up + SwiGLU
template <int CPL, int LPR>
__global__ void __launch_bounds__(256) decode_gateup_kernel(DecodeArgs a, int NB) {
    constexpr int RW = kWave / LPR;  // rows per wave
    constexpr int RG = 2 * RW;       // gate rows (and up rows) per workgroup
    __shared__ int scratch[8];
    __shared__ float vals[kDecodeMaxT][2][RG];

    const int ai = blockIdx.x / NB, nb = blockIdx.x % NB;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    if (blockIdx.x == 0)
        for (int i = tid; i < (a.H + 63) / 64; i += 256) a.counters[i] = 0;
    int n_total;
    const int e = find_active<256>(a, ai, &n_total, scratch);
    if (e < 0) return;
    const uint8_t* slot = slot_ptr(a, e);
    const bool is_shared = e == a.E;
    const int p0 = __builtin_amdgcn_readfirstlane(is_shared ? a.T * a.k : a.offsets[e]);
    // A token routes to an expert at most once, so ne <= T <= 16; the clamp
    // only guards the LDS array against routing not made by moe_route_topk.
    const int ne = min(kDecodeMaxT, __builtin_amdgcn_readfirstlane(is_shared ? a.T : a.offsets[e + 1] - p0));

    // Shared gate: s_t = sigmoid(x_t . w_g), once per layer call.
    if (is_shared && nb == 0) {
        for (int t = wave; t < a.T; t += 4) {
            float acc = 0.0f;
            for (int c = lane; c < a.H; c += kWave)
                acc += bf16_bits_f32(a.x[(size_t)t * a.H + c]) * bf16_bits_f32(a.wg[c]);
            acc = wave_sum(acc);
            if (lane == 0) a.sbuf[t] = sigmoidf_(acc);
        }
    }

    const int H = a.H, I = a.I;
    const int part = wave >> 1, sub = wave & 1;
    const int lir = lane % LPR, rsub = lane / LPR;
    const int irow = nb * RG + sub * RW + rsub;
    const bool valid = irow < I;
    const int grow = part * I + (valid ? irow : 0);

    const uint8_t* codes = slot + a.gu_codes + (size_t)grow * (H / 2);
    const uint8_t* scales = slot + a.gu_scales + (size_t)grow * (H / 16);
    const float g = reinterpret_cast<const float*>(slot + a.gu_glob)[grow];

    u32x4_t cw[CPL];
    uint32_t sc[CPL];
#pragma unroll
    for (int j = 0; j < CPL; ++j) {
        const int c = lir + LPR * j;
        cw[j] = *reinterpret_cast<const u32x4_t*>(codes + c * 16);
        sc[j] = *reinterpret_cast<const uint16_t*>(scales + c * 2);
    }

    for (int ti = 0; ti < ne; ++ti) {
        const int t = is_shared ? ti : a.sorted_assign[p0 + ti] / a.k;
        const uint16_t* xr = a.x + (size_t)t * H;
        float acc = 0.0f;
#pragma unroll
        for (int j = 0; j < CPL; ++j) {
            const int c = lir + LPR * j;
            const u32x4_t* xp = reinterpret_cast<const u32x4_t*>(xr + c * 32);
            uint32_t xw[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                u32x4_t v = xp[q];
                xw[4 * q + 0] = v.x; xw[4 * q + 1] = v.y; xw[4 * q + 2] = v.z; xw[4 * q + 3] = v.w;
            }
            const float p_lo = block16_dot_bf16(cw[j].x, cw[j].y, xw);
            const float p_hi = block16_dot_bf16(cw[j].z, cw[j].w, xw + 8);
            acc += e4m3_f32<0>(sc[j]) * p_lo + e4m3_f32<1>(sc[j]) * p_hi;
        }
        acc = group_sum<LPR>(acc);
        if (lir == 0 && valid) vals[ti][part][sub * RW + rsub] = acc * g;
    }
    __syncthreads();
    for (int idx = tid; idx < ne * RG; idx += 256) {
        const int ti = idx / RG, il = idx % RG, i = nb * RG + il;
        if (i < I) {
            const float gate = vals[ti][0][il], up = vals[ti][1][il];
            a.hbuf[(size_t)(p0 + ti) * I + i] = gate * sigmoidf_(gate) * up;
        }
    }
}

// ------------------------------------------------------------------ down + combine
constexpr int kDownMaxI = 1024;

__global__ void __launch_bounds__(64) decode_down_kernel(DecodeArgs a, int NB, const float* __restrict__ hb) {
    constexpr int ROWS = kWave;
    constexpr int PITCH_MAX = kDownMaxI / 2 + 16;
    constexpr int SPITCH_MAX = kDownMaxI / 16 + 4;
    __shared__ __attribute__((aligned(16))) uint8_t lds_codes[ROWS * PITCH_MAX];
    __shared__ __attribute__((aligned(16))) uint8_t lds_sc[ROWS * SPITCH_MAX];
    __shared__ int scratch[4];

    const int ai = blockIdx.x / NB, rb = blockIdx.x % NB;
    const int lane = threadIdx.x;
    const int H = a.H, I = a.I, T = a.T, k = a.k;
    const int r0 = rb * ROWS;
    const int rows_here = min(ROWS, H - r0);
    int n_total;
    const int e = find_active<64>(a, ai, &n_total, scratch);

    if (e >= 0) {
        const uint8_t* slot = slot_ptr(a, e);
        const bool is_shared = e == a.E;
        const int p0 = __builtin_amdgcn_readfirstlane(is_shared ? T * k : a.offsets[e]);
        const int ne = __builtin_amdgcn_readfirstlane(is_shared ? T : a.offsets[e + 1] - p0);
        const int cpr = I / 32;               // 16-byte code chunks per row
        const int pitch = I / 2 + 16;         // padded LDS row pitch of codes (bank spread)
        const int spitch = I / 16 + 4;        // padded LDS row pitch of scales

        // Stage this block's rows: codes (I/2 bytes per row) and scales (I/16 per row).
        const uint8_t* gcodes = slot + a.dn_codes + (size_t)r0 * (I / 2);
        const uint8_t* gsc = slot + a.dn_scales + (size_t)r0 * (I / 16);
        const int pieces = rows_here * cpr;
        for (int q = lane; q < pieces; q += kWave) {
            const int row = q / cpr, c = q % cpr;
            *reinterpret_cast<u32x4_t*>(lds_codes + row * pitch + c * 16) =
                *reinterpret_cast<const u32x4_t*>(gcodes + (size_t)q * 16);
            *reinterpret_cast<uint16_t*>(lds_sc + row * spitch + c * 2) =
                *reinterpret_cast<const uint16_t*>(gsc + (size_t)q * 2);
        }
        __syncthreads();

        const bool valid = lane < rows_here;
        const int row = r0 + (valid ? lane : 0);
        const float g = reinterpret_cast<const float*>(slot + a.dn_glob)[row];
        const uint8_t* my_codes = lds_codes + lane * pitch;
        const uint8_t* my_sc = lds_sc + lane * spitch;

        for (int tb = 0; tb < ne; tb += 4) {
            const int nt = min(4, ne - tb);
            float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
            for (int c = 0; c < cpr; ++c) {
                const u32x4_t cwv = *reinterpret_cast<const u32x4_t*>(my_codes + c * 16);
                const uint32_t s16 = *reinterpret_cast<const uint16_t*>(my_sc + c * 2);
                const float s0 = e4m3_f32<0>(s16), s1 = e4m3_f32<1>(s16);
                float wv[32];
                const uint32_t words[4] = {cwv.x, cwv.y, cwv.z, cwv.w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    f32x2_t v0 = e2m1x2_f32<0>(words[q]);
                    f32x2_t v1 = e2m1x2_f32<1>(words[q]);
                    f32x2_t v2 = e2m1x2_f32<2>(words[q]);
                    f32x2_t v3 = e2m1x2_f32<3>(words[q]);
                    wv[8 * q + 0] = v0.x; wv[8 * q + 1] = v0.y; wv[8 * q + 2] = v1.x; wv[8 * q + 3] = v1.y;
                    wv[8 * q + 4] = v2.x; wv[8 * q + 5] = v2.y; wv[8 * q + 6] = v3.x; wv[8 * q + 7] = v3.y;
                }
#pragma unroll
                for (int tt = 0; tt < 4; ++tt) {
                    if (tt < nt) {
                        const float* hp = hb + (size_t)(p0 + tb + tt) * I + c * 32;
                        float lo = 0.0f, hi = 0.0f;
#pragma unroll
                        for (int i = 0; i < 16; ++i) lo += wv[i] * hp[i];
#pragma unroll
                        for (int i = 16; i < 32; ++i) hi += wv[i] * hp[i];
                        acc[tt] += s0 * lo + s1 * hi;
                    }
                }
            }
#pragma unroll
            for (int tt = 0; tt < 4; ++tt)
                if (tt < nt && valid) a.obuf[(size_t)(p0 + tb + tt) * H + row] = acc[tt] * g;
        }
    }

    // Arrival: the last workgroup of this row block combines it for all tokens.
    bool combine;
    if (n_total == 0) {
        combine = ai == 0;  // nothing active: the first workgroup writes 0 (or leaves y)
    } else {
        if (e < 0) return;
        __threadfence();
        if (lane == 0) scratch[1] = atomicAdd(&a.counters[rb], 1);
        __syncthreads();
        combine = scratch[1] == n_total - 1;
        if (combine) __threadfence();
    }
    if (!combine) return;
    if (lane < rows_here) {
        const int row = r0 + lane;
        for (int t = 0; t < T; ++t) {
            float acc = 0.0f;
            for (int j = 0; j < k; ++j) {
                const int aidx = t * k + j;
                const int ej = a.ids[aidx];
                if (a.slot_of_expert[ej] >= 0) acc += a.w[aidx] * a.obuf[(size_t)a.assign_pos[aidx] * H + row];
            }
            if (a.shared != nullptr) acc += a.sbuf[t] * a.obuf[(size_t)(T * k + t) * H + row];
            float* yp = a.y + (size_t)t * H + row;
            *yp = a.accumulate ? *yp + acc : acc;
        }
    }
    if (n_total > 0 && lane == 0) a.counters[rb] = 0;
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
hipError_t launch_gateup_cpl(int lpr, const DecodeArgs& a, int nblocks_expert, int grid, hipStream_t s) {
    switch (lpr) {
#define CASE(L)                                                                                          \
    case L:                                                                                              \
        hipLaunchKernelGGL((decode_gateup_kernel<CPL, L>), dim3(grid), dim3(256), 0, s, a, nblocks_expert); \
        return hipGetLastError();
        CASE(1) CASE(2) CASE(4) CASE(8) CASE(16) CASE(32) CASE(64)
#undef CASE
    }
    return hipErrorInvalidValue;
}

}  // namespace

bool decode_shape_supported(int H, int I) {
    GateupCfg c = gateup_cfg(H);
    return c.cpl >= 1 && c.cpl <= 8 && I <= kDownMaxI;
}

hipError_t launch_decode(const Layer& L, const uint16_t* x, int T, const float* w, const int32_t* ids,
                         const int32_t* offsets, const int32_t* sorted_assign, const int32_t* assign_pos, float* y,
                         int accumulate, void* ws, hipStream_t s) {
    const int H = L.H, I = L.I, E = L.E, k = L.k;
    const int nrows_all = T * k + T;
    uint8_t* p = static_cast<uint8_t*>(ws);
    DecodeArgs a;
    a.bank = L.bank;
    a.slot_bytes = L.slot_bytes;
    a.slot_of_expert = L.slot_of_expert;
    a.shared = L.shared;
    a.wg = L.wg;
    a.x = x;
    a.T = T; a.H = H; a.I = I; a.E = E; a.k = k;
    a.w = w; a.ids = ids; a.offsets = offsets; a.sorted_assign = sorted_assign; a.assign_pos = assign_pos;
    a.hbuf = reinterpret_cast<float*>(p);
    p += (size_t)nrows_all * I * 4;
    a.obuf = reinterpret_cast<float*>(p);
    p += (size_t)nrows_all * H * 4;
    a.sbuf = reinterpret_cast<float*>(p);
    p += 256 * ((T * 4 + 255) / 256);
    a.counters = reinterpret_cast<int*>(p);
    a.y = y;
    a.accumulate = accumulate;
    SlotGeom gm = slot_geom(H, I);
    a.gu_codes = gm.gu_codes; a.gu_scales = gm.gu_scales; a.gu_glob = gm.gu_glob;
    a.dn_codes = gm.dn_codes; a.dn_scales = gm.dn_scales; a.dn_glob = gm.dn_glob;

    const int na_max = min(E, T * k) + (L.shared ? 1 : 0);
    GateupCfg c = gateup_cfg(H);
    const int rg = 2 * (64 / c.lpr);
    const int nb_gu = ceil_div(I, rg);
    hipError_t err = hipSuccess;
    if (na_max > 0) {
        switch (c.cpl) {
            case 1: err = launch_gateup_cpl<1>(c.lpr, a, nb_gu, na_max * nb_gu, s); break;
            case 2: err = launch_gateup_cpl<2>(c.lpr, a, nb_gu, na_max * nb_gu, s); break;
            case 3: err = launch_gateup_cpl<3>(c.lpr, a, nb_gu, na_max * nb_gu, s); break;
            case 4: err = launch_gateup_cpl<4>(c.lpr, a, nb_gu, na_max * nb_gu, s); break;
            case 5: err = launch_gateup_cpl<5>(c.lpr, a, nb_gu, na_max * nb_gu, s); break;
            case 6: err = launch_gateup_cpl<6>(c.lpr, a, nb_gu, na_max * nb_gu, s); break;
            case 7: err = launch_gateup_cpl<7>(c.lpr, a, nb_gu, na_max * nb_gu, s); break;
            case 8: err = launch_gateup_cpl<8>(c.lpr, a, nb_gu, na_max * nb_gu, s); break;
            default: return hipErrorInvalidValue;
        }
        if (err != hipSuccess) return err;
    }
    const int nb_dn = ceil_div(H, 64);
    const int grid_dn = max(1, na_max) * nb_dn;
    hipLaunchKernelGGL(decode_down_kernel, dim3(grid_dn), dim3(64), 0, s, a, nb_dn, (const float*)a.hbuf);
    return hipGetLastError();
}

}  // namespace moe
