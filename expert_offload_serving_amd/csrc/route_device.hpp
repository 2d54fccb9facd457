// Device-side top-k routing for one token per wave (shared by the routing
// kernels and the decode kernels that route in their prologue).
//
// Routing follows the replicated router with norm_topk_prob of the pages
// (issue #62, R9700 interim report): the k largest logits are selected and
// their weights are the softmax over those k logits, which equals a full
// softmax renormalised over the selected experts.  Selection order is
// (logit descending, expert index ascending); -0 ties with +0.
#pragma once

#include "nvfp4_device.hpp"

namespace moe {

constexpr int kRouteMaxE = 1024;
constexpr int kRouteVPL = kRouteMaxE / kWave;  // logits held per lane at most

// DPP row operations of the GCN/CDNA ISA (gfx9 encodings).
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr3 = 0x113, kDppRowShr4 = 0x114,
              kDppRowShr8 = 0x118, kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;

// Logits are compared as order-preserving unsigned keys: the float bits with
// the sign bit set for non-negative values and all bits inverted for negative
// ones, after folding -0 onto +0.  Key 0 (an all-ones NaN) marks "no
// candidate": it is never the maximum while a real logit remains.
__device__ __forceinline__ uint32_t order_key(float v) {
    const uint32_t u = __float_as_uint(v + 0.0f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_logit(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// One step of a wave maximum: take the key DPP control CTRL brings in when it
// is larger.  Lanes the masks disable, or whose source lies outside the row,
// see 0 (the identity of the maximum), which lets the move fold into the max
// as its DPP source (one instruction per step).
template <int CTRL, int ROW_MASK, int BANK_MASK>
__device__ __forceinline__ uint32_t umax_dpp_step(uint32_t v) {
    const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, BANK_MASK, false);
    return v > o ? v : o;
}

// Wave-wide maximum key, returned to every lane.  The DPP sequence leaves the
// result in lane 63 (shifts within each 16-lane row, then the row
// broadcasts); max tolerates the overlapping inputs.
__device__ __forceinline__ uint32_t wave_umax_dpp(uint32_t v) {
    v = umax_dpp_step<kDppRowShr1, 0xF, 0xF>(v);
    v = umax_dpp_step<kDppRowShr2, 0xF, 0xF>(v);
    v = umax_dpp_step<kDppRowShr3, 0xF, 0xF>(v);
    v = umax_dpp_step<kDppRowShr4, 0xF, 0xE>(v);
    v = umax_dpp_step<kDppRowShr8, 0xF, 0xC>(v);
    v = umax_dpp_step<kDppRowBcast15, 0xA, 0xF>(v);
    v = umax_dpp_step<kDppRowBcast31, 0xC, 0xF>(v);
    return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// One wave selects the top-k of row `l` (E <= 64 * VPL logits; lane L holds
// experts L + 64 i; every lane passes the same row) and writes ids and weights
// (global or LDS pointers).
// Each of the k rounds takes the wave maximum of the remaining keys, then the
// lowest expert index holding it (a second wave maximum, over ~index of the
// entries equal to the first).  A selected key becomes 0.
// A NaN logit (a precondition violation) only changes which valid, distinct
// experts come out.  Weights: softmax over the k selected logits in double
// (exp(l_j - l_max) / sum), summed in selection order, rounded to f32.
template <int VPL>
__device__ void topk_one_token(const float* __restrict__ l, int E, int k, int32_t* __restrict__ ids,
                               float* __restrict__ w, int lane) {
    static_assert(VPL <= kRouteVPL, "too many logits per lane");
    // every logit load is issued before any is used, with no branch around them (buffer loads past the row
    // return zeros, masked to "no candidate" below), so they wait for one another only once
    // the row is the same for the whole wave; readfirstlane lets the compiler keep its resource scalar
    const uint64_t lp = reinterpret_cast<uint64_t>(l);
    const uint32_t lp_lo = __builtin_amdgcn_readfirstlane((uint32_t)lp);
    const uint32_t lp_hi = __builtin_amdgcn_readfirstlane((uint32_t)(lp >> 32));
    const rsrc_t lres = make_rsrc(reinterpret_cast<const float*>(((uint64_t)lp_hi << 32) | lp_lo), (uint32_t)E * 4);
    uint32_t lv[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) lv[i] = buf_load4(lres, 4 * (lane + kWave * i));
    uint32_t v[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) v[i] = order_key(__uint_as_float(lv[i])) & (lane + kWave * i < E ? ~0u : 0u);
    float held = 0.0f;  // selection j's logit, kept by lane j (j < 64)
    float m = 0.0f;
    for (int j = 0; j < k; ++j) {
        uint32_t lm = v[0];
#pragma unroll
        for (int i = 1; i < VPL; ++i) lm = v[i] > lm ? v[i] : lm;
        const uint32_t M = wave_umax_dpp(lm);
        // lowest index holding M: each lane offers its lowest slot holding M as ~index, the wave takes the
        // largest (all on the vector units: with many waves per CU the shared scalar unit would be the limit)
        uint32_t cand = 0;
#pragma unroll
        for (int i = VPL - 1; i >= 0; --i) cand = v[i] == M ? ~(uint32_t)(lane + kWave * i) : cand;
        const uint32_t best = wave_umax_dpp(cand);
        // M is a key some lane holds, so best != 0; the clamp only keeps the index in range
        const int bi = best != 0 ? (int)~best : 0;
        const int owner_slot = bi / kWave, owner_lane = bi % kWave;
#pragma unroll
        for (int i = 0; i < VPL; ++i) v[i] = (i == owner_slot && lane == owner_lane) ? 0u : v[i];
        const float bv = key_logit(M);
        if (j == 0) m = bv;
        if ((j % kWave) == lane) ids[j] = bi;
        if (j == lane) held = bv;
        if (j >= kWave && (j % kWave) == lane) w[j] = bv;  // parked logit, replaced below
    }
    // exp of each selected logit relative to the largest, in double
    if (k <= kWave) {
        const double ex = lane < k ? exp((double)held - (double)m) : 0.0;
        double sum = 0.0;
        for (int j = 0; j < k; ++j) {
            const int lo = __builtin_amdgcn_readlane((int)(uint32_t)__double_as_longlong(ex), j);
            const int hi = __builtin_amdgcn_readlane((int)(uint32_t)(__double_as_longlong(ex) >> 32), j);
            sum += __longlong_as_double(((long long)(uint32_t)hi << 32) | (uint32_t)lo);
        }
        if (lane < k) w[lane] = (float)(ex / sum);
    } else {
        // rare: more selections than lanes; logits of selections >= 64 were parked in w
        double sum = 0.0;
        for (int j = 0; j < k; ++j) sum += exp((double)(j < kWave ? __shfl(held, j, kWave) : w[j]) - (double)m);
        for (int j = lane; j < k; j += kWave) {
            const float lj = j < kWave ? held : w[j];
            w[j] = (float)(exp((double)lj - (double)m) / sum);
        }
    }
}

}  // namespace moe
