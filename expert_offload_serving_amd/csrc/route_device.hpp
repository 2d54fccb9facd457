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
// ones, after folding -0 onto +0.  Key 0 marks "no candidate": the one float
// pattern that would map to it (an all-ones NaN, a precondition violation)
// takes key 1 instead, so 0 is never the maximum while a logit remains.
__device__ __forceinline__ uint32_t order_key(float v) {
    const uint32_t u = __float_as_uint(v + 0.0f);
    const uint32_t key = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return key > 1u ? key : 1u;
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
// Each lane first orders its VPL keys (descending; equal keys keep index
// order, as the insertion network below is stable), so its head is its best
// remaining candidate.  Each of the k rounds takes the wave maximum M of the
// heads; the selection is the lowest expert index holding M, which is the
// head of the lowest lane among those whose head is M and whose slot i is the
// smallest (one ballot, or one per slot when heads tie), and that lane drops
// its head.  Selection j is kept by lane j % 64 and stored after the rounds.
// Weights: softmax over the k selected logits in double (exp(l_j - l_max) /
// sum), summed in selection order, rounded to f32.
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
    uint32_t kk[VPL];  // this lane's remaining keys, best first
    int ss[VPL];       // their slots i (expert lane + 64 i); VPL once dropped
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        kk[i] = order_key(__uint_as_float(lv[i])) & (lane + kWave * i < E ? ~0u : 0u);
        ss[i] = i;
    }
#pragma unroll
    for (int i = 1; i < VPL; ++i)
#pragma unroll
        for (int j = i; j > 0; --j) {
            const bool sw = kk[j] > kk[j - 1];
            const uint32_t ka = kk[j - 1], kb = kk[j];
            const int sa = ss[j - 1], sb = ss[j];
            kk[j - 1] = sw ? kb : ka;
            kk[j] = sw ? ka : kb;
            ss[j - 1] = sw ? sb : sa;
            ss[j] = sw ? sa : sb;
        }
    float held = 0.0f;  // selection j's logit, kept by lane j (j < 64)
    int held_id = 0;    // and its expert
    float m = 0.0f;
    for (int j = 0; j < k; ++j) {
        const uint32_t M = wave_umax_dpp(kk[0]);
        uint64_t hit = __ballot(kk[0] == M);
        int slot;
        if (__popcll(hit) == 1) {  // uniform; the usual case
            slot = __builtin_amdgcn_readlane(ss[0], (int)__builtin_ctzll(hit));
        } else {  // heads tie on M: the smallest slot holding M, then its lowest lane
            slot = 0;
            for (int i = 0; i < VPL; ++i) {
                const uint64_t b = __ballot(kk[0] == M && ss[0] == i);
                if (b != 0) {
                    hit = b;
                    slot = i;
                    break;
                }
            }
        }
        // M >= 1 is the head of some lane (k <= E valid keys), so hit != 0
        const int owner = (int)__builtin_ctzll(hit);
        const int bi = min(slot * kWave + owner, E - 1);  // the clamp only keeps the index in range
        if (lane == owner) {
#pragma unroll
            for (int i = 0; i + 1 < VPL; ++i) {
                kk[i] = kk[i + 1];
                ss[i] = ss[i + 1];
            }
            kk[VPL - 1] = 0u;
            ss[VPL - 1] = VPL;
        }
        const float bv = key_logit(M);
        if (j == 0) m = bv;
        if (j == lane) {
            held = bv;
            held_id = bi;
        }
        if (j >= kWave && (j % kWave) == lane) {  // rare: more selections than lanes; logit parked in w
            ids[j] = bi;
            w[j] = bv;
        }
    }
    if (lane < k) ids[lane] = held_id;
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
