// MXFP4 bank format for gfx950: the decode path (T <= 16) of the routed-MoE
// layer, the dequant hooks and the bank slicer.
//
// MXFP4 (issue #62 "What it touches" names it as a bank format whose
// checkpoints are transposed, blocks_t [K//2, N], with 32-wide fp4 scale
// blocks): E2M1 elements with one E8M0 scale per 32 consecutive elements
// along the contraction axis, no per-row global.  gfx950 multiplies that
// format natively: v_mfma_scale_f32_16x16x128_f8f6f4 takes fp4 codes as
// they are stored and applies one E8M0 scale per (row, 32-element block)
// itself, so gate_up needs no decode on the vector ALUs at all.
//
// Work item = (expert, 32-row slice of I), one wave per item (as the NVFP4
// wave kernel; 64-row slices when 32-row items would outnumber the waves,
// which halves the items and their partial sums):
//   gate_up  16-row x 128-column records (lane 16a + i: row i, the 32
//            columns [32a, 32a + 32), i.e. one scale block) are the A operand
//            of the scaled MFMA as loaded; the activations are its B operand
//            in fp8 E4M3 as two terms with their own E8M0 block scales
//            (x = 2^s_hi * hi + 2^s_lo * lo: the bf16 value's 8 significant
//            bits split 4 + 4, so the product is exact up to fp32 summation);
//   SwiGLU   h = silu(gate) * up in fp32, then two bf16 terms (h_hi + h_lo
//            carries 16 significant bits);
//   down     the slice's 32 (or 64) columns of every row: 64-row x 32-column records
//            decoded exactly to bf16 by v_cvt_scalef32_pk_bf16_fp4, which
//            applies the block's E8M0 scale in the conversion (e2m1 * 2^e is
//            exact in bf16 for every E8M0 value), into
//            v_mfma_f32_16x16x32_bf16 against h_hi and h_lo.  (A scaled
//            MFMA contracts 128 columns per instruction: the item's 32-wide
//            slice would fill a quarter of it.)
// The per-(row, slice) partials times the routing weight go to the same
// fixed-order combine as the NVFP4 path, which has no globals to apply here.
//
// Operand lane layouts of v_mfma_scale_f32_16x16x128_f8f6f4 (measured on
// gfx950): fp4 operand, lane 16a + i: row (column) i, k = 32a + [0, 32),
// the even k in the low nibble; fp8 operand, lane 16g + c: column c,
// bytes 0-15 k = 16g + [0, 16), bytes 16-31 k = 64 + 16g + [0, 16); the E8M0
// scale operand of lane 16g + c belongs to k-block g; the result as for
// every 16x16 MFMA, lane 16g + c holds rows 4g + [0, 4) of column c.
#include <map>
#include <mutex>
#include <set>
#include <utility>

#include "decode_common.hpp"

namespace moe {

SlotGeom mx_slot_geom(int H, int I) {
    SlotGeom g;
    size_t off = 0;
    g.gu_codes = off; off += (size_t)2 * I * H / 2;
    g.gu_scales = off; off += (size_t)2 * I * H / 32;
    g.gu_glob = off;
    g.dn_codes = off; off += (size_t)H * I / 2;
    g.dn_scales = off; off += (size_t)H * I / 32;
    g.dn_glob = off;
    g.total = off;
    return g;
}

namespace {

typedef int v8i_t __attribute__((ext_vector_type(8)));

constexpr int kMW = 8;               // waves per workgroup
constexpr int kMT = kMW * kWave;     // threads per workgroup
constexpr int kXB = 2560 + 16;       // LDS bytes per staged activation row (H <= 2560; 16-byte pad)

// LDS bytes for T tokens plus the zero row: fp8 hi and lo rows, then their E8M0 scale rows.
__host__ __device__ inline size_t mx_lds_bytes(int T, int H) { return (size_t)(T + 1) * (2 * kXB + 2 * (H / 32)); }

__device__ __forceinline__ float e8m0_as_f32(uint32_t b) { return __uint_as_float((b & 0xFF) << 23); }

// Two bf16 terms of v: hi = bf16(v), lo = bf16(v - hi), packed per pair.
__device__ __forceinline__ void split_bf16x2(float v0, float v1, uint32_t& hi, uint32_t& lo) {
    const __bf16 h0 = (__bf16)v0, h1 = (__bf16)v1;
    const __bf16 l0 = (__bf16)(v0 - (float)h0), l1 = (__bf16)(v1 - (float)h1);
    hi = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
    lo = (uint32_t)__builtin_bit_cast(uint16_t, l0) | ((uint32_t)__builtin_bit_cast(uint16_t, l1) << 16);
}

// E8M0 byte of a block whose largest magnitude is amax, such that amax / 2^(byte - 127) lies in [128, 256)
// (below the E4M3 maximum 448); 0 (2^-127) for amax == 0 or below the E8M0 range.
__device__ __forceinline__ int mx_block_exp(float amax) {
    int e = 0;
    if (amax > 0.0f) (void)frexpf(amax, &e);  // amax = m * 2^e, m in [0.5, 1)
    const int b = amax > 0.0f ? (e - 1 - 7) + 127 : 0;
    return b < 0 ? 0 : (b > 254 ? 254 : b);
}

// Activations to LDS as two fp8 terms per 32-block: lane holds chunks (8 bf16) lane + 64 i of token t; the
// four lanes 4m..4m+3 hold one 32-block.
__device__ __forceinline__ void mx_stage_x(const DecArgs& a, const XRegs<kMW>& xr, uint8_t* xs, int tid, int lane,
                                           int wave) {
    const int H = a.H, T = a.T, NB = H / 32;
    uint8_t* srow = xs + (size_t)(T + 1) * 2 * kXB;  // scale rows: hi [(T + 1) x NB], then lo
#pragma unroll
    for (int p = 0; p < XRegs<kMW>::XT; ++p) {
        const int t = wave + kMW * p;
#pragma unroll
        for (int i = 0; i < XRegs<kMW>::XC; ++i) {
            const int ch = lane + kWave * i;  // chunk of 8 values; block ch / 4
            float v[8];
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint32_t w = word_of(xr.v[p][i], d);
                v[2 * d] = __uint_as_float(w << 16);
                v[2 * d + 1] = __uint_as_float(w & 0xFFFF0000u);
            }
            float am = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf(v[e]));
            am = quad_max(am);
            const int bh = mx_block_exp(am);
            const float inv_h = ldexpf(1.0f, 127 - bh);
            float r[8];
            uint32_t hw[2];
#pragma unroll
            for (int d = 0; d < 2; ++d) {
                int pk = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * d] * inv_h, v[4 * d + 1] * inv_h, 0, false);
                pk = __builtin_amdgcn_cvt_pk_fp8_f32(v[4 * d + 2] * inv_h, v[4 * d + 3] * inv_h, pk, true);
                hw[d] = (uint32_t)pk;
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    r[4 * d + e] = v[4 * d + e] * inv_h - (e == 0 ? __builtin_amdgcn_cvt_f32_fp8(pk, 0)
                                                            : e == 1 ? __builtin_amdgcn_cvt_f32_fp8(pk, 1)
                                                            : e == 2 ? __builtin_amdgcn_cvt_f32_fp8(pk, 2)
                                                                     : __builtin_amdgcn_cvt_f32_fp8(pk, 3));
            }
            // the residuals (exact in f32) in units of the block's own second scale
            float ar = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) ar = fmaxf(ar, fabsf(r[e]));
            ar = quad_max(ar);
            const int bl_rel = mx_block_exp(ar);  // exponent of the residual in units of 2^(bh - 127)
            int bl = bl_rel - 127 + bh;           // as an absolute E8M0 byte
            const bool lo_zero = ar == 0.0f || bl < 0;
            bl = lo_zero ? 0 : bl;
            const float inv_l = lo_zero ? 0.0f : ldexpf(1.0f, 127 - bl_rel);
            uint32_t lw[2];
#pragma unroll
            for (int d = 0; d < 2; ++d) {
                int pk = __builtin_amdgcn_cvt_pk_fp8_f32(r[4 * d] * inv_l, r[4 * d + 1] * inv_l, 0, false);
                pk = __builtin_amdgcn_cvt_pk_fp8_f32(r[4 * d + 2] * inv_l, r[4 * d + 3] * inv_l, pk, true);
                lw[d] = (uint32_t)pk;
            }
            if (t < T && ch < H / 8) {
                *reinterpret_cast<uint2*>(xs + (size_t)t * 2 * kXB + 8 * ch) = make_uint2(hw[0], hw[1]);
                *reinterpret_cast<uint2*>(xs + (size_t)t * 2 * kXB + kXB + 8 * ch) = make_uint2(lw[0], lw[1]);
                if ((ch & 3) == 0) {
                    srow[t * NB + ch / 4] = (uint8_t)bh;
                    srow[(T + 1) * NB + t * NB + ch / 4] = (uint8_t)bl;
                }
            }
        }
    }
    // the zero row (columns of the MFMA without a token): zero values, scale byte 0
    for (int q = tid; q < (2 * kXB) / 16; q += kMT)
        *reinterpret_cast<u32x4_t*>(xs + (size_t)T * 2 * kXB + 16 * q) = u32x4_t{0, 0, 0, 0};
    for (int q = tid; q < NB; q += kMT) {
        srow[T * NB + q] = 0;
        srow[(T + 1) * NB + T * NB + q] = 0;
    }
}

struct MxRing {
    u32x4_t cd[8];
    uint32_t sc[8];
};

// Item geometry for SL intermediate rows (32 or 64): the slice has NTT gate tiles (rows SL s + 16 r) and the NTT
// matching up tiles; a gate_up group is 8 records, CPG chunks of 128 columns of the 2 NTT tiles; the slice's SL
// down columns are CH chunks of 32, and a down group is RGG row groups of 64 times those CH chunks.
template <int SL>
struct MxGeom {
    static constexpr int NTT = SL / 16;
    static constexpr int CPG = 4 / NTT;
    static constexpr int CH = SL / 32;
    static constexpr int RGG = 8 / CH;
};

// gate_up group ga: chunks q = CPG ga + qq, each the slice's NTT gate and NTT up tiles (entry 2 NTT qq + r).
template <int SL>
__device__ __forceinline__ void mx_issue_a(const DecArgs& a, const Item& it, int ga, int lane, MxRing& R) {
    using G = MxGeom<SL>;
    const int KQ = a.H / 128, NT = 2 * a.I / 16, up = a.I / 16;
#pragma unroll
    for (int qq = 0; qq < G::CPG; ++qq) {
        const int q = G::CPG * ga + qq;
#pragma unroll
        for (int r = 0; r < 2 * G::NTT; ++r) {
            const int rec = q * NT + (r < G::NTT ? 0 : up) + G::NTT * it.s + r % G::NTT;
            R.cd[2 * G::NTT * qq + r] = buf_load16(it.sres, q < KQ ? a.gu_codes + rec * kRecBytes + 16 * lane : kOob);
            R.sc[2 * G::NTT * qq + r] = __builtin_amdgcn_raw_buffer_load_b8(
                it.sres, q < KQ ? a.gu_scales + rec * 64 + lane : kOob, 0, 0);
        }
    }
}

// down group gb: records (chunk CH s + r % CH, row group RGG gb + r / CH), entry r.
template <int SL>
__device__ __forceinline__ void mx_issue_b(const DecArgs& a, const Item& it, int gb, int lane, MxRing& R) {
    using G = MxGeom<SL>;
    const int NG = a.H / 64;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const int p = G::RGG * gb + r / G::CH;
        const int rec = (G::CH * it.s + r % G::CH) * NG + p;
        R.cd[r] = buf_load16(it.sres, p < NG ? a.dn_codes + rec * kRecBytes + 16 * lane : kOob);
        R.sc[r] = buf_load4(it.sres, p < NG ? a.dn_scales + rec * 64 + 4 * (lane & 15) : kOob);
    }
}

// fp8 B operand (two 16-byte halves) and its E8M0 byte for chunk q of staged row `row`, lane (c, g).
__device__ __forceinline__ void mx_x_operand(const uint8_t* xs, int T, int NB, int row, int q, int g, v8i_t& bh,
                                             v8i_t& bl, int& sh, int& sl) {
    const uint8_t* p = xs + (size_t)row * 2 * kXB + 128 * q + 16 * g;
    const u32x4_t h0 = *reinterpret_cast<const u32x4_t*>(p), h1 = *reinterpret_cast<const u32x4_t*>(p + 64);
    const u32x4_t l0 = *reinterpret_cast<const u32x4_t*>(p + kXB), l1 = *reinterpret_cast<const u32x4_t*>(p + kXB + 64);
    bh = v8i_t{(int)h0.x, (int)h0.y, (int)h0.z, (int)h0.w, (int)h1.x, (int)h1.y, (int)h1.z, (int)h1.w};
    bl = v8i_t{(int)l0.x, (int)l0.y, (int)l0.z, (int)l0.w, (int)l1.x, (int)l1.y, (int)l1.z, (int)l1.w};
    const uint8_t* srow = xs + (size_t)(T + 1) * 2 * kXB;
    sh = srow[row * NB + 4 * q + g];
    sl = srow[(T + 1) * NB + row * NB + 4 * q + g];
}

template <int SL>
__device__ __forceinline__ void mx_compute_a(const DecArgs& a, const MxRing& R, int ga, const uint8_t* xs, int row,
                                             int g, f32x4_t (&acc)[2 * MxGeom<SL>::NTT]) {
    using G = MxGeom<SL>;
    const int KQ = a.H / 128, NB = a.H / 32;
#pragma unroll
    for (int qq = 0; qq < G::CPG; ++qq) {
        const int q = G::CPG * ga + qq;
        if (q >= KQ) continue;  // uniform: a padded chunk
        v8i_t bh, bl;
        int sh, sl;
        mx_x_operand(xs, a.T, NB, row, q, g, bh, bl, sh, sl);
#pragma unroll
        for (int r = 0; r < 2 * G::NTT; ++r) {
            const u32x4_t c = R.cd[2 * G::NTT * qq + r];
            const v8i_t A = v8i_t{(int)c.x, (int)c.y, (int)c.z, (int)c.w, 0, 0, 0, 0};
            const int sa = (int)R.sc[2 * G::NTT * qq + r];
            acc[r] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, bh, acc[r], 4, 0, 0, sa, 0, sh);
            acc[r] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, bl, acc[r], 4, 0, 0, sa, 0, sl);
        }
    }
}

// One down record's tile j (rows 16 j + i of the 64-row group, the slice's 32 columns [8g, 8g + 8) of lane
// (i, g)) decoded exactly to bf16 with its E8M0 scale (byte j of the lane's scale dword).
__device__ __forceinline__ bf16x8_t mx_down_frag(uint32_t code_word, uint32_t scale_dword, int j) {
    const float sc = e8m0_as_f32(scale_dword >> (8 * j));
    const bf16x2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(code_word, sc, 0);
    const bf16x2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(code_word, sc, 1);
    const bf16x2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(code_word, sc, 2);
    const bf16x2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(code_word, sc, 3);
    const u32x4_t u = {__builtin_bit_cast(uint32_t, v0), __builtin_bit_cast(uint32_t, v1),
                       __builtin_bit_cast(uint32_t, v2), __builtin_bit_cast(uint32_t, v3)};
    return __builtin_bit_cast(bf16x8_t, u);
}

// The group's row groups: each 16-row tile j summed over the slice's CH column chunks, then stored.
template <int SL>
__device__ __forceinline__ void mx_compute_b(const DecArgs& a, const MxRing& R, int gb,
                                             const bf16x8_t (&Bh)[MxGeom<SL>::CH], const bf16x8_t (&Bl)[MxGeom<SL>::CH],
                                             float wc, const rsrc_t& pres, int pbase) {
    using G = MxGeom<SL>;
    const int NG = a.H / 64;
#pragma unroll
    for (int rg = 0; rg < G::RGG; ++rg) {
        const int p = G::RGG * gb + rg;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f32x4_t D = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int cc = 0; cc < G::CH; ++cc) {
                const int r = G::CH * rg + cc;
                const bf16x8_t A = mx_down_frag(word_of(R.cd[r], j), R.sc[r], j);
                D = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Bh[cc], D, 0, 0, 0);
                D = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Bl[cc], D, 0, 0, 0);
            }
            buf_store16(pres, p < NG ? pbase + 4 * (64 * p + 16 * j) : kOob, D * wc);
        }
    }
}

// SwiGLU on this lane's rows 4g + [0, 4) of each tile (token c), then the down operand of each 32-column chunk
// cc (tiles 2 cc and 2 cc + 1): lane (c, g') needs chunk rows 8g' + [0, 8): tile g' / 2 of the pair, from lanes
// (c, 2 (g' & 1)) and (c, 2 (g' & 1) + 1)
template <int SL>
__device__ __forceinline__ void mx_swiglu(const f32x4_t (&acc)[2 * MxGeom<SL>::NTT], int c, int g,
                                          bf16x8_t (&Bh)[MxGeom<SL>::CH], bf16x8_t (&Bl)[MxGeom<SL>::CH]) {
    using G = MxGeom<SL>;
#pragma unroll
    for (int cc = 0; cc < G::CH; ++cc) {
        uint32_t PH[2][2], PL[2][2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int d = 0; d < 2; ++d) {
                const int gt = 2 * cc + tt;
                const float h0 = silu_fast(acc[gt][2 * d]) * acc[G::NTT + gt][2 * d];
                const float h1 = silu_fast(acc[gt][2 * d + 1]) * acc[G::NTT + gt][2 * d + 1];
                split_bf16x2(h0, h1, PH[tt][d], PL[tt][d]);
            }
        const int src0 = c + 32 * (g & 1), src1 = src0 + 16;
        const bool hi = g >= 2;
        uint32_t bh[4], bl[4];
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            const uint32_t h00 = (uint32_t)__shfl((int)PH[0][d], src0, kWave);
            const uint32_t h10 = (uint32_t)__shfl((int)PH[1][d], src0, kWave);
            const uint32_t h01 = (uint32_t)__shfl((int)PH[0][d], src1, kWave);
            const uint32_t h11 = (uint32_t)__shfl((int)PH[1][d], src1, kWave);
            const uint32_t l00 = (uint32_t)__shfl((int)PL[0][d], src0, kWave);
            const uint32_t l10 = (uint32_t)__shfl((int)PL[1][d], src0, kWave);
            const uint32_t l01 = (uint32_t)__shfl((int)PL[0][d], src1, kWave);
            const uint32_t l11 = (uint32_t)__shfl((int)PL[1][d], src1, kWave);
            bh[d] = hi ? h10 : h00;
            bh[2 + d] = hi ? h11 : h01;
            bl[d] = hi ? l10 : l00;
            bl[2 + d] = hi ? l11 : l01;
        }
        Bh[cc] = __builtin_bit_cast(bf16x8_t, u32x4_t{bh[0], bh[1], bh[2], bh[3]});
        Bl[cc] = __builtin_bit_cast(bf16x8_t, u32x4_t{bl[0], bl[1], bl[2], bl[3]});
    }
}

constexpr int kMU = 4;  // waves per workgroup that take items of their own under COOP: one per SIMD

// Spin on an LDS counter until it reaches target (every wave it waits for is in this workgroup and arrives).
__device__ __forceinline__ void mx_lds_wait_count(int* p, int target) {
    while (__hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < target) __builtin_amdgcn_s_sleep(1);
}

// Persistent over items v = wave * grid + block + j * 8 * grid.  MULTI: some wave has more than one item.
// ROUTE: the kernel routes the tokens itself in its prologue (from a.logits) and writes the routing outputs.
// SL: rows per item, 32, or 64 when 32-row items would outnumber the waves (half the items and partial sums).
// COOP (with !MULTI): only the first kMU waves of a workgroup take items of their own; each item past kMU per
// workgroup (a leftover) is run by the other kMU waves of one workgroup together, beside the first waves' items
// from the start: wave kMU + w streams the gate_up groups w, w + kMU, ... and the down groups w, w + kMU, ...,
// and the gate_up partial sums meet in LDS, added in wave order, before SwiGLU.  (A leftover run by one wave
// would share one SIMD with another item for the whole call.)
template <int SL, bool MULTI, bool ROUTE, bool COOP = false>
__global__ void __launch_bounds__(kMT) mx_wave_kernel(DecArgs a, int nsl) {
    using G = MxGeom<SL>;
    extern __shared__ __attribute__((aligned(16))) uint8_t xs[];
    __shared__ Tables tb;
    __shared__ f32x4_t coop_red[COOP ? kMU : 1][COOP ? 2 * G::NTT : 1][kWave];
    __shared__ int coop_cnt[2];  // partial sums written, partial sums read (counted per wave, never reset)
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int H = a.H, T = a.T, k = a.k;
    XRegs<kMW> xv;
    const int n_act = ROUTE ? stage_route<kMW>(a, tb, xv, tid, lane, wave, [] {})
                            : stage_tables<kMW>(a, tb, xv, tid, lane, wave);
    const int n_items = (n_act + (a.shared != nullptr ? 1 : 0)) * nsl;
    const int stride = (int)gridDim.x * kMW;
    int v = __builtin_amdgcn_readfirstlane(COOP && wave >= kMU ? n_items : wave * (int)gridDim.x + (int)blockIdx.x);
    if (COOP && tid < 2) coop_cnt[tid] = 0;
    const int c = lane & 15, g = lane >> 4;
    const int KQ = H / 128, NG = H / 64;
    const int NGA = (KQ + G::CPG - 1) / G::CPG;  // gate_up groups of CPG chunks
    const int NGB = (NG + G::RGG - 1) / G::RGG;  // down groups of RGG row groups
    const rsrc_t pres = make_rsrc(a.part, (uint32_t)((size_t)(T * k + T) * nsl * H * 4));

    Item cur = decode_item(a, tb, n_act, nsl, v, v < n_items, c);
    MxRing R0, R1;
    mx_issue_a<SL>(a, cur, 0, lane, R0);
    mx_issue_a<SL>(a, cur, 1, lane, R1);
    __builtin_amdgcn_sched_barrier(0);
    mx_stage_x(a, xv, xs, tid, lane, wave);
    __syncthreads();
    const bool coop_wave = COOP && wave >= kMU;  // runs leftover items, none of its own
    if (v >= n_items && !coop_wave) return;      // uniform per wave; no barrier follows
    if (v < n_items) do {
        const Item nxt = decode_item(a, tb, n_act, nsl, v + stride, MULTI && v + stride < n_items, c);
        const int row = cur.tok >= 0 ? cur.tok : T;

        // ---- gate_up on the scaled matrix cores: the slice's two gate and two up tiles over all of K
        f32x4_t acc[2 * G::NTT];
#pragma unroll
        for (int r = 0; r < 2 * G::NTT; ++r) acc[r] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        int ga = 0;
        for (; ga + 2 < NGA; ga += 2) {
            mx_compute_a<SL>(a, R0, ga, xs, row, g, acc);
            __builtin_amdgcn_sched_barrier(0);
            mx_issue_a<SL>(a, cur, ga + 2, lane, R0);
            __builtin_amdgcn_sched_barrier(0);
            mx_compute_a<SL>(a, R1, ga + 1, xs, row, g, acc);
            __builtin_amdgcn_sched_barrier(0);
            mx_issue_a<SL>(a, cur, ga + 3, lane, R1);
            __builtin_amdgcn_sched_barrier(0);
        }
        mx_compute_a<SL>(a, R0, ga, xs, row, g, acc);
        __builtin_amdgcn_sched_barrier(0);
        mx_issue_b<SL>(a, cur, 0, lane, R0);
        __builtin_amdgcn_sched_barrier(0);
        mx_compute_a<SL>(a, R1, ga + 1, xs, row, g, acc);
        __builtin_amdgcn_sched_barrier(0);
        mx_issue_b<SL>(a, cur, 1, lane, R1);
        __builtin_amdgcn_sched_barrier(0);

        bf16x8_t Bh[G::CH], Bl[G::CH];
        mx_swiglu<SL>(acc, c, g, Bh, Bl);

        // ---- down: the slice's SL columns of all H rows, partial sums times the routing weight
        const int pbase = c < cur.ne ? 4 * ((cur.prow * nsl + cur.s) * H + 4 * g) : kOob;
        int gb = 0;
        for (; gb + 2 < NGB; gb += 2) {
            mx_compute_b<SL>(a, R0, gb, Bh, Bl, cur.wc, pres, pbase);
            __builtin_amdgcn_sched_barrier(0);
            mx_issue_b<SL>(a, cur, gb + 2, lane, R0);
            __builtin_amdgcn_sched_barrier(0);
            mx_compute_b<SL>(a, R1, gb + 1, Bh, Bl, cur.wc, pres, pbase);
            __builtin_amdgcn_sched_barrier(0);
            mx_issue_b<SL>(a, cur, gb + 3, lane, R1);
            __builtin_amdgcn_sched_barrier(0);
        }
        mx_compute_b<SL>(a, R0, gb, Bh, Bl, cur.wc, pres, pbase);
        if (!MULTI) {
            mx_compute_b<SL>(a, R1, gb + 1, Bh, Bl, cur.wc, pres, pbase);
            break;
        }
        __builtin_amdgcn_sched_barrier(0);
        mx_issue_a<SL>(a, nxt, 0, lane, R0);
        __builtin_amdgcn_sched_barrier(0);
        mx_compute_b<SL>(a, R1, gb + 1, Bh, Bl, cur.wc, pres, pbase);
        __builtin_amdgcn_sched_barrier(0);
        mx_issue_a<SL>(a, nxt, 1, lane, R1);
        __builtin_amdgcn_sched_barrier(0);
        cur = nxt;
        v += stride;
    } while (v < n_items);

    if (coop_wave) {
        // leftover items kMU * grid + b + grid * r of workgroup b, run by its waves kMU .. 2 kMU - 1 together
        // (each takes part in every round, so all kMU of them arrive at every count below)
        const int cw = wave - kMU;
        const int grid = (int)gridDim.x;
        for (int r = 0;; ++r) {
            const int lv = kMU * grid + (int)blockIdx.x + grid * r;
            if (lv >= n_items) break;  // uniform over the workgroup's leftover waves
            const Item it = decode_item(a, tb, n_act, nsl, lv, true, c);
            const int row = it.tok >= 0 ? it.tok : T;
            f32x4_t acc[2 * G::NTT];
#pragma unroll
            for (int q = 0; q < 2 * G::NTT; ++q) acc[q] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            // gate_up groups cw, cw + kMU, ...: groups past NGA load zeros and their chunks are skipped
            int ga = cw;
            mx_issue_a<SL>(a, it, ga, lane, R0);
            mx_issue_a<SL>(a, it, ga + kMU, lane, R1);
            __builtin_amdgcn_sched_barrier(0);
            for (; ga + 2 * kMU < NGA; ga += 2 * kMU) {
                mx_compute_a<SL>(a, R0, ga, xs, row, g, acc);
                __builtin_amdgcn_sched_barrier(0);
                mx_issue_a<SL>(a, it, ga + 2 * kMU, lane, R0);
                __builtin_amdgcn_sched_barrier(0);
                mx_compute_a<SL>(a, R1, ga + kMU, xs, row, g, acc);
                __builtin_amdgcn_sched_barrier(0);
                mx_issue_a<SL>(a, it, ga + 3 * kMU, lane, R1);
                __builtin_amdgcn_sched_barrier(0);
            }
            mx_compute_a<SL>(a, R0, ga, xs, row, g, acc);
            __builtin_amdgcn_sched_barrier(0);
            mx_compute_a<SL>(a, R1, ga + kMU, xs, row, g, acc);
            __builtin_amdgcn_sched_barrier(0);
            // the kMU partial sums meet in LDS (the previous round's have all been read)
            mx_lds_wait_count(&coop_cnt[1], kMU * r);
#pragma unroll
            for (int q = 0; q < 2 * G::NTT; ++q) coop_red[cw][q][lane] = acc[q];
            if (lane == 0) __hip_atomic_fetch_add(&coop_cnt[0], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
            mx_lds_wait_count(&coop_cnt[0], kMU * (r + 1));
#pragma unroll
            for (int q = 0; q < 2 * G::NTT; ++q) {
                f32x4_t t = coop_red[0][q][lane];
#pragma unroll
                for (int w = 1; w < kMU; ++w) t += coop_red[w][q][lane];
                acc[q] = t;
                __builtin_amdgcn_sched_barrier(0);  // a tile at a time
            }
            if (lane == 0) __hip_atomic_fetch_add(&coop_cnt[1], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
            bf16x8_t Bh[G::CH], Bl[G::CH];
            mx_swiglu<SL>(acc, c, g, Bh, Bl);
            // down groups cw, cw + kMU, ...: groups past NGB load zeros and store nothing
            __builtin_amdgcn_sched_barrier(0);
            mx_issue_b<SL>(a, it, cw, lane, R0);
            mx_issue_b<SL>(a, it, cw + kMU, lane, R1);
            __builtin_amdgcn_sched_barrier(0);
            const int pbase = c < it.ne ? 4 * ((it.prow * nsl + it.s) * H + 4 * g) : kOob;
            int gb = cw;
            for (; gb + 2 * kMU < NGB; gb += 2 * kMU) {
                mx_compute_b<SL>(a, R0, gb, Bh, Bl, it.wc, pres, pbase);
                __builtin_amdgcn_sched_barrier(0);
                mx_issue_b<SL>(a, it, gb + 2 * kMU, lane, R0);
                __builtin_amdgcn_sched_barrier(0);
                mx_compute_b<SL>(a, R1, gb + kMU, Bh, Bl, it.wc, pres, pbase);
                __builtin_amdgcn_sched_barrier(0);
                mx_issue_b<SL>(a, it, gb + 3 * kMU, lane, R1);
                __builtin_amdgcn_sched_barrier(0);
            }
            mx_compute_b<SL>(a, R0, gb, Bh, Bl, it.wc, pres, pbase);
            __builtin_amdgcn_sched_barrier(0);
            mx_compute_b<SL>(a, R1, gb + kMU, Bh, Bl, it.wc, pres, pbase);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

// ------------------------------------------------------------------ dequant hooks

// Transposed checkpoint layout: one thread per byte (j, n) of blocks_t: out[n, 2j] and out[n, 2j + 1], decoded by
// the converter the down phase uses (fp4 -> bf16 with the E8M0 scale applied), widened to f32.
__global__ void __launch_bounds__(256) mx_dequant_t_kernel(const uint8_t* __restrict__ blocks_t,
                                                           const uint8_t* __restrict__ scales_t, int N, int K,
                                                           float* __restrict__ out) {
    const long q = (long)blockIdx.x * 256 + threadIdx.x;
    if (q >= (long)N * (K / 2)) return;
    const long j = q / N;
    const int n = (int)(q % N);
    const uint32_t code = blocks_t[q];
    const float sc = e8m0_as_f32(scales_t[(j / 16) * N + n]);
    const bf16x2_t v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(code, sc, 0);
    out[(size_t)n * K + 2 * j] = (float)v.x;
    out[(size_t)n * K + 2 * j + 1] = (float)v.y;
}

// A slot's gate_up through the scaled matrix cores (as the forward consumes it): record (q, t) times one-hot fp8
// columns, eight products per record give its 16 x 128 values.  down: the bf16 converter, as the forward.
__global__ void __launch_bounds__(64) mx_dequant_gu_kernel(const uint8_t* __restrict__ slot, int H, int I,
                                                           float* __restrict__ out, int gu_codes, int gu_scales) {
    const int rec = blockIdx.x, lane = threadIdx.x, i = lane & 15, g = lane >> 4;
    const int NT = 2 * I / 16, q = rec / NT, t = rec % NT;
    const u32x4_t cw = *reinterpret_cast<const u32x4_t*>(slot + gu_codes + (size_t)rec * kRecBytes + 16 * lane);
    const int sa = slot[gu_scales + (size_t)rec * 64 + lane];
    const v8i_t A = v8i_t{(int)cw.x, (int)cw.y, (int)cw.z, (int)cw.w, 0, 0, 0, 0};
    for (int m = 0; m < 8; ++m) {
        // B[k][col] = 1 where k = 16 m + col: in lane (col, g), half m / 4, when g == m % 4, byte col
        uint32_t w[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (g == m % 4) w[4 * (m / 4) + i / 4] = 0x38u << (8 * (i % 4));
        const v8i_t B = v8i_t{(int)w[0], (int)w[1], (int)w[2], (int)w[3], (int)w[4], (int)w[5], (int)w[6], (int)w[7]};
        const f32x4_t D = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, 4,
                                                                           0, 0, sa, 0, 127);
#pragma unroll
        for (int v = 0; v < 4; ++v)
            out[(size_t)(16 * t + 4 * g + v) * H + 128 * q + 16 * m + i] = D[v];
    }
}

__global__ void __launch_bounds__(256) mx_dequant_dn_kernel(const uint8_t* __restrict__ slot, int H, int I,
                                                            float* __restrict__ out, int dn_codes, int dn_scales) {
    const long lanes = (long)H * I / 32;
    const long q = (long)blockIdx.x * 256 + threadIdx.x;
    if (q >= lanes) return;
    const long rec = q / kWave;
    const int lane = (int)(q % kWave), i = lane & 15, g = lane >> 4;
    const int NG = H / 64, kc = (int)(rec / NG), p = (int)(rec % NG);
    const u32x4_t cw = *reinterpret_cast<const u32x4_t*>(slot + dn_codes + rec * kRecBytes + 16 * lane);
    const uint32_t sd = *reinterpret_cast<const uint32_t*>(slot + dn_scales + rec * 64 + 4 * i);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const bf16x8_t v = mx_down_frag(word_of(cw, j), sd, j);
        float* o = out + (size_t)(64 * p + 16 * j + i) * I + 32 * kc + 8 * g;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[e] = (float)v[e];
    }
}

// ------------------------------------------------------------------ one item per workgroup
// When the items fit the CUs one per workgroup (one token at top-8 and
// I = 640: 180 items), a wave per item leaves most of each CU idle, and one
// wave's loads in flight are too few to stream an item's ~120 KB in time.
// Then the eight waves of a workgroup share its item: wave w takes the
// 128-column gate_up chunks q = w + 8 i (all four tiles of the slice) and the
// 64-row down groups w + 8 i.  The gate_up partial sums meet in LDS and are
// added over the waves in a fixed order; every wave forms SwiGLU for exactly
// the down operand it needs (as the wave kernel does, from the summed tiles).
// A wave issues its gate_up loads first and one down group after each
// gate_up chunk, so it computes on the chunks that have arrived while the
// down records stream in.
constexpr int kMxQW = 3;  // most gate_up chunks per wave (H <= 2560: 20 chunks over 8 waves)
constexpr int kMxBW = 5;  // most down groups per wave (H <= 2560: 40 groups over 8 waves)

template <bool ROUTE>
__global__ void __launch_bounds__(kMT) mx_fused_kernel(DecArgs a, int nsl) {
    extern __shared__ __attribute__((aligned(16))) uint8_t xs[];
    __shared__ Tables tb;
    __shared__ f32x4_t red[kMW][4][kWave];  // gate_up partial sums of every wave
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int H = a.H, T = a.T, k = a.k;
    const int c = lane & 15, g = lane >> 4;
    const int KQ = H / 128, NG = H / 64, NB = H / 32;
    XRegs<kMW> xv;
    const int n_act = ROUTE ? stage_route<kMW>(a, tb, xv, tid, lane, wave, [] {})
                            : stage_tables<kMW>(a, tb, xv, tid, lane, wave);
    const int n_items = (n_act + (a.shared != nullptr ? 1 : 0)) * nsl;
    if ((int)blockIdx.x >= n_items) return;  // uniform
    const Item it = decode_item(a, tb, n_act, nsl, (int)blockIdx.x, true, c);

    // ---- gate_up loads of this wave's chunks: tiles 0, 1 (gate rows 32 s + 16 r), 2, 3 (the matching up rows)
    const int NTT = 2 * a.I / 16, up = a.I / 16;
    u32x4_t ac[kMxQW][4];
    uint32_t as[kMxQW][4];
#pragma unroll
    for (int i = 0; i < kMxQW; ++i) {
        const int q = wave + kMW * i;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int rec = q * NTT + (r < 2 ? 0 : up) + 2 * it.s + (r & 1);
            ac[i][r] = buf_load16(it.sres, q < KQ ? a.gu_codes + rec * kRecBytes + 16 * lane : kOob);
            as[i][r] = __builtin_amdgcn_raw_buffer_load_b8(it.sres, q < KQ ? a.gu_scales + rec * 64 + lane : kOob, 0, 0);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    mx_stage_x(a, xv, xs, tid, lane, wave);
    __syncthreads();

    // ---- gate_up on the scaled matrix cores; a down group is issued after each chunk
    const int row = it.tok >= 0 ? it.tok : T;
    u32x4_t bc[kMxBW];
    uint32_t bs[kMxBW];
    f32x4_t acc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    constexpr int NSTEP = kMxQW > kMxBW ? kMxQW : kMxBW;
#pragma unroll
    for (int i = 0; i < NSTEP; ++i) {
        const int q = wave + kMW * i;
        if (i < kMxQW && q < KQ) {  // uniform per wave
            v8i_t bh, bl;
            int sh, sl;
            mx_x_operand(xs, T, NB, row, q, g, bh, bl, sh, sl);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const u32x4_t cw = ac[i][r];
                const v8i_t A = v8i_t{(int)cw.x, (int)cw.y, (int)cw.z, (int)cw.w, 0, 0, 0, 0};
                const int sa = (int)as[i][r];
                acc[r] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, bh, acc[r], 4, 0, 0, sa, 0, sh);
                acc[r] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, bl, acc[r], 4, 0, 0, sa, 0, sl);
            }
        }
        if (i < kMxBW) {
            __builtin_amdgcn_sched_barrier(0);
            const int rg = wave + kMW * i;
            const int rec = it.s * NG + rg;
            bc[i] = buf_load16(it.sres, rg < NG ? a.dn_codes + rec * kRecBytes + 16 * lane : kOob);
            bs[i] = buf_load4(it.sres, rg < NG ? a.dn_scales + rec * 64 + 4 * (lane & 15) : kOob);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) red[wave][r][lane] = acc[r];
    __syncthreads();

    // ---- SwiGLU for this lane's down operand: lane (c, g) needs slice rows 8 g + [0, 8) of token c, i.e. rows
    // 8 (g & 1) + [0, 4) and + [4, 8) of tile g >> 1, held by lanes 32 (g & 1) + c and + 16 of each wave's sums
    bf16x8_t Bh, Bl;
    {
        const int tt = g >> 1, L0 = 32 * (g & 1) + c;
        f32x4_t gs0 = {0.0f, 0.0f, 0.0f, 0.0f}, gs1 = gs0, us0 = gs0, us1 = gs0;
#pragma unroll
        for (int w = 0; w < kMW; ++w) {
            gs0 += red[w][tt][L0];
            gs1 += red[w][tt][L0 + 16];
            us0 += red[w][2 + tt][L0];
            us1 += red[w][2 + tt][L0 + 16];
        }
        float h[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float gv = e < 4 ? gs0[e] : gs1[e - 4], uv = e < 4 ? us0[e] : us1[e - 4];
            h[e] = silu_fast(gv) * uv;
        }
        uint32_t bh[4], bl[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) split_bf16x2(h[2 * d], h[2 * d + 1], bh[d], bl[d]);
        Bh = __builtin_bit_cast(bf16x8_t, u32x4_t{bh[0], bh[1], bh[2], bh[3]});
        Bl = __builtin_bit_cast(bf16x8_t, u32x4_t{bl[0], bl[1], bl[2], bl[3]});
    }

    // ---- down: this wave's row groups of the slice's 32 columns, partial sums times the routing weight
    const rsrc_t pres = make_rsrc(a.part, (uint32_t)((size_t)(T * k + T) * nsl * H * 4));
    const int pbase = c < it.ne ? 4 * ((it.prow * nsl + it.s) * H + 4 * g) : kOob;
#pragma unroll
    for (int i = 0; i < kMxBW; ++i) {
        const int rg = wave + kMW * i;
        if (rg >= NG) break;  // uniform per wave
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const bf16x8_t A = mx_down_frag(word_of(bc[i], j), bs[i], j);
            f32x4_t D = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Bh, f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
            D = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, Bl, D, 0, 0, 0);
            buf_store16(pres, pbase + 4 * (64 * rg + 16 * j), D * it.wc);
        }
    }
}

hipError_t allow_mx_lds(const void* fn) {
    static std::mutex mu;
    static std::set<std::pair<const void*, int>> done;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(mu);
    if (done.count({fn, dev})) return hipSuccess;
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)mx_lds_bytes(kDecodeMaxT, 2560));
    if (e == hipSuccess) done.insert({fn, dev});
    return e;
}

hipError_t mx_device_cus(int& ncu) {
    static std::mutex mu;
    static std::map<int, int> cus;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(mu);
    auto it = cus.find(dev);
    if (it != cus.end()) {
        ncu = it->second;
        return hipSuccess;
    }
    e = hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
    if (e == hipSuccess) cus[dev] = ncu;
    return e;
}

}  // namespace

bool mx_decode_shape_supported(int H, int I) { return H % 128 == 0 && I % 32 == 0 && H <= 2560; }

namespace {
template <int SL, bool ROUTE>
hipError_t launch_mx_wave(const DecArgs& a, int items_max, int nsl, int grid, size_t lds, hipStream_t s) {
    hipError_t e;
    if ((e = allow_mx_lds(reinterpret_cast<const void*>(&mx_wave_kernel<SL, true, ROUTE>))) != hipSuccess) return e;
    if ((e = allow_mx_lds(reinterpret_cast<const void*>(&mx_wave_kernel<SL, false, ROUTE>))) != hipSuccess) return e;
    if ((e = allow_mx_lds(reinterpret_cast<const void*>(&mx_wave_kernel<SL, false, ROUTE, true>))) != hipSuccess)
        return e;
    if (items_max > grid * kMW)
        hipLaunchKernelGGL((mx_wave_kernel<SL, true, ROUTE>), dim3(grid), dim3(kMT), lds, s, a, nsl);
    else if (items_max > grid * kMU && items_max <= grid * (kMU + 2))  // a few leftovers: up to two rounds
        hipLaunchKernelGGL((mx_wave_kernel<SL, false, ROUTE, true>), dim3(grid), dim3(kMT), lds, s, a, nsl);
    else
        hipLaunchKernelGGL((mx_wave_kernel<SL, false, ROUTE>), dim3(grid), dim3(kMT), lds, s, a, nsl);
    return hipGetLastError();
}

// rows_max: most routed rows plus the shared expert's.  nsl (out): slices per expert of the items launched.
template <bool ROUTE>
hipError_t launch_mx_kernels(const DecArgs& a, int rows_max, int I, int& nsl, int ncu, size_t lds, hipStream_t s) {
    hipError_t e;
    nsl = I / 32;
    const int items_max = rows_max * nsl;
    if (items_max <= ncu) {  // one item per workgroup, shared by its waves
        if ((e = allow_mx_lds(reinterpret_cast<const void*>(&mx_fused_kernel<ROUTE>))) != hipSuccess) return e;
        hipLaunchKernelGGL(mx_fused_kernel<ROUTE>, dim3(items_max), dim3(kMT), lds, s, a, nsl);
        return hipGetLastError();
    }
    if (items_max > ncu * kMW && I % 64 == 0) {  // 32-row items would outnumber the waves: 64-row items
        nsl = I / 64;
        return launch_mx_wave<64, ROUTE>(a, rows_max * nsl, nsl, ncu, lds, s);
    }
    return launch_mx_wave<32, ROUTE>(a, items_max, nsl, ncu, lds, s);
}
}  // namespace

hipError_t launch_mx_decode(const Layer& L, const uint16_t* x, int T, const float* w, const int32_t* offsets,
                            const int32_t* sorted_assign, float* y, int accumulate, void* ws, hipStream_t s,
                            const RouteOut* route) {
    const int H = L.H, I = L.I, E = L.E, k = L.k;
    const WsLayout wl = ws_layout(T, H, I, E, k);
    DecArgs a{};
    a.bank = L.bank; a.slot_bytes = L.slot_bytes; a.num_slots = L.num_slots; a.slot_of_expert = L.slot_of_expert;
    a.shared = L.shared; a.wg = L.wg; a.x = x;
    a.T = T; a.H = H; a.I = I; a.E = E; a.k = k;
    a.w = w; a.offsets = offsets; a.sorted_assign = sorted_assign;
    a.part = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + wl.part);
    a.rowslot = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(ws) + wl.dg);
    a.dgrow = nullptr;
    a.n_spare = 0;
    a.y = y; a.accumulate = accumulate;
    const SlotGeom gm = mx_slot_geom(H, I);
    a.gu_codes = (int)gm.gu_codes; a.gu_scales = (int)gm.gu_scales; a.gu_glob = 0;
    a.dn_codes = (int)gm.dn_codes; a.dn_scales = (int)gm.dn_scales; a.dn_glob = 0;
    a.no_glob = 1;
    a.route_wg = 0;  // workgroup 0 writes the routing outputs when the kernels route
    a.logits = route ? route->logits : nullptr;
    a.r_ids = route ? route->ids : nullptr;
    a.r_w = route ? route->w : nullptr;
    a.r_offsets = route ? route->offsets : nullptr;
    a.r_sorted = route ? route->sorted_assign : nullptr;
    a.r_pos = route ? route->assign_pos : nullptr;
    int ncu = 0;
    hipError_t e = mx_device_cus(ncu);
    if (e != hipSuccess) return e;
    int nsl = 0;
    const int rows_max = (T * k < E ? T * k : E) + 1;
    const size_t lds = mx_lds_bytes(T, H);
    e = route ? launch_mx_kernels<true>(a, rows_max, I, nsl, ncu, lds, s)
              : launch_mx_kernels<false>(a, rows_max, I, nsl, ncu, lds, s);
    if (e != hipSuccess) return e;
    const int nch = H / 64;
    if (nsl <= 10) hipLaunchKernelGGL(dcombine_kernel<10>, dim3(T * nch), dim3(256), 0, s, a, nsl, nch);
    else if (nsl <= 20) hipLaunchKernelGGL(dcombine_kernel<20>, dim3(T * nch), dim3(256), 0, s, a, nsl, nch);
    else hipLaunchKernelGGL(dcombine_kernel<32>, dim3(T * nch), dim3(256), 0, s, a, nsl, nch);
    return hipGetLastError();
}

hipError_t launch_mx_dequant_t(const uint8_t* blocks_t, const uint8_t* scales_t, int N, int K, float* out,
                               hipStream_t s) {
    const long n = (long)N * (K / 2);
    hipLaunchKernelGGL(mx_dequant_t_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, blocks_t, scales_t, N,
                       K, out);
    return hipGetLastError();
}

hipError_t launch_mx_dequant_slot(const uint8_t* slot, int H, int I, int matrix, float* out, hipStream_t s) {
    const SlotGeom gm = mx_slot_geom(H, I);
    if (matrix == 0) {
        const int recs = (H / 128) * (2 * I / 16);
        hipLaunchKernelGGL(mx_dequant_gu_kernel, dim3(recs), dim3(64), 0, s, slot, H, I, out, (int)gm.gu_codes,
                           (int)gm.gu_scales);
    } else {
        const long lanes = (long)H * I / 32;
        hipLaunchKernelGGL(mx_dequant_dn_kernel, dim3((unsigned)((lanes + 255) / 256)), dim3(256), 0, s, slot, H, I,
                           out, (int)gm.dn_codes, (int)gm.dn_scales);
    }
    return hipGetLastError();
}

}  // namespace moe
