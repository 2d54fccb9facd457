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
// Both phases stream their weights with one 16-byte load per lane per record.
// The kernel is persistent (one workgroup per CU): while an item reduces,
// runs SwiGLU and its down phase, the next item's loads are already in
// flight.  A second kernel scales each row's slice sum by the expert's
// down-row globals and adds the rows of a token in a fixed order with the
// shared expert's sigmoid-gated term (PR #385 "What this adds": routed +
// sigmoid(gate) * shared before one reduction).
//
// Arithmetic: v_mfma_f32_16x16x32_f16 with the weights as the 16-row operand
// and up to 16 tokens as the 16 columns.  Weights decode exactly to fp16
// (frag_f16).  Activations enter as fp16 times a power of two per (wave,
// token) that puts the wave's largest magnitude in [2^14, 2^15), so the
// bf16 -> fp16 conversion is exact in the fp16 normal range; the scale is
// undone exactly on the fp32 result.  The hidden slice is rescaled the same
// way before phase B.  Accumulation is fp32 and every sum runs in a fixed
// order, so results are bit-reproducible.
#include <map>
#include <mutex>
#include <set>
#include <utility>

#include "decode_common.hpp"

namespace moe {
namespace {

// Per-lane loads of one item: phase A (gate/up records, their scales and the
// SwiGLU thread's two row globals) and phase B (down records and scales).
template <int KQW>
struct ALoads {
    u32x4_t ar[KQW][2];
    uint32_t asc[KQW][2];
    float glob;  // lane l < 32: gate global of slice row l; lane l >= 32: up global of slice row l - 32
};
template <int NRGW>
struct BLoads {
    u32x4_t br[NRGW];
    uint32_t bsc[NRGW];
};

// Phase A split: wave w takes the two gate tiles (w < 4) or the two up tiles
// (w >= 4) of the slice, over the 128-column steps kq = w % 4 + 4 i.
template <int KQW>
__device__ __forceinline__ void issue_a(const DecArgs& a, const Item& it, int wave, int lane, int tid,
                                        ALoads<KQW>& L) {
    const int H = a.H, I = a.I, KQ = H / 128, NT = 2 * I / 16;
    const int s = it.s;
    const int t0 = (wave >> 2) * (I / 16) + 2 * s;  // first of this wave's two tiles
    const int soff = lane_scale_off(lane);
#pragma unroll
    for (int i = 0; i < KQW; ++i) {
        const int kq = (wave & 3) + 4 * i;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
            const int rec = kq * NT + t0 + tt;
            L.ar[i][tt] = buf_load16(it.sres, kq < KQ ? a.gu_codes + rec * kRecBytes + 16 * lane : kOob);
            L.asc[i][tt] = buf_load4(it.sres, kq < KQ ? a.gu_scales + rec * kRecScaleBytes + soff : kOob);
        }
    }
    (void)tid;
    L.glob = __uint_as_float(buf_load4(it.sres, a.gu_glob + 4 * ((lane >> 5) * I + kSl * s + (lane & 31))));
}

// Phase B loads of row group wave + 8 i (one record and its scales).
template <int NRGW>
__device__ __forceinline__ void issue_b_one(const DecArgs& a, const Item& it, int wave, int lane, BLoads<NRGW>& L,
                                            int i) {
    const int NG = a.H / 64, soff = lane_scale_off(lane);
    const int rg = wave + kDW * i;
    const int rec = it.s * NG + rg;
    L.br[i] = buf_load16(it.sres, rg < NG ? a.dn_codes + rec * kRecBytes + 16 * lane : kOob);
    L.bsc[i] = buf_load4(it.sres, rg < NG ? a.dn_scales + rec * kRecScaleBytes + soff : kOob);
}

template <int NRGW>
__device__ __forceinline__ void issue_b(const DecArgs& a, const Item& it, int wave, int lane, BLoads<NRGW>& L) {
#pragma unroll
    for (int i = 0; i < NRGW; ++i) issue_b_one<NRGW>(a, it, wave, lane, L, i);
}

// Workgroup LDS besides the activations.
struct DecShared {
    f32x4_t red[2][kDW][2][kWave];  // phase A partial sums of every wave, double-buffered by item parity
    int xsh[kDecodeMaxT + 1];       // per-token activation exponent shift (row T: the zero row)
    Tables tb;
};

// One work item.  Consumes LA (phase A) and LB (phase B) of `cur`; with PF,
// refills LA with the loads of item na and, after phase B, LB with those of
// item nb (without PF, when no workgroup has a next item, nothing is
// prefetched: even out-of-range loads take the CU's address units).
// With ILB the caller has issued only the phase A loads: phase B's are issued
// one row group after each 128-column step of phase A.  A CU holds a limited
// number of loads in flight and a wave that issues past that limit stalls, so
// this keeps the waves computing phase A on the records that have arrived
// while the rest stream in.
template <int KQW, int NRGW, bool PF, bool ILB = false>
__device__ __forceinline__ void run_item(const DecArgs& a, DecShared& sh, const _Float16* x16, int XP, int nsl,
                                         const rsrc_t& pres, const Item& cur, ALoads<KQW>& LA, BLoads<NRGW>& LB,
                                         const Item& na, const Item& nb, int tid, int lane, int wave, int par) {
    const int H = a.H, T = a.T, k = a.k, KQ = H / 128, NG = H / 64;
    const int c = lane & 15, g = lane >> 4;
    const int xrow = cur.tok >= 0 ? cur.tok : T;  // this lane's activation row (T: zeros)
    const _Float16* xr = x16 + xrow * XP + 8 * g;

    // ---- phase A: this wave's two tiles of the slice over its share of K
    f32x4_t acc[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) acc[tt] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
    constexpr int NSTEP = KQW > NRGW ? KQW : NRGW;
#pragma unroll
    for (int i = 0; i < NSTEP; ++i) {
        const int kq = (wave & 3) + 4 * i;
        if (i < KQW && kq < KQ) {  // uniform per wave
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const f16x8_t X =
                    __builtin_bit_cast(f16x8_t, *reinterpret_cast<const u32x4_t*>(xr + 128 * kq + 32 * m));
#pragma unroll
                for (int tt = 0; tt < 2; ++tt) {
                    f16x2_t S;
                    if (m == 0) S = scale_f16x2<0>(LA.asc[i][tt]);
                    else if (m == 1) S = scale_f16x2<1>(LA.asc[i][tt]);
                    else if (m == 2) S = scale_f16x2<2>(LA.asc[i][tt]);
                    else S = scale_f16x2<3>(LA.asc[i][tt]);
                    const f16x8_t A = frag_f16(word_of(LA.ar[i][tt], m), S);
                    acc[tt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, X, acc[tt], 0, 0, 0);
                }
            }
        }
        if (ILB && i < NRGW) {
            __builtin_amdgcn_sched_barrier(0);
            issue_b_one<NRGW>(a, cur, wave, lane, LB, i);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    const float glob = LA.glob;
    // slice 0 records, per output row of the item, where the expert's down globals live
    if (cur.s == 0)
        for (int cc = tid; cc < cur.ne; cc += kDT)
            a.rowslot[cur.shared ? T * k + cc : sh.tb.sorted[cur.begin + cc]] = cur.slot_index;

    // ---- the registers of phase A are free: item na's phase A loads stream from here on
    if (PF) {
        __builtin_amdgcn_sched_barrier(0);
        issue_a<KQW>(a, na, wave, lane, tid, LA);
        __builtin_amdgcn_sched_barrier(0);
    }

    const float xinv = ldexpf(1.0f, -sh.xsh[xrow]);
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) sh.red[par][wave][tt][lane] = acc[tt] * xinv;
    __syncthreads();

    // ---- SwiGLU, computed by every wave for exactly the values its phase B
    // operand needs: lane (c, g) takes hidden rows 8g + [0, 8) of token c.
    // Gate sums come from waves 0-3 and up sums from waves 4-7, added in order.
    f16x8_t B;
    float oscale;
    {
        const int tt = g >> 1, L0 = 32 * (g & 1) + c;  // rows 8(g & 1) + [0,4) and + [4,8) of tile tt
        f32x4_t gs0 = {0.0f, 0.0f, 0.0f, 0.0f}, gs1 = gs0, us0 = gs0, us1 = gs0;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            gs0 += sh.red[par][w][tt][L0];
            gs1 += sh.red[par][w][tt][L0 + 16];
            us0 += sh.red[par][4 + w][tt][L0];
            us1 += sh.red[par][4 + w][tt][L0 + 16];
        }
        float h[8];
        float hm = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float gsum = e < 4 ? gs0[e] : gs1[e - 4], usum = e < 4 ? us0[e] : us1[e - 4];
            const float gv = gsum * __shfl(glob, 8 * g + e, kWave);
            const float uv = usum * __shfl(glob, 32 + 8 * g + e, kWave);
            h[e] = silu_fast(gv) * uv;
            hm = fmaxf(hm, fabsf(h[e]));
        }
        hm = fmaxf(hm, __shfl_xor(hm, 16, kWave));
        hm = fmaxf(hm, __shfl_xor(hm, 32, kWave));
        const int hsh = fp16_shift(hm);
        const float hsc = ldexpf(1.0f, hsh);
        uint32_t hw[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) {
            const f16x2_t q = {(_Float16)(h[2 * d] * hsc), (_Float16)(h[2 * d + 1] * hsc)};
            hw[d] = __builtin_bit_cast(uint32_t, q);
        }
        B = __builtin_bit_cast(f16x8_t, u32x4_t{hw[0], hw[1], hw[2], hw[3]});
        oscale = ldexpf(1.0f, -hsh) * cur.wc;
    }

    // ---- phase B: the slice's 32 down columns for this wave's row groups
    const int pbase = c < cur.ne ? 4 * ((cur.prow * nsl + cur.s) * H + 4 * g) : kOob;
#pragma unroll
    for (int i = 0; i < NRGW; ++i) {
        const int rg = wave + kDW * i;
        if (rg >= NG) break;  // uniform per wave
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f16x2_t S;
            if (j == 0) S = scale_f16x2<0>(LB.bsc[i]);
            else if (j == 1) S = scale_f16x2<1>(LB.bsc[i]);
            else if (j == 2) S = scale_f16x2<2>(LB.bsc[i]);
            else S = scale_f16x2<3>(LB.bsc[i]);
            const f16x8_t A = frag_f16(word_of(LB.br[i], j), S);
            const f32x4_t D = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, B, f32x4_t{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
            buf_store16(pres, pbase + 4 * (64 * rg + 16 * j), D * oscale);
        }
    }

    // ---- item nb's phase B loads
    if (PF) {
        __builtin_amdgcn_sched_barrier(0);
        issue_b<NRGW>(a, nb, wave, lane, LB);
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <int NW>
__device__ __forceinline__ void stage_x(const DecArgs& a, const XRegs<NW>& xr, int* xsh, _Float16* x16, int XP,
                                        int tid, int lane, int wave) {
    const int H = a.H, T = a.T;
#pragma unroll
    for (int p = 0; p < XRegs<NW>::XT; ++p) {
        const int t = wave + NW * p;
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < XRegs<NW>::XC; ++i)
#pragma unroll
            for (int d = 0; d < 4; ++d) {
                const uint32_t wv = word_of(xr.v[p][i], d);
                amax = fmaxf(amax, fmaxf(fabsf(__uint_as_float(wv << 16)), fabsf(__uint_as_float(wv & 0xFFFF0000u))));
            }
        amax = wave_max(amax);
        const int sh_t = fp16_shift(amax);
        const float sc = ldexpf(1.0f, sh_t);
        if (t < T) {
            if (lane == 0) xsh[t] = sh_t;
#pragma unroll
            for (int i = 0; i < XRegs<NW>::XC; ++i) {
                const int ch = lane + kWave * i;
                if (ch >= H / 8) continue;
                uint32_t hw[4];
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const uint32_t wv = word_of(xr.v[p][i], d);
                    const f16x2_t q = {(_Float16)(__uint_as_float(wv << 16) * sc),
                                       (_Float16)(__uint_as_float(wv & 0xFFFF0000u) * sc)};
                    hw[d] = __builtin_bit_cast(uint32_t, q);
                }
                *reinterpret_cast<u32x4_t*>(x16 + t * XP + 8 * ch) = u32x4_t{hw[0], hw[1], hw[2], hw[3]};
            }
        }
    }
    for (int ch = tid; ch < XP / 8; ch += NW * kWave)  // the zero row
        *reinterpret_cast<u32x4_t*>(x16 + T * XP + 8 * ch) = u32x4_t{0, 0, 0, 0};
    if (tid == 0) xsh[T] = 0;
}

// Spare workgroups (launched past the items when CUs are free) copy the
// down-row globals of every output row into dgrow, so the combine reads them
// at its start instead of first reading the row's slot.  Row p in sorted
// order: p < T*k is assignment sorted[p] of the last active expert whose
// group starts at or before p; p >= T*k is shared row p.  Each spare
// workgroup takes rows j, j + n_spare, ... in batches of 8, every load of a
// batch issued before its stores.
constexpr int kDgBatch = 8;
__device__ void copy_down_globals(const DecArgs& a, const Tables& tb, int n_act, int j, int n_spare, int tid) {
    const int T = a.T, k = a.k, n = T * k, rows = n + T, H4 = a.H / 4;
    const rsrc_t dres = make_rsrc(a.dgrow, (uint32_t)((size_t)rows * a.H * 4));
    for (int p0 = j; p0 < rows; p0 += kDgBatch * n_spare) {
        f32x4_t v[kDgBatch][2];
        int row[kDgBatch];
#pragma unroll
        for (int b = 0; b < kDgBatch; ++b) {
            const int p = p0 + b * n_spare;
            rsrc_t res = make_rsrc(a.bank, 0u);
            row[b] = -1;
            if (p < n) {
                int lo = 0, hi = n_act - 1;
                while (lo < hi) {
                    const int mid = (lo + hi + 1) / 2;
                    if (tb.off[tb.act[mid]] <= p) lo = mid; else hi = mid - 1;
                }
                const int sl = tb.slot[tb.act[lo]];
                row[b] = tb.sorted[p];
                if (sl >= 0) res = make_rsrc(a.bank + (size_t)sl * a.slot_bytes, (uint32_t)a.slot_bytes);
            } else if (p < rows) {
                row[b] = p;
                if (a.shared != nullptr) res = make_rsrc(a.shared, (uint32_t)a.slot_bytes);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int c4 = tid + kDT * i;
                v[b][i] = __builtin_bit_cast(f32x4_t, buf_load16(res, c4 < H4 ? a.dn_glob + 16 * c4 : kOob));
            }
        }
#pragma unroll
        for (int b = 0; b < kDgBatch; ++b)
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                const int c4 = tid + kDT * i;
                buf_store16(dres, row[b] >= 0 && c4 < H4 ? 16 * (row[b] * H4 + c4) : kOob, v[b][i]);
            }
    }
}

// Persistent over work items u = blockIdx.x + j * gridDim.x; item u is
// (the shared expert for u < nsl, else expert act[u / nsl - 1]; slice u % nsl).  Every token's
// activations are staged in LDS once, as fp16 times a per-token power of two.
// Phase A loads run two items ahead and phase B loads one item ahead, so the
// next items stream while this one reduces, runs SwiGLU and finishes.
// KQW: most 128-column steps of K = H per wave (steps wave % 4 + 4 i);
// NRGW: most 64-row down groups per wave (groups wave + 8 i).
// MULTI: a workgroup may have several items (items beyond the grid); otherwise each has at most one.
template <int KQW, int NRGW, bool ROUTE, bool MULTI>
__global__ void __launch_bounds__(kDT) fused_kernel(DecArgs a, int nsl) {
    extern __shared__ __attribute__((aligned(16))) _Float16 x16[];  // (T + 1) rows of XP halves; row T is zero
    __shared__ DecShared sh;

    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int H = a.H, T = a.T, k = a.k;
    const int XP = H + 8;  // padded row: rows of different tokens start 16 bytes apart modulo the LDS banks
    Tables& tb = sh.tb;

    XRegs<kDW> xv;
    const int G = (int)gridDim.x, c = lane & 15;
    ALoads<KQW> LA0, LA1;
    BLoads<NRGW> LB;
    Item it0;
    // a workgroup whose one item is the shared expert's (items 0 .. nsl-1) needs no routing for it: its weights
    // start streaming before the kernel routes
    const bool early = ROUTE && !MULTI && a.shared != nullptr && (int)blockIdx.x < nsl;  // uniform
    const auto start_early = [&]() {
        if (early) {
            it0 = decode_item(a, tb, 0, nsl, blockIdx.x, true, c);
            issue_a<KQW>(a, it0, wave, lane, tid, LA0);
        }
    };
    const int n_act = ROUTE ? stage_route<kDW>(a, tb, xv, tid, lane, wave, start_early)
                            : stage_tables<kDW>(a, tb, xv, tid, lane, wave);
    const int n_items = (n_act + (a.shared != nullptr ? 1 : 0)) * nsl;
    int u = blockIdx.x;
    if (u >= n_items) {  // uniform: a workgroup without items; spare ones copy the down-row globals
        if (a.dgrow != nullptr && u >= (int)gridDim.x - a.n_spare)
            copy_down_globals(a, tb, n_act, u - ((int)gridDim.x - a.n_spare), a.n_spare, tid);
        return;
    }

    // ---- the first items' weights start streaming, then the activations go to LDS
    const rsrc_t pres = make_rsrc(a.part, (uint32_t)((size_t)(T * k + T) * nsl * H * 4));
    // the first item's loads, the activations to LDS, then the second item's loads (issuing loads is paced
    // by the CU's address units, so loads the first item does not need would delay the staging)
    // (a workgroup with one item issues phase B's loads during phase A).  With one item the activations go to
    // LDS first: they arrived with the routing, and a workgroup that started early has slack to wait for them.
    if (!MULTI) stage_x<kDW>(a, xv, sh.xsh, x16, XP, tid, lane, wave);
    if (!early) {
        it0 = decode_item(a, tb, n_act, nsl, u, true, c);
        issue_a<KQW>(a, it0, wave, lane, tid, LA0);
        if (MULTI) issue_b<NRGW>(a, it0, wave, lane, LB);
        __builtin_amdgcn_sched_barrier(0);
    }
    if (MULTI) stage_x<kDW>(a, xv, sh.xsh, x16, XP, tid, lane, wave);
    __syncthreads();
    if (!MULTI) {
        run_item<KQW, NRGW, false, true>(a, sh, x16, XP, nsl, pres, it0, LA0, LB, it0, it0, tid, lane, wave, 0);
        return;
    }
    Item it1 = decode_item(a, tb, n_act, nsl, u + G, u + G < n_items, c);
    issue_a<KQW>(a, it1, wave, lane, tid, LA1);
    __builtin_amdgcn_sched_barrier(0);

    for (;;) {
        const Item it2 = decode_item(a, tb, n_act, nsl, u + 2 * G, u + 2 * G < n_items, c);
        run_item<KQW, NRGW, true>(a, sh, x16, XP, nsl, pres, it0, LA0, LB, it2, it1, tid, lane, wave, 0);
        if (u + G >= n_items) break;
        const Item it3 = decode_item(a, tb, n_act, nsl, u + 3 * G, u + 3 * G < n_items, c);
        run_item<KQW, NRGW, true>(a, sh, x16, XP, nsl, pres, it1, LA1, LB, it3, it2, tid, lane, wave, 1);
        if (u + 2 * G >= n_items) break;
        u += 2 * G;
        it0 = it2;
        it1 = it3;
    }
}

// ------------------------------------------------------------------ wave-item kernel
// For batches with many active experts the items outnumber the workgroups
// several times over, and the per-item barrier of the fused kernel leaves
// each CU waiting on its slowest wave.  Here each wave runs whole items on
// its own (same items, same partial outputs, same combine): phase A
// accumulates the slice's four tiles over all of K in registers, SwiGLU is
// wave-local, phase B follows, and no barrier is taken after the prologue.
// A wave streams its item as groups of records through a two-slot register
// ring (one group in flight while the other is consumed; a third slot
// measured slower): a gate_up group is two 128-column steps of the four
// tiles, a down group four 64-row record groups of the slice's 32 columns.
// The last groups of an item prefetch the first groups of the wave's next
// item.  Group counts are padded to even numbers with zero records (reads
// past the slot return zeros, stores past the partials are dropped, padded
// K steps are skipped).
constexpr int kWW = 8;             // waves per workgroup
constexpr int kWT = kWW * kWave;   // threads per workgroup
constexpr int kWU = 4;             // waves per workgroup that take items of their own under COOP: one per SIMD
#ifndef MOE_WAVE_MIN_ITEMS
#define MOE_WAVE_MIN_ITEMS 600     // work items from which decode runs the wave-item kernel (about T >= 4)
#endif

struct WaveShared {
    int xsh[kDecodeMaxT + 1];
    Tables tb;
};

struct Ring8 {
    u32x4_t cd[8];
    uint32_t sc[8];
};

__device__ __forceinline__ f16x2_t scale_of(uint32_t sdw, int m) {
    return m == 0 ? scale_f16x2<0>(sdw) : (m == 1 ? scale_f16x2<1>(sdw) : (m == 2 ? scale_f16x2<2>(sdw) : scale_f16x2<3>(sdw)));
}

// SL: intermediate rows per item (32 or 64).  A slice has NTT = SL/16 gate
// tiles (rows SL*s + [0, SL)) and the NTT matching up tiles; a gate_up group
// is 8 records: 8/(2 NTT) steps of the 2 NTT tiles.  A down group is 4 row
// groups p of the slice's SL/32 column chunks.
template <int SL>
struct WaveGeom {
    static constexpr int NTT = SL / 16;           // gate (and up) tiles per slice
    static constexpr int SPG = 8 / (2 * NTT);     // 128-column steps per gate_up group
    static constexpr int NB = SL / 32;            // 32-column chunks (phase B operands) per slice
};

template <int SL>
__device__ __forceinline__ void wv_issue_a(const DecArgs& a, const Item& it, int ga, int lane, Ring8& R) {
    using W = WaveGeom<SL>;
    const int KQ = a.H / 128, NT = 2 * a.I / 16, up = a.I / 16, soff = lane_scale_off(lane);
#pragma unroll
    for (int qq = 0; qq < W::SPG; ++qq) {
        const int q = W::SPG * ga + qq;
#pragma unroll
        for (int r = 0; r < 2 * W::NTT; ++r) {
            const int rec = q * NT + (r < W::NTT ? 0 : up) + W::NTT * it.s + r % W::NTT;
            R.cd[2 * W::NTT * qq + r] = buf_load16(it.sres, q < KQ ? a.gu_codes + rec * kRecBytes + 16 * lane : kOob);
            R.sc[2 * W::NTT * qq + r] = buf_load4(it.sres, q < KQ ? a.gu_scales + rec * kRecScaleBytes + soff : kOob);
        }
    }
}

// down group gb: records (column chunk NB s + f, row group 4 gb + r) in entry NB r + f.
template <int SL>
__device__ __forceinline__ void wv_issue_b(const DecArgs& a, const Item& it, int gb, int lane, Ring8& R) {
    using W = WaveGeom<SL>;
    const int NG = a.H / 64, soff = lane_scale_off(lane);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int p = 4 * gb + r;
#pragma unroll
        for (int f = 0; f < W::NB; ++f) {
            const int rec = (W::NB * it.s + f) * NG + p;
            R.cd[W::NB * r + f] = buf_load16(it.sres, p < NG ? a.dn_codes + rec * kRecBytes + 16 * lane : kOob);
            R.sc[W::NB * r + f] = buf_load4(it.sres, p < NG ? a.dn_scales + rec * kRecScaleBytes + soff : kOob);
        }
    }
}

// Row globals of this lane's accumulator rows 4g + [0, 4) of the slice's gate and up tiles.
template <int SL>
__device__ __forceinline__ void wv_issue_glob(const DecArgs& a, const Item& it, int lane,
                                              f32x4_t (&gl)[2 * WaveGeom<SL>::NTT]) {
    using W = WaveGeom<SL>;
    const int g = lane >> 4;
#pragma unroll
    for (int r = 0; r < 2 * W::NTT; ++r) {
        const int row = (r < W::NTT ? 0 : a.I) + SL * it.s + 16 * (r % W::NTT) + 4 * g;
        gl[r] = __builtin_bit_cast(f32x4_t, buf_load16(it.sres, a.gu_glob + 4 * row));
    }
}

template <int SL>
__device__ __forceinline__ void wv_compute_a(const DecArgs& a, const Ring8& R, int ga, const _Float16* xr,
                                             f32x4_t (&acc)[2 * WaveGeom<SL>::NTT]) {
    using W = WaveGeom<SL>;
    const int KQ = a.H / 128;
#pragma unroll
    for (int qq = 0; qq < W::SPG; ++qq) {
        const int q = W::SPG * ga + qq;
        if (q >= KQ) continue;  // uniform: a padded step (its activations would lie past the row)
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            const f16x8_t X = __builtin_bit_cast(f16x8_t, *reinterpret_cast<const u32x4_t*>(xr + 128 * q + 32 * m));
#pragma unroll
            for (int r = 0; r < 2 * W::NTT; ++r) {
                const int e = 2 * W::NTT * qq + r;
                const f16x8_t A = frag_f16(word_of(R.cd[e], m), scale_of(R.sc[e], m));
                acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, X, acc[r], 0, 0, 0);
            }
        }
    }
}

template <int SL>
__device__ __forceinline__ void wv_compute_b(const DecArgs& a, const Ring8& R, int gb,
                                             const f16x8_t (&B)[WaveGeom<SL>::NB], float oscale, const rsrc_t& pres,
                                             int pbase) {
    using W = WaveGeom<SL>;
    const int NG = a.H / 64;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        const int p = 4 * gb + r;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            f32x4_t D = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int f = 0; f < W::NB; ++f) {
                const int e = W::NB * r + f;
                D = __builtin_amdgcn_mfma_f32_16x16x32_f16(frag_f16(word_of(R.cd[e], j), scale_of(R.sc[e], j)), B[f],
                                                           D, 0, 0, 0);
            }
            buf_store16(pres, p < NG ? pbase + 4 * (64 * p + 16 * j) : kOob, D * oscale);
        }
    }
}

// SwiGLU on this lane's rows 4g + [0, 4) of each gate/up tile pair (acc: the slice's gate and up tiles over all
// of K), then the phase B operands: operand f of lane (c, g') holds slice rows 32f + 8g' + [0, 8) of token c,
// taken from lanes (c, 2(g' & 1)) and (c, 2(g' & 1) + 1) of tile 2f + (g' >> 1).  The hidden values go to fp16
// times a power of two that puts the wave's largest one in [2^14, 2^15); oscale undoes it (times the column
// weight wc) on the down result.
template <int SL>
__device__ __forceinline__ void wv_swiglu(const f32x4_t (&acc)[2 * WaveGeom<SL>::NTT],
                                          const f32x4_t (&gl)[2 * WaveGeom<SL>::NTT], float xinv, float wc, int c,
                                          int g, f16x8_t (&B)[WaveGeom<SL>::NB], float& oscale) {
    using W = WaveGeom<SL>;
    float h[W::NTT][4];
    float hm = 0.0f;
#pragma unroll
    for (int tt = 0; tt < W::NTT; ++tt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const float gv = acc[tt][r] * xinv * gl[tt][r];
            const float uv = acc[W::NTT + tt][r] * xinv * gl[W::NTT + tt][r];
            h[tt][r] = silu_fast(gv) * uv;
            hm = fmaxf(hm, fabsf(h[tt][r]));
        }
    hm = fmaxf(hm, __shfl_xor(hm, 16, kWave));
    hm = fmaxf(hm, __shfl_xor(hm, 32, kWave));
    const int hsh = fp16_shift(hm);
    const float hsc = ldexpf(1.0f, hsh);
    uint32_t P[W::NTT][2];
#pragma unroll
    for (int tt = 0; tt < W::NTT; ++tt)
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            const f16x2_t q = {(_Float16)(h[tt][2 * d] * hsc), (_Float16)(h[tt][2 * d + 1] * hsc)};
            P[tt][d] = __builtin_bit_cast(uint32_t, q);
        }
    const int src0 = c + 32 * (g & 1), src1 = src0 + 16;
    const bool hi = g >= 2;
#pragma unroll
    for (int f = 0; f < W::NB; ++f) {
        uint32_t bw[4];
#pragma unroll
        for (int d = 0; d < 2; ++d) {
            const uint32_t a0 = (uint32_t)__shfl((int)P[2 * f][d], src0, kWave);
            const uint32_t a1 = (uint32_t)__shfl((int)P[2 * f + 1][d], src0, kWave);
            const uint32_t b0 = (uint32_t)__shfl((int)P[2 * f][d], src1, kWave);
            const uint32_t b1 = (uint32_t)__shfl((int)P[2 * f + 1][d], src1, kWave);
            bw[d] = hi ? a1 : a0;
            bw[2 + d] = hi ? b1 : b0;
        }
        B[f] = __builtin_bit_cast(f16x8_t, u32x4_t{bw[0], bw[1], bw[2], bw[3]});
    }
    oscale = ldexpf(1.0f, -hsh) * wc;
}

// Waits until the LDS counter *p reaches target (the waves that raise it never wait on this one).
__device__ __forceinline__ void lds_wait_count(int* p, int target) {
    while (__hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) < target) __builtin_amdgcn_s_sleep(1);
}

// MULTI: a wave may have several items (more items than waves); otherwise each wave has at most one and
// nothing of a next item is prefetched (even out-of-range loads take the CU's address units).
// COOP (with !MULTI): only the first kWU waves of a workgroup (one per SIMD) take items of their own; the
// items past kWU per workgroup (leftovers) are each run by the other kWU waves of one workgroup together,
// beside the first waves' items from the start: wave kWU + w streams the gate_up groups w, w + kWU, ... and the
// down groups w, w + kWU, ..., and the gate_up partial sums meet in LDS, added in wave order, before SwiGLU.
// One wave running a leftover beside an item would share one SIMD's VALU (the fp4 decode) for the whole call
// with one wave's loads in flight; split over kWU waves it spreads over the four SIMDs.
template <int SL, bool ROUTE, bool MULTI, bool COOP = false>
__global__ void __launch_bounds__(kWT) wave_kernel(DecArgs a, int nsl) {
    using W = WaveGeom<SL>;
    extern __shared__ __attribute__((aligned(16))) _Float16 x16[];  // (T + 1) rows of XP halves; row T is zero
    __shared__ WaveShared sh;
    __shared__ f32x4_t coop_red[COOP ? kWU : 1][COOP ? 2 * W::NTT : 1][kWave];
    __shared__ int coop_cnt[2];  // partial sums written, partial sums read (counted per wave, never reset)

    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int H = a.H, T = a.T, k = a.k;
    const int XP = H + 8;
    XRegs<kWW> xv;
    const int n_act = ROUTE ? stage_route<kWW>(a, sh.tb, xv, tid, lane, wave, [] {})
                            : stage_tables<kWW>(a, sh.tb, xv, tid, lane, wave);
    const int n_items = (n_act + (a.shared != nullptr ? 1 : 0)) * nsl;
    const int stride = (int)gridDim.x * kWW;
    // consecutive items go to different CUs; readfirstlane tells the compiler the item is wave-uniform
    int v = __builtin_amdgcn_readfirstlane(COOP && wave >= kWU ? n_items : wave * (int)gridDim.x + (int)blockIdx.x);
    if (COOP && tid < 2) coop_cnt[tid] = 0;

    const int c = lane & 15, g = lane >> 4;
    const int KQ = H / 128, NG = H / 64;
    const int NGA = 2 * ((KQ + 2 * W::SPG - 1) / (2 * W::SPG));  // gate_up groups, an even number
    const int NGB = 2 * ((NG + 7) / 8);                          // down groups, an even number
    const rsrc_t pres = make_rsrc(a.part, (uint32_t)((size_t)(T * k + T) * nsl * H * 4));
    const rsrc_t rres = make_rsrc(a.rowslot, (uint32_t)(T * k + T) * 4);

    // the first item's weights start streaming (a wave without items loads nothing), then the activations go
    // to LDS; after the barrier a wave without items leaves
    Item cur = decode_item(a, sh.tb, n_act, nsl, v, v < n_items, c);
    Ring8 R0, R1;
    f32x4_t gl[2 * W::NTT];
    wv_issue_glob<SL>(a, cur, lane, gl);
    wv_issue_a<SL>(a, cur, 0, lane, R0);
    wv_issue_a<SL>(a, cur, 1, lane, R1);
    __builtin_amdgcn_sched_barrier(0);
    stage_x<kWW>(a, xv, sh.xsh, x16, XP, tid, lane, wave);
    __syncthreads();
    const bool coop_wave = COOP && wave >= kWU;  // runs leftover items, none of its own
    if (v >= n_items && !coop_wave) return;      // uniform per wave; no barrier follows
    if (v < n_items) do {
        const Item nxt = decode_item(a, sh.tb, n_act, nsl, v + stride, MULTI && v + stride < n_items, c);
        const int xrow = cur.tok >= 0 ? cur.tok : T;
        const _Float16* xr = x16 + xrow * XP + 8 * g;

        // ---- phase A: the slice's gate and up tiles over all of K
        f32x4_t acc[2 * W::NTT];
#pragma unroll
        for (int r = 0; r < 2 * W::NTT; ++r) acc[r] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        int ga = 0;
        for (; ga + 2 < NGA; ga += 2) {
            wv_compute_a<SL>(a, R0, ga, xr, acc);
            __builtin_amdgcn_sched_barrier(0);
            wv_issue_a<SL>(a, cur, ga + 2, lane, R0);
            __builtin_amdgcn_sched_barrier(0);
            wv_compute_a<SL>(a, R1, ga + 1, xr, acc);
            __builtin_amdgcn_sched_barrier(0);
            wv_issue_a<SL>(a, cur, ga + 3, lane, R1);
            __builtin_amdgcn_sched_barrier(0);
        }
        wv_compute_a<SL>(a, R0, ga, xr, acc);
        __builtin_amdgcn_sched_barrier(0);
        wv_issue_b<SL>(a, cur, 0, lane, R0);
        __builtin_amdgcn_sched_barrier(0);
        wv_compute_a<SL>(a, R1, ga + 1, xr, acc);
        __builtin_amdgcn_sched_barrier(0);
        wv_issue_b<SL>(a, cur, 1, lane, R1);
        __builtin_amdgcn_sched_barrier(0);

        // ---- SwiGLU, then the phase B operands
        f16x8_t B[W::NB];
        float oscale;
        wv_swiglu<SL>(acc, gl, ldexpf(1.0f, -sh.xsh[xrow]), cur.wc, c, g, B, oscale);
        // slice 0 records, per output row of the item, where the expert's down globals live
        __builtin_amdgcn_raw_buffer_store_b32((uint32_t)cur.slot_index, rres,
                                              cur.s == 0 && g == 0 && c < cur.ne ? 4 * cur.prow : kOob, 0, 0);

        // ---- phase B: the slice's SL down columns for all H outputs
        const int pbase = c < cur.ne ? 4 * ((cur.prow * nsl + cur.s) * H + 4 * g) : kOob;
        int gb = 0;
        for (; gb + 2 < NGB; gb += 2) {
            wv_compute_b<SL>(a, R0, gb, B, oscale, pres, pbase);
            __builtin_amdgcn_sched_barrier(0);
            wv_issue_b<SL>(a, cur, gb + 2, lane, R0);
            __builtin_amdgcn_sched_barrier(0);
            wv_compute_b<SL>(a, R1, gb + 1, B, oscale, pres, pbase);
            __builtin_amdgcn_sched_barrier(0);
            wv_issue_b<SL>(a, cur, gb + 3, lane, R1);
            __builtin_amdgcn_sched_barrier(0);
        }
        // ---- the next item's first groups start streaming
        wv_compute_b<SL>(a, R0, gb, B, oscale, pres, pbase);
        if (!MULTI) {
            wv_compute_b<SL>(a, R1, gb + 1, B, oscale, pres, pbase);
            break;
        }
        __builtin_amdgcn_sched_barrier(0);
        wv_issue_glob<SL>(a, nxt, lane, gl);
        wv_issue_a<SL>(a, nxt, 0, lane, R0);
        __builtin_amdgcn_sched_barrier(0);
        wv_compute_b<SL>(a, R1, gb + 1, B, oscale, pres, pbase);
        __builtin_amdgcn_sched_barrier(0);
        wv_issue_a<SL>(a, nxt, 1, lane, R1);
        __builtin_amdgcn_sched_barrier(0);
        cur = nxt;
        v += stride;
    } while (v < n_items);

    if (coop_wave) {
        // leftover items kWU * grid + b + grid * r of workgroup b, run by its waves kWU .. 2 kWU - 1 together
        // (each takes part in every round, so all kWU of them arrive at every count below)
        const int cw = wave - kWU;
        const int grid = (int)gridDim.x;
        for (int r = 0;; ++r) {
            const int lv = kWU * grid + (int)blockIdx.x + grid * r;
            if (lv >= n_items) break;  // uniform over the workgroup's leftover waves
            const Item it = decode_item(a, sh.tb, n_act, nsl, lv, true, c);
            const int xrow = it.tok >= 0 ? it.tok : T;
            const _Float16* xr = x16 + xrow * XP + 8 * g;
            f32x4_t acc[2 * W::NTT];
#pragma unroll
            for (int q = 0; q < 2 * W::NTT; ++q) acc[q] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
            wv_issue_glob<SL>(a, it, lane, gl);
            // gate_up groups cw, cw + kWU, ...: groups past NGA load zeros and their steps are skipped
            int ga = cw;
            wv_issue_a<SL>(a, it, ga, lane, R0);
            wv_issue_a<SL>(a, it, ga + kWU, lane, R1);
            __builtin_amdgcn_sched_barrier(0);
            for (; ga + 2 * kWU < NGA; ga += 2 * kWU) {
                wv_compute_a<SL>(a, R0, ga, xr, acc);
                __builtin_amdgcn_sched_barrier(0);
                wv_issue_a<SL>(a, it, ga + 2 * kWU, lane, R0);
                __builtin_amdgcn_sched_barrier(0);
                wv_compute_a<SL>(a, R1, ga + kWU, xr, acc);
                __builtin_amdgcn_sched_barrier(0);
                wv_issue_a<SL>(a, it, ga + 3 * kWU, lane, R1);
                __builtin_amdgcn_sched_barrier(0);
            }
            wv_compute_a<SL>(a, R0, ga, xr, acc);
            __builtin_amdgcn_sched_barrier(0);
            wv_compute_a<SL>(a, R1, ga + kWU, xr, acc);
            __builtin_amdgcn_sched_barrier(0);
            // the kWU partial sums meet in LDS (the previous round's have all been read)
            lds_wait_count(&coop_cnt[1], kWU * r);
#pragma unroll
            for (int q = 0; q < 2 * W::NTT; ++q) coop_red[cw][q][lane] = acc[q];
            if (lane == 0) __hip_atomic_fetch_add(&coop_cnt[0], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
            lds_wait_count(&coop_cnt[0], kWU * (r + 1));
#pragma unroll
            for (int q = 0; q < 2 * W::NTT; ++q) {
                f32x4_t t = coop_red[0][q][lane];
#pragma unroll
                for (int w = 1; w < kWU; ++w) t += coop_red[w][q][lane];
                acc[q] = t;
                __builtin_amdgcn_sched_barrier(0);  // a tile at a time
            }
            if (lane == 0) __hip_atomic_fetch_add(&coop_cnt[1], 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
            f16x8_t B[W::NB];
            float oscale;
            wv_swiglu<SL>(acc, gl, ldexpf(1.0f, -sh.xsh[xrow]), it.wc, c, g, B, oscale);
            // the down records are issued only now: in flight across the reduction and SwiGLU they would push
            // the kernel past its registers
            __builtin_amdgcn_sched_barrier(0);
            wv_issue_b<SL>(a, it, cw, lane, R0);
            wv_issue_b<SL>(a, it, cw + kWU, lane, R1);
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_raw_buffer_store_b32((uint32_t)it.slot_index, rres,
                                                  cw == 0 && it.s == 0 && g == 0 && c < it.ne ? 4 * it.prow : kOob,
                                                  0, 0);
            // down groups cw, cw + kWU, ...: groups past NGB load zeros and store nothing
            const int pbase = c < it.ne ? 4 * ((it.prow * nsl + it.s) * H + 4 * g) : kOob;
            int gb = cw;
            for (; gb + 2 * kWU < NGB; gb += 2 * kWU) {
                wv_compute_b<SL>(a, R0, gb, B, oscale, pres, pbase);
                __builtin_amdgcn_sched_barrier(0);
                wv_issue_b<SL>(a, it, gb + 2 * kWU, lane, R0);
                __builtin_amdgcn_sched_barrier(0);
                wv_compute_b<SL>(a, R1, gb + kWU, B, oscale, pres, pbase);
                __builtin_amdgcn_sched_barrier(0);
                wv_issue_b<SL>(a, it, gb + 3 * kWU, lane, R1);
                __builtin_amdgcn_sched_barrier(0);
            }
            wv_compute_b<SL>(a, R0, gb, B, oscale, pres, pbase);
            __builtin_amdgcn_sched_barrier(0);
            wv_compute_b<SL>(a, R1, gb + kWU, B, oscale, pres, pbase);
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

constexpr size_t kXLdsMax = (size_t)(kDecodeMaxT + 1) * (2560 + 8) * 2;

// Compute units of the current device (queried once per device; thread-safe).
hipError_t device_cus(int& ncu) {
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

// The dynamic LDS limit of a kernel raised to what the activations need, once per (kernel, device); thread-safe.
hipError_t allow_lds(const void* fn) {
    static std::mutex mu;
    static std::set<std::pair<const void*, int>> done;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(mu);
    if (done.count({fn, dev})) return hipSuccess;
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kXLdsMax);
    if (e == hipSuccess) done.insert({fn, dev});
    return e;
}

template <int KQW, int NRGW, bool ROUTE>
hipError_t launch_fused(DecArgs& a, int items_max, int nsl, int ncu, hipStream_t s) {
    hipError_t e = allow_lds(reinterpret_cast<const void*>(&fused_kernel<KQW, NRGW, ROUTE, true>));
    if (e == hipSuccess) e = allow_lds(reinterpret_cast<const void*>(&fused_kernel<KQW, NRGW, ROUTE, false>));
    if (e != hipSuccess) return e;
    const bool multi = items_max > ncu;  // otherwise every workgroup has at most one item
    // a kernel that routes itself has every workgroup route; workgroup 0 must exist to write the routing.
    // CUs the items leave free get spare workgroups that copy the down-row globals for the combine.
    // (a.dgrow stays set only when they run, which tells the combine where to read the globals)
    int grid = items_max < ncu ? items_max : ncu;
    a.n_spare = 0;
    if (grid < ncu && a.dgrow != nullptr) {
        const int rows = a.T * a.k + a.T;
        a.n_spare = min(ncu - grid, (rows + kDgBatch - 1) / kDgBatch);
        grid += a.n_spare;
    } else {
        a.dgrow = nullptr;
    }
    // the routing outputs come from a spare workgroup when there is one (it has no item to delay)
    a.route_wg = a.n_spare > 0 ? grid - 1 : 0;
    const size_t lds = (size_t)(a.T + 1) * (a.H + 8) * 2;
    if (multi)
        hipLaunchKernelGGL((fused_kernel<KQW, NRGW, ROUTE, true>), dim3(grid), dim3(kDT), lds, s, a, nsl);
    else
        hipLaunchKernelGGL((fused_kernel<KQW, NRGW, ROUTE, false>), dim3(grid), dim3(kDT), lds, s, a, nsl);
    return hipGetLastError();
}

template <int SL, bool ROUTE>
hipError_t launch_wave(const DecArgs& a, int items_max, int nsl, int ncu, hipStream_t s) {
    hipError_t e = allow_lds(reinterpret_cast<const void*>(&wave_kernel<SL, ROUTE, true>));
    if (e == hipSuccess) e = allow_lds(reinterpret_cast<const void*>(&wave_kernel<SL, ROUTE, false>));
    if (e == hipSuccess) e = allow_lds(reinterpret_cast<const void*>(&wave_kernel<SL, ROUTE, false, true>));
    if (e != hipSuccess) return e;
    const int grid = items_max < ncu ? items_max : ncu;
    const size_t lds = (size_t)(a.T + 1) * (a.H + 8) * 2;
    if (items_max > grid * kWW)  // some wave has a second item
        hipLaunchKernelGGL((wave_kernel<SL, ROUTE, true>), dim3(grid), dim3(kWT), lds, s, a, nsl);
    else if (items_max > grid * kWU && items_max <= grid * (kWU + 2))  // a few leftovers: up to two rounds
        hipLaunchKernelGGL((wave_kernel<SL, ROUTE, false, true>), dim3(grid), dim3(kWT), lds, s, a, nsl);
    else
        hipLaunchKernelGGL((wave_kernel<SL, ROUTE, false>), dim3(grid), dim3(kWT), lds, s, a, nsl);
    return hipGetLastError();
}

template <bool ROUTE>
hipError_t launch_main(DecArgs& a, int I, int T, int k, int E, int& nsl, int ncu, hipStream_t s) {
    // 32-row items; when they would outnumber the waves of one pass, 64-row items (half the partials)
    nsl = I / kSl;
    const int rows_max = (T * k < E ? T * k : E) + 1;
    if (rows_max * nsl < MOE_WAVE_MIN_ITEMS) return launch_fused<5, 5, ROUTE>(a, rows_max * nsl, nsl, ncu, s);
    a.dgrow = nullptr;  // the wave-item kernel leaves the combine to read the globals through the row slots
    if (rows_max * nsl > ncu * kWW && I % 64 == 0) {
        nsl = I / 64;
        return launch_wave<64, ROUTE>(a, rows_max * nsl, nsl, ncu, s);
    }
    return launch_wave<32, ROUTE>(a, rows_max * nsl, nsl, ncu, s);
}

}  // namespace

// Per-wave register budget: the kernel keeps an item's loads in flight at
// once (up to 5 steps of 128 columns and 5 row groups of 64 per wave), sized
// for H up to 2560; larger H runs the prefill path.
bool decode_shape_supported(int H, int I) { return H % 128 == 0 && I % kSl == 0 && H <= 2560; }

size_t decode_part_bytes(int T, int H, int I, int k) { return (size_t)(T * k + T) * (I / kSl) * H * 4; }
size_t decode_rowslot_bytes(int T, int k) { return (size_t)(T * k + T) * 4; }
size_t decode_dgrow_bytes(int T, int H, int k) { return (size_t)(T * k + T) * H * 4; }

// In-kernel routing (the prologue handles up to two tokens per wave).
#ifndef MOE_ROUTE_IN_KERNEL_MAX_T
#define MOE_ROUTE_IN_KERNEL_MAX_T 8   // two tokens per wave (T = 12, 16) measured slower than a routing launch
#endif
bool decode_routes_in_kernel(int T, int E) { return E <= kRouteInKernelMaxE && T <= MOE_ROUTE_IN_KERNEL_MAX_T; }

hipError_t launch_decode(const Layer& L, const uint16_t* x, int T, const float* w, const int32_t* ids,
                         const int32_t* offsets, const int32_t* sorted_assign, const int32_t* assign_pos, float* y,
                         int accumulate, void* ws, hipStream_t s, const RouteOut* route) {
    (void)ids;
    (void)assign_pos;
    const int H = L.H, I = L.I, E = L.E, k = L.k;
    const WsLayout wl = ws_layout(T, H, I, E, k);
    // the regions must not overlap (a kernel would read another region's data as its own)
    if (wl.dg < wl.part + decode_part_bytes(T, H, I, k) ||
        wl.dgrow < wl.dg + decode_rowslot_bytes(T, k) || wl.total < wl.dgrow + decode_dgrow_bytes(T, H, k))
        return hipErrorInvalidValue;
    DecArgs a;
    a.bank = L.bank; a.slot_bytes = L.slot_bytes; a.num_slots = L.num_slots; a.slot_of_expert = L.slot_of_expert;
    a.shared = L.shared; a.wg = L.wg; a.x = x;
    a.T = T; a.H = H; a.I = I; a.E = E; a.k = k;
    a.w = w; a.offsets = offsets; a.sorted_assign = sorted_assign;
    a.part = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + wl.part);
    a.rowslot = reinterpret_cast<int32_t*>(static_cast<uint8_t*>(ws) + wl.dg);
    a.dgrow = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + wl.dgrow);
    a.n_spare = 0;
    a.y = y; a.accumulate = accumulate;
    const SlotGeom gm = slot_geom(H, I);
    a.gu_codes = (int)gm.gu_codes; a.gu_scales = (int)gm.gu_scales; a.gu_glob = (int)gm.gu_glob;
    a.dn_codes = (int)gm.dn_codes; a.dn_scales = (int)gm.dn_scales; a.dn_glob = (int)gm.dn_glob;
    a.no_glob = 0;

    a.route_wg = 0;
    a.logits = route ? route->logits : nullptr;
    a.r_ids = route ? route->ids : nullptr;
    a.r_w = route ? route->w : nullptr;
    a.r_offsets = route ? route->offsets : nullptr;
    a.r_sorted = route ? route->sorted_assign : nullptr;
    a.r_pos = route ? route->assign_pos : nullptr;
    int ncu = 0;
    hipError_t e = device_cus(ncu);
    if (e != hipSuccess) return e;
    int nsl = 0;
    e = route ? launch_main<true>(a, I, T, k, E, nsl, ncu, s) : launch_main<false>(a, I, T, k, E, nsl, ncu, s);
    if (e != hipSuccess) return e;
    const int nch = H / 64;
    if (nsl <= 10) hipLaunchKernelGGL(dcombine_kernel<10>, dim3(T * nch), dim3(256), 0, s, a, nsl, nch);
    else if (nsl <= 20) hipLaunchKernelGGL(dcombine_kernel<20>, dim3(T * nch), dim3(256), 0, s, a, nsl, nch);
    else hipLaunchKernelGGL(dcombine_kernel<32>, dim3(T * nch), dim3(256), 0, s, a, nsl, nch);
    return hipGetLastError();
}

}  // namespace moe
