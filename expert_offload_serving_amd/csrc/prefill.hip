// Prefill path (T > 16) of the NVFP4 routed-MoE layer for gfx950.
//
// With thousands of tokens each expert sees a dense block of rows, so the
// expert FFN becomes a grouped GEMM over the permuted tokens (the
// permutation groups the T*k assignments by expert; the shared expert is one
// more group holding every token).  The contraction runs on
// v_mfma_f32_16x16x32_f16 with fp32 accumulation:
//  - weights: e2m1 * e4m3 has at most 6 significant bits and lies in
//    [2^-10, 2688], so every dequantised weight is exact in fp16.  Each wave
//    dequantises its own B fragments from the packed codes in registers
//    (v_cvt_scalef32_pk_f16_fp4 with unit scale, then v_pk_mul_f16 by the
//    block scale), so weights never pass through LDS; the per-row global
//    multiplies the accumulator in the epilogue.
//  - activations: each token row is multiplied by a power of two that puts
//    its largest magnitude in [2^14, 2^15), which makes the bf16 -> fp16
//    conversion exact in the fp16 normal range (values more than 28 binades
//    below the row maximum round to fp16 subnormals); the epilogue undoes
//    the scale exactly.
//  - hidden state: silu(gate) * up is stored in fp16 as the A operand of
//    the down GEMM, each (token row, 128-column tile) times its own power of
//    two that puts the tile's largest magnitude in [2^14, 2^15) (the tile's
//    exponent is kept beside it).  The down GEMM, whose 128-column K steps
//    are exactly those tiles, brings a row's tiles to the row's smallest
//    exponent while staging them (exact unless a value falls below the fp16
//    range relative to the row maximum) and undoes that exponent on the fp32
//    result, so the hidden state neither saturates nor loses precision to
//    fp16 subnormals whatever its magnitude.
// K is consumed in steps of 128 (four 32-column MFMA chunks).  Weight
// fragments come straight from the slot's operand-order records: a gate_up
// record holds one 16-row tile for all four chunks of a step, a down record
// holds four 16-row tiles for one chunk, so each lane loads 16 bytes per
// record and every byte feeds an MFMA.  The activation tile in LDS is read as
// the matching operand: lane (row i, group g) takes columns [32m + 8g, +8) of
// the step for chunk m.
//
//   prep:     per-token scale, fp16 activations, shared gate sigmoid(x_t . w_g);
//             in the same launch, the plan: (group, m0) tiles of 128 rows plus
//             one 32/64/128-row remainder per group
//   gate_up:  C = x W_gu^T over 64 gate and the 64 matching up rows per tile,
//             epilogue h = silu(gate) * up -> fp16
//   down:     O = h W_dn^T over 128 output rows per tile -> fp16, each (row, 256-column chunk) times
//             its own power of two (the chunk's largest magnitude in [2^14, 2^15)), undone by the combine
//   combine:  y_t = sum_j w_tj O[pos(t,j)] + s_t O[shared row t] (fixed order, fp32)
//
// MXFP4 banks (E2M1 with one E8M0 scale per 32 elements, no globals) run the
// same kernels with MX set: the weights are decoded exactly to bf16 by
// v_cvt_scalef32_pk_bf16_fp4, which applies the block's E8M0 scale itself
// (e2m1 * 2^e is exact in bf16 for every E8M0 value), into
// v_mfma_f32_16x16x32_bf16.  gate_up takes the bf16 activations as they are
// (no per-token scale); its records give lane (row i, a) the 32 columns
// [32a, 32a + 32) of the step (one scale block), so MFMA m of a step uses
// dword m of every lane's record and the activation columns 32a + 8m + [0, 8)
// of the same lane position: the four MFMAs still cover the step's 128
// columns once.  The hidden state is stored as two bf16 terms (h_hi = bf16(h),
// h_lo = bf16(h - h_hi): 16 significant bits, fp32's range, no exponents) and
// down multiplies each decoded weight fragment by both.
#include <map>
#include <mutex>

#include "internal.hpp"
#include "nvfp4_device.hpp"

namespace moe {
namespace {

constexpr int BK = 128;           // contraction step
constexpr int APITCH = BK + 8;    // LDS row pitch of the activation tile, in fp16 elements
constexpr int kClasses = 3;       // row-tile classes: 128, 64, 32 rows

struct PrefillArgs {
    const uint8_t* bank;
    size_t slot_bytes;
    int num_slots;
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
    _Float16* hbuf;   // fp16 [(T*k + T), I], tile (row, c) scaled by 2^hexp[row, c]
    uint16_t* hmx;    // MXFP4: bf16 [(T*k + T), I] high terms, then the low terms
    int mx;           // MXFP4 bank (the prep skips the fp16 activations)
    int* hexp;        // i32  [(T*k + T), KT]: exponent of each 128-column tile of hbuf (kNoExp: all zero)
    int KT;           // 128-column tiles of I
    _Float16* obuf;   // fp16 [(T*k + T), H], chunk (row, c) scaled by 2^oexp[row, c]
    int* oexp;        // i32  [(T*k + T), OT]: exponent of each 256-column chunk of obuf (kNoExp: all zero)
    int OT;           // 256-column chunks of H
    _Float16* x16;    // fp16 [T, H] scaled activations
    float* xinv;      // f32  [T] inverse activation scale
    float* sbuf;      // f32  [T] shared gate
    int* tiles;       // [4 + kClasses * 2 * cap]: per-class counts, then (group, m0) pairs per class
    int cap;
    float* y;
    int accumulate;
    size_t gu_codes, gu_scales, gu_glob, dn_codes, dn_scales, dn_glob;
};

// Group g < E: routed expert g, rows [offsets[g], offsets[g+1]); g == E: the
// shared expert, rows [T*k, T*k + T).
__device__ __forceinline__ int group_begin(const PrefillArgs& a, int g) {
    return g < a.E ? a.offsets[g] : a.T * a.k;
}
__device__ __forceinline__ int group_end(const PrefillArgs& a, int g) {
    return g < a.E ? a.offsets[g + 1] : a.T * a.k + a.T;
}
// An expert whose slot index is negative or not below num_slots is left out.
__device__ __forceinline__ bool slot_in_bank(const PrefillArgs& a, int sl) { return sl >= 0 && sl < a.num_slots; }
__device__ __forceinline__ bool group_active(const PrefillArgs& a, int g) {
    if (g == a.E) return a.shared != nullptr;
    return a.offsets[g + 1] > a.offsets[g] && slot_in_bank(a, a.slot_of_expert[g]);
}
__device__ __forceinline__ const uint8_t* group_slot(const PrefillArgs& a, int g) {
    return g == a.E ? a.shared : a.bank + (size_t)a.slot_of_expert[g] * a.slot_bytes;
}

// ------------------------------------------------------------------ prep
// One 256-thread workgroup per token t.
__device__ __forceinline__ void prep_token(const PrefillArgs& a, int t, float (&red)[2][4]) {
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int H = a.H, nvec = H / 8;
    const u32x4_t* xr = reinterpret_cast<const u32x4_t*>(a.x + (size_t)t * H);
    const u32x4_t* wr = reinterpret_cast<const u32x4_t*>(a.wg);
    constexpr int kMaxV = 4;  // H <= 8192
    u32x4_t xv[kMaxV];
    float amax = 0.0f, dot = 0.0f;
#pragma unroll
    for (int q = 0; q < kMaxV; ++q) {
        const int v = tid + 256 * q;
        xv[q] = v < nvec ? xr[v] : u32x4_t{0, 0, 0, 0};
        const uint32_t ws[4] = {xv[q].x, xv[q].y, xv[q].z, xv[q].w};
        u32x4_t wv = (a.shared != nullptr && v < nvec) ? wr[v] : u32x4_t{0, 0, 0, 0};
        const uint32_t gs[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            amax = fmaxf(amax, fabsf(bf16_bits_f32(ws[m] & 0xFFFF)));
            amax = fmaxf(amax, fabsf(bf16_bits_f32(ws[m] >> 16)));
            dot = dot2_bf16(as_bf16x2(ws[m]), as_bf16x2(gs[m]), dot);
        }
    }
    amax = wave_max(amax);
    dot = wave_sum(dot);
    if (lane == 0) red[0][wave] = amax, red[1][wave] = dot;
    __syncthreads();
    amax = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
    // scale = 2^(14 - floor(log2 amax)) puts the row maximum in [2^14, 2^15)
    int e = 0;
    if (amax > 0.0f) (void)frexpf(amax, &e);  // amax = m * 2^e, m in [0.5, 1)
    const int shift = amax > 0.0f ? 15 - e : 0;
    const float sc = ldexpf(1.0f, shift);
    if (tid == 0) {
        a.xinv[t] = ldexpf(1.0f, -shift);
        if (a.shared != nullptr) a.sbuf[t] = sigmoidf_(red[1][0] + red[1][1] + red[1][2] + red[1][3]);
    }
    if (a.mx) return;  // the MXFP4 GEMMs read the bf16 activations directly
    f16x2_t* dst = reinterpret_cast<f16x2_t*>(a.x16 + (size_t)t * H);
#pragma unroll
    for (int q = 0; q < kMaxV; ++q) {
        const int v = tid + 256 * q;
        if (v >= nvec) continue;
        const uint32_t ws[4] = {xv[q].x, xv[q].y, xv[q].z, xv[q].w};
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            f16x2_t h2;
            h2.x = (_Float16)(bf16_bits_f32(ws[m] & 0xFFFF) * sc);
            h2.y = (_Float16)(bf16_bits_f32(ws[m] >> 16) * sc);
            dst[v * 4 + m] = h2;
        }
    }
}

// ------------------------------------------------------------------ plan
__device__ __forceinline__ int tile_class(int rows) { return rows > 64 ? 0 : (rows > 32 ? 1 : 2); }

// One 256-thread workgroup lists every tile.
__device__ __forceinline__ void plan_tiles(const PrefillArgs& a, int (&wsum)[kClasses][4]) {
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int G = a.E + 1;
    const int per = (G + 255) / 256;
    const int g0 = tid * per, g1 = min(G, g0 + per);
    int cnt[kClasses] = {0, 0, 0};
    for (int g = g0; g < g1; ++g) {
        if (!group_active(a, g)) continue;
        const int n = group_end(a, g) - group_begin(a, g);
        cnt[0] += n / 128;
        if (n % 128) cnt[tile_class(n % 128)] += 1;
    }
    int pos[kClasses];
#pragma unroll
    for (int c = 0; c < kClasses; ++c) {
        int incl = cnt[c];
#pragma unroll
        for (int off = 1; off < kWave; off <<= 1) {
            const int o = __shfl_up(incl, off, kWave);
            if (lane >= off) incl += o;
        }
        if (lane == kWave - 1) wsum[c][wave] = incl;
        pos[c] = incl - cnt[c];
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < kClasses; ++c) {
        int before = 0, total = 0;
        for (int i = 0; i < 4; ++i) {
            if (i < wave) before += wsum[c][i];
            total += wsum[c][i];
        }
        pos[c] += before;
        if (tid == 0) a.tiles[c] = total;
    }
    for (int g = g0; g < g1; ++g) {
        if (!group_active(a, g)) continue;
        const int n = group_end(a, g) - group_begin(a, g);
        for (int m0 = 0; m0 < n; m0 += 128) {
            const int c = (n - m0 >= 128) ? 0 : tile_class(n - m0);
            int* e = a.tiles + 4 + 2 * (c * a.cap + pos[c]);
            e[0] = g;
            e[1] = m0;
            ++pos[c];
        }
    }
}

// Workgroup 0 plans the tiles (it reads only the routing offsets), workgroups
// 1..T prepare the tokens: one launch, and the plan overlaps the preparation.
__global__ void __launch_bounds__(256) prep_plan_kernel(PrefillArgs a) {
    __shared__ float red[2][4];
    __shared__ int wsum[kClasses][4];
    if (blockIdx.x == 0) plan_tiles(a, wsum);
    else prep_token(a, (int)blockIdx.x - 1, red);
}

// ------------------------------------------------------------------ grouped GEMM (gate_up and down)

__device__ __forceinline__ f16x8_t lds_frag(const _Float16* p) {
    return __builtin_bit_cast(f16x8_t, *reinterpret_cast<const u32x4_t*>(p));
}

// Exponent of a hidden-state tile that is all zero: larger than any real one,
// so it never is a row's minimum, and aligning to a real one gives zeros.
constexpr int kNoExp = 1 << 20;

__device__ __forceinline__ int tile_shift(float amax) { return amax > 0.0f ? fp16_shift(amax) : kNoExp; }

// 2^n as an fp16 pair for n in [-24, 0] (subnormal below -14); 0 below -24.
__device__ __forceinline__ f16x2_t pow2_f16x2(int n) {
    const uint16_t b = n < -24 ? 0 : (n < -14 ? (uint16_t)(1u << (n + 24)) : (uint16_t)((n + 15) << 10));
    const _Float16 v = __builtin_bit_cast(_Float16, b);
    return f16x2_t{v, v};
}

// Eight fp16 values times 2^d (d <= 0), in two exact power-of-two steps
// (the second rounds only results below the fp16 normal range).
__device__ __forceinline__ u32x4_t scale_h8(u32x4_t v, int d) {
    const int d1 = d > -14 ? d : -14;
    const f16x2_t f1 = pow2_f16x2(d1), f2 = pow2_f16x2(d - d1);
    u32x4_t o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const f16x2_t h = __builtin_bit_cast(f16x2_t, word_of(v, i)) * f1 * f2;
        const uint32_t u = __builtin_bit_cast(uint32_t, h);
        if (i == 0) o.x = u; else if (i == 1) o.y = u; else if (i == 2) o.z = u; else o.w = u;
    }
    return o;
}

// MXFP4: E8M0 byte as an f32 power of two; eight E2M1 codes (one dword) times 2^(e - 127), exactly, in bf16.
__device__ __forceinline__ float e8m0_f32(uint32_t b) { return __uint_as_float((b & 0xFF) << 23); }
__device__ __forceinline__ bf16x8_t mx_frag_bf16(uint32_t cw, float sc) {
    const bf16x2_t v0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, sc, 0);
    const bf16x2_t v1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, sc, 1);
    const bf16x2_t v2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, sc, 2);
    const bf16x2_t v3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw, sc, 3);
    const u32x4_t u = {__builtin_bit_cast(uint32_t, v0), __builtin_bit_cast(uint32_t, v1),
                       __builtin_bit_cast(uint32_t, v2), __builtin_bit_cast(uint32_t, v3)};
    return __builtin_bit_cast(bf16x8_t, u);
}
// bf16 bits of the two terms of h: hi = bf16(h), lo = bf16(h - hi) (both round to nearest even)
__device__ __forceinline__ void split_bf16(float h, uint16_t& hi, uint16_t& lo) {
    const __bf16 bh = (__bf16)h;
    const __bf16 bl = (__bf16)(h - (float)bh);
    hi = __builtin_bit_cast(uint16_t, bh);
    lo = __builtin_bit_cast(uint16_t, bl);
}

// 16 bytes per lane from a buffer straight into LDS: lane L's bytes land at lds + 16 L (lds is wave-uniform;
// checked with a probe on this part).  A device function of its own: written inside the kernel template, the
// builtin made the host compilation drop the kernel's launch stub without a diagnostic.
__device__ __forceinline__ void lds_load16(rsrc_t r, _Float16* lds, int off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, off, 0, 0, 0);
}

// ------------------------------------------------------------------ grouped GEMM tiles
// One workgroup (NW waves) computes a BM-token tile (BM = 128, 64 or 32)
// against a block of weight rows: gate_up: matching gate and up rows, down:
// output rows.  Wave (wm, wn) owns tokens [BM/WM wm, +BM/WM) and NB 16-row
// weight blocks (gate_up: NB/2 gate tiles and the matching up tiles; down:
// NB/4 record groups), so each dequantised weight fragment feeds BM/16/WM
// MFMAs.  Four waves with 512 registers each (twice the weight rows per
// wave) measured slower for 128-row tiles: a single wave per SIMD could not
// hide its dequantisation behind the matrix cores.  Per 128-column step the
// activation tile (BM x 128) sits in LDS one step ahead; each wave's weight
// records are loaded two steps ahead into a register ping-pong.  gate_up
// loads its activation tiles straight into LDS (16-byte buffer loads to LDS,
// no register staging and no store phase: 429 against 438 us per 2,048-token
// NVFP4 step, 409 against 419 for MXFP4); down stages them through registers,
// since each hidden-state row is rescaled on the way.  Load order per step
// end: activations of step s + 2, then weights of step s + 2, so waiting for
// either never waits for the other's newer loads.  Every load is an
// unconditional buffer load (past the end it reads zeros), which keeps the
// compiler's wait counts exact.
template <bool GATEUP, int BM, int NW, int WM, int NB, int MINW, bool MX>
__global__ void __launch_bounds__(NW * kWave, MINW) tile_gemm_kernel(PrefillArgs a, int cls, int n_tiles_n) {
    constexpr int NWN = NW / WM;             // waves along the weight rows (WM along the tokens)
    constexpr int MI = BM / 16 / WM;         // 16-row token blocks per wave
    constexpr int NT = NW * kWave;           // threads
    constexpr int AQ = BM * 16 / NT;         // activation chunks per thread per step
    // a gate_up workgroup's h-columns are exactly one 128-column K step of the down GEMM (one exponent tile)
    static_assert(!GATEUP || NWN * 8 * NB == BK, "gate_up column tile must match the down K step");
    constexpr int NA = MX && !GATEUP ? 2 : 1;  // activation tiles per step: MXFP4 down stages h_hi and h_lo
    // gate_up: the activation tile goes straight from memory into LDS (no register staging).  One array per
    // buffer, so the compiler never makes a read of one wait for the loads in flight into the other; rows of BK
    // elements without padding (a load fills 64 consecutive 16-byte slots), the 16-byte chunk c of row r at
    // slot c ^ (r & 15), so the 16 rows of a fragment read fall in 16 different bank groups.
    constexpr bool DMA = GATEUP;
    constexpr int DQ = DMA ? BM * BK * 2 / (NW * 1024) : 1;  // 1 KiB loads per wave per step
    __shared__ __attribute__((aligned(16))) _Float16 sA[2][DMA ? 8 : NA * BM * APITCH];
    __shared__ __attribute__((aligned(1024))) _Float16 sD0[DMA ? BM * BK : 8];
    __shared__ __attribute__((aligned(1024))) _Float16 sD1[DMA ? BM * BK : 8];
    __shared__ int tok[BM];
    // per-(row, wave along the weight rows) maximum of |h| (gate_up) or |o| (down); down: each row's smallest
    // hidden-state tile exponent
    __shared__ float smax[NWN][BM];
    __shared__ int semin[BM];

    // XCD-aware order: workgroups are dealt round-robin to the 8 XCDs (block b to XCD b % 8), so the active
    // blocks of XCD x take one contiguous range of (tile, column tile) pairs.  The column tiles of a row tile,
    // and the tiles of one expert, then share that XCD's L2: the activation tile and the expert's weights are
    // fetched from HBM once per XCD instead of once per workgroup.
    const int n_active = a.tiles[cls] * n_tiles_n;
    if ((int)blockIdx.x >= n_active) return;
    const int per_xcd = n_active / 8, extra = n_active % 8, xcd = (int)blockIdx.x % 8;
    const int lb = xcd * per_xcd + min(xcd, extra) + (int)blockIdx.x / 8;
    const int tile = lb / n_tiles_n, nt = lb % n_tiles_n;
    const int* te = a.tiles + 4 + 2 * (cls * a.cap + tile);
    const int g = te[0], m0 = te[1];
    const int gb = group_begin(a, g), cnt = min(BM, group_end(a, g) - gb - m0);
    const uint8_t* slot = group_slot(a, g);
    const int H = a.H, I = a.I, T = a.T, k = a.k;
    const int K = GATEUP ? H : I;
    const int nsteps = (K + BK - 1) / BK;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int wm = wave / NWN, wn = wave % NWN;
    const int l16 = lane & 15, q4 = lane >> 4;

    if (GATEUP) {
        for (int m = tid; m < BM; m += NT) {
            int t = -1;
            if (m < cnt) {
                const int p = gb + m0 + m;
                t = g < a.E ? a.sorted_assign[p] / k : p - T * k;
            }
            tok[m] = t;
        }
        __syncthreads();
    }

    // ---- activation loader: thread -> 16-byte chunk (tid & 15) of rows (tid >> 4) + (NT / 16) q
    const int ach = tid & 15, arow0 = tid >> 4;
    const int rows = T * k + T;
    const rsrc_t ares = GATEUP ? make_rsrc(MX ? static_cast<const void*>(a.x) : static_cast<const void*>(a.x16),
                                           (uint32_t)T * H * 2)
                               : (MX ? make_rsrc(a.hmx, (uint32_t)((size_t)rows * I * 4))
                                     : make_rsrc(a.hbuf, (uint32_t)((size_t)rows * I * 2)));
    int aoff[AQ];
#pragma unroll
    for (int q = 0; q < AQ; ++q) {
        const int m = arow0 + (NT / 16) * q;
        const int mm = m < cnt ? m : 0;  // rows past the group read a valid row; their outputs are dropped
        aoff[q] = GATEUP ? 2 * tok[mm] * H : 2 * (gb + m0 + mm) * I;
    }
    // down: the hidden-state tiles of a row carry their own exponents; each is brought to the row's smallest
    // (the exponent of its largest tile) while staged, and that one is undone in the epilogue
    const rsrc_t xres = make_rsrc(a.hexp, GATEUP || MX ? 0u : (uint32_t)((size_t)rows * a.KT * 4));
    int emin[GATEUP ? 1 : AQ], eoff[GATEUP ? 1 : AQ];
    if (!GATEUP && !MX) {
        int ev[AQ][4];
#pragma unroll
        for (int q = 0; q < AQ; ++q) {
            const int m = arow0 + (NT / 16) * q;
            eoff[q] = 4 * (gb + m0 + (m < cnt ? m : 0)) * a.KT;
#pragma unroll
            for (int j = 0; j < 4; ++j) ev[q][j] = (int)buf_load4(xres, j < a.KT ? eoff[q] + 4 * j : kOob);
        }
#pragma unroll
        for (int q = 0; q < AQ; ++q) {
            int e = kNoExp;
#pragma unroll
            for (int j = 0; j < 4; ++j) e = j < a.KT ? min(e, ev[q][j]) : e;
            for (int j = 4; j < a.KT; ++j) e = min(e, (int)buf_load4(xres, eoff[q] + 4 * j));
            emin[q] = e;
            if (ach == 0) semin[arow0 + (NT / 16) * q] = e;
        }
    }
    // DMA: wave load j covers tile rows 4 (NW j + wave) + [0, 4): lane -> row + lane / 16, the chunk that belongs
    // in slot lane % 16, (lane % 16) ^ (row % 16); rows past the group read a valid row (their outputs are dropped)
    int doff[DQ];
    if (DMA) {
#pragma unroll
        for (int j = 0; j < DQ; ++j) {
            const int r = 4 * (NW * j + wave) + lane / 16;
            doff[j] = 2 * tok[r < cnt ? r : 0] * H + 16 * ((lane & 15) ^ (r & 15));
        }
    }
    auto dma_a = [&](int step, _Float16* dst) {
#pragma unroll
        for (int j = 0; j < DQ; ++j)
            lds_load16(ares, dst + 512 * (NW * j + wave), step < nsteps ? doff[j] + 2 * BK * step : kOob);
    };
    u32x4_t ra[AQ], rl[NA == 2 ? AQ : 1];
    int rex[GATEUP ? 1 : AQ];
    auto load_a = [&](int step) {
        const int kk = step * BK + 8 * ach;
        const bool ok = step < nsteps && kk < K;
        if (!GATEUP && !MX) {
#pragma unroll
            for (int q = 0; q < AQ; ++q) rex[q] = (int)buf_load4(xres, step < nsteps ? eoff[q] + 4 * step : kOob);
        }
#pragma unroll
        for (int q = 0; q < AQ; ++q) ra[q] = buf_load16(ares, ok ? aoff[q] + 2 * kk : kOob);
        if (NA == 2) {
#pragma unroll
            for (int q = 0; q < AQ; ++q) rl[NA == 2 ? q : 0] = buf_load16(ares, ok ? 2 * rows * I + aoff[q] + 2 * kk : kOob);
        }
    };
    auto store_a = [&](int buf) {
#pragma unroll
        for (int q = 0; q < AQ; ++q) {
            const u32x4_t v = GATEUP || MX ? ra[q] : scale_h8(ra[q], emin[GATEUP ? 0 : q] - rex[GATEUP ? 0 : q]);
            *reinterpret_cast<u32x4_t*>(&sA[buf][(arow0 + (NT / 16) * q) * APITCH + 8 * ach]) = v;
            if (NA == 2)
                *reinterpret_cast<u32x4_t*>(&sA[buf][BM * APITCH + (arow0 + (NT / 16) * q) * APITCH + 8 * ach]) =
                    rl[NA == 2 ? q : 0];
        }
    };

    // ---- weight records of this wave
    const rsrc_t sres = make_rsrc(slot, (uint32_t)a.slot_bytes);
    // scales: NVFP4 one dword per lane (its four E4M3 bytes); MXFP4 gate_up one E8M0 byte per lane, down one dword
    // per lane (the four rows' E8M0 bytes), 64 bytes per record
    const int soff = MX ? (GATEUP ? lane : 4 * (lane & 15)) : lane_scale_off(lane);
    const int sstride = MX ? 64 : kRecScaleBytes;
    const int codes = (int)(GATEUP ? a.gu_codes : a.dn_codes), scales = (int)(GATEUP ? a.gu_scales : a.dn_scales);
    const int hc0 = 8 * NB * (NWN * nt + wn);      // gate_up: first h-column of the wave (NB / 2 tiles)
    const int grp0 = (NB / 4) * (NWN * nt + wn);   // down: first record group of the wave (NB / 4 groups)
    struct BRegs {
        u32x4_t c[NB];
        uint32_t s[NB];
    };
    // gate_up: record b < NB/2 is gate tile hc0/16 + b, b >= NB/2 the matching up tile (one 128-column step each).
    // down: record 4 gi + m is group grp0 + gi at 32-column chunk 4 step + m.
    auto load_b = [&](int step, BRegs& r) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            int rec;
            bool ok = step < nsteps;
            if (GATEUP) {
                const int hcb = hc0 + 16 * (b % (NB / 2));
                ok = ok && hcb < I;
                rec = step * (2 * I / 16) + (b / (NB / 2)) * (I / 16) + hcb / 16;
            } else {
                const int gi = b >> 2, kc = 4 * step + (b & 3);
                ok = ok && kc < I / 32 && 64 * (grp0 + gi) < H;
                rec = kc * (H / 64) + grp0 + gi;
            }
            r.c[b] = buf_load16(sres, ok ? codes + rec * kRecBytes + 16 * lane : kOob);
            if (MX && GATEUP)
                r.s[b] = __builtin_amdgcn_raw_buffer_load_b8(sres, ok ? scales + rec * sstride + soff : kOob, 0, 0);
            else
                r.s[b] = buf_load4(sres, ok ? scales + rec * sstride + soff : kOob);
        }
    };

    f32x4_t acc[MI][NB];
#pragma unroll
    for (int i = 0; i < MI; ++i)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[i][b] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};

    auto compute = [&](int buf, const BRegs& r) {
        if constexpr (DMA) {
            // every weight fragment of chunk m first, then one activation fragment at a time (few registers live)
            const _Float16* sd = buf ? sD1 : sD0;
#pragma unroll
            for (int m = 0; m < 4; ++m) {
                const int col = MX ? 32 * q4 + 8 * m : 32 * m + 8 * q4;
                f16x8_t fb[NB];
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const uint32_t cw = word_of(r.c[b], m);
                    if (MX) {
                        fb[b] = __builtin_bit_cast(f16x8_t, mx_frag_bf16(cw, e8m0_f32(r.s[b])));
                    } else {
                        f16x2_t S;
                        if (m == 0) S = scale_f16x2<0>(r.s[b]);
                        else if (m == 1) S = scale_f16x2<1>(r.s[b]);
                        else if (m == 2) S = scale_f16x2<2>(r.s[b]);
                        else S = scale_f16x2<3>(r.s[b]);
                        fb[b] = frag_f16(cw, S);
                    }
                }
#pragma unroll
                for (int i = 0; i < MI; ++i) {
                    const f16x8_t fa = lds_frag(sd + (16 * i + l16) * BK + 8 * ((col / 8) ^ l16));
#pragma unroll
                    for (int b = 0; b < NB; ++b) {
                        if (MX)
                            acc[i][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                                __builtin_bit_cast(bf16x8_t, fa), __builtin_bit_cast(bf16x8_t, fb[b]), acc[i][b], 0, 0, 0);
                        else
                            acc[i][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa, fb[b], acc[i][b], 0, 0, 0);
                    }
                }
            }
            return;
        }
#pragma unroll
        for (int m = 0; m < 4; ++m) {
            // MXFP4 gate_up: MFMA m takes dword m of every lane's record, columns 32 q4 + 8 m + [0, 8)
            const int col = MX && GATEUP ? 32 * q4 + 8 * m : 32 * m + 8 * q4;
            f16x8_t fa[MI];
#pragma unroll
            for (int i = 0; i < MI; ++i) fa[i] = lds_frag(&sA[buf][(16 * MI * wm + 16 * i + l16) * APITCH + col]);
            if (MX) {
                bf16x8_t fl[NA == 2 ? MI : 1];
                if (NA == 2) {
#pragma unroll
                    for (int i = 0; i < MI; ++i)
                        fl[NA == 2 ? i : 0] = __builtin_bit_cast(
                            bf16x8_t, lds_frag(&sA[buf][BM * APITCH + (16 * MI * wm + 16 * i + l16) * APITCH + col]));
                }
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const int ri = GATEUP ? b : 4 * (b >> 2) + m;
                    const int d = GATEUP ? m : (b & 3);
                    const float sc = e8m0_f32(GATEUP ? r.s[ri] : r.s[ri] >> (8 * d));
                    const bf16x8_t fb = mx_frag_bf16(word_of(r.c[ri], d), sc);
#pragma unroll
                    for (int i = 0; i < MI; ++i) {
                        acc[i][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, fa[i]), fb,
                                                                            acc[i][b], 0, 0, 0);
                        if (NA == 2)
                            acc[i][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fl[NA == 2 ? i : 0], fb, acc[i][b],
                                                                                0, 0, 0);
                    }
                }
                continue;
            }
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                // gate_up: record b holds chunk m in dword m; down: record 4 gi + m holds tile j in dword j
                const int ri = GATEUP ? b : 4 * (b >> 2) + m;
                const int d = GATEUP ? m : (b & 3);
                const uint32_t cw = word_of(r.c[ri], d);
                f16x2_t S;
                if (d == 0) S = scale_f16x2<0>(r.s[ri]);
                else if (d == 1) S = scale_f16x2<1>(r.s[ri]);
                else if (d == 2) S = scale_f16x2<2>(r.s[ri]);
                else S = scale_f16x2<3>(r.s[ri]);
                const f16x8_t fb = frag_f16(cw, S);
#pragma unroll
                for (int i = 0; i < MI; ++i) acc[i][b] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa[i], fb, acc[i][b], 0, 0, 0);
            }
        }
    };

    // the issue order of the loads is part of the design (see above): pin it
#define MOE_PIN() __builtin_amdgcn_sched_barrier(0)
    BRegs rb0, rb1;
    if constexpr (DMA) {
        // Before the barrier that ends a step each wave waits for its own loads into the next step's buffer
        // (vmcnt(n): all but the newest n loads have landed; the newest are the step's weight loads, issued after
        // them), then a bare s_barrier: a full workgroup barrier would also wait for every weight load in flight.
        // The empty asm statements keep the compiler from moving LDS accesses across the barrier.
        constexpr int kVm = 2 * NB;  // a step's weight loads, issued after its activation loads
        constexpr int kWaitAct = (kVm & 15) | ((kVm >> 4) << 14) | 0x70 | 0xF00;
        constexpr int kWaitAct0 = ((2 * kVm + DQ) & 15) | (((2 * kVm + DQ) >> 4) << 14) | 0x70 | 0xF00;
#define MOE_SYNC(W)                              \
    do {                                         \
        asm volatile("" ::: "memory");           \
        __builtin_amdgcn_s_waitcnt(W);           \
        __builtin_amdgcn_s_barrier();            \
        asm volatile("" ::: "memory");           \
    } while (0)
        dma_a(0, sD0);
        MOE_PIN();
        load_b(0, rb0);
        MOE_PIN();
        dma_a(1, sD1);
        MOE_PIN();
        load_b(1, rb1);
        MOE_PIN();
        MOE_SYNC(kWaitAct0);  // step 0's activations
        int s = 0;
        for (; s + 1 < nsteps; s += 2) {
            compute(0, rb0);
            MOE_PIN();
            MOE_SYNC(kWaitAct);  // step s + 1's activations landed; every wave is done with buffer 0
            dma_a(s + 2, sD0);
            MOE_PIN();
            load_b(s + 2, rb0);
            MOE_PIN();
            compute(1, rb1);
            MOE_PIN();
            MOE_SYNC(kWaitAct);
            dma_a(s + 3, sD1);
            MOE_PIN();
            load_b(s + 3, rb1);
            MOE_PIN();
        }
        if (s < nsteps) compute(0, rb0);
        __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): no load into LDS outlives the loop
#undef MOE_SYNC
    } else {
        load_a(0);
        MOE_PIN();
        load_b(0, rb0);
        MOE_PIN();
        store_a(0);
        MOE_PIN();
        load_a(1);
        MOE_PIN();
        load_b(1, rb1);
        MOE_PIN();
        __syncthreads();
        int s = 0;
        for (; s + 1 < nsteps; s += 2) {  // one exit: keeps the loop-carried loads' wait counts exact
            compute(0, rb0);
            MOE_PIN();
            store_a(1);           // activations of step s + 1
            MOE_PIN();
            load_a(s + 2);
            MOE_PIN();
            load_b(s + 2, rb0);
            MOE_PIN();
            __syncthreads();
            compute(1, rb1);
            MOE_PIN();
            store_a(0);           // activations of step s + 2
            MOE_PIN();
            load_a(s + 3);
            MOE_PIN();
            load_b(s + 3, rb1);
            MOE_PIN();
            __syncthreads();
        }
        if (s < nsteps) compute(0, rb0);  // odd number of steps: the last one sits in buffer 0
    }
#undef MOE_PIN

    // ---- epilogue: lane holds token rows 4 q4 + [0, 4) of column l16 of each 16x16 block
    const rsrc_t gres = make_rsrc(slot, (uint32_t)a.slot_bytes);
    if (GATEUP && MX) {
        // h = silu(gate) * up in fp32 (MXFP4 has no globals and the activations no scale), stored as two bf16 terms
        constexpr int NC = NB / 2;
        const size_t lo_off = (size_t)rows * I;
#pragma unroll
        for (int cb = 0; cb < NC; ++cb) {
            const int hc = hc0 + 16 * cb + l16;
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = 16 * MI * wm + 16 * i + 4 * q4 + r;
                    if (hc < I && m < cnt) {
                        uint16_t hi, lo;
                        split_bf16(silu_fast(acc[i][cb][r]) * acc[i][NB / 2 + cb][r], hi, lo);
                        const size_t at = (size_t)(gb + m0 + m) * I + hc;
                        a.hmx[at] = hi;
                        a.hmx[lo_off + at] = lo;
                    }
                }
        }
    } else if (GATEUP) {
        // h = silu(gate) * up in fp32; the tile's 128 columns are this workgroup's: its largest |h| per row
        // (over the 16 lanes of a column block, the wave's blocks, then the waves) sets the row's exponent
        constexpr int NC = NB / 2;
        float hv[NC][MI][4];
        float rmax[MI][4];
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) rmax[i][r] = 0.0f;
#pragma unroll
        for (int cb = 0; cb < NC; ++cb) {
            const int hc = hc0 + 16 * cb + l16;
            const bool cok = hc < I;
            const float gg = __uint_as_float(buf_load4(gres, cok ? (int)a.gu_glob + 4 * hc : kOob));
            const float gu = __uint_as_float(buf_load4(gres, cok ? (int)a.gu_glob + 4 * (I + hc) : kOob));
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = 16 * MI * wm + 16 * i + 4 * q4 + r;
                    const bool ok = cok && m < cnt;
                    const float inv = a.xinv[tok[ok ? m : 0] >= 0 ? tok[ok ? m : 0] : 0];
                    const float gate = acc[i][cb][r] * inv * gg;
                    const float up = acc[i][NB / 2 + cb][r] * inv * gu;
                    const float h = ok ? silu_fast(gate) * up : 0.0f;
                    hv[cb][i][r] = h;
                    rmax[i][r] = fmaxf(rmax[i][r], fabsf(h));
                }
        }
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float v = row16_max(rmax[i][r]);
                if (l16 == 0) smax[wn][16 * MI * wm + 16 * i + 4 * q4 + r] = v;
            }
        __syncthreads();
        const int KT = a.KT;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = 16 * MI * wm + 16 * i + 4 * q4 + r;
                float tmax = 0.0f;
#pragma unroll
                for (int w = 0; w < NWN; ++w) tmax = fmaxf(tmax, smax[w][m]);
                const int e = tile_shift(tmax);
                if (m < cnt && wn == 0 && l16 == 0) a.hexp[(size_t)(gb + m0 + m) * KT + nt] = e;
                const float sc = ldexpf(1.0f, e == kNoExp ? 0 : e);
#pragma unroll
                for (int cb = 0; cb < NC; ++cb) {
                    const int hc = hc0 + 16 * cb + l16;
                    if (hc < I && m < cnt) a.hbuf[(size_t)(gb + m0 + m) * I + hc] = (_Float16)(hv[cb][i][r] * sc);
                }
            }
    } else {
        // o = acc * 2^-emin * gd; a wave's NB / 4 record groups are 64 output columns of one 256-column chunk
        // (chunk (NWN nt + wn) / 4: column tiles are 256 or 512 wide, so the waves of a chunk share a workgroup).
        // The chunk's largest |o| per row (16 lanes, the wave's blocks, then the chunk's four waves) sets the
        // power of two the row's chunk is stored under in fp16.
        static_assert(GATEUP || (NB == 4 && NWN % 4 == 0), "a down wave covers 64 columns; four make a 256-column chunk");
        float ov[NB][MI][4];
        float rmax[MI][4];
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) rmax[i][r] = 0.0f;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            const int oc = 64 * grp0 + 16 * b + l16;
            const bool cok = oc < H;
            // MXFP4: no row globals, and the hidden state carries no exponent
            const float gd = MX ? 1.0f : __uint_as_float(buf_load4(gres, cok ? (int)a.dn_glob + 4 * oc : kOob));
#pragma unroll
            for (int i = 0; i < MI; ++i)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                    const int m = 16 * MI * wm + 16 * i + 4 * q4 + r;
                    const int e = MX ? 0 : semin[m];
                    const float o = cok && m < cnt ? ldexpf(acc[i][b][r], e == kNoExp ? 0 : -e) * gd : 0.0f;
                    ov[b][i][r] = o;
                    rmax[i][r] = fmaxf(rmax[i][r], fabsf(o));
                }
        }
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const float v = row16_max(rmax[i][r]);
                if (l16 == 0) smax[wn][16 * MI * wm + 16 * i + 4 * q4 + r] = v;
            }
        __syncthreads();
        const int OT = a.OT, ch = grp0 / 4, w0 = wn & ~3;
#pragma unroll
        for (int i = 0; i < MI; ++i)
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = 16 * MI * wm + 16 * i + 4 * q4 + r;
                const float cmax = fmaxf(fmaxf(smax[w0][m], smax[w0 + 1][m]), fmaxf(smax[w0 + 2][m], smax[w0 + 3][m]));
                const int e = tile_shift(cmax);
                if (m < cnt && wn == w0 && l16 == 0 && ch < OT) a.oexp[(size_t)(gb + m0 + m) * OT + ch] = e;
                const float sc = ldexpf(1.0f, e == kNoExp ? 0 : e);
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const int oc = 64 * grp0 + 16 * b + l16;
                    if (oc < H && m < cnt) a.obuf[(size_t)(gb + m0 + m) * H + oc] = (_Float16)(ov[b][i][r] * sc);
                }
            }
    }
}

// gate_up: one wave per 128 tokens (each dequantised weight fragment feeds 8
// MFMAs, no weight record loaded twice) measured faster than two; down keeps
// two waves along the tokens and whole 64-row record groups per wave.
// Remainder tiles (32 and 64 rows) run the same kernel with one wave along
// the tokens; their smaller register and LDS footprint lets several
// workgroups share a CU.  Four-wave workgroups (two per CU) made the 128-row
// gate_up faster in isolation but the whole forward slower, as they leave
// no room on a CU for the remainder tiles of the side stream.
template <bool GATEUP, int BM>
struct TileCfg;
template <> struct TileCfg<true, 128> { static constexpr int NW = 8, WM = 1, NB = 2, MINW = 2; };
template <> struct TileCfg<false, 128> { static constexpr int NW = 8, WM = 2, NB = 4, MINW = 2; };
template <> struct TileCfg<true, 64> { static constexpr int NW = 8, WM = 1, NB = 2, MINW = 4; };
template <> struct TileCfg<false, 64> { static constexpr int NW = 8, WM = 1, NB = 4, MINW = 2; };
template <> struct TileCfg<true, 32> { static constexpr int NW = 8, WM = 1, NB = 2, MINW = 6; };
template <> struct TileCfg<false, 32> { static constexpr int NW = 8, WM = 1, NB = 4, MINW = 4; };

template <bool GATEUP, int BM, bool MX>
hipError_t launch_tiles(const PrefillArgs& a, int cls, int max_tiles, hipStream_t s) {
    using C = TileCfg<GATEUP, BM>;
    const int cols = GATEUP ? (C::NW / C::WM) * 8 * C::NB : (C::NW / C::WM) * 16 * C::NB;  // h-columns or output rows
    const int ntn = ceil_div(GATEUP ? a.I : a.H, cols);
    // the MXFP4 32-row down (two activation fragments per MFMA step) needs more registers than four waves per SIMD
    constexpr int MINW = MX && !GATEUP && BM == 32 ? 3 : C::MINW;
    hipLaunchKernelGGL((tile_gemm_kernel<GATEUP, BM, C::NW, C::WM, C::NB, MINW, MX>), dim3(max_tiles * ntn),
                       dim3(C::NW * kWave), 0, s, a, cls, ntn);
    return hipGetLastError();
}

// ------------------------------------------------------------------ combine
// One thread per 8 output columns of token t (one 16-byte load per expert
// row; 8 columns never straddle a 256-column exponent chunk); the k expert
// rows are read in groups of 8 with every load of a group in flight before the
// first add (rows past k read as zero), brought back to fp32 by their chunk's
// exponent and added in assignment order.
struct O8 {
    f32x4_t lo, hi;
};
__device__ __forceinline__ O8 load_o8(const rsrc_t& ores, const rsrc_t& xres, int row, int c8, int H8, int OT,
                                      bool valid) {
    const int ch = (8 * c8) / 256;
    const int e = (int)buf_load4(xres, valid ? 4 * (row * OT + ch) : kOob);
    const u32x4_t h = buf_load16(ores, valid ? 16 * (row * H8 + c8) : kOob);
    const float sc = e == kNoExp ? 0.0f : ldexpf(1.0f, -e);
    // word_of, not h.y: __builtin_bit_cast of a vector element (h.y) compiles here to a cast of element 0
    const f16x2_t h0 = __builtin_bit_cast(f16x2_t, word_of(h, 0)), h1 = __builtin_bit_cast(f16x2_t, word_of(h, 1));
    const f16x2_t h2 = __builtin_bit_cast(f16x2_t, word_of(h, 2)), h3 = __builtin_bit_cast(f16x2_t, word_of(h, 3));
    return O8{f32x4_t{(float)h0.x, (float)h0.y, (float)h1.x, (float)h1.y} * sc,
              f32x4_t{(float)h2.x, (float)h2.y, (float)h3.x, (float)h3.y} * sc};
}

__global__ void __launch_bounds__(256) combine_kernel(PrefillArgs a, int nchunk) {
    const int t = blockIdx.x / nchunk, chunk = blockIdx.x % nchunk;
    const int H = a.H, T = a.T, k = a.k, H8 = H / 8, OT = a.OT;
    const int c8 = chunk * 256 + (int)threadIdx.x;
    if (c8 >= H8) return;
    const int rows = T * k + T;
    const rsrc_t ores = make_rsrc(a.obuf, (uint32_t)((size_t)rows * H * 2));
    const rsrc_t xres = make_rsrc(a.oexp, (uint32_t)((size_t)rows * OT * 4));
    f32x4_t lo = {0.0f, 0.0f, 0.0f, 0.0f}, hi = lo;
    for (int j0 = 0; j0 < k; j0 += 8) {
        O8 v[8];
        float wj[8];
        bool ok[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int j = j0 + i, aidx = t * k + j;
            const bool valid = j < k;
            const int p = valid ? a.assign_pos[aidx] : 0;
            v[i] = load_o8(ores, xres, p, c8, H8, OT, valid);
            wj[i] = valid ? a.w[aidx] : 0.0f;
            ok[i] = valid && slot_in_bank(a, a.slot_of_expert[a.ids[aidx]]);
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (ok[i]) lo += wj[i] * v[i].lo, hi += wj[i] * v[i].hi;
    }
    if (a.shared != nullptr) {
        const O8 vs = load_o8(ores, xres, T * k + t, c8, H8, OT, true);
        lo += a.sbuf[t] * vs.lo;
        hi += a.sbuf[t] * vs.hi;
    }
    f32x4_t* yp = reinterpret_cast<f32x4_t*>(a.y + (size_t)t * H) + 2 * c8;
    if (a.accumulate) lo += yp[0], hi += yp[1];
    yp[0] = lo;
    yp[1] = hi;
}

// The 128-row tiles (matrix-core bound) and the 32/64-row remainder tiles
// (bound by streaming their experts' weights) are independent until the
// combine, so the remainder GEMMs run on a second stream forked from and
// joined back to the caller's stream with events: the two kinds of work share
// the chip instead of following each other.  One side stream and event pair
// per caller stream (calls on one stream are ordered, so their events can be
// reused); default priority.
struct Fork {
    hipStream_t side = nullptr;
    hipEvent_t forked = nullptr, joined = nullptr;
};

std::mutex g_fork_mu;
std::map<hipStream_t, Fork> g_forks;

hipError_t fork_for(hipStream_t s, Fork& out) {
    std::lock_guard<std::mutex> lock(g_fork_mu);
    auto it = g_forks.find(s);
    if (it != g_forks.end()) {
        out = it->second;
        return hipSuccess;
    }
    Fork f;
    hipError_t e = hipStreamCreateWithFlags(&f.side, hipStreamNonBlocking);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&f.forked, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&f.joined, hipEventDisableTiming);
    if (e != hipSuccess) {  // nothing half-made is kept
        if (f.joined) (void)hipEventDestroy(f.joined);
        if (f.forked) (void)hipEventDestroy(f.forked);
        if (f.side) (void)hipStreamDestroy(f.side);
        return e;
    }
    g_forks[s] = f;
    out = f;
    return hipSuccess;
}

}  // namespace

// Every side stream and event pair the prefill path created: each side stream is synchronised, then destroyed.
hipError_t release_side_streams() {
    std::lock_guard<std::mutex> lock(g_fork_mu);
    hipError_t first = hipSuccess;
    for (auto& kv : g_forks) {
        Fork& f = kv.second;
        hipError_t e = hipStreamSynchronize(f.side);
        if (e == hipSuccess) e = hipEventDestroy(f.forked);
        if (e == hipSuccess) e = hipEventDestroy(f.joined);
        if (e == hipSuccess) e = hipStreamDestroy(f.side);
        if (e != hipSuccess && first == hipSuccess) first = e;
    }
    g_forks.clear();
    return first;
}

bool prefill_shape_supported(int H, int I) { return H % 128 == 0 && I % 32 == 0 && H <= 8192; }

namespace {

// prep + plan, the grouped GEMMs (remainder tiles on the side stream), the combine
template <bool MX>
hipError_t run_prefill(const PrefillArgs& a, hipStream_t s) {
    const int rows = a.T * a.k + a.T;
    const int G = a.E + 1;
    const int max128 = min(a.cap, rows / 128 + G);
    const int maxsmall = min(a.cap, G);
    // the side stream and its events exist before anything is enqueued, so a failure here enqueues nothing
    Fork f;
    hipError_t e = fork_for(s, f);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(prep_plan_kernel, dim3(a.T + 1), dim3(256), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    // remainder tiles on the side stream, 128-row tiles on the caller's stream
    if ((e = hipEventRecord(f.forked, s)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(f.side, f.forked, 0)) != hipSuccess) return e;
    if ((e = launch_tiles<true, 64, MX>(a, 1, maxsmall, f.side)) != hipSuccess) return e;
    if ((e = launch_tiles<true, 32, MX>(a, 2, maxsmall, f.side)) != hipSuccess) return e;
    if ((e = launch_tiles<false, 64, MX>(a, 1, maxsmall, f.side)) != hipSuccess) return e;
    if ((e = launch_tiles<false, 32, MX>(a, 2, maxsmall, f.side)) != hipSuccess) return e;
    if ((e = hipEventRecord(f.joined, f.side)) != hipSuccess) return e;
    if ((e = launch_tiles<true, 128, MX>(a, 0, max128, s)) != hipSuccess) return e;
    if ((e = launch_tiles<false, 128, MX>(a, 0, max128, s)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(s, f.joined, 0)) != hipSuccess) return e;
    const int nchunk = ceil_div(a.H / 8, 256);
    hipLaunchKernelGGL(combine_kernel, dim3(a.T * nchunk), dim3(256), 0, s, a, nchunk);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(const Layer& L, const uint16_t* x, int T, const float* w, const int32_t* ids,
                          const int32_t* offsets, const int32_t* sorted_assign, const int32_t* assign_pos, float* y,
                          int accumulate, void* ws, hipStream_t s, bool mx) {
    const int H = L.H, I = L.I, E = L.E, k = L.k;
    uint8_t* p = static_cast<uint8_t*>(ws);
    const WsLayout wl = ws_layout(T, H, I, E, k, mx);
    PrefillArgs a;
    a.bank = L.bank; a.slot_bytes = L.slot_bytes; a.num_slots = L.num_slots; a.slot_of_expert = L.slot_of_expert;
    a.shared = L.shared; a.wg = L.wg; a.x = x;
    a.T = T; a.H = H; a.I = I; a.E = E; a.k = k;
    a.w = w; a.ids = ids; a.offsets = offsets; a.sorted_assign = sorted_assign; a.assign_pos = assign_pos;
    a.hbuf = reinterpret_cast<_Float16*>(p + wl.h);
    a.hmx = reinterpret_cast<uint16_t*>(p + wl.h);
    a.mx = mx ? 1 : 0;
    a.hexp = reinterpret_cast<int*>(p + wl.hx);
    a.KT = ceil_div(I, BK);
    a.obuf = reinterpret_cast<_Float16*>(p + wl.o);
    a.oexp = reinterpret_cast<int*>(p + wl.ox);
    a.OT = ceil_div(H, 256);
    a.x16 = reinterpret_cast<_Float16*>(p + wl.x16);
    a.xinv = reinterpret_cast<float*>(p + wl.xinv);
    a.sbuf = reinterpret_cast<float*>(p + wl.s);
    a.tiles = reinterpret_cast<int*>(p + wl.tiles);
    a.cap = wl.tile_cap;
    a.y = y; a.accumulate = accumulate;
    const SlotGeom gm = mx ? mx_slot_geom(H, I) : slot_geom(H, I);
    a.gu_codes = gm.gu_codes; a.gu_scales = gm.gu_scales; a.gu_glob = gm.gu_glob;
    a.dn_codes = gm.dn_codes; a.dn_scales = gm.dn_scales; a.dn_glob = gm.dn_glob;
    return mx ? run_prefill<true>(a, s) : run_prefill<false>(a, s);
}

}  // namespace moe
