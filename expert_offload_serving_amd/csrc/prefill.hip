// Prefill path (T > 16) of the NVFP4 routed-MoE layer for gfx950.
//
// With thousands of tokens each expert sees a dense block of rows, so the
// expert FFN becomes a grouped GEMM over the permuted tokens (the
// permutation groups the T*k assignments by expert; the shared expert is one
// more group holding every token).  NVFP4 is not an MFMA input format with
// E4M3 16-blocks, but e2m1 * e4m3 has at most 6 significant bits, so each
// weight tile is dequantised exactly to bf16 in LDS and fed to
// v_mfma_f32_32x32x16_bf16 with fp32 accumulation; the per-row global
// multiplies the accumulator in the epilogue.
//
//   plan:     list the (group, 128-row m-tile) work items of active groups
//   gate_up:  C[m, n] = sum_h x[tok(m), h] W_gu[n, h] for 64 gate rows and the
//             matching 64 up rows per tile; epilogue h = silu(gate) * up -> bf16
//   down:     O[m, n] = sum_i h[m, i] W_dn[n, i] -> fp32 per assignment row
//   combine:  y_t = sum_j w_tj O[pos(t,j)] + sigmoid(x_t . w_g) O[shared row t]
// The hidden state is rounded to bf16 (the MFMA input type); everything else
// accumulates in fp32, and the combine order is fixed.
#include "internal.hpp"
#include "nvfp4_device.hpp"

namespace moe {
namespace {

constexpr int BM = 128;        // tokens per tile
constexpr int BN = 128;        // weight rows per tile (gate_up: 64 gate + 64 up)
constexpr int BK = 64;         // contraction step
constexpr int LDSP = BK + 8;   // LDS row pitch in bf16 elements (144 B: spreads rows over banks)

struct PrefillArgs {
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
    uint16_t* hbuf;   // bf16 [(T*k + T), I]
    float* obuf;      // f32  [(T*k + T), H]
    int* tiles;       // [1 + 2 * max_tiles]: count, then (group, m0) pairs
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
__device__ __forceinline__ bool group_active(const PrefillArgs& a, int g) {
    if (g == a.E) return a.shared != nullptr;
    return a.offsets[g + 1] > a.offsets[g] && a.slot_of_expert[g] >= 0;
}
__device__ __forceinline__ const uint8_t* group_slot(const PrefillArgs& a, int g) {
    return g == a.E ? a.shared : a.bank + (size_t)a.slot_of_expert[g] * a.slot_bytes;
}

__global__ void __launch_bounds__(256) plan_kernel(PrefillArgs a) {
    __shared__ int wsum[4];
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int G = a.E + 1;
    const int per = (G + 255) / 256;
    const int g0 = tid * per, g1 = min(G, g0 + per);
    int cnt = 0;
    for (int g = g0; g < g1; ++g)
        if (group_active(a, g)) cnt += ceil_div(group_end(a, g) - group_begin(a, g), BM);
    int incl = cnt;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        int o = __shfl_up(incl, off, kWave);
        if (lane >= off) incl += o;
    }
    if (lane == kWave - 1) wsum[wave] = incl;
    __syncthreads();
    int before = 0, total = 0;
    for (int i = 0; i < 4; ++i) {
        if (i < wave) before += wsum[i];
        total += wsum[i];
    }
    int pos = before + incl - cnt;
    for (int g = g0; g < g1; ++g) {
        if (!group_active(a, g)) continue;
        const int n = group_end(a, g) - group_begin(a, g);
        for (int m0 = 0; m0 < n; m0 += BM) {
            a.tiles[1 + 2 * pos] = g;
            a.tiles[2 + 2 * pos] = m0;
            ++pos;
        }
    }
    if (tid == 0) a.tiles[0] = total;
}

// Dequantise 32 consecutive elements (16 code bytes, 2 scale bytes) to bf16 in LDS.
__device__ __forceinline__ void dequant32_to_lds(u32x4_t cw, uint32_t s16, __bf16* dst) {
    const float s0 = e4m3_f32<0>(s16), s1 = e4m3_f32<1>(s16);
    const uint32_t words[4] = {cw.x, cw.y, cw.z, cw.w};
    uint32_t packed[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float s = q < 2 ? s0 : s1;
        f32x2_t v0 = e2m1x2_f32<0>(words[q]), v1 = e2m1x2_f32<1>(words[q]);
        f32x2_t v2 = e2m1x2_f32<2>(words[q]), v3 = e2m1x2_f32<3>(words[q]);
        // products are exact in bf16; the conversion only drops zero bits
        bf16x2_t b0 = {(__bf16)(v0.x * s), (__bf16)(v0.y * s)};
        bf16x2_t b1 = {(__bf16)(v1.x * s), (__bf16)(v1.y * s)};
        bf16x2_t b2 = {(__bf16)(v2.x * s), (__bf16)(v2.y * s)};
        bf16x2_t b3 = {(__bf16)(v3.x * s), (__bf16)(v3.y * s)};
        packed[4 * q + 0] = __builtin_bit_cast(uint32_t, b0);
        packed[4 * q + 1] = __builtin_bit_cast(uint32_t, b1);
        packed[4 * q + 2] = __builtin_bit_cast(uint32_t, b2);
        packed[4 * q + 3] = __builtin_bit_cast(uint32_t, b3);
    }
    u32x4_t* d = reinterpret_cast<u32x4_t*>(dst);
#pragma unroll
    for (int q = 0; q < 4; ++q) d[q] = u32x4_t{packed[4 * q], packed[4 * q + 1], packed[4 * q + 2], packed[4 * q + 3]};
}

__device__ __forceinline__ bf16x8_t lds_frag(const __bf16* p) {
    return __builtin_bit_cast(bf16x8_t, *reinterpret_cast<const u32x4_t*>(p));
}

// Row i (0..31 within a 32x32 block) of accumulator register r for lane l.
__device__ __forceinline__ int acc_row(int r, int lane) { return (r / 4) * 8 + (lane / 32) * 4 + (r % 4); }

// ------------------------------------------------------------------ gate_up + SwiGLU
__global__ void __launch_bounds__(256) gateup_mfma_kernel(PrefillArgs a) {
    __shared__ __attribute__((aligned(16))) __bf16 sA[BM * LDSP];
    __shared__ __attribute__((aligned(16))) __bf16 sB[BN * LDSP];
    __shared__ int tok[BM];

    const int n_tiles_n = ceil_div(a.I, BN / 2);
    const int tile = blockIdx.x / n_tiles_n, nt = blockIdx.x % n_tiles_n;
    if (tile >= a.tiles[0]) return;
    const int g = a.tiles[1 + 2 * tile], m0 = a.tiles[2 + 2 * tile];
    const int gb = group_begin(a, g), cnt = min(BM, group_end(a, g) - gb - m0);
    const uint8_t* slot = group_slot(a, g);
    const int H = a.H, I = a.I;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int wm = wave >> 1, wn = wave & 1;
    const int n0 = nt * (BN / 2);  // first h column (gate row) of the tile

    for (int m = tid; m < BM; m += 256) {
        int t = -1;
        if (m < cnt) {
            const int p = gb + m0 + m;
            t = g < a.E ? a.sorted_assign[p] / a.k : p - a.T * a.k;
        }
        tok[m] = t;
    }
    __syncthreads();

    // loader roles: row = tid / 2, 32-element half = tid % 2
    const int lrow = tid >> 1, lhalf = tid & 1;
    const int my_tok = tok[lrow];
    // B row: tile rows [0, 64) are gate rows n0.., [64, 128) are up rows I + n0..
    const int hcol = n0 + (lrow & 63);
    const bool brow_ok = hcol < I;
    const int wrow = (lrow < 64 ? 0 : I) + (brow_ok ? hcol : 0);
    const uint8_t* bcodes = slot + a.gu_codes + (size_t)wrow * (H / 2);
    const uint8_t* bscales = slot + a.gu_scales + (size_t)wrow * (H / 16);
    const uint16_t* xrow = a.x + (size_t)(my_tok < 0 ? 0 : my_tok) * H;

    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    for (int k0 = 0; k0 < H; k0 += BK) {
        const int kc = k0 + 32 * lhalf;
        const bool kok = kc < H;
        // A: 32 activations of row lrow
        u32x4_t av[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) av[q] = u32x4_t{0, 0, 0, 0};
        if (my_tok >= 0 && kok) {
            const u32x4_t* src = reinterpret_cast<const u32x4_t*>(xrow + kc);
#pragma unroll
            for (int q = 0; q < 4; ++q) av[q] = src[q];
        }
        // B: 32 weights of row lrow
        u32x4_t cw = u32x4_t{0, 0, 0, 0};
        uint32_t s16 = 0;
        if (brow_ok && kok) {
            cw = *reinterpret_cast<const u32x4_t*>(bcodes + kc / 2);
            s16 = *reinterpret_cast<const uint16_t*>(bscales + kc / 16);
        }
        __syncthreads();
        u32x4_t* da = reinterpret_cast<u32x4_t*>(sA + lrow * LDSP + 32 * lhalf);
#pragma unroll
        for (int q = 0; q < 4; ++q) da[q] = av[q];
        dequant32_to_lds(cw, s16, sB + lrow * LDSP + 32 * lhalf);
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < BK; kk += 16) {
            const int ko = kk + 8 * (lane / 32);
            bf16x8_t fa[2], fb[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) fa[i] = lds_frag(sA + (64 * wm + 32 * i + lane % 32) * LDSP + ko);
            // j = 0: gate rows, j = 1: up rows, both for h columns [32 wn, 32 wn + 32)
#pragma unroll
            for (int j = 0; j < 2; ++j) fb[j] = lds_frag(sB + (64 * j + 32 * wn + lane % 32) * LDSP + ko);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
    }

    // epilogue: lane holds column (lane % 32) of each 32x32 block
    const int col = n0 + 32 * wn + lane % 32;
    if (col < I) {
        const float* gl = reinterpret_cast<const float*>(slot + a.gu_glob);
        const float gg = gl[col], gu = gl[I + col];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = 64 * wm + 32 * i + acc_row(r, lane);
                if (m < cnt) {
                    const float gate = acc[i][0][r] * gg, up = acc[i][1][r] * gu;
                    const __bf16 hv = (__bf16)(gate * sigmoidf_(gate) * up);
                    a.hbuf[(size_t)(gb + m0 + m) * I + col] = __builtin_bit_cast(uint16_t, hv);
                }
            }
    }
}

// ------------------------------------------------------------------ down
__global__ void __launch_bounds__(256) down_mfma_kernel(PrefillArgs a) {
    __shared__ __attribute__((aligned(16))) __bf16 sA[BM * LDSP];
    __shared__ __attribute__((aligned(16))) __bf16 sB[BN * LDSP];

    const int n_tiles_n = ceil_div(a.H, BN);
    const int tile = blockIdx.x / n_tiles_n, nt = blockIdx.x % n_tiles_n;
    if (tile >= a.tiles[0]) return;
    const int g = a.tiles[1 + 2 * tile], m0 = a.tiles[2 + 2 * tile];
    const int gb = group_begin(a, g), cnt = min(BM, group_end(a, g) - gb - m0);
    const uint8_t* slot = group_slot(a, g);
    const int H = a.H, I = a.I;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int wm = wave >> 1, wn = wave & 1;
    const int n0 = nt * BN;

    const int lrow = tid >> 1, lhalf = tid & 1;
    const bool arow_ok = lrow < cnt;
    const uint16_t* hrow = a.hbuf + (size_t)(gb + m0 + (arow_ok ? lrow : 0)) * I;
    const int orow = n0 + lrow;
    const bool brow_ok = orow < H;
    const uint8_t* bcodes = slot + a.dn_codes + (size_t)(brow_ok ? orow : 0) * (I / 2);
    const uint8_t* bscales = slot + a.dn_scales + (size_t)(brow_ok ? orow : 0) * (I / 16);

    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    for (int k0 = 0; k0 < I; k0 += BK) {
        const int kc = k0 + 32 * lhalf;
        const bool kok = kc < I;
        u32x4_t av[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) av[q] = u32x4_t{0, 0, 0, 0};
        if (arow_ok && kok) {
            const u32x4_t* src = reinterpret_cast<const u32x4_t*>(hrow + kc);
#pragma unroll
            for (int q = 0; q < 4; ++q) av[q] = src[q];
        }
        u32x4_t cw = u32x4_t{0, 0, 0, 0};
        uint32_t s16 = 0;
        if (brow_ok && kok) {
            cw = *reinterpret_cast<const u32x4_t*>(bcodes + kc / 2);
            s16 = *reinterpret_cast<const uint16_t*>(bscales + kc / 16);
        }
        __syncthreads();
        u32x4_t* da = reinterpret_cast<u32x4_t*>(sA + lrow * LDSP + 32 * lhalf);
#pragma unroll
        for (int q = 0; q < 4; ++q) da[q] = av[q];
        dequant32_to_lds(cw, s16, sB + lrow * LDSP + 32 * lhalf);
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < BK; kk += 16) {
            const int ko = kk + 8 * (lane / 32);
            bf16x8_t fa[2], fb[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) fa[i] = lds_frag(sA + (64 * wm + 32 * i + lane % 32) * LDSP + ko);
#pragma unroll
            for (int j = 0; j < 2; ++j) fb[j] = lds_frag(sB + (64 * wn + 32 * j + lane % 32) * LDSP + ko);
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fa[i], fb[j], acc[i][j], 0, 0, 0);
        }
    }

    const float* gl = reinterpret_cast<const float*>(slot + a.dn_glob);
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int col = n0 + 64 * wn + 32 * j + lane % 32;
        if (col >= H) continue;
        const float gd = gl[col];
#pragma unroll
        for (int i = 0; i < 2; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = 64 * wm + 32 * i + acc_row(r, lane);
                if (m < cnt) a.obuf[(size_t)(gb + m0 + m) * H + col] = acc[i][j][r] * gd;
            }
    }
}

// ------------------------------------------------------------------ combine
__global__ void __launch_bounds__(256) combine_kernel(PrefillArgs a) {
    __shared__ float red[4];
    __shared__ float s_sh;
    const int t = blockIdx.x;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int H = a.H, T = a.T, k = a.k;
    if (a.shared != nullptr) {
        float acc = 0.0f;
        for (int c = tid; c < H; c += 256)
            acc += bf16_bits_f32(a.x[(size_t)t * H + c]) * bf16_bits_f32(a.wg[c]);
        acc = wave_sum(acc);
        if (lane == 0) red[wave] = acc;
        __syncthreads();
        if (tid == 0) s_sh = sigmoidf_(red[0] + red[1] + red[2] + red[3]);
        __syncthreads();
    }
    for (int n = tid; n < H; n += 256) {
        float acc = 0.0f;
        for (int j = 0; j < k; ++j) {
            const int aidx = t * k + j;
            if (a.slot_of_expert[a.ids[aidx]] >= 0) acc += a.w[aidx] * a.obuf[(size_t)a.assign_pos[aidx] * H + n];
        }
        if (a.shared != nullptr) acc += s_sh * a.obuf[(size_t)(T * k + t) * H + n];
        float* yp = a.y + (size_t)t * H + n;
        *yp = a.accumulate ? *yp + acc : acc;
    }
}

}  // namespace

bool prefill_shape_supported(int H, int I) { return H % 32 == 0 && I % 32 == 0; }

hipError_t launch_prefill(const Layer& L, const uint16_t* x, int T, const float* w, const int32_t* ids,
                          const int32_t* offsets, const int32_t* sorted_assign, const int32_t* assign_pos, float* y,
                          int accumulate, void* ws, hipStream_t s) {
    const int H = L.H, I = L.I, E = L.E, k = L.k;
    const int nrows_all = T * k + T;
    uint8_t* p = static_cast<uint8_t*>(ws);
    PrefillArgs a;
    a.bank = L.bank; a.slot_bytes = L.slot_bytes; a.slot_of_expert = L.slot_of_expert;
    a.shared = L.shared; a.wg = L.wg; a.x = x;
    a.T = T; a.H = H; a.I = I; a.E = E; a.k = k;
    a.w = w; a.ids = ids; a.offsets = offsets; a.sorted_assign = sorted_assign; a.assign_pos = assign_pos;
    a.hbuf = reinterpret_cast<uint16_t*>(p);
    p += (size_t)nrows_all * I * 4;  // sized for the f32 decode layout; bf16 uses half
    a.obuf = reinterpret_cast<float*>(p);
    p += (size_t)nrows_all * H * 4;
    p += 256 * ((T * 4 + 255) / 256);
    p += 256 * (((H + 63) / 64 * 4 + 255) / 256);
    a.tiles = reinterpret_cast<int*>(p);
    a.y = y; a.accumulate = accumulate;
    SlotGeom gm = slot_geom(H, I);
    a.gu_codes = gm.gu_codes; a.gu_scales = gm.gu_scales; a.gu_glob = gm.gu_glob;
    a.dn_codes = gm.dn_codes; a.dn_scales = gm.dn_scales; a.dn_glob = gm.dn_glob;

    const int max_tiles = ceil_div(nrows_all, BM) + E + 1;
    hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(256), 0, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(gateup_mfma_kernel, dim3(max_tiles * ceil_div(I, BN / 2)), dim3(256), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(down_mfma_kernel, dim3(max_tiles * ceil_div(H, BN)), dim3(256), 0, s, a);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(combine_kernel, dim3(T), dim3(256), 0, s, a);
    return hipGetLastError();
}

size_t forward_ws_bytes(int T, int H, int I, int E, int k) {
    const size_t nrows_all = (size_t)T * k + T;
    size_t b = nrows_all * I * 4 + nrows_all * H * 4;
    b += 256 * (((size_t)T * 4 + 255) / 256);
    b += 256 * ((((size_t)H + 63) / 64 * 4 + 255) / 256);
    const size_t max_tiles = (nrows_all + BM - 1) / BM + E + 1;
    b += 256 * (((1 + 2 * max_tiles) * 4 + 255) / 256);
    return b;
}

}  // namespace moe
