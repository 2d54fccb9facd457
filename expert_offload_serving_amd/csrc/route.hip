// Top-k routing with renormalised weights and the deterministic permutation
// of assignments by expert, for gfx950.
//
// Routing follows the replicated router with norm_topk_prob of the pages
// (issue #62, R9700 interim report: "norm_topk_prob defaults True and the
// router is replicated"): the k largest logits are selected and their
// weights are the softmax over those k logits, which equals a full softmax
// renormalised over the selected experts.  Selection order is (logit
// descending, expert index ascending).  The permutation groups the T*k
// assignments by expert with a stable counting sort (per-expert counts,
// exclusive scan, then stable ranks from wave ballots), so the grouping is
// bit-reproducible: no atomic operation decides an order (atomics only count).
#include "internal.hpp"
#include "nvfp4_device.hpp"

namespace moe {
namespace {

constexpr int kMaxE = 1024;
constexpr int kVPL = kMaxE / kWave;  // logits held per lane

// Selection order as one unsigned 64-bit key per (logit, expert): the high
// word maps the logit monotonically onto uint32 (-0 folded onto +0, so equal
// logits tie), the low word is ~index, so a larger key ranks first and ties
// go to the lower index.  Key 0 means "no candidate" (every real key has a
// nonzero low word).  A NaN logit maps to some key; NaN input is a
// precondition violation and only has to leave a valid, untaken expert.
__device__ __forceinline__ uint64_t rank_key(float v, int idx) {
    uint32_t u = __float_as_uint(v + 0.0f);
    u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)u << 32) | (uint32_t)~(uint32_t)idx;
}
__device__ __forceinline__ int key_index(uint64_t key) { return (int)~(uint32_t)key; }
// The logit of a key (a -0 logit comes back as +0, which no later step can tell apart).
__device__ __forceinline__ float key_value(uint64_t key) {
    const uint32_t u = (uint32_t)(key >> 32);
    return __uint_as_float((u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u);
}

// DPP row operations of the GCN/CDNA ISA (gfx9 encodings).
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr3 = 0x113, kDppRowShr4 = 0x114,
              kDppRowShr8 = 0x118, kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;

// One branch-free step of a wave max over 64-bit keys: take the key DPP
// control CTRL brings in when it is larger; lanes the masks disable keep
// their own (old operand = own key).
template <int CTRL, int ROW_MASK, int BANK_MASK>
__device__ __forceinline__ uint64_t kmax_step(uint64_t key) {
    const uint32_t lo = (uint32_t)key, hi = (uint32_t)(key >> 32);
    const uint32_t olo = (uint32_t)__builtin_amdgcn_update_dpp((int)lo, (int)lo, CTRL, ROW_MASK, BANK_MASK, false);
    const uint32_t ohi = (uint32_t)__builtin_amdgcn_update_dpp((int)hi, (int)hi, CTRL, ROW_MASK, BANK_MASK, false);
    const uint64_t other = ((uint64_t)ohi << 32) | olo;
    return other > key ? other : key;
}

// Wave-wide maximum key, returned to every lane.  The DPP sequence leaves
// the result in lane 63 (shifts within each 16-lane row, then the row
// broadcasts); max tolerates the overlapping inputs.
__device__ __forceinline__ uint64_t wave_max_key(uint64_t key) {
    key = kmax_step<kDppRowShr1, 0xF, 0xF>(key);
    key = kmax_step<kDppRowShr2, 0xF, 0xF>(key);
    key = kmax_step<kDppRowShr3, 0xF, 0xF>(key);
    key = kmax_step<kDppRowShr4, 0xF, 0xE>(key);
    key = kmax_step<kDppRowShr8, 0xF, 0xC>(key);
    key = kmax_step<kDppRowBcast15, 0xA, 0xF>(key);
    key = kmax_step<kDppRowBcast31, 0xC, 0xF>(key);
    const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)key, 63);
    const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)(key >> 32), 63);
    return ((uint64_t)hi << 32) | lo;
}

// One wave selects the top-k of row `l` (E <= 64 * VPL logits) and writes
// ids and weights.  Selection: k rounds of a wave maximum over each lane's
// best remaining key.  Weights: softmax over the k selected logits in
// double (exp(l_j - l_max) / sum), summed in selection order, rounded to f32.
template <int VPL>
__device__ void topk_one_token(const float* __restrict__ l, int E, int k, int32_t* __restrict__ ids,
                               float* __restrict__ w, int lane) {
    static_assert(VPL <= kVPL, "too many logits per lane");
    uint64_t key[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        const int idx = lane + kWave * i;
        key[i] = idx < E ? rank_key(l[idx], idx) : 0ull;
    }
    float held = 0.0f;  // selection j's logit, kept by lane j (j < 64)
    float m = 0.0f;
    for (int j = 0; j < k; ++j) {
        uint64_t best = key[0];
#pragma unroll
        for (int i = 1; i < VPL; ++i) best = key[i] > best ? key[i] : best;
        best = wave_max_key(best);
        const int bi = key_index(best);
        const int owner_slot = bi / kWave, owner_lane = bi % kWave;
        const float bv = key_value(best);
#pragma unroll
        for (int i = 0; i < VPL; ++i) key[i] = (i == owner_slot && lane == owner_lane) ? 0ull : key[i];
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

template <int VPL>
__global__ void __launch_bounds__(256) topk_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                    int32_t* __restrict__ ids, float* __restrict__ w) {
    int t = blockIdx.x * 4 + threadIdx.x / kWave;
    if (t >= T) return;
    int lane = threadIdx.x % kWave;
    topk_one_token<VPL>(logits + (size_t)t * E, E, k, ids + (size_t)t * k, w + (size_t)t * k, lane);
}

// Multi-workgroup stable counting sort for large batches.  Block b owns the
// assignments [1024 b, 1024 b + 1024).  perm_count writes each block's
// per-expert histogram; perm_scatter (one workgroup per block again) adds the
// histograms of the earlier blocks and the per-expert totals to get where its
// assignments of each expert start, then ranks them stably inside the block
// (wave ballots, waves in order) and scatters them.
constexpr int kPermBlock = 1024;

__global__ void __launch_bounds__(1024) perm_count_kernel(const int32_t* __restrict__ ids, int n, int E,
                                                           int32_t* __restrict__ block_hist) {
    __shared__ int hist[kMaxE];
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += 1024) hist[e] = 0;
    __syncthreads();
    const int a = blockIdx.x * kPermBlock + tid;
    if (a < n) atomicAdd(&hist[ids[a]], 1);
    __syncthreads();
    for (int e = tid; e < E; e += 1024) block_hist[(size_t)blockIdx.x * E + e] = hist[e];
}

__global__ void __launch_bounds__(1024) perm_scatter_kernel(const int32_t* __restrict__ ids, int n, int E, int nblocks,
                                                             const int32_t* __restrict__ block_hist,
                                                             int32_t* __restrict__ offsets,
                                                             int32_t* __restrict__ sorted_assign,
                                                             int32_t* __restrict__ assign_pos) {
    __shared__ int run[kMaxE];
    __shared__ int wsum[16];
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int b = blockIdx.x;
    // per expert (one per thread): total over all blocks, and the part in blocks before b
    int total = 0, before_b = 0;
    if (tid < E) {
        for (int bb = 0; bb < nblocks; ++bb) {
            const int h = block_hist[(size_t)bb * E + tid];
            total += h;
            if (bb < b) before_b += h;
        }
    }
    // exclusive scan of the totals over experts
    int incl = total;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const int o = __shfl_up(incl, off, kWave);
        if (lane >= off) incl += o;
    }
    if (lane == kWave - 1) wsum[wave] = incl;
    __syncthreads();
    int wbefore = 0;
    for (int i = 0; i < wave; ++i) wbefore += wsum[i];
    const int excl = wbefore + incl - total;
    if (tid < E) {
        run[tid] = excl + before_b;
        if (b == 0) offsets[tid] = excl;
    }
    if (b == 0 && tid == 0) offsets[E] = n;
    __syncthreads();
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int a = b * kPermBlock + tid;
    const bool valid = a < n;
    const int e = valid ? ids[a] : 0;
    uint64_t peers = __ballot(valid);
    for (int bit = 0; bit < nbits; ++bit) {
        const bool on = (e >> bit) & 1;
        const uint64_t m = __ballot(on);
        peers &= on ? m : ~m;
    }
    const int rank = __popcll(peers & lt_mask);
    const int cw = __popcll(peers);
    const int last_wave = (min(kPermBlock, n - b * kPermBlock) - 1) / kWave;
    for (int w2 = 0; w2 <= last_wave; ++w2) {
        if (wave == w2 && valid) {
            const int b0 = run[e];
            const int pos = b0 + rank;
            if (rank == 0) run[e] = b0 + cw;
            sorted_assign[pos] = a;
            assign_pos[a] = pos;
        }
        __syncthreads();
    }
}

// Decode batches (T <= 16, T*k <= kDirectMaxAssign): one workgroup with one
// wave per token selects the top-k, then ranks every assignment directly:
//   offsets[e] = #{assignments with expert < e}
//   pos(a)     = #{a' : (e', a') < (e, a)}   (expert, then flat index)
// which is the same stable grouping as the counting sort, in one launch.
constexpr int kDirectMaxAssign = 256;

template <int VPL>
__global__ void __launch_bounds__(1024) route_small_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                            int32_t* __restrict__ ids, float* __restrict__ w,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ sorted_assign,
                                                            int32_t* __restrict__ assign_pos) {
    __shared__ __attribute__((aligned(16))) int32_t ids_lds[kDirectMaxAssign + 4];
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    if (wave < T) topk_one_token<VPL>(logits + (size_t)wave * E, E, k, ids_lds + wave * k, w + (size_t)wave * k, lane);
    const int n = T * k, n4 = (n + 3) / 4;
    if ((int)threadIdx.x < 4 * n4 - n) ids_lds[n + threadIdx.x] = 0x7FFFFFFF;  // pad: ranks after every expert
    __syncthreads();
    const int4* ids4 = reinterpret_cast<const int4*>(ids_lds);
    // pos(a) = #{b : (e_b, b) < (e_a, a)}, scanned four assignments per LDS read
    for (int a = threadIdx.x; a < n; a += blockDim.x) {
        const int e = ids_lds[a];
        int pos = 0;
        for (int q = 0; q < n4; ++q) {
            const int4 v = ids4[q];
            const int b = 4 * q;
            pos += (v.x < e || (v.x == e && b < a)) + (v.y < e || (v.y == e && b + 1 < a)) +
                   (v.z < e || (v.z == e && b + 2 < a)) + (v.w < e || (v.w == e && b + 3 < a));
        }
        ids[a] = e;
        sorted_assign[pos] = a;
        assign_pos[a] = pos;
    }
    // offsets[e] = #{b : e_b < e}
    for (int e = threadIdx.x; e <= E; e += blockDim.x) {
        int c = 0;
        for (int q = 0; q < n4; ++q) {
            const int4 v = ids4[q];
            c += (v.x < e) + (v.y < e) + (v.z < e) + (v.w < e);
        }
        offsets[e] = c;
    }
}

template <int VPL>
hipError_t launch_route_vpl(const float* logits, int T, int E, int k, int32_t* ids, float* w, int32_t* offsets,
                            int32_t* sorted_assign, int32_t* assign_pos, int32_t* ws, hipStream_t s) {
    if (T <= 16 && T * k <= kDirectMaxAssign) {
        const int threads = kWave * max(4, T);
        hipLaunchKernelGGL(route_small_kernel<VPL>, dim3(1), dim3(threads), 0, s, logits, T, E, k, ids, w, offsets,
                           sorted_assign, assign_pos);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(topk_kernel<VPL>, dim3(ceil_div(T, 4)), dim3(256), 0, s, logits, T, E, k, ids, w);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int n = T * k, nblocks = ceil_div(n, kPermBlock);
    hipLaunchKernelGGL(perm_count_kernel, dim3(nblocks), dim3(1024), 0, s, ids, n, E, ws);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    hipLaunchKernelGGL(perm_scatter_kernel, dim3(nblocks), dim3(1024), 0, s, ids, n, E, nblocks,
                       static_cast<const int32_t*>(ws), offsets, sorted_assign, assign_pos);
    return hipGetLastError();
}

}  // namespace

size_t route_ws_bytes(int T, int E, int k) {
    // per-block expert histograms of the multi-workgroup permutation
    const long n = (long)T * k;
    return (size_t)((n + kPermBlock - 1) / kPermBlock) * (size_t)E * 4;
}

hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* w, int32_t* offsets,
                        int32_t* sorted_assign, int32_t* assign_pos, void* ws_v, hipStream_t s) {
    int32_t* ws = static_cast<int32_t*>(ws_v);
    const int vpl = ceil_div(E, kWave);
    if (vpl <= 1) return launch_route_vpl<1>(logits, T, E, k, ids, w, offsets, sorted_assign, assign_pos, ws, s);
    if (vpl <= 2) return launch_route_vpl<2>(logits, T, E, k, ids, w, offsets, sorted_assign, assign_pos, ws, s);
    if (vpl <= 4) return launch_route_vpl<4>(logits, T, E, k, ids, w, offsets, sorted_assign, assign_pos, ws, s);
    if (vpl <= 8) return launch_route_vpl<8>(logits, T, E, k, ids, w, offsets, sorted_assign, assign_pos, ws, s);
    return launch_route_vpl<16>(logits, T, E, k, ids, w, offsets, sorted_assign, assign_pos, ws, s);
}

}  // namespace moe
