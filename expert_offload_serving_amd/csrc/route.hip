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
// bit-reproducible: no atomic operation decides an order.
#include "internal.hpp"
#include "nvfp4_device.hpp"

namespace moe {
namespace {

constexpr int kMaxE = 1024;
constexpr int kVPL = kMaxE / kWave;  // logits held per lane

// (va, ia) ranks before (vb, ib): larger logit first, lower index on ties.
// With a NaN operand neither comparison holds and the index decides, so the
// result is always a valid, untaken expert.
__device__ __forceinline__ bool ranks_before(float va, int ia, float vb, int ib) {
    if (ia < 0) return false;
    if (ib < 0) return true;
    if (va > vb) return true;
    if (va < vb) return false;
    return ia < ib;
}

// One wave selects the top-k of row `l` (E <= 64 * VPL logits) and writes ids and weights.
template <int VPL>
__device__ void topk_one_token(const float* __restrict__ l, int E, int k, int32_t* __restrict__ ids,
                               float* __restrict__ w, int lane) {
    static_assert(VPL <= kVPL, "too many logits per lane");
    float v[VPL];
    uint32_t taken = 0;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        int idx = lane + kWave * i;
        v[i] = idx < E ? l[idx] : 0.0f;
    }
    float held_v[VPL];  // logit of selection j is kept by lane j % 64 in slot j / 64
#pragma unroll
    for (int i = 0; i < VPL; ++i) held_v[i] = 0.0f;
    float m = 0.0f;
    for (int j = 0; j < k; ++j) {
        float bv = 0.0f;
        int bi = -1;
#pragma unroll
        for (int i = 0; i < VPL; ++i) {
            int idx = lane + kWave * i;
            bool ok = idx < E && !((taken >> i) & 1u);
            if (ok && ranks_before(v[i], idx, bv, bi)) bv = v[i], bi = idx;
        }
#pragma unroll
        for (int off = kWave / 2; off > 0; off >>= 1) {
            float ov = __shfl_xor(bv, off, kWave);
            int oi = __shfl_xor(bi, off, kWave);
            if (ranks_before(ov, oi, bv, bi)) bv = ov, bi = oi;
        }
        // bi is the same on every lane (a strict total order without NaN).
        if (bi >= 0 && (bi % kWave) == lane) taken |= 1u << (bi / kWave);
        if (j == 0) m = bv;
        if ((j % kWave) == lane) {
            held_v[j / kWave] = bv;
            ids[j] = bi;
        }
    }
    // Softmax over the selected logits in double, summed in selection order.
    double ex[VPL];
#pragma unroll
    for (int i = 0; i < VPL; ++i) ex[i] = (lane + kWave * i < k) ? exp((double)held_v[i] - (double)m) : 0.0;
    double sum = 0.0;
    for (int j = 0; j < k; ++j) {
        double e = 0.0;
#pragma unroll
        for (int i = 0; i < VPL; ++i)
            if (i == j / kWave) e = ex[i];
        sum += __shfl(e, j % kWave, kWave);
    }
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
        int j = lane + kWave * i;
        if (j < k) w[j] = (float)(ex[i] / sum);
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

// Stable counting sort of n = T*k assignments by expert, one workgroup of
// 1024 threads.  `ids` may be global or LDS memory.
__device__ void permute_block(const int32_t* ids, int n, int E, int32_t* __restrict__ offsets,
                              int32_t* __restrict__ sorted_assign, int32_t* __restrict__ assign_pos, int* cnt,
                              int* run, int* wsum) {
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    for (int e = tid; e < E; e += 1024) cnt[e] = 0;
    __syncthreads();
    for (int a = tid; a < n; a += 1024) atomicAdd(&cnt[ids[a]], 1);
    __syncthreads();
    // Exclusive scan of cnt[0..E) (E <= 1024: one entry per thread).
    int c = tid < E ? cnt[tid] : 0;
    int incl = c;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        int o = __shfl_up(incl, off, kWave);
        if (lane >= off) incl += o;
    }
    if (lane == kWave - 1) wsum[wave] = incl;
    __syncthreads();
    if (tid == 0) {
        int acc = 0;
        for (int i = 0; i < 16; ++i) {
            int s = wsum[i];
            wsum[i] = acc;
            acc += s;
        }
    }
    __syncthreads();
    int excl = incl - c + wsum[wave];
    if (tid < E) {
        offsets[tid] = excl;
        run[tid] = excl;
    }
    if (tid == 0) offsets[E] = n;
    __syncthreads();
    int nbits = 0;
    while ((1 << nbits) < E) ++nbits;
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    for (int base = 0; base < n; base += 1024) {
        int a = base + tid;
        bool valid = a < n;
        int e = valid ? ids[a] : 0;
        uint64_t peers = __ballot(valid);
        for (int b = 0; b < nbits; ++b) {
            bool bit = (e >> b) & 1;
            uint64_t m = __ballot(bit);
            peers &= bit ? m : ~m;
        }
        int rank = __popcll(peers & lt_mask);
        int cw = __popcll(peers);
        int last_wave = min(15, (n - base - 1) / kWave);
        for (int w2 = 0; w2 <= last_wave; ++w2) {
            if (wave == w2 && valid) {
                int b0 = run[e];
                int pos = b0 + rank;
                if (rank == 0) run[e] = b0 + cw;
                sorted_assign[pos] = a;
                assign_pos[a] = pos;
            }
            __syncthreads();
        }
    }
}

__global__ void __launch_bounds__(1024) permute_kernel(const int32_t* __restrict__ ids, int n, int E,
                                                        int32_t* __restrict__ offsets,
                                                        int32_t* __restrict__ sorted_assign,
                                                        int32_t* __restrict__ assign_pos) {
    __shared__ int cnt[kMaxE];
    __shared__ int run[kMaxE];
    __shared__ int wsum[16];
    permute_block(ids, n, E, offsets, sorted_assign, assign_pos, cnt, run, wsum);
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
    __shared__ int32_t ids_lds[kDirectMaxAssign];
    const int wave = threadIdx.x / kWave, lane = threadIdx.x % kWave;
    if (wave < T) topk_one_token<VPL>(logits + (size_t)wave * E, E, k, ids_lds + wave * k, w + (size_t)wave * k, lane);
    __syncthreads();
    const int n = T * k;
    for (int a = threadIdx.x; a < n; a += blockDim.x) {
        const int e = ids_lds[a];
        int pos = 0;
        for (int b = 0; b < n; ++b) {
            const int eb = ids_lds[b];
            pos += (eb < e || (eb == e && b < a)) ? 1 : 0;
        }
        ids[a] = e;
        sorted_assign[pos] = a;
        assign_pos[a] = pos;
    }
    for (int e = threadIdx.x; e <= E; e += blockDim.x) {
        int c = 0;
        for (int b = 0; b < n; ++b) c += ids_lds[b] < e ? 1 : 0;
        offsets[e] = c;
    }
}

template <int VPL>
hipError_t launch_route_vpl(const float* logits, int T, int E, int k, int32_t* ids, float* w, int32_t* offsets,
                            int32_t* sorted_assign, int32_t* assign_pos, hipStream_t s) {
    if (T <= 16 && T * k <= kDirectMaxAssign) {
        const int threads = kWave * max(4, T);
        hipLaunchKernelGGL(route_small_kernel<VPL>, dim3(1), dim3(threads), 0, s, logits, T, E, k, ids, w, offsets,
                           sorted_assign, assign_pos);
        return hipGetLastError();
    }
    hipLaunchKernelGGL(topk_kernel<VPL>, dim3(ceil_div(T, 4)), dim3(256), 0, s, logits, T, E, k, ids, w);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(permute_kernel, dim3(1), dim3(1024), 0, s, ids, T * k, E, offsets, sorted_assign,
                       assign_pos);
    return hipGetLastError();
}

}  // namespace

size_t route_ws_bytes(int, int, int) { return 0; }

hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* w, int32_t* offsets,
                        int32_t* sorted_assign, int32_t* assign_pos, void*, hipStream_t s) {
    const int vpl = ceil_div(E, kWave);
    if (vpl <= 1) return launch_route_vpl<1>(logits, T, E, k, ids, w, offsets, sorted_assign, assign_pos, s);
    if (vpl <= 2) return launch_route_vpl<2>(logits, T, E, k, ids, w, offsets, sorted_assign, assign_pos, s);
    if (vpl <= 4) return launch_route_vpl<4>(logits, T, E, k, ids, w, offsets, sorted_assign, assign_pos, s);
    if (vpl <= 8) return launch_route_vpl<8>(logits, T, E, k, ids, w, offsets, sorted_assign, assign_pos, s);
    return launch_route_vpl<16>(logits, T, E, k, ids, w, offsets, sorted_assign, assign_pos, s);
}

}  // namespace moe
