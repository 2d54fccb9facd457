// Top-k routing with renormalised weights (route_device.hpp) and the
// deterministic permutation of assignments by expert, for gfx950.  The
// permutation groups the T*k assignments by expert with a stable counting
// sort (per-expert counts, exclusive scan, then stable ranks from wave
// ballots), so the grouping is bit-reproducible: no atomic operation decides
// an order (atomics only count).
#include "internal.hpp"
#include "nvfp4_device.hpp"
#include "route_device.hpp"

namespace moe {
namespace {

constexpr int kMaxE = kRouteMaxE;

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
// assignments of each expert start, then ranks them stably inside the block:
// wave ballots give each assignment's rank among its wave's assignments of
// the same expert, and a per-(wave, expert) count table scanned over the
// waves gives each wave's start, so all waves scatter at once.
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
    __shared__ int wcnt[16][kMaxE];  // per wave: its assignments of each expert, then where they start
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int b = blockIdx.x;
    // per expert (one per thread): total over all blocks, and the part in blocks before b
    int total = 0, before_b = 0;
    if (tid < E) {
        // unrolled so that the histogram loads are in flight together rather than one round trip each
#pragma unroll 8
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
    for (int i = tid; i < 16 * E; i += 1024) wcnt[i / E][i % E] = 0;
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
    __syncthreads();  // wcnt cleared, run set
    if (valid && rank == 0) wcnt[wave][e] = __popcll(peers);
    __syncthreads();
    if (tid < E) {  // each wave's start for expert tid: run[tid] plus the counts of the waves before it
        int acc = run[tid];
        for (int w2 = 0; w2 < 16; ++w2) {
            const int c = wcnt[w2][tid];
            wcnt[w2][tid] = acc;
            acc += c;
        }
    }
    __syncthreads();
    if (valid) {
        const int pos = wcnt[wave][e] + rank;
        sorted_assign[pos] = a;
        assign_pos[a] = pos;
    }
}

// Decode batches (T <= 16, T*k <= kDirectMaxAssign): one workgroup with one
// wave per token selects the top-k, then ranks every assignment directly:
//   pos(a)     = #{a' : (e', a') < (e, a)}   (expert, then flat index)
//   offsets[e] = #{assignments with expert < e}
// which is the same stable grouping as the counting sort, in one launch.
// P threads (a power of two, up to 16) share one assignment's count, each
// scanning every P-th group of four ids, and add their parts with lane
// shuffles; the offsets are then a binary search of the sorted expert list.
constexpr int kDirectMaxAssign = 256;

template <int VPL>
__global__ void __launch_bounds__(1024) route_small_kernel(const float* __restrict__ logits, int T, int E, int k,
                                                            int32_t* __restrict__ ids, float* __restrict__ w,
                                                            int32_t* __restrict__ offsets,
                                                            int32_t* __restrict__ sorted_assign,
                                                            int32_t* __restrict__ assign_pos) {
    __shared__ __attribute__((aligned(16))) int32_t ids_lds[kDirectMaxAssign + 4];
    __shared__ int32_t sorted_e[kDirectMaxAssign];
    const int tid = threadIdx.x, nthr = blockDim.x;
    const int wave = tid / kWave, lane = tid % kWave;
    if (wave < T) topk_one_token<VPL>(logits + (size_t)wave * E, E, k, ids_lds + wave * k, w + (size_t)wave * k, lane);
    const int n = T * k, n4 = (n + 3) / 4;
    if (tid < 4 * n4 - n) ids_lds[n + tid] = 0x7FFFFFFF;  // pad: ranks after every expert
    __syncthreads();
    int P = 1;
    while (P < 16 && 2 * P * n <= nthr) P *= 2;
    const int4* ids4 = reinterpret_cast<const int4*>(ids_lds);
    // the P threads of an assignment are consecutive lanes of one wave, all active together
    for (int idx = tid; idx < n * P; idx += nthr) {
        const int a = idx / P, part = idx % P;
        const int e = ids_lds[a];
        int pos = 0;
#pragma unroll 4
        for (int q = part; q < n4; q += P) {
            const int4 v = ids4[q];
            const int b = 4 * q;
            pos += (v.x < e || (v.x == e && b < a)) + (v.y < e || (v.y == e && b + 1 < a)) +
                   (v.z < e || (v.z == e && b + 2 < a)) + (v.w < e || (v.w == e && b + 3 < a));
        }
        for (int off = 1; off < P; off <<= 1) pos += __shfl_xor(pos, off, kWave);
        if (part == 0) {
            ids[a] = e;
            sorted_assign[pos] = a;
            assign_pos[a] = pos;
            sorted_e[pos] = e;
        }
    }
    __syncthreads();
    // offsets[e] = #{b : e_b < e}: the first sorted position holding an expert >= e
    for (int e = tid; e <= E; e += nthr) {
        int lo = 0, hi = n;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (sorted_e[mid] < e) lo = mid + 1;
            else hi = mid;
        }
        offsets[e] = lo;
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
