// Offload engine: one MoE layer-step over an HBM expert cache filled from
// pinned host banks (issue #62 "Why TP=2 loses today": a fraction of the
// experts lives in a GPU slot cache, the rest is streamed over PCIe each
// step; PR #385 "Measurements": prefill serves cache hits from device memory).
//
// A device-side directory (cache slot of every (layer, expert), -1 when not
// cached) lets the GPU find the hits by itself: the step routes, looks the
// routed experts up in the directory and starts the hits-only forward at
// once.  Before that forward, in stream order, the lookup's small result
// (the routed experts and whether each is cached) is copied to pinned host
// memory; the host waits for that copy only, so its planning overlaps the
// hits forward.  The host's LRU manager (the one behind moe_cache_plan)
// then touches the hits, assigns the misses their slots (never a slot the
// hits forward reads: those were just touched), copies the misses on the
// copy stream, updates the directory and runs the misses-only forward
// accumulating into the same output.  A step without misses costs one such
// wait and no second forward.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <vector>

#include "internal.hpp"
#include "moe_nvfp4.h"

namespace moe {
namespace {

// info[e]: slot of routed expert e when cached, -2 when routed but not cached, -1 when not routed;
// hit_map[e]: the slot for cached routed experts, else -1.  One thread per expert (routed: a nonempty group).
__global__ void __launch_bounds__(256) lookup_kernel(const int32_t* __restrict__ offsets,
                                                     const int32_t* __restrict__ dir, int E, int32_t* __restrict__ info,
                                                     int32_t* __restrict__ hit_map) {
    const int e = blockIdx.x * 256 + threadIdx.x;
    if (e >= E) return;
    const bool routed = offsets[e + 1] > offsets[e];
    const int s = dir[e];
    info[e] = routed ? (s >= 0 ? s : -2) : -1;
    hit_map[e] = routed && s >= 0 ? s : -1;
}

// Directory updates (index into dir, value) and the misses-only slot map.
__global__ void __launch_bounds__(256) update_kernel(const int32_t* __restrict__ upd, int n_upd, int32_t* __restrict__ dir,
                                                     const int32_t* __restrict__ miss_pairs, int n_miss, int E,
                                                     int32_t* __restrict__ miss_map) {
    const int t = blockIdx.x * 256 + threadIdx.x;
    if (t < n_upd) dir[upd[2 * t]] = upd[2 * t + 1];
    if (t < E) {
        int s = -1;
        for (int i = 0; i < n_miss; ++i)
            if (miss_pairs[2 * i] == t) s = miss_pairs[2 * i + 1];
        miss_map[t] = s;
    }
}

__global__ void __launch_bounds__(256) fill_kernel(int32_t* __restrict__ p, long n, int32_t v) {
    const long i = (long)blockIdx.x * 256 + threadIdx.x;
    if (i < n) p[i] = v;
}

}  // namespace
}  // namespace moe

// Device workspace carve-up (256-byte aligned regions).
struct OffloadDev {
    int32_t *dir, *info, *hit_map, *miss_map, *upd, *ids, *offsets, *sorted, *pos;
    float* w;
    uint8_t *route_ws, *fwd_ws;
    size_t route_ws_bytes, fwd_ws_bytes, total;
};

static OffloadDev offload_layout(uint8_t* base, int L, int E, int T_max, int k, int H, int I) {
    OffloadDev d{};
    size_t off = 0;
    auto take = [&](size_t bytes) {
        uint8_t* p = base ? base + off : nullptr;
        off += moe::align256(bytes);
        return p;
    };
    const size_t n = (size_t)T_max * k;
    d.dir = reinterpret_cast<int32_t*>(take((size_t)L * E * 4));
    d.info = reinterpret_cast<int32_t*>(take((size_t)E * 4));
    d.hit_map = reinterpret_cast<int32_t*>(take((size_t)E * 4));
    d.miss_map = reinterpret_cast<int32_t*>(take((size_t)E * 4));
    d.upd = reinterpret_cast<int32_t*>(take((size_t)(4 * E + 2 * E) * 4));  // updates then the miss pairs
    d.ids = reinterpret_cast<int32_t*>(take(n * 4));
    d.w = reinterpret_cast<float*>(take(n * 4));
    d.offsets = reinterpret_cast<int32_t*>(take((size_t)(E + 1) * 4));
    d.sorted = reinterpret_cast<int32_t*>(take(n * 4));
    d.pos = reinterpret_cast<int32_t*>(take(n * 4));
    d.route_ws_bytes = moe::route_ws_bytes(T_max, E, k);
    d.route_ws = take(d.route_ws_bytes);
    // decode workspaces grow with T up to 16, prefill ones with T: the largest is at min(T_max, 16) or T_max
    const size_t fw = std::max(moe::forward_ws_bytes(std::min(T_max, moe::kDecodeMaxT), H, I, E, k),
                               moe::forward_ws_bytes(T_max, H, I, E, k));
    d.fwd_ws_bytes = fw;
    d.fwd_ws = take(fw);
    d.total = off;
    return d;
}

struct moe_offload {
    int L, E, k, H, I, T_max, num_slots;
    size_t slot_bytes;
    uint8_t* cache;
    std::vector<const void*> host_slots;  // [L * E] pinned
    moe_expert_cache_t* lru;
    OffloadDev dev;
    int32_t* h_info = nullptr;   // pinned [E]
    int32_t* h_upd = nullptr;    // pinned [6 E]: directory updates (index, value), then (miss expert, slot)
    hipEvent_t info_ready = nullptr, filled = nullptr, filled2 = nullptr;
    hipStream_t copy2 = nullptr;  // a second copy stream (default priority): the misses alternate between the two
    std::vector<int32_t> ids, som, miss_e, miss_s, evicted;
};

extern "C" {

size_t moe_offload_device_bytes(int num_layers, int num_experts, int k, int T_max, int H, int I) {
    if (num_layers < 1 || num_experts < 1 || num_experts > 1024 || k < 1 || k > num_experts || T_max < 1 ||
        moe_nvfp4_slot_bytes(H, I) == 0)
        return 0;
    return offload_layout(nullptr, num_layers, num_experts, T_max, k, H, I).total;
}

moe_offload_t* moe_offload_create(int num_layers, int num_experts, int k, int H, int I, int T_max, void* cache_base,
                                  int num_slots, const void* const* host_slots, void* dev_ws, size_t dev_ws_bytes,
                                  hipStream_t stream) {
    const size_t need = moe_offload_device_bytes(num_layers, num_experts, k, T_max, H, I);
    if (need == 0) {
        moe::set_error(MOE_ERR_UNSUPPORTED_SHAPE, "moe_offload_create: bad sizes");
        return nullptr;
    }
    if (!cache_base || num_slots < 1 || !host_slots || !dev_ws || dev_ws_bytes < need ||
        reinterpret_cast<uintptr_t>(dev_ws) % 256 != 0 || reinterpret_cast<uintptr_t>(cache_base) % 256 != 0) {
        moe::set_error(MOE_ERR_INVALID_ARGUMENT,
                       "moe_offload_create: cache, host slots and a 256-byte aligned device workspace of %zu bytes "
                       "are required", need);
        return nullptr;
    }
    for (long i = 0; i < (long)num_layers * num_experts; ++i) {
        hipPointerAttribute_t attr;
        if (!host_slots[i] || hipPointerGetAttributes(&attr, host_slots[i]) != hipSuccess ||
            attr.type != hipMemoryTypeHost) {
            (void)hipGetLastError();
            moe::set_error(MOE_ERR_NOT_PINNED, "moe_offload_create: host slot %ld is not page-locked", i);
            return nullptr;
        }
    }
    auto* o = new moe_offload;
    o->L = num_layers; o->E = num_experts; o->k = k; o->H = H; o->I = I; o->T_max = T_max;
    o->num_slots = num_slots;
    o->slot_bytes = moe_nvfp4_slot_bytes(H, I);
    o->cache = static_cast<uint8_t*>(cache_base);
    o->host_slots.assign(host_slots, host_slots + (size_t)num_layers * num_experts);
    o->lru = moe_cache_create(num_layers, num_experts, num_slots);
    o->dev = offload_layout(static_cast<uint8_t*>(dev_ws), num_layers, num_experts, T_max, k, H, I);
    hipError_t e = hipHostMalloc(reinterpret_cast<void**>(&o->h_info), (size_t)num_experts * 4, hipHostMallocDefault);
    if (e == hipSuccess) e = hipHostMalloc(reinterpret_cast<void**>(&o->h_upd), (size_t)6 * num_experts * 4,
                                           hipHostMallocDefault);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&o->info_ready, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&o->filled, hipEventDisableTiming);
    if (e == hipSuccess) e = hipEventCreateWithFlags(&o->filled2, hipEventDisableTiming);
    if (e == hipSuccess) e = hipStreamCreateWithFlags(&o->copy2, hipStreamNonBlocking);
    if (e == hipSuccess) {
        const long n = (long)num_layers * num_experts;
        hipLaunchKernelGGL(moe::fill_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream, o->dev.dir, n,
                           -1);
        e = hipGetLastError();
    }
    if (e != hipSuccess || !o->lru) {
        moe::set_error(MOE_ERR_HIP, "moe_offload_create: %s", hipGetErrorString(e));
        moe_offload_destroy(o);
        return nullptr;
    }
    return o;
}

void moe_offload_destroy(moe_offload_t* o) {
    if (!o) return;
    if (o->info_ready) (void)hipEventDestroy(o->info_ready);
    if (o->filled) (void)hipEventDestroy(o->filled);
    if (o->filled2) (void)hipEventDestroy(o->filled2);
    if (o->copy2) {
        (void)hipStreamSynchronize(o->copy2);
        (void)hipStreamDestroy(o->copy2);
    }
    if (o->h_info) (void)hipHostFree(o->h_info);
    if (o->h_upd) (void)hipHostFree(o->h_upd);
    if (o->lru) moe_cache_destroy(o->lru);
    delete o;
}

int moe_offload_layer(moe_offload_t* o, int layer, const float* logits, const uint16_t* x, int T,
                      const void* shared_slot, const uint16_t* shared_gate_w, float* y, hipStream_t stream,
                      hipStream_t copy_stream, int* n_hit, int* n_miss) {
    if (!o || layer < 0 || layer >= o->L || T < 1 || T > o->T_max || !logits || !x || !y || !n_hit || !n_miss)
        return moe::set_error(MOE_ERR_INVALID_ARGUMENT, "moe_offload_layer: bad arguments");
    const int E = o->E, k = o->k;
    OffloadDev& d = o->dev;
    int rc = moe_route_topk(logits, T, E, k, d.ids, d.w, d.offsets, d.sorted, d.pos, d.route_ws, d.route_ws_bytes,
                            stream);
    if (rc != MOE_OK) return rc;
    hipLaunchKernelGGL(moe::lookup_kernel, dim3((unsigned)((E + 255) / 256)), dim3(256), 0, stream, d.offsets,
                       d.dir + (size_t)layer * E, E, d.info, d.hit_map);
    hipError_t e = hipGetLastError();
    if (e == hipSuccess) e = hipMemcpyAsync(o->h_info, d.info, (size_t)E * 4, hipMemcpyDeviceToHost, stream);
    if (e == hipSuccess) e = hipEventRecord(o->info_ready, stream);
    if (e != hipSuccess) return moe::set_error(MOE_ERR_HIP, "moe_offload_layer lookup: %s", hipGetErrorString(e));
    // the hits forward starts at once (with the shared expert); the host plans meanwhile
    moe_nvfp4_layer_t Lh{o->H, o->I, E, k, o->cache, o->slot_bytes, o->num_slots, d.hit_map, shared_slot,
                         shared_gate_w};
    rc = moe_nvfp4_forward(&Lh, x, T, d.ids, d.w, d.offsets, d.sorted, d.pos, y, 0, d.fwd_ws, d.fwd_ws_bytes, stream);
    if (rc != MOE_OK) return rc;
    if ((e = hipEventSynchronize(o->info_ready)) != hipSuccess)
        return moe::set_error(MOE_ERR_HIP, "moe_offload_layer wait: %s", hipGetErrorString(e));
    o->ids.clear();
    for (int ex = 0; ex < E; ++ex)
        if (o->h_info[ex] != -1) o->ids.push_back(ex);
    o->som.assign(E, -1);
    o->miss_e.assign(o->ids.size() + 1, 0);
    o->miss_s.assign(o->ids.size() + 1, 0);
    int nm = 0, nh = 0;
    o->evicted.assign(o->ids.size() + 1, -1);
    rc = moe::cache_plan(o->lru, layer, o->ids.data(), (int)o->ids.size(), o->som.data(), o->miss_e.data(),
                         o->miss_s.data(), &nm, &nh, o->evicted.data());
    if (rc != MOE_OK) return rc;
    *n_hit = nh;
    *n_miss = nm;
    if (nm == 0) return MOE_OK;
    // the directory changes: each evicted (layer, expert) leaves it, each miss enters at its slot
    int nu = 0;
    for (int i = 0; i < nm; ++i) {
        const int32_t prev = o->evicted[i];
        if (prev >= 0) {
            o->h_upd[2 * nu] = prev;
            o->h_upd[2 * nu + 1] = -1;
            ++nu;
        }
    }
    for (int i = 0; i < nm; ++i) {
        o->h_upd[2 * nu] = layer * E + o->miss_e[i];
        o->h_upd[2 * nu + 1] = o->miss_s[i];
        ++nu;
    }
    int32_t* pairs = o->h_upd + 2 * nu;  // (miss expert, slot) for the misses-only map
    for (int i = 0; i < nm; ++i) {
        pairs[2 * i] = o->miss_e[i];
        pairs[2 * i + 1] = o->miss_s[i];
    }
    // the copies alternate between the caller's copy stream and the engine's second one (two DMA queues move
    // more than one over the host link); each stream's event is waited on before the misses forward
    for (int i = 0; i < nm; ++i) {
        e = hipMemcpyAsync(o->cache + (size_t)o->miss_s[i] * o->slot_bytes,
                           o->host_slots[(size_t)layer * E + o->miss_e[i]], o->slot_bytes, hipMemcpyHostToDevice,
                           (i & 1) ? o->copy2 : copy_stream);
        if (e != hipSuccess) return moe::set_error(MOE_ERR_HIP, "moe_offload_layer fill: %s", hipGetErrorString(e));
    }
    if ((e = hipEventRecord(o->filled2, o->copy2)) != hipSuccess ||
        (e = hipStreamWaitEvent(stream, o->filled2, 0)) != hipSuccess ||
        (e = hipEventRecord(o->filled, copy_stream)) != hipSuccess ||
        (e = hipMemcpyAsync(d.upd, o->h_upd, (size_t)(2 * nu + 2 * nm) * 4, hipMemcpyHostToDevice, stream)) !=
            hipSuccess)
        return moe::set_error(MOE_ERR_HIP, "moe_offload_layer update: %s", hipGetErrorString(e));
    const int th = std::max(nu, E);
    hipLaunchKernelGGL(moe::update_kernel, dim3((unsigned)((th + 255) / 256)), dim3(256), 0, stream, d.upd, nu, d.dir,
                       d.upd + 2 * nu, nm, E, d.miss_map);
    if ((e = hipGetLastError()) != hipSuccess || (e = hipStreamWaitEvent(stream, o->filled, 0)) != hipSuccess)
        return moe::set_error(MOE_ERR_HIP, "moe_offload_layer update: %s", hipGetErrorString(e));
    moe_nvfp4_layer_t Lm{o->H, o->I, E, k, o->cache, o->slot_bytes, o->num_slots, d.miss_map, nullptr, nullptr};
    return moe_nvfp4_forward(&Lm, x, T, d.ids, d.w, d.offsets, d.sorted, d.pos, y, 1, d.fwd_ws, d.fwd_ws_bytes,
                             stream);
}

}  // extern "C"
