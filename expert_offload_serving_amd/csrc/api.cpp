// C ABI of the NVFP4 routed-MoE library: argument validation, error
// reporting, dispatch to the gfx950 kernels, the expert-cache fill and the
// host-side cache slot manager.  See include/moe_nvfp4.h for the contract.
#include "moe_nvfp4.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "internal.hpp"

namespace moe {

SlotGeom slot_geom(int H, int I) {
    SlotGeom g;
    size_t off = 0;
    g.gu_codes = off; off += (size_t)2 * I * H / 2;
    g.gu_scales = off; off += (size_t)2 * I * H / 16;
    g.gu_glob = off; off += (size_t)2 * I * 4;
    g.dn_codes = off; off += (size_t)H * I / 2;
    g.dn_scales = off; off += (size_t)H * I / 16;
    g.dn_glob = off; off += (size_t)H * 4;
    g.total = off;
    return g;
}

}  // namespace moe

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

// Largest buffer the kernels address (32-bit byte offsets in buffer resources).
constexpr size_t kMaxBuffer = (size_t)1 << 31;

// The slot format's tile: H % 128 == 0, I % 32 == 0 (the fp4 scale-block guard of issue #62).
bool shape_ok(int H, int I) { return H > 0 && I > 0 && H % 128 == 0 && I % 32 == 0; }

int check_route_shape(int T, int E, int k) {
    if (T < 0) return fail(MOE_ERR_INVALID_ARGUMENT, "T must be >= 0 (got %d)", T);
    if (E < 1 || E > 1024) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "E must be in [1, 1024] (got %d)", E);
    if (k < 1 || k > E) return fail(MOE_ERR_INVALID_ARGUMENT, "k must be in [1, E] (got k=%d, E=%d)", k, E);
    if ((long)T * k > (1L << 30)) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "T*k too large");
    return MOE_OK;
}

int forward_impl(const moe_nvfp4_layer_t* layer, const uint16_t* x, int T, const int32_t* topk_ids,
                 const float* topk_w, const int32_t* expert_offsets, const int32_t* sorted_assign,
                 const int32_t* assign_pos, float* y, int accumulate, void* ws, size_t ws_bytes, hipStream_t stream,
                 const moe::RouteOut* route);
int validate_forward(const moe_nvfp4_layer_t* layer, const uint16_t* x, int T, const int32_t* topk_ids,
                     const float* topk_w, const int32_t* expert_offsets, const int32_t* sorted_assign,
                     const int32_t* assign_pos, float* y, int accumulate, void* ws, size_t ws_bytes);
moe::Layer layer_of(const moe_nvfp4_layer_t& L);

}  // namespace

namespace moe {

int set_error(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return code;
}

}  // namespace moe

extern "C" {

const char* moe_last_error(void) { return g_last_error.c_str(); }

size_t moe_nvfp4_slot_bytes(int H, int I) {
    if (!shape_ok(H, I)) return 0;
    return moe::slot_geom(H, I).total;
}

size_t moe_route_workspace_bytes(int T, int E, int k) {
    if (check_route_shape(T, E, k) != MOE_OK) return 0;
    return moe::route_ws_bytes(T, E, k);
}

int moe_route_topk(const float* logits, int T, int E, int k, int32_t* topk_ids, float* topk_w,
                   int32_t* expert_offsets, int32_t* sorted_assign, int32_t* assign_pos, void* ws, size_t ws_bytes,
                   hipStream_t stream) {
    int rc = check_route_shape(T, E, k);
    if (rc != MOE_OK) return rc;
    if (T == 0) return MOE_OK;
    if (!logits || !topk_ids || !topk_w || !expert_offsets || !sorted_assign || !assign_pos)
        return fail(MOE_ERR_INVALID_ARGUMENT, "moe_route_topk: null pointer argument");
    const size_t need = moe::route_ws_bytes(T, E, k);
    if (ws_bytes < need || (need > 0 && !ws))
        return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "route workspace %zu < %zu bytes", ws_bytes, need);
    hipError_t e = moe::launch_route(logits, T, E, k, topk_ids, topk_w, expert_offsets, sorted_assign, assign_pos,
                                     ws, stream);
    if (e != hipSuccess) return hip_fail(e, "moe_route_topk launch");
    return MOE_OK;
}

int moe_router_logits(const uint16_t* x, const uint16_t* w_router, int T, int H, int E, float* logits,
                      hipStream_t stream) {
    if (T < 0) return fail(MOE_ERR_INVALID_ARGUMENT, "T must be >= 0 (got %d)", T);
    if (E < 1 || E > 1024) return fail(MOE_ERR_UNSUPPORTED_SHAPE, "E must be in [1, 1024] (got %d)", E);
    if (!moe::router_shape_supported(T, H, E))
        return fail(MOE_ERR_UNSUPPORTED_SHAPE, "router shape T=%d H=%d E=%d unsupported (H %% 256 == 0, H <= 16384)",
                    T, H, E);
    if (T == 0) return MOE_OK;
    if (!x || !w_router || !logits) return fail(MOE_ERR_INVALID_ARGUMENT, "moe_router_logits: null pointer argument");
    hipError_t e = moe::launch_router(x, w_router, T, H, E, logits, stream);
    if (e != hipSuccess) return hip_fail(e, "moe_router_logits launch");
    return MOE_OK;
}

int moe_router_topk(const uint16_t* x, const uint16_t* w_router, int T, int H, int E, int k, float* logits,
                    int32_t* topk_ids, float* topk_w, int32_t* expert_offsets, int32_t* sorted_assign,
                    int32_t* assign_pos, void* ws, size_t ws_bytes, hipStream_t stream) {
    // every argument is checked before anything is enqueued
    int rc = check_route_shape(T, E, k);
    if (rc != MOE_OK) return rc;
    if (!moe::router_shape_supported(T, H, E))
        return fail(MOE_ERR_UNSUPPORTED_SHAPE, "router shape T=%d H=%d E=%d unsupported (H %% 256 == 0, H <= 16384)",
                    T, H, E);
    if (T == 0) return MOE_OK;
    if (!x || !w_router || !logits || !topk_ids || !topk_w || !expert_offsets || !sorted_assign || !assign_pos)
        return fail(MOE_ERR_INVALID_ARGUMENT, "moe_router_topk: null pointer argument");
    const size_t need = moe::route_ws_bytes(T, E, k);
    if (ws_bytes < need || (need > 0 && !ws))
        return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "route workspace %zu < %zu bytes", ws_bytes, need);
    hipError_t e = moe::launch_router(x, w_router, T, H, E, logits, stream);
    if (e != hipSuccess) return hip_fail(e, "moe_router_topk: router launch");
    e = moe::launch_route(logits, T, E, k, topk_ids, topk_w, expert_offsets, sorted_assign, assign_pos, ws, stream);
    if (e != hipSuccess) return hip_fail(e, "moe_router_topk: routing launch");
    return MOE_OK;
}

size_t moe_nvfp4_forward_workspace_bytes(int T, int H, int I, int E, int k) {
    if (!shape_ok(H, I) || check_route_shape(T, E, k) != MOE_OK) return 0;
    return moe::forward_ws_bytes(T, H, I, E, k);
}

int moe_nvfp4_forward(const moe_nvfp4_layer_t* layer, const uint16_t* x, int T, const int32_t* topk_ids,
                      const float* topk_w, const int32_t* expert_offsets, const int32_t* sorted_assign,
                      const int32_t* assign_pos, float* y, int accumulate, void* ws, size_t ws_bytes,
                      hipStream_t stream) {
    return forward_impl(layer, x, T, topk_ids, topk_w, expert_offsets, sorted_assign, assign_pos, y, accumulate, ws,
                        ws_bytes, stream, nullptr);
}

size_t moe_nvfp4_route_forward_workspace_bytes(int T, int H, int I, int E, int k) {
    if (!shape_ok(H, I) || check_route_shape(T, E, k) != MOE_OK) return 0;
    return moe::align256(moe::forward_ws_bytes(T, H, I, E, k)) + moe::route_ws_bytes(T, E, k);
}

int moe_nvfp4_route_forward(const moe_nvfp4_layer_t* layer, const float* logits, const uint16_t* x, int T,
                            int32_t* topk_ids, float* topk_w, int32_t* expert_offsets, int32_t* sorted_assign,
                            int32_t* assign_pos, float* y, int accumulate, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
    if (!layer) return fail(MOE_ERR_INVALID_ARGUMENT, "moe_nvfp4_route_forward: layer is NULL");
    const moe_nvfp4_layer_t& L = *layer;
    int rc = check_route_shape(T, L.E, L.k);
    if (rc != MOE_OK) return rc;
    if (T == 0) return forward_impl(layer, x, T, topk_ids, topk_w, expert_offsets, sorted_assign, assign_pos, y,
                                    accumulate, ws, ws_bytes, stream, nullptr);
    if (!logits) return fail(MOE_ERR_INVALID_ARGUMENT, "moe_nvfp4_route_forward: logits is NULL");
    if (!shape_ok(L.H, L.I))
        return fail(MOE_ERR_UNSUPPORTED_SHAPE, "H must be a positive multiple of 128 and I of 32 (got H=%d, I=%d)",
                    L.H, L.I);
    const size_t fws = moe::align256(moe::forward_ws_bytes(T, L.H, L.I, L.E, L.k));
    const size_t need = fws + moe::route_ws_bytes(T, L.E, L.k);
    if (!ws || ws_bytes < need)
        return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "route_forward workspace %zu < %zu bytes", ws_bytes, need);
    if (moe::decode_path(T, L.H, L.I, L.k) && moe::decode_routes_in_kernel(T, L.E)) {
        const moe::RouteOut ro{logits, topk_ids, topk_w, expert_offsets, sorted_assign, assign_pos};
        return forward_impl(layer, x, T, topk_ids, topk_w, expert_offsets, sorted_assign, assign_pos, y, accumulate,
                            ws, fws, stream, &ro);
    }
    // routing as its own launch (its workspace after the forward's), then the forward; every argument is checked
    // before the first launch
    if (!topk_ids || !topk_w || !expert_offsets || !sorted_assign || !assign_pos)
        return fail(MOE_ERR_INVALID_ARGUMENT, "moe_nvfp4_route_forward: null routing output");
    rc = validate_forward(layer, x, T, topk_ids, topk_w, expert_offsets, sorted_assign, assign_pos, y, accumulate, ws,
                          fws);
    if (rc != MOE_OK) return rc;
    const moe::Layer ml = layer_of(L);
    hipError_t e = moe::launch_route(logits, T, L.E, L.k, topk_ids, topk_w, expert_offsets, sorted_assign,
                                     assign_pos, static_cast<uint8_t*>(ws) + fws, stream);
    if (e == hipSuccess) {
        if (moe::decode_path(T, L.H, L.I, L.k))
            e = moe::launch_decode(ml, x, T, topk_w, topk_ids, expert_offsets, sorted_assign, assign_pos, y,
                                   accumulate, ws, stream, nullptr);
        else
            e = moe::launch_prefill(ml, x, T, topk_w, topk_ids, expert_offsets, sorted_assign, assign_pos, y,
                                    accumulate, ws, stream);
    }
    if (e != hipSuccess) return hip_fail(e, "moe_nvfp4_route_forward launch");
    return MOE_OK;
}

}  // extern "C"

namespace {

// Every check of a forward call (nothing is enqueued here).
int validate_forward(const moe_nvfp4_layer_t* layer, const uint16_t* x, int T, const int32_t* topk_ids,
                     const float* topk_w, const int32_t* expert_offsets, const int32_t* sorted_assign,
                     const int32_t* assign_pos, float* y, int accumulate, void* ws, size_t ws_bytes) {
    if (!layer) return fail(MOE_ERR_INVALID_ARGUMENT, "moe_nvfp4_forward: layer is NULL");
    const moe_nvfp4_layer_t& L = *layer;
    if (!shape_ok(L.H, L.I))
        return fail(MOE_ERR_UNSUPPORTED_SHAPE, "H must be a positive multiple of 128 and I of 32 (got H=%d, I=%d)",
                    L.H, L.I);
    int rc = check_route_shape(T, L.E, L.k);
    if (rc != MOE_OK) return rc;
    if (accumulate != 0 && accumulate != 1) return fail(MOE_ERR_INVALID_ARGUMENT, "accumulate must be 0 or 1");
    const size_t sb = moe::slot_geom(L.H, L.I).total;
    if (L.slot_bytes != sb)
        return fail(MOE_ERR_INVALID_ARGUMENT, "slot_bytes %zu does not match H=%d, I=%d (%zu bytes)", L.slot_bytes,
                    L.H, L.I, sb);
    // the kernels address every buffer through 32-bit offsets: each must stay below 2 GiB
    if (sb >= kMaxBuffer || (size_t)T * L.H * 4 >= kMaxBuffer ||
        moe::forward_ws_bytes(T, L.H, L.I, L.E, L.k) >= kMaxBuffer)
        return fail(MOE_ERR_UNSUPPORTED_SHAPE, "T=%d H=%d I=%d k=%d: a slot, x, y or the workspace reaches 2 GiB", T,
                    L.H, L.I, L.k);
    if (T == 0) return MOE_OK;
    if (!L.bank_base || !L.slot_of_expert || L.num_slots < 1)
        return fail(MOE_ERR_INVALID_ARGUMENT, "layer bank, slot map and num_slots are required");
    if (reinterpret_cast<uintptr_t>(L.bank_base) % 256 != 0)
        return fail(MOE_ERR_INVALID_ARGUMENT, "bank_base must be 256-byte aligned");
    if (L.shared_slot && (reinterpret_cast<uintptr_t>(L.shared_slot) % 64 != 0))
        return fail(MOE_ERR_INVALID_ARGUMENT, "shared_slot must be 64-byte aligned");
    if (L.shared_slot && !L.shared_gate_w)
        return fail(MOE_ERR_INVALID_ARGUMENT, "shared_gate_w is required with a shared expert");
    if (!x || !topk_ids || !topk_w || !expert_offsets || !sorted_assign || !assign_pos || !y)
        return fail(MOE_ERR_INVALID_ARGUMENT, "moe_nvfp4_forward: null pointer argument");
    const size_t need = moe::forward_ws_bytes(T, L.H, L.I, L.E, L.k);
    if (!ws || ws_bytes < need)
        return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "forward workspace %zu < %zu bytes", ws_bytes, need);
    if (reinterpret_cast<uintptr_t>(ws) % 256 != 0)
        return fail(MOE_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
    if (!moe::decode_path(T, L.H, L.I, L.k) && !moe::prefill_shape_supported(L.H, L.I))
        return fail(MOE_ERR_UNSUPPORTED_SHAPE, "prefill path does not support H=%d, I=%d", L.H, L.I);
    return MOE_OK;
}

moe::Layer layer_of(const moe_nvfp4_layer_t& L) {
    return moe::Layer{L.H, L.I, L.E, L.k, static_cast<const uint8_t*>(L.bank_base), L.slot_bytes, L.num_slots,
                      L.slot_of_expert, static_cast<const uint8_t*>(L.shared_slot), L.shared_gate_w};
}

int forward_impl(const moe_nvfp4_layer_t* layer, const uint16_t* x, int T, const int32_t* topk_ids,
                 const float* topk_w, const int32_t* expert_offsets, const int32_t* sorted_assign,
                 const int32_t* assign_pos, float* y, int accumulate, void* ws, size_t ws_bytes, hipStream_t stream,
                 const moe::RouteOut* route) {
    int rc = validate_forward(layer, x, T, topk_ids, topk_w, expert_offsets, sorted_assign, assign_pos, y, accumulate,
                              ws, ws_bytes);
    if (rc != MOE_OK || T == 0) return rc;
    const moe::Layer ml = layer_of(*layer);
    hipError_t e;
    if (moe::decode_path(T, ml.H, ml.I, ml.k))
        e = moe::launch_decode(ml, x, T, topk_w, topk_ids, expert_offsets, sorted_assign, assign_pos, y, accumulate,
                               ws, stream, route);
    else
        e = moe::launch_prefill(ml, x, T, topk_w, topk_ids, expert_offsets, sorted_assign, assign_pos, y, accumulate,
                                ws, stream);
    if (e != hipSuccess) return hip_fail(e, "moe_nvfp4_forward launch");
    return MOE_OK;
}

}  // namespace

extern "C" {

int expert_cache_fill(void* cache_base, size_t slot_bytes, int num_slots, const int32_t* dst_slots,
                      const void* const* src, int n, hipStream_t copy_stream, hipEvent_t done) {
    if (n < 0) return fail(MOE_ERR_INVALID_ARGUMENT, "n must be >= 0");
    if (n > 0 && (!cache_base || !dst_slots || !src || slot_bytes == 0 || num_slots < 1))
        return fail(MOE_ERR_INVALID_ARGUMENT, "expert_cache_fill: missing cache, slots or sources");
    for (int i = 0; i < n; ++i) {
        if (dst_slots[i] < 0 || dst_slots[i] >= num_slots)
            return fail(MOE_ERR_INVALID_ARGUMENT, "dst_slots[%d] = %d outside [0, %d)", i, dst_slots[i], num_slots);
        if (!src[i]) return fail(MOE_ERR_INVALID_ARGUMENT, "src[%d] is NULL", i);
    }
    for (int i = 0; i < n; ++i) {
        hipPointerAttribute_t attr;
        hipError_t e = hipPointerGetAttributes(&attr, src[i]);
        if (e != hipSuccess || attr.type != hipMemoryTypeHost) {
            (void)hipGetLastError();
            return fail(MOE_ERR_NOT_PINNED, "src[%d] is not page-locked host memory", i);
        }
    }
    uint8_t* base = static_cast<uint8_t*>(cache_base);
    for (int i = 0; i < n; ++i) {
        hipError_t e = hipMemcpyAsync(base + (size_t)dst_slots[i] * slot_bytes, src[i], slot_bytes,
                                      hipMemcpyHostToDevice, copy_stream);
        if (e != hipSuccess) return hip_fail(e, "expert_cache_fill copy");
    }
    if (done) {
        hipError_t e = hipEventRecord(done, copy_stream);
        if (e != hipSuccess) return hip_fail(e, "expert_cache_fill event");
    }
    return MOE_OK;
}

int moe_nvfp4_slice_bank(const void* src_bank, int num_slots, int H, int I, int r, int n, void* dst_bank,
                         hipStream_t stream) {
    if (!shape_ok(H, I))
        return fail(MOE_ERR_UNSUPPORTED_SHAPE, "H must be a positive multiple of 128 and I of 32");
    if (n < 1 || r < 0 || r >= n || I % n != 0 || (I / n) % 32 != 0)
        return fail(MOE_ERR_UNSUPPORTED_SHAPE, "slice %d of %d: I/n must be a multiple of 32 (I=%d)", r, n, I);
    if (num_slots < 0) return fail(MOE_ERR_INVALID_ARGUMENT, "num_slots must be >= 0");
    if (num_slots == 0) return MOE_OK;
    if (!src_bank || !dst_bank) return fail(MOE_ERR_INVALID_ARGUMENT, "null bank pointer");
    hipError_t e = moe::launch_slice_bank(static_cast<const uint8_t*>(src_bank), num_slots, H, I, r, n,
                                          static_cast<uint8_t*>(dst_bank), stream);
    if (e != hipSuccess) return hip_fail(e, "moe_nvfp4_slice_bank launch");
    return MOE_OK;
}

int moe_nvfp4_dequant(const uint8_t* codes, const uint8_t* scales, const float* globals, int rows, int K, float* out,
                      hipStream_t stream) {
    if (rows < 0 || K <= 0 || K % 16 != 0)
        return fail(MOE_ERR_UNSUPPORTED_SHAPE, "rows must be >= 0 and K a positive multiple of 16 (rows=%d, K=%d)", rows,
                    K);
    if (rows == 0) return MOE_OK;
    if (!codes || !scales || !globals || !out) return fail(MOE_ERR_INVALID_ARGUMENT, "null pointer argument");
    if (reinterpret_cast<uintptr_t>(codes) % 4 != 0 || reinterpret_cast<uintptr_t>(out) % 16 != 0)
        return fail(MOE_ERR_INVALID_ARGUMENT, "codes must be 4-byte and out 16-byte aligned");
    hipError_t e = moe::launch_dequant_rows(codes, scales, globals, rows, K, out, stream);
    if (e != hipSuccess) return hip_fail(e, "moe_nvfp4_dequant launch");
    return MOE_OK;
}

int moe_nvfp4_dequant_slot(const void* slot, int H, int I, int matrix, float* out, hipStream_t stream) {
    if (!shape_ok(H, I))
        return fail(MOE_ERR_UNSUPPORTED_SHAPE, "H must be a positive multiple of 128 and I of 32");
    if (matrix != 0 && matrix != 1) return fail(MOE_ERR_INVALID_ARGUMENT, "matrix must be 0 (gate_up) or 1 (down)");
    if (!slot || !out) return fail(MOE_ERR_INVALID_ARGUMENT, "null pointer argument");
    if (reinterpret_cast<uintptr_t>(slot) % 16 != 0 || reinterpret_cast<uintptr_t>(out) % 16 != 0)
        return fail(MOE_ERR_INVALID_ARGUMENT, "slot and out must be 16-byte aligned");
    hipError_t e = moe::launch_dequant(static_cast<const uint8_t*>(slot), H, I, matrix, out, stream);
    if (e != hipSuccess) return hip_fail(e, "moe_nvfp4_dequant_slot launch");
    return MOE_OK;
}

int moe_release_streams(void) {
    hipError_t e = moe::release_side_streams();
    if (e != hipSuccess) return hip_fail(e, "moe_release_streams");
    return MOE_OK;
}

}  // extern "C"

// ------------------------------------------------------------------ MXFP4 bank format

namespace {

// Every check of an MXFP4 forward call (nothing is enqueued here).
int validate_mx_forward(const moe_nvfp4_layer_t* layer, const uint16_t* x, int T, const int32_t* topk_ids,
                        const float* topk_w, const int32_t* expert_offsets, const int32_t* sorted_assign,
                        const int32_t* assign_pos, float* y, int accumulate, void* ws, size_t ws_bytes) {
    if (!layer) return fail(MOE_ERR_INVALID_ARGUMENT, "moe_mxfp4_forward: layer is NULL");
    const moe_nvfp4_layer_t& L = *layer;
    if (!shape_ok(L.H, L.I))
        return fail(MOE_ERR_UNSUPPORTED_SHAPE, "H must be a positive multiple of 128 and I of 32 (got H=%d, I=%d)",
                    L.H, L.I);
    int rc = check_route_shape(T, L.E, L.k);
    if (rc != MOE_OK) return rc;
    if (accumulate != 0 && accumulate != 1) return fail(MOE_ERR_INVALID_ARGUMENT, "accumulate must be 0 or 1");
    const size_t sb = moe::mx_slot_geom(L.H, L.I).total;
    if (L.slot_bytes != sb)
        return fail(MOE_ERR_INVALID_ARGUMENT, "slot_bytes %zu does not match an MXFP4 slot at H=%d, I=%d (%zu bytes)",
                    L.slot_bytes, L.H, L.I, sb);
    const bool decode = moe::decode_path(T, L.H, L.I, L.k);
    // the kernels address every buffer through 32-bit offsets: each must stay below 2 GiB
    if (sb >= kMaxBuffer || (size_t)T * L.H * 4 >= kMaxBuffer ||
        moe::forward_ws_bytes(T, L.H, L.I, L.E, L.k, true) >= kMaxBuffer)
        return fail(MOE_ERR_UNSUPPORTED_SHAPE, "T=%d H=%d I=%d k=%d: a slot, x, y or the workspace reaches 2 GiB", T,
                    L.H, L.I, L.k);
    if (T == 0) return MOE_OK;
    if (decode ? !moe::mx_decode_shape_supported(L.H, L.I) : !moe::prefill_shape_supported(L.H, L.I))
        return fail(MOE_ERR_UNSUPPORTED_SHAPE, "MXFP4 %s path does not support H=%d, I=%d",
                    decode ? "decode" : "prefill", L.H, L.I);
    if (!L.bank_base || !L.slot_of_expert || L.num_slots < 1)
        return fail(MOE_ERR_INVALID_ARGUMENT, "layer bank, slot map and num_slots are required");
    if (reinterpret_cast<uintptr_t>(L.bank_base) % 256 != 0)
        return fail(MOE_ERR_INVALID_ARGUMENT, "bank_base must be 256-byte aligned");
    if (L.shared_slot && (reinterpret_cast<uintptr_t>(L.shared_slot) % 64 != 0))
        return fail(MOE_ERR_INVALID_ARGUMENT, "shared_slot must be 64-byte aligned");
    if (L.shared_slot && !L.shared_gate_w)
        return fail(MOE_ERR_INVALID_ARGUMENT, "shared_gate_w is required with a shared expert");
    if (!x || !topk_ids || !topk_w || !expert_offsets || !sorted_assign || !assign_pos || !y)
        return fail(MOE_ERR_INVALID_ARGUMENT, "moe_mxfp4_forward: null pointer argument");
    const size_t need = moe::forward_ws_bytes(T, L.H, L.I, L.E, L.k, true);
    if (!ws || ws_bytes < need)
        return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "forward workspace %zu < %zu bytes", ws_bytes, need);
    if (reinterpret_cast<uintptr_t>(ws) % 256 != 0)
        return fail(MOE_ERR_INVALID_ARGUMENT, "workspace must be 256-byte aligned");
    return MOE_OK;
}

}  // namespace

extern "C" {

size_t moe_mxfp4_slot_bytes(int H, int I) {
    if (!shape_ok(H, I)) return 0;
    return moe::mx_slot_geom(H, I).total;
}

size_t moe_mxfp4_forward_workspace_bytes(int T, int H, int I, int E, int k) {
    if (!shape_ok(H, I) || check_route_shape(T, E, k) != MOE_OK) return 0;
    if (moe::decode_path(T, H, I, k) ? !moe::mx_decode_shape_supported(H, I) : !moe::prefill_shape_supported(H, I))
        return 0;
    return moe::forward_ws_bytes(T, H, I, E, k, true);
}

int moe_mxfp4_forward(const moe_nvfp4_layer_t* layer, const uint16_t* x, int T, const int32_t* topk_ids,
                      const float* topk_w, const int32_t* expert_offsets, const int32_t* sorted_assign,
                      const int32_t* assign_pos, float* y, int accumulate, void* ws, size_t ws_bytes,
                      hipStream_t stream) {
    int rc = validate_mx_forward(layer, x, T, topk_ids, topk_w, expert_offsets, sorted_assign, assign_pos, y,
                                 accumulate, ws, ws_bytes);
    if (rc != MOE_OK || T == 0) return rc;
    const moe::Layer ml = layer_of(*layer);
    hipError_t e = moe::decode_path(T, ml.H, ml.I, ml.k)
                       ? moe::launch_mx_decode(ml, x, T, topk_w, expert_offsets, sorted_assign, y, accumulate, ws,
                                               stream)
                       : moe::launch_prefill(ml, x, T, topk_w, topk_ids, expert_offsets, sorted_assign, assign_pos, y,
                                             accumulate, ws, stream, true);
    if (e != hipSuccess) return hip_fail(e, "moe_mxfp4_forward launch");
    return MOE_OK;
}

size_t moe_mxfp4_route_forward_workspace_bytes(int T, int H, int I, int E, int k) {
    const size_t f = moe_mxfp4_forward_workspace_bytes(T, H, I, E, k);
    if (f == 0) return 0;
    return moe::align256(f) + moe::route_ws_bytes(T, E, k);
}

int moe_mxfp4_route_forward(const moe_nvfp4_layer_t* layer, const float* logits, const uint16_t* x, int T,
                            int32_t* topk_ids, float* topk_w, int32_t* expert_offsets, int32_t* sorted_assign,
                            int32_t* assign_pos, float* y, int accumulate, void* ws, size_t ws_bytes,
                            hipStream_t stream) {
    if (!layer) return fail(MOE_ERR_INVALID_ARGUMENT, "moe_mxfp4_route_forward: layer is NULL");
    const moe_nvfp4_layer_t& L = *layer;
    int rc = check_route_shape(T, L.E, L.k);
    if (rc != MOE_OK) return rc;
    // every check of the forward, against its share of the workspace (the routing's follows it)
    const size_t f = moe::forward_ws_bytes(T, L.H, L.I, L.E, L.k, true);
    const size_t fws = moe::align256(f);
    rc = validate_mx_forward(layer, x, T, topk_ids, topk_w, expert_offsets, sorted_assign, assign_pos, y, accumulate,
                             ws, ws_bytes < fws ? ws_bytes : fws);
    if (rc != MOE_OK || T == 0) return rc;
    if (!logits) return fail(MOE_ERR_INVALID_ARGUMENT, "moe_mxfp4_route_forward: logits is NULL");
    const size_t need = fws + moe::route_ws_bytes(T, L.E, L.k);
    if (ws_bytes < need)
        return fail(MOE_ERR_WORKSPACE_TOO_SMALL, "route_forward workspace %zu < %zu bytes", ws_bytes, need);
    const moe::Layer ml = layer_of(L);
    hipError_t e;
    if (moe::decode_routes_in_kernel(T, L.E)) {
        const moe::RouteOut ro{logits, topk_ids, topk_w, expert_offsets, sorted_assign, assign_pos};
        e = moe::launch_mx_decode(ml, x, T, topk_w, expert_offsets, sorted_assign, y, accumulate, ws, stream, &ro);
    } else {
        e = moe::launch_route(logits, T, L.E, L.k, topk_ids, topk_w, expert_offsets, sorted_assign, assign_pos,
                              static_cast<uint8_t*>(ws) + fws, stream);
        if (e == hipSuccess)
            e = moe::decode_path(T, L.H, L.I, L.k)
                    ? moe::launch_mx_decode(ml, x, T, topk_w, expert_offsets, sorted_assign, y, accumulate, ws, stream)
                    : moe::launch_prefill(ml, x, T, topk_w, topk_ids, expert_offsets, sorted_assign, assign_pos, y,
                                          accumulate, ws, stream, true);
    }
    if (e != hipSuccess) return hip_fail(e, "moe_mxfp4_route_forward launch");
    return MOE_OK;
}

int moe_mxfp4_dequant(const uint8_t* blocks_t, const uint8_t* scales_t, int N, int K, float* out,
                      hipStream_t stream) {
    if (N < 0 || K <= 0 || K % 32 != 0)
        return fail(MOE_ERR_UNSUPPORTED_SHAPE, "N must be >= 0 and K a positive multiple of 32 (N=%d, K=%d)", N, K);
    if (N == 0) return MOE_OK;
    if (!blocks_t || !scales_t || !out) return fail(MOE_ERR_INVALID_ARGUMENT, "null pointer argument");
    hipError_t e = moe::launch_mx_dequant_t(blocks_t, scales_t, N, K, out, stream);
    if (e != hipSuccess) return hip_fail(e, "moe_mxfp4_dequant launch");
    return MOE_OK;
}

int moe_mxfp4_dequant_slot(const void* slot, int H, int I, int matrix, float* out, hipStream_t stream) {
    if (!shape_ok(H, I))
        return fail(MOE_ERR_UNSUPPORTED_SHAPE, "H must be a positive multiple of 128 and I of 32");
    if (matrix != 0 && matrix != 1) return fail(MOE_ERR_INVALID_ARGUMENT, "matrix must be 0 (gate_up) or 1 (down)");
    if (!slot || !out) return fail(MOE_ERR_INVALID_ARGUMENT, "null pointer argument");
    if (reinterpret_cast<uintptr_t>(slot) % 16 != 0 || reinterpret_cast<uintptr_t>(out) % 16 != 0)
        return fail(MOE_ERR_INVALID_ARGUMENT, "slot and out must be 16-byte aligned");
    hipError_t e = moe::launch_mx_dequant_slot(static_cast<const uint8_t*>(slot), H, I, matrix, out, stream);
    if (e != hipSuccess) return hip_fail(e, "moe_mxfp4_dequant_slot launch");
    return MOE_OK;
}

int moe_mxfp4_slice_bank(const void* src_bank, int num_slots, int H, int I, int r, int n, void* dst_bank,
                         hipStream_t stream) {
    if (!shape_ok(H, I))
        return fail(MOE_ERR_UNSUPPORTED_SHAPE, "H must be a positive multiple of 128 and I of 32");
    if (n < 1 || r < 0 || r >= n || I % n != 0 || (I / n) % 32 != 0)
        return fail(MOE_ERR_UNSUPPORTED_SHAPE, "slice %d of %d: I/n must be a multiple of 32 (I=%d)", r, n, I);
    if (num_slots < 0) return fail(MOE_ERR_INVALID_ARGUMENT, "num_slots must be >= 0");
    if (num_slots == 0) return MOE_OK;
    if (!src_bank || !dst_bank) return fail(MOE_ERR_INVALID_ARGUMENT, "null bank pointer");
    hipError_t e = moe::launch_mx_slice_bank(static_cast<const uint8_t*>(src_bank), num_slots, H, I, r, n,
                                             static_cast<uint8_t*>(dst_bank), stream);
    if (e != hipSuccess) return hip_fail(e, "moe_mxfp4_slice_bank launch");
    return MOE_OK;
}

}  // extern "C"

// ------------------------------------------------------------------ host cache slot manager

struct moe_expert_cache {
    int L, E, C;
    std::vector<int32_t> where;  // (layer * E + expert) -> slot or -1
    std::vector<int32_t> owner;  // slot -> layer * E + expert or -1
    std::vector<int32_t> prev, next;  // recency list over slots; head = least recent
    int head = -1, tail = -1;
    int never_used = 0;          // slots [never_used, C) were never assigned
    std::vector<uint8_t> mark;   // scratch [E]

    void unlink(int c) {
        if (prev[c] >= 0) next[prev[c]] = next[c]; else head = next[c];
        if (next[c] >= 0) prev[next[c]] = prev[c]; else tail = prev[c];
        prev[c] = next[c] = -1;
    }
    void push_recent(int c) {
        prev[c] = tail;
        next[c] = -1;
        if (tail >= 0) next[tail] = c; else head = c;
        tail = c;
    }
};

extern "C" {

moe_expert_cache_t* moe_cache_create(int num_layers, int num_experts, int num_slots) {
    if (num_layers < 1 || num_experts < 1 || num_slots < 1) {
        fail(MOE_ERR_INVALID_ARGUMENT, "moe_cache_create: sizes must be positive");
        return nullptr;
    }
    auto* c = new moe_expert_cache;
    c->L = num_layers;
    c->E = num_experts;
    c->C = num_slots;
    c->where.assign((size_t)num_layers * num_experts, -1);
    c->owner.assign(num_slots, -1);
    c->prev.assign(num_slots, -1);
    c->next.assign(num_slots, -1);
    c->mark.assign(num_experts, 0);
    return c;
}

void moe_cache_destroy(moe_expert_cache_t* cache) { delete cache; }

int moe_cache_plan(moe_expert_cache_t* c, int layer, const int32_t* ids, int n, int32_t* slot_of_expert,
                   int32_t* miss_experts, int32_t* miss_slots, int* n_miss, int* n_hit) {
    return moe::cache_plan(c, layer, ids, n, slot_of_expert, miss_experts, miss_slots, n_miss, n_hit, nullptr);
}

}  // extern "C"

// moe_cache_plan; evicted (optional, one entry per miss): the (layer * E + expert) whose slot the miss took, or
// -1 when the slot had never been used.
int moe::cache_plan(moe_expert_cache_t* c, int layer, const int32_t* ids, int n, int32_t* slot_of_expert,
                    int32_t* miss_experts, int32_t* miss_slots, int* n_miss, int* n_hit, int32_t* evicted) {
    if (!c || layer < 0 || layer >= c->L || n < 0 || (n > 0 && !ids) || !slot_of_expert || !n_miss || !n_hit ||
        (n > 0 && (!miss_experts || !miss_slots)))
        return fail(MOE_ERR_INVALID_ARGUMENT, "moe_cache_plan: bad arguments");
    const int E = c->E;
    std::fill(c->mark.begin(), c->mark.end(), 0);
    int distinct = 0;
    for (int i = 0; i < n; ++i) {
        if (ids[i] < 0 || ids[i] >= E) return fail(MOE_ERR_INVALID_ARGUMENT, "routed id %d outside [0, %d)", ids[i], E);
        if (!c->mark[ids[i]]) c->mark[ids[i]] = 1, ++distinct;
    }
    if (distinct > c->C)
        return fail(MOE_ERR_INVALID_ARGUMENT, "layer-step needs %d distinct experts, pool has %d slots", distinct, c->C);
    const size_t base = (size_t)layer * E;
    int hits = 0, misses = 0;
    for (int e = 0; e < E; ++e) {  // hits become most recent, ascending
        if (!c->mark[e]) continue;
        const int s = c->where[base + e];
        if (s >= 0) {
            c->unlink(s);
            c->push_recent(s);
            ++hits;
        }
    }
    for (int e = 0; e < E; ++e) {  // misses take a never-used slot, else evict the least recent
        if (!c->mark[e] || c->where[base + e] >= 0) continue;
        int s, prev = -1;
        if (c->never_used < c->C) {
            s = c->never_used++;
        } else {
            s = c->head;
            c->unlink(s);
            prev = c->owner[s];
            c->where[prev] = -1;
        }
        if (evicted) evicted[misses] = prev;
        c->owner[s] = (int32_t)(base + e);
        c->where[base + e] = s;
        c->push_recent(s);
        miss_experts[misses] = e;
        miss_slots[misses] = s;
        ++misses;
    }
    for (int e = 0; e < E; ++e) slot_of_expert[e] = c->mark[e] ? c->where[base + e] : -1;
    *n_miss = misses;
    *n_hit = hits;
    return MOE_OK;
}


extern "C" {

}  // extern "C"
