// Internal launch interface between the C ABI layer (api.cpp) and the kernels.
// Every launcher assumes its arguments were validated by api.cpp and returns
// the hipError_t of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

struct moe_expert_cache;  // the host slot manager (api.cpp)

namespace moe {

__host__ __device__ inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

// moe_cache_plan with the evicted (layer * E + expert) of each miss, or -1 for a never-used slot (api.cpp).
int cache_plan(::moe_expert_cache* c, int layer, const int32_t* ids, int n, int32_t* slot_of_expert,
               int32_t* miss_experts, int32_t* miss_slots, int* n_miss, int* n_hit, int32_t* evicted);

// Records the calling thread's last-error message (api.cpp) and returns code.
int set_error(int code, const char* fmt, ...);

// Routing (route.hip)
size_t route_ws_bytes(int T, int E, int k);
hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* w, int32_t* offsets,
                        int32_t* sorted_assign, int32_t* assign_pos, void* ws, hipStream_t s);

// Router projection (router.hip): logits [T, E] = x [T, H] . w_r [E, H]^T.
bool router_shape_supported(int T, int H, int E);
hipError_t launch_router(const uint16_t* x, const uint16_t* wr, int T, int H, int E, float* logits, hipStream_t s);

// Layer description after validation.
struct Layer {
    int H, I, E, k;
    const uint8_t* bank;
    size_t slot_bytes;
    int num_slots;              // slot indices outside [0, num_slots) leave their expert out
    const int32_t* slot_of_expert;
    const uint8_t* shared;      // nullptr: no shared expert
    const uint16_t* wg;         // bf16 [H]
};

// Byte offsets of the six slot regions.
struct SlotGeom {
    size_t gu_codes, gu_scales, gu_glob, dn_codes, dn_scales, dn_glob, total;
};
SlotGeom slot_geom(int H, int I);

// Decode path, T <= 16 (decode.hip): shapes it covers and the bytes of its
// per-(row, slice) partial outputs.  Other shapes run the prefill path.
constexpr int kDecodeMaxT = 16;
constexpr int kDecodeMaxAssign = 1024;  // T*k
bool decode_shape_supported(int H, int I);
size_t decode_part_bytes(int T, int H, int I, int k);
size_t decode_rowslot_bytes(int T, int k);
size_t decode_dgrow_bytes(int T, int H, int k);
inline bool decode_path(int T, int H, int I, int k) {
    return T <= kDecodeMaxT && T * k <= kDecodeMaxAssign && decode_shape_supported(H, I);
}

// Forward workspace: byte offsets of its regions (each 256-byte aligned).
// The decode path uses `part` (per-(row, slice) partial outputs), `dg`
// (per-row slot of the row's expert) and `dgrow` (per-row copies of the
// expert's down-row globals); the prefill path uses the others:
//   h      hidden state, (T*k + T) rows of I fp16 values (MXFP4 bank: the bf16
//          high terms of all rows, then the bf16 low terms)
//   hx     the exponent of each 128-column tile of h, (T*k + T) rows of ceil(I/128) i32 (MXFP4: empty)
//   o      per-assignment expert outputs, (T*k + T) rows of H fp16, chunk (row, c) scaled by 2^ox[row, c]
//   ox     the exponent of each 256-column chunk of o, (T*k + T) rows of ceil(H/256) i32
//   s      shared-gate sigmoid per token, T f32
//   x16    scaled fp16 activations [T, H]; xinv: their inverse scales [T]
//   tiles  work lists: 4 counts, then 3 classes x tile_cap (group, m0) pairs
struct WsLayout {
    size_t part, dg, dgrow, h, hx, o, ox, s, x16, xinv, tiles, total;
    int tile_cap;
};
inline size_t align256(size_t b) { return (b + 255) / 256 * 256; }
inline WsLayout ws_layout(int T, int H, int I, int E, int k, bool mx = false) {
    WsLayout L{};
    if (decode_path(T, H, I, k)) {
        L.part = 0;
        L.dg = L.part + align256(decode_part_bytes(T, H, I, k));
        L.dgrow = L.dg + align256(decode_rowslot_bytes(T, k));
        L.total = L.dgrow + align256(decode_dgrow_bytes(T, H, k));
        return L;
    }
    const size_t rows = (size_t)T * k + T;
    L.h = 0;
    L.hx = L.h + align256(rows * I * (mx ? 4 : 2));
    L.o = L.hx + (mx ? 0 : align256(rows * (size_t)ceil_div(I, 128) * 4));
    L.ox = L.o + align256(rows * H * 2);
    L.s = L.ox + align256(rows * (size_t)ceil_div(H, 256) * 4);
    L.x16 = L.s + align256((size_t)T * 4);
    L.xinv = L.x16 + align256((size_t)T * H * 2);
    L.tiles = L.xinv + align256((size_t)T * 4);
    L.tile_cap = (int)((rows + 31) / 32 + E + 1);
    L.total = L.tiles + align256((4 + 3 * 2 * (size_t)L.tile_cap) * 4);
    return L;
}
inline size_t forward_ws_bytes(int T, int H, int I, int E, int k, bool mx = false) {
    return ws_layout(T, H, I, E, k, mx).total;
}

// Routing computed inside the decode kernels (route_forward): the logits and
// the routing outputs, which the kernels fill as moe_route_topk would.
struct RouteOut {
    const float* logits;
    int32_t* ids;
    float* w;
    int32_t* offsets;
    int32_t* sorted_assign;
    int32_t* assign_pos;
};
bool decode_routes_in_kernel(int T, int E);

// route == nullptr: the routing tensors are inputs; otherwise the kernels
// route from route->logits and write the routing tensors.
hipError_t launch_decode(const Layer& L, const uint16_t* x, int T, const float* w, const int32_t* ids,
                         const int32_t* offsets, const int32_t* sorted_assign, const int32_t* assign_pos, float* y,
                         int accumulate, void* ws, hipStream_t s, const RouteOut* route = nullptr);

// Prefill path, T > 16 (prefill.hip)
bool prefill_shape_supported(int H, int I);
hipError_t release_side_streams();
// mx: the bank holds MXFP4 slots (mx_slot_geom) instead of NVFP4 ones.
hipError_t launch_prefill(const Layer& L, const uint16_t* x, int T, const float* w, const int32_t* ids,
                          const int32_t* offsets, const int32_t* sorted_assign, const int32_t* assign_pos, float* y,
                          int accumulate, void* ws, hipStream_t s, bool mx = false);

// MXFP4 bank format (mxfp4.hip, slicer in util.hip): slot regions (globals empty), the decode path (T <= 16), the
// dequant hooks (checkpoint-transposed matrix; one matrix of a slot through the forward's own decode).
SlotGeom mx_slot_geom(int H, int I);
bool mx_decode_shape_supported(int H, int I);
// route == nullptr: the routing tensors are inputs; otherwise the kernels route from route->logits.
hipError_t launch_mx_decode(const Layer& L, const uint16_t* x, int T, const float* w, const int32_t* offsets,
                            const int32_t* sorted_assign, float* y, int accumulate, void* ws, hipStream_t s,
                            const RouteOut* route = nullptr);
hipError_t launch_mx_dequant_t(const uint8_t* blocks_t, const uint8_t* scales_t, int N, int K, float* out,
                               hipStream_t s);
hipError_t launch_mx_dequant_slot(const uint8_t* slot, int H, int I, int matrix, float* out, hipStream_t s);
hipError_t launch_mx_slice_bank(const uint8_t* src, int num_slots, int H, int I, int r, int n, uint8_t* dst,
                                hipStream_t s);

// Utilities (util.hip)
hipError_t launch_dequant(const uint8_t* slot, int H, int I, int matrix, float* out, hipStream_t s);
hipError_t launch_dequant_rows(const uint8_t* codes, const uint8_t* scales, const float* globals, int rows, int K,
                               float* out, hipStream_t s);
hipError_t launch_slice_bank(const uint8_t* src, int num_slots, int H, int I, int r, int n, uint8_t* dst,
                             hipStream_t s);


}  // namespace moe
