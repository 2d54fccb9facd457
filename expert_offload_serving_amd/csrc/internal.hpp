// Internal launch interface between the C ABI layer (api.cpp) and the kernels.
// Every launcher assumes its arguments were validated by api.cpp and returns
// the hipError_t of its launches.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Routing (route.hip)
size_t route_ws_bytes(int T, int E, int k);
hipError_t launch_route(const float* logits, int T, int E, int k, int32_t* ids, float* w, int32_t* offsets,
                        int32_t* sorted_assign, int32_t* assign_pos, void* ws, hipStream_t s);

// Layer description after validation.
struct Layer {
    int H, I, E, k;
    const uint8_t* bank;
    size_t slot_bytes;
    const int32_t* slot_of_expert;
    const uint8_t* shared;      // nullptr: no shared expert
    const uint16_t* wg;         // bf16 [H]
};

// Byte offsets of the six slot regions.
struct SlotGeom {
    size_t gu_codes, gu_scales, gu_glob, dn_codes, dn_scales, dn_glob, total;
};
SlotGeom slot_geom(int H, int I);

// Forward workspace (forward.cpp)
size_t forward_ws_bytes(int T, int H, int I, int E, int k);

// Decode path, T <= 16 (decode.hip)
constexpr int kDecodeMaxT = 16;
bool decode_shape_supported(int H, int I);
hipError_t launch_decode(const Layer& L, const uint16_t* x, int T, const float* w, const int32_t* ids,
                         const int32_t* offsets, const int32_t* sorted_assign, const int32_t* assign_pos, float* y,
                         int accumulate, void* ws, hipStream_t s);

// Prefill path, T > 16 (prefill.hip)
bool prefill_shape_supported(int H, int I);
hipError_t launch_prefill(const Layer& L, const uint16_t* x, int T, const float* w, const int32_t* ids,
                          const int32_t* offsets, const int32_t* sorted_assign, const int32_t* assign_pos, float* y,
                          int accumulate, void* ws, hipStream_t s);

// Utilities (util.hip)
hipError_t launch_dequant(const uint8_t* codes, const uint8_t* scales, const float* globals, int rows, int K,
                          float* out, hipStream_t s);
hipError_t launch_slice_bank(const uint8_t* src, int num_slots, int H, int I, int r, int n, uint8_t* dst,
                             hipStream_t s);

__host__ __device__ inline int ceil_div(int a, int b) { return (a + b - 1) / b; }

}  // namespace moe
