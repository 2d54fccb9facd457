// moe_nvfp4_route_forward_noalloc: the decode-path layer call with its
// workspace in a fixed device array instead of a caller-provided buffer, for
// callers that cannot allocate (code under graph capture, tight serving
// loops, harnesses that forbid allocation).
//
// The array lives in the library's code object: each GPU the library runs on
// holds its own copy (kScratchBytes) until the process ends.  Host code never
// passes the array's name to a kernel (on the host that name is a stand-in,
// not a device address): the first call on a device, with that device
// current, asks the runtime for the array's device address and keeps it per
// device; every later use goes through that address.  Every call on a device
// shares its array, so calls that overlap on one GPU race.
#include <map>
#include <mutex>

#include "internal.hpp"
#include "moe_nvfp4.h"

namespace {

// Largest route_forward workspace served: the decode path at T = 16, H = 2560, I = 640, k = 8 needs 29.6 MiB.
constexpr size_t kScratchBytes = (size_t)32 << 20;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mu;
std::map<int, void*> g_scratch_ptr;  // device -> device address of `scratch`

hipError_t scratch_on_current_device(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    auto it = g_scratch_ptr.find(dev);
    if (it != g_scratch_ptr.end()) {
        *out = it->second;
        return hipSuccess;
    }
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
    *out = p;
    return hipSuccess;
}

}  // namespace

extern "C" {

size_t moe_nvfp4_noalloc_scratch_bytes(void) { return kScratchBytes; }

int moe_nvfp4_route_forward_noalloc(const moe_nvfp4_layer_t* layer, const float* logits, const uint16_t* x, int T,
                                    int32_t* topk_ids, float* topk_w, int32_t* expert_offsets,
                                    int32_t* sorted_assign, int32_t* assign_pos, float* y, int accumulate,
                                    hipStream_t stream) {
    if (!layer) return moe::set_error(MOE_ERR_INVALID_ARGUMENT, "moe_nvfp4_route_forward_noalloc: layer is NULL");
    const moe_nvfp4_layer_t& L = *layer;
    if (T > moe::kDecodeMaxT)
        return moe::set_error(MOE_ERR_UNSUPPORTED_SHAPE,
                              "moe_nvfp4_route_forward_noalloc covers the decode path only (T <= %d, got T=%d)",
                              moe::kDecodeMaxT, T);
    const size_t need = moe_nvfp4_route_forward_workspace_bytes(T, L.H, L.I, L.E, L.k);
    if (T <= 0 || need == 0)  // T = 0 (a no-op) and bad shapes: the regular entry point handles and reports them
        return moe_nvfp4_route_forward(layer, logits, x, T, topk_ids, topk_w, expert_offsets, sorted_assign,
                                       assign_pos, y, accumulate, nullptr, 0, stream);
    if (need > kScratchBytes)
        return moe::set_error(MOE_ERR_WORKSPACE_TOO_SMALL,
                              "moe_nvfp4_route_forward_noalloc: T=%d H=%d I=%d E=%d k=%d needs %zu workspace bytes; "
                              "the fixed scratch holds %zu",
                              T, L.H, L.I, L.E, L.k, need, kScratchBytes);
    if (!moe::decode_path(T, L.H, L.I, L.k))
        return moe::set_error(MOE_ERR_UNSUPPORTED_SHAPE,
                              "moe_nvfp4_route_forward_noalloc covers the decode path only (H <= 2560, T*k <= 1024)");
    void* ws = nullptr;
    hipError_t e = scratch_on_current_device(&ws);
    if (e != hipSuccess)
        return moe::set_error(MOE_ERR_HIP, "moe_nvfp4_route_forward_noalloc: scratch address: %s",
                              hipGetErrorString(e));
    // Nothing in the workspace has to start at zero: every region the decode kernels read in a call is written
    // earlier in the same call.
    return moe_nvfp4_route_forward(layer, logits, x, T, topk_ids, topk_w, expert_offsets, sorted_assign, assign_pos,
                                   y, accumulate, ws, kScratchBytes, stream);
}

}  // extern "C"
