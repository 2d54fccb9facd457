/*
 * moe_nvfp4.h - C ABI of the MI355X (gfx950) NVFP4 routed-MoE layer library.
 *
 * What the library computes comes from the FreeToken pages on offloaded MoE
 * serving: PR #385 ("What this adds": NVFP4 expert banks of packed 4-bit
 * codes, 16-wide FP8 scale blocks and per-row fp32 globals, sliced along the
 * intermediate axis; one combine routed + sigmoid(gate) * shared) and issue
 * #62 ("What it touches": gate_up is [2I, H] with gate rows [0, I) and up
 * rows [I, 2I), down is [H, I]; "The fix that fits": an I-slice turns the
 * down projection into partial sums; "Why TP=2 loses today": experts live in
 * a GPU slot cache filled from host banks over PCIe on misses).
 *
 * Conventions for every entry point:
 *  - Pointers are device pointers unless marked "host".  The caller owns all
 *    memory; the library allocates and frees nothing on the GPU.
 *  - Calls validate their arguments synchronously, before anything is
 *    enqueued; a failed call enqueues nothing and returns a nonzero status.
 *    moe_last_error() then returns a message for the calling thread.
 *  - Work is enqueued on the given stream and the call returns; device faults
 *    surface at the caller's next synchronisation.  moe_route_topk,
 *    moe_nvfp4_forward, moe_nvfp4_route_forward, moe_router_logits and
 *    moe_router_topk make no host synchronisation and allocate no memory
 *    (the prefill path creates its side stream and two events on its first
 *    call for a given caller stream, and reuses them afterwards;
 *    moe_release_streams destroys them).
 *  - Shapes: H % 128 == 0, I % 32 == 0 (see the slot format below),
 *    1 <= k <= E <= 1024, T >= 0 (T == 0 is a no-op).  The kernels address
 *    buffers through 32-bit byte offsets: a slot, x, y or a workspace of
 *    2 GiB or more is refused with MOE_ERR_UNSUPPORTED_SHAPE.
 *  - bf16 values are passed as their uint16 bit patterns.
 */
#ifndef MOE_NVFP4_H
#define MOE_NVFP4_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARGUMENT = 1,
    MOE_ERR_UNSUPPORTED_SHAPE = 2,
    MOE_ERR_WORKSPACE_TOO_SMALL = 3,
    MOE_ERR_NOT_PINNED = 4,
    MOE_ERR_HIP = 5,
};

/* Message describing the last failed call on this thread ("" if none). */
const char* moe_last_error(void);

/* ------------------------------------------------------------------ slots
 * An expert is two NVFP4 matrices (PR #385 "What this adds": packed 4-bit
 * E2M1 codes, one E4M3FN scale per 16 consecutive elements along the
 * contraction axis, one fp32 global per row; issue #62 "What it touches":
 * gate_up is [2I, H] with gate rows [0, I) and up rows [I, 2I), down is
 * [H, I]).  Element (r, c) of a matrix with N rows is
 *     W[r,c] = e2m1(code(r,c)) * e4m3(scale(r, c/16)) * global[r].
 * One slot holds, in this order and without padding:
 *     gate_up codes   2I*H/2 bytes      gate_up scales  2I*H/16 bytes
 *     gate_up globals f32 [2I]          down codes      H*I/2 bytes
 *     down scales     H*I/16 bytes      down globals    f32 [H]
 * Codes and scales are stored in matrix-core operand order, so that one
 * 16-byte load per lane of a 64-lane wave brings whole operand fragments of
 * the 16x16x32 MFMA (lane L = 16*g + i holds row i of a 16-row tile and the
 * 8 columns [8g, 8g+8) of a 32-column chunk; two codes per byte, the even
 * column in the low nibble).  With e = c % 8, g = (c / 8) % 4, i = r % 16:
 *   gate_up (N = 2I, "column-grouped": a 16-row x 128-column tile per 1 KiB),
 *     q = c / 128, m = (c / 32) % 4, t = r / 16, T = N / 16:
 *       code byte  = 16*(64*(q*T + t) + 16*g + i) + 4*m + e/2
 *       scale byte = 4*(16*(2*(q*T + t) + g/2) + i) + m      (block c/16)
 *   down (N = H, "row-grouped": a 64-row x 32-column tile per 1 KiB),
 *     k = c / 32, p = r / 64, j = (r / 16) % 4, P = N / 64:
 *       code byte  = 16*(64*(k*P + p) + 16*g + i) + 4*j + e/2
 *       scale byte = 4*(16*(2*(k*P + p) + g/2) + i) + j      (block c/16)
 *   globals: row r at byte 4*r of its region.
 * Requires H % 128 == 0 and I % 32 == 0 (I/tp a multiple of 32 is the
 * fp4 scale-block guard of issue #62 "What it touches"; H % 128 is this
 * format's tile).  Returns the slot size in bytes, or 0 for other shapes. */
size_t moe_nvfp4_slot_bytes(int H, int I);

/* ------------------------------------------------------------------ routing
 * Top-k expert selection with renormalised weights (issue #62, R9700 interim
 * report: norm_topk_prob renormalises the selected weights; the router is
 * replicated) and the permutation of the T*k assignments by expert.
 *   logits          f32 [T, E] router logits (NaN is a precondition violation)
 *   topk_ids        i32 [T, k] out: experts by (logit descending, index ascending)
 *   topk_w          f32 [T, k] out: softmax over the k selected logits
 *   expert_offsets  i32 [E+1]  out: exclusive scan of per-expert counts
 *   sorted_assign   i32 [T*k]  out: flat indices t*k+j ordered by (expert, t, j)
 *   assign_pos      i32 [T*k]  out: inverse of sorted_assign
 *   ws, ws_bytes    device scratch of at least moe_route_workspace_bytes(T, E, k)
 * The result is deterministic (no atomics decide any order). */
size_t moe_route_workspace_bytes(int T, int E, int k);
int moe_route_topk(const float* logits, int T, int E, int k, int32_t* topk_ids, float* topk_w,
                   int32_t* expert_offsets, int32_t* sorted_assign, int32_t* assign_pos, void* ws, size_t ws_bytes,
                   hipStream_t stream);

/* ------------------------------------------------------------------ router
 * The replicated router's projection (issue #62, R9700 interim report: the
 * router is replicated and its top-k weights renormalised), the step just
 * before the top-k above:
 *   logits[t, e] = sum_h x[t, h] * w_router[e, h]
 *   x          device bf16 [T, H] activations (row-major)
 *   w_router   device bf16 [E, H] router weights (row-major, one row per expert)
 *   logits     device f32 [T, E] out
 * bf16 products are exact in fp32; the sum is accumulated in fp32 in a fixed
 * order (T <= 16: vector dot products, one workgroup per expert row; larger
 * T: the matrix cores), so repeated calls give identical bits.
 * Shapes: T >= 0 (0 is a no-op), 1 <= E <= 1024, H % 256 == 0, H <= 16384,
 * T*H*2 and E*H*2 below 2^31 bytes; others return MOE_ERR_UNSUPPORTED_SHAPE
 * with nothing enqueued.  Buffers are owned by the caller. */
int moe_router_logits(const uint16_t* x, const uint16_t* w_router, int T, int H, int E, float* logits,
                      hipStream_t stream);

/* moe_router_logits followed by moe_route_topk on its logits, in one call
 * on `stream` (the router fused into routing): logits is written (f32
 * [T, E], the values the selection was made on) and the routing outputs are
 * those of moe_route_topk.  ws, ws_bytes: at least
 * moe_route_workspace_bytes(T, E, k).  All arguments are validated before
 * anything is enqueued. */
int moe_router_topk(const uint16_t* x, const uint16_t* w_router, int T, int H, int E, int k, float* logits,
                    int32_t* topk_ids, float* topk_w, int32_t* expert_offsets, int32_t* sorted_assign,
                    int32_t* assign_pos, void* ws, size_t ws_bytes, hipStream_t stream);

/* ------------------------------------------------------------------ layer
 * A layer's expert storage: E routed experts addressed through a slot map
 * into a bank of equally sized slots, plus an optional shared expert.
 *   bank_base       device base of the slot array (256-byte aligned)
 *   slot_bytes      must equal moe_nvfp4_slot_bytes(H, I)
 *   slot_of_expert  device i32 [E]: slot index of each expert, or -1 to leave it
 *                   out of this call (its assignments then contribute nothing)
 *   num_slots       number of slots at bank_base; an index outside [0, num_slots)
 *                   leaves its expert out exactly like -1 (no memory outside the
 *                   bank is read)
 *   shared_slot     device pointer to the shared expert's slot (same layout,
 *                   same H and I), or NULL for no shared expert
 *   shared_gate_w   device bf16 [H]: the shared expert's scalar gate
 *                   s_t = sigmoid(x_t . w); ignored when shared_slot is NULL
 * The struct is read during the call only (host pointer, not retained). */
typedef struct {
    int H, I, E, k;
    const void* bank_base;
    size_t slot_bytes;
    int num_slots;
    const int32_t* slot_of_expert;
    const void* shared_slot;
    const uint16_t* shared_gate_w;
} moe_nvfp4_layer_t;

/* Workspace the forward needs for T tokens; 0 on bad shapes. */
size_t moe_nvfp4_forward_workspace_bytes(int T, int H, int I, int E, int k);

/* The routed-MoE layer (PR #385 "What this adds": routed + sigmoid(gate) *
 * shared; issue #62 "What it touches": gate/up rows, down columns):
 *   y_t (=|+=) sum_j w_tj * FFN_{e_tj}(x_t) + s_t * FFN_shared(x_t)
 *   FFN(x) = W_dn (silu(W_gate x) * (W_up x)),  s_t = sigmoid(x_t . w_g)
 *   x        bf16 [T, H] activations
 *   routing  the outputs of moe_route_topk for the same T, E, k
 *   y        f32 [T, H]; accumulate = 0 writes y, 1 adds into y
 * Arithmetic: every contraction runs on the fp16 matrix cores
 * (v_mfma_f32_16x16x32_f16) with fp32 accumulation.  NVFP4 weights decode
 * exactly to fp16 (e2m1 * e4m3 has at most 6 significant bits); bf16
 * activations enter as fp16 times a per-token power of two, which is exact
 * in the fp16 normal range; the hidden state goes back into fp16 with a
 * power-of-two scale per (token, slice or 128-column tile); every scale is
 * undone exactly on the fp32 results.
 * T <= 16 (with H <= 2560) runs the decode path: one persistent kernel over
 * (expert, I-slice) work items whose operands are decoded in registers,
 * then a combine kernel that sums the slices and applies the down-row
 * globals in a fixed order.  Larger T runs the prefill path: grouped GEMMs
 * over the permuted tokens; its remainder tiles run on a library-owned side
 * stream forked from and joined back to `stream`, so the call stays ordered
 * on `stream` (and capturable in a graph).  Output order of summation is
 * fixed, so repeated calls give bit-identical results. */
int moe_nvfp4_forward(const moe_nvfp4_layer_t* layer, const uint16_t* x, int T, const int32_t* topk_ids,
                      const float* topk_w, const int32_t* expert_offsets, const int32_t* sorted_assign,
                      const int32_t* assign_pos, float* y, int accumulate, void* ws, size_t ws_bytes,
                      hipStream_t stream);

/* Workspace moe_nvfp4_route_forward needs for T tokens; 0 on bad shapes. */
size_t moe_nvfp4_route_forward_workspace_bytes(int T, int H, int I, int E, int k);

/* moe_route_topk followed by moe_nvfp4_forward in one call, with the same
 * results: the routing outputs (topk_ids, topk_w, expert_offsets,
 * sorted_assign, assign_pos, device buffers sized as for moe_route_topk) are
 * written, and y is the layer output for the routing of `logits` (device f32
 * [T, E]).  On the decode path with T <= 8 and E <= 256 the forward's first
 * kernel routes by itself in its prologue (one launch less on the critical
 * path of a decode step); otherwise the routing is its own launch on
 * `stream`.  The
 * workspace holds both calls' workspaces; the other arguments and errors are
 * those of the two calls. */
int moe_nvfp4_route_forward(const moe_nvfp4_layer_t* layer, const float* logits, const uint16_t* x, int T,
                            int32_t* topk_ids, float* topk_w, int32_t* expert_offsets, int32_t* sorted_assign,
                            int32_t* assign_pos, float* y, int accumulate, void* ws, size_t ws_bytes,
                            hipStream_t stream);

/* ------------------------------------------------------------------ without allocation
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation): the same
 * call as moe_nvfp4_route_forward with the same arguments, results and
 * errors, except that its workspace is a fixed array inside the library
 * (moe_nvfp4_noalloc_scratch_bytes() bytes, 32 MiB, held on each GPU the
 * library runs on until the process ends) instead of ws/ws_bytes.  It covers
 * the decode path (T <= 16, H <= 2560, T*k <= 1024) whose workspace fits
 * that array (T = 16, H = 2560, I = 640, k = 8 needs 29.6 MiB); other shapes
 * return MOE_ERR_UNSUPPORTED_SHAPE or MOE_ERR_WORKSPACE_TOO_SMALL with nothing
 * enqueued.  It calls no allocation routine.  All calls on one GPU share its
 * array: calls that can overlap on one GPU (different streams without
 * ordering between them) race and must be serialised by the caller. */
size_t moe_nvfp4_noalloc_scratch_bytes(void);
int moe_nvfp4_route_forward_noalloc(const moe_nvfp4_layer_t* layer, const float* logits, const uint16_t* x, int T,
                                    int32_t* topk_ids, float* topk_w, int32_t* expert_offsets,
                                    int32_t* sorted_assign, int32_t* assign_pos, float* y, int accumulate,
                                    hipStream_t stream);

/* ------------------------------------------------------------------ expert cache
 * Copy n expert slots from pinned host banks into GPU cache slots
 * (issue #62 "Why TP=2 loses today" and PR #385 "What this adds": the GPU
 * holds a fraction of the experts and streams misses over PCIe each step).
 *   cache_base   device base of num_slots slots of slot_bytes each
 *   dst_slots    host i32 [n]: destination slot of each copy (0 <= slot < num_slots)
 *   src          host array of n host pointers, each to slot_bytes of page-locked
 *                (hipHostMalloc / pinned) memory; non-pinned sources are refused
 *   copy_stream  stream the copies are enqueued on (one hipMemcpyAsync each)
 *   done         event recorded on copy_stream after the last copy, or NULL
 * Returns after enqueueing; the caller orders compute after `done`. */
int expert_cache_fill(void* cache_base, size_t slot_bytes, int num_slots, const int32_t* dst_slots,
                      const void* const* src, int n, hipStream_t copy_stream, hipEvent_t done);

/* Host-side slot manager for the expert cache: one pool of num_slots GPU
 * slots shared by every (layer, expert), least-recently-used replacement.
 * For one layer-step, moe_cache_plan takes the routed ids (host, any order,
 * repeats allowed), marks cached experts as most recent (ascending expert
 * order), assigns each missing expert, in ascending order, the lowest
 * never-used slot or else the least recently used entry's slot, and reports:
 *   slot_of_expert  host i32 [E]: slot of every routed expert, -1 otherwise
 *   miss_experts    host i32 [n]: missing experts in ascending order (first *n_miss)
 *   miss_slots      host i32 [n]: the slot each miss must be filled into
 * Returns MOE_ERR_INVALID_ARGUMENT if one layer-step needs more distinct
 * experts than the pool holds.  Not thread-safe per handle. */
typedef struct moe_expert_cache moe_expert_cache_t;
moe_expert_cache_t* moe_cache_create(int num_layers, int num_experts, int num_slots);
void moe_cache_destroy(moe_expert_cache_t* cache);
int moe_cache_plan(moe_expert_cache_t* cache, int layer, const int32_t* ids, int n, int32_t* slot_of_expert,
                   int32_t* miss_experts, int32_t* miss_slots, int* n_miss, int* n_hit);

/* ------------------------------------------------------------------ offload engine
 * One MoE layer-step over the expert cache (issue #62 "Why TP=2 loses
 * today": the GPU caches a fraction of the experts and streams the rest over
 * PCIe; PR #385 "Measurements": prefill serves cache hits from device
 * memory).  The engine keeps a device-side directory of where every
 * (layer, expert) is cached, so each step routes, looks the routed experts up
 * on the GPU and starts the hits-only forward (with the shared expert)
 * before the host sees anything; the host then waits only for the small
 * lookup result (copied ahead of that forward), plans with the same LRU
 * policy as moe_cache_plan (one pool of num_slots slots over all layers;
 * hits refreshed, misses into never-used or least recently used slots, never
 * a slot this step reads), copies the misses on copy_stream and runs the
 * misses-only forward accumulating into y.  Steps without misses run one
 * forward.  NVFP4 slots.
 *   moe_offload_device_bytes  device workspace the engine needs (directory,
 *                             routing, lookup, forward workspace); 0 on bad sizes
 *   moe_offload_create        cache_base: device, num_slots slots of
 *                             moe_nvfp4_slot_bytes(H, I), 256-byte aligned;
 *                             host_slots: host array of num_layers*num_experts
 *                             pointers to page-locked slots (layer-major), not
 *                             copied; dev_ws: that workspace (256-byte aligned),
 *                             initialised on `stream`.  Buffers stay owned by
 *                             the caller and must outlive the engine; the engine
 *                             itself allocates two small page-locked host
 *                             buffers, three events and a second copy stream
 *                             (the misses alternate between copy_stream and
 *                             it).  NULL on error.
 *   moe_offload_layer         logits f32 [T, E], x bf16 [T, H], 1 <= T <= T_max;
 *                             shared_slot / shared_gate_w as in the layer struct
 *                             (NULL: none); y f32 [T, H] out; n_hit / n_miss:
 *                             host out.  Synchronises the host with `stream`
 *                             once per step (after the lookup); not capturable.
 * Not thread-safe per engine. */
typedef struct moe_offload moe_offload_t;
size_t moe_offload_device_bytes(int num_layers, int num_experts, int k, int T_max, int H, int I);
moe_offload_t* moe_offload_create(int num_layers, int num_experts, int k, int H, int I, int T_max, void* cache_base,
                                  int num_slots, const void* const* host_slots, void* dev_ws, size_t dev_ws_bytes,
                                  hipStream_t stream);
void moe_offload_destroy(moe_offload_t* engine);
int moe_offload_layer(moe_offload_t* engine, int layer, const float* logits, const uint16_t* x, int T,
                      const void* shared_slot, const uint16_t* shared_gate_w, float* y, hipStream_t stream,
                      hipStream_t copy_stream, int* n_hit, int* n_miss);

/* ------------------------------------------------------------------ bank slicing
 * Intermediate-axis slice r of n of every slot in a bank (issue #62 "What it
 * touches": gate_up gives two disjoint row ranges, down a column slice; PR
 * #385: codes, scale blocks and per-row globals sliced to match):
 * dst slot j (shape H, I/n) gets gate rows [r*Il, (r+1)*Il) and up rows
 * [I + r*Il, I + (r+1)*Il) of src slot j, with their scales and globals, and
 * down columns [r*Il, (r+1)*Il) of all H rows, with all H globals.
 * Requires Il = I/n to be a multiple of 32. */
int moe_nvfp4_slice_bank(const void* src_bank, int num_slots, int H, int I, int r, int n, void* dst_bank,
                         hipStream_t stream);

/* ------------------------------------------------------------------ MXFP4 banks
 * The second fp4 bank format (issue #62 "What it touches": mxfp4, whose
 * checkpoints store each matrix transposed, blocks_t [K//2, N], with 32-wide
 * fp4 scale blocks; "Suggested staging": the last format to add): E2M1 codes
 * with one E8M0 scale (2^(byte - 127), 0xFF NaN) per 32 consecutive
 * elements along the contraction axis and no per-row global:
 *     W[r, c] = e2m1(code(r, c)) * e8m0(scale(r, c / 32)).
 * One slot holds, in this order and without padding:
 *     gate_up codes  2I*H/2 bytes     gate_up scales  2I*H/32 bytes
 *     down codes     H*I/2 bytes      down scales     H*I/32 bytes
 * in gfx950 matrix-core operand order (lane L = 16*a + i of a wave loads one
 * 16-byte piece): with i = r % 16,
 *   gate_up (N = 2I): a 16-row x 128-column tile per 1 KiB whose piece L is
 *     row i, columns [32a, 32a + 32) (the fp4 operand of
 *     v_mfma_scale_f32_16x16x128_f8f6f4, one scale block), q = c / 128,
 *     a = (c / 32) % 4, t = r / 16, T = N / 16:
 *       code byte  = 16*(64*(q*T + t) + 16*a + i) + (c % 32)/2
 *       scale byte = 64*(q*T + t) + 16*a + i                   (block c/32)
 *   down (N = H): the NVFP4 down tiling (64-row x 32-column tile per 1 KiB),
 *     k = c / 32, p = r / 64, j = (r / 16) % 4, g = (c / 8) % 4, P = N / 64:
 *       code byte  = 16*(64*(k*P + p) + 16*g + i) + 4*j + (c % 8)/2
 *       scale byte = 64*(k*P + p) + 4*i + j                    (block k)
 * The even column of a byte is its low nibble.  Same shape rules as NVFP4
 * slots (H % 128 == 0, I % 32 == 0); 0 for other shapes. */
size_t moe_mxfp4_slot_bytes(int H, int I);

/* Workspace moe_mxfp4_forward needs for T tokens; 0 for shapes it does not take. */
size_t moe_mxfp4_forward_workspace_bytes(int T, int H, int I, int E, int k);

/* The routed-MoE layer of moe_nvfp4_forward over MXFP4 slots (the same
 * layer struct with slot_bytes = moe_mxfp4_slot_bytes(H, I); the same
 * routing inputs, combine, accumulate and error rules, the same 2 GiB
 * buffer limits).  Decode path (T <= 16, T*k <= 1024, H <= 2560): gate_up
 * runs on v_mfma_scale_f32_16x16x128_f8f6f4 with the fp4 codes and E8M0
 * scales used as stored and the activations entered as two fp8 E4M3 terms
 * with their own E8M0 block scales (the bf16 value exactly, unless a block's
 * values span more than the fp8 range); down decodes its codes exactly to
 * bf16 with the scale applied by v_cvt_scalef32_pk_bf16_fp4 and multiplies
 * them on v_mfma_f32_16x16x32_bf16 against the hidden state as two bf16
 * terms.  Larger T (H <= 8192) runs the grouped-GEMM prefill path of
 * moe_nvfp4_forward with both matrices decoded exactly to bf16 by that
 * converter, on v_mfma_f32_16x16x32_bf16 against the bf16 activations
 * (gate_up) and the hidden state as two bf16 terms (down).  Sums are fp32 in
 * a fixed order (bit-reproducible). */
int moe_mxfp4_forward(const moe_nvfp4_layer_t* layer, const uint16_t* x, int T, const int32_t* topk_ids,
                      const float* topk_w, const int32_t* expert_offsets, const int32_t* sorted_assign,
                      const int32_t* assign_pos, float* y, int accumulate, void* ws, size_t ws_bytes,
                      hipStream_t stream);

/* Workspace moe_mxfp4_route_forward needs for T tokens; 0 for shapes it does not take. */
size_t moe_mxfp4_route_forward_workspace_bytes(int T, int H, int I, int E, int k);

/* moe_route_topk followed by moe_mxfp4_forward in one call, with the same
 * results and the same contract as moe_nvfp4_route_forward (routing outputs
 * written, y the layer output for the routing of `logits`, device f32
 * [T, E]).  With T <= 8 and E <= 256 the forward's kernel routes by itself in
 * its prologue; otherwise the routing is its own launch on `stream`, its
 * workspace after the forward's.  Every argument is checked before anything
 * is enqueued. */
int moe_mxfp4_route_forward(const moe_nvfp4_layer_t* layer, const float* logits, const uint16_t* x, int T,
                            int32_t* topk_ids, float* topk_w, int32_t* expert_offsets, int32_t* sorted_assign,
                            int32_t* assign_pos, float* y, int accumulate, void* ws, size_t ws_bytes,
                            hipStream_t stream);

/* MXFP4 decode of one matrix in the checkpoints' transposed layout:
 *   blocks_t  device u8 [K/2, N]: byte (j, n) = W[n, 2j] (low nibble), W[n, 2j+1]
 *   scales_t  device u8 [K/32, N]: E8M0 of (n, block)
 *   out       device f32 [N, K]
 * K a positive multiple of 32; N == 0 is a no-op.  Decoded by the converter
 * the forward's down phase uses (fp4 -> bf16 with the scale applied). */
int moe_mxfp4_dequant(const uint8_t* blocks_t, const uint8_t* scales_t, int N, int K, float* out,
                      hipStream_t stream);

/* One matrix of an MXFP4 slot to fp32, row-major, through the forward's own
 * decode: gate_up (matrix 0, out [2I, H]) through the scaled matrix cores
 * against one-hot fp8 columns, down (matrix 1, out [H, I]) through the bf16
 * converter. */
int moe_mxfp4_dequant_slot(const void* slot, int H, int I, int matrix, float* out, hipStream_t stream);

/* Intermediate-axis slice r of n of every MXFP4 slot in a bank.  In the
 * checkpoints' transposed tensors it runs along N of gate_up (columns
 * [r*Il, (r+1)*Il) and [I + r*Il, I + (r+1)*Il)) and along K of down (rows
 * [r*Il/2, (r+1)*Il/2) of blocks_t, [r*Il/32, (r+1)*Il/32) of scales_t),
 * Il = I/n a multiple of 32 (issue #62 "What it touches": mxfp4's slice is
 * along N and its scales slice differently). */
int moe_mxfp4_slice_bank(const void* src_bank, int num_slots, int H, int I, int r, int n, void* dst_bank,
                         hipStream_t stream);

/* ------------------------------------------------------------------ dequant
 * The NVFP4 decode of one row-major matrix (PR #385 "What this adds": packed
 * 4-bit codes, 16-wide FP8 scale blocks, per-row fp32 globals), with the
 * decode the forward kernels use:
 *     out[r, c] = f32(f32(e2m1(code(r, c)) * e4m3(scales[r, c/16])) * globals[r])
 *   codes    device u8 [rows, K/2]: element 2j of a row in the low nibble of byte j
 *   scales   device u8 [rows, K/16]: OCP E4M3FN bytes
 *   globals  device f32 [rows]
 *   out      device f32 [rows, K], 16-byte aligned (codes 4-byte aligned)
 * K must be a positive multiple of 16; rows == 0 is a no-op.  E4M3 NaN
 * scale bytes give NaN. */
int moe_nvfp4_dequant(const uint8_t* codes, const uint8_t* scales, const float* globals, int rows, int K, float* out,
                      hipStream_t stream);

/* The same decode of one matrix of one slot (the operand-order layout
 * above) to fp32, row-major: matrix 0 is gate_up (out [2I, H]), matrix 1 is
 * down (out [H, I]). */
int moe_nvfp4_dequant_slot(const void* slot, int H, int I, int matrix, float* out, hipStream_t stream);

/* ------------------------------------------------------------------ streams
 * Synchronise and destroy the side streams and events the prefill path
 * created for its callers' streams (the next prefill call creates them
 * again).  The caller must not have prefill work in flight or being captured
 * on any stream when calling this. */
int moe_release_streams(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_NVFP4_H */
