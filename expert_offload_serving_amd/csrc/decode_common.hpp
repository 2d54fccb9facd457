// Pieces shared by the decode-path kernels of both bank formats (NVFP4 in
// decode.hip, MXFP4 in mxfp4.hip): the kernel arguments, the routing tables
// staged in LDS, the work-item decode, the prologue that stages tables and
// activations (or routes in-kernel), and the combine that sums each row's
// slice partials in a fixed order with the shared expert's gated term.
#pragma once

#include "internal.hpp"
#include "nvfp4_device.hpp"
#include "route_device.hpp"

namespace moe {
namespace {
constexpr int kDW = 8;              // waves per workgroup
constexpr int kDT = kDW * kWave;    // threads per workgroup
constexpr int kSl = 32;             // intermediate rows per work item
constexpr int kMaxE = 1024;         // experts (64 per ballot chunk)

struct DecArgs {
    const uint8_t* bank;
    size_t slot_bytes;
    int num_slots;
    const int32_t* slot_of_expert;
    const uint8_t* shared;
    const uint16_t* wg;
    const uint16_t* x;
    int T, H, I, E, k;
    const float* w;
    const int32_t* offsets;
    const int32_t* sorted_assign;
    float* part;   // [(T*k + T) * nsl, H]: row (assignment or T*k + token) * nsl + slice, times the row's weight
    int32_t* rowslot;  // [(T*k + T)]: slot of each row's expert (-1 left out, -2 shared)
    float* dgrow;      // [(T*k + T), H]: the rows' down-row globals, when spare workgroups copy them (else null)
    int n_spare;       // spare workgroups at the end of the grid
    float* y;
    int accumulate;
    int gu_codes, gu_scales, gu_glob, dn_codes, dn_scales, dn_glob;  // region offsets in a slot
    int no_glob;       // 1: the format has no down-row globals (MXFP4); the partials are final
    // routing inside the kernel (route_forward): the logits in, the routing outputs (written by workgroup 0)
    const float* logits;
    int32_t *r_ids, *r_offsets, *r_sorted, *r_pos;
    float* r_w;
    int route_wg;      // the workgroup that writes the routing outputs
};

// A slot index outside [0, num_slots) leaves its expert out (-1), like a
// negative one: the kernels never address memory outside the bank.
__device__ __forceinline__ int slot_or_skip(int sl, int num_slots) { return sl >= 0 && sl < num_slots ? sl : -1; }

// Routing tables staged in LDS once per workgroup.
struct Tables {
    alignas(16) int ids[kDecodeMaxAssign];   // top-k ids, when the kernel routes (first: 16-byte aligned)
    int off[kMaxE + 1];          // expert_offsets
    int slot[kMaxE];             // slot_of_expert
    int sorted[kDecodeMaxAssign];
    float w[kDecodeMaxAssign];
    int act[kMaxE];              // experts with assignments, ascending
    int n_act;
};
constexpr int kRouteInKernelMaxE = 256;  // experts the decode kernels route themselves (4 logits per lane)

// A work item as seen by one lane: its slice, its tokens (the MFMA's 16
// columns) and the expert's slot as a buffer resource (0 bytes when the
// expert is left out or there is no item, so every load reads zeros).
struct Item {
    int s, ne, begin;
    bool shared;     // the shared expert (rows T*k + token) rather than a routed one
    int slot_index;  // the expert's slot, -1 when left out, -2 for the shared expert
    int tok, prow;   // this lane's column: token (-1: none) and output row
    float wc;        // this lane's column weight
    rsrc_t sres;
};

// Branch-free on purpose: with a divergent branch (c < ne) inside the
// routed/shared choice, the compiler would treat the slot as divergent and
// wrap every buffer load in a readfirstlane loop.  n_act must be
// wave-uniform (read with readfirstlane).
__device__ __forceinline__ Item decode_item(const DecArgs& a, const Tables& tb, int n_act, int nsl, int u, bool valid,
                                            int c) {
    Item it;
    const int ui = u / nsl;
    it.s = u % nsl;
    // the shared expert's items come first: they need no routing, so a kernel can start them before it routes
    const bool has_sh = a.shared != nullptr;
    const int ri = has_sh ? ui - 1 : ui;
    const bool shared = valid && has_sh && ui == 0;
    const bool routed = valid && !shared && ri < n_act;
    const int e = __builtin_amdgcn_readfirstlane(tb.act[routed ? ri : 0]);
    const int e_ok = routed ? e : 0;
    const int b0 = __builtin_amdgcn_readfirstlane(tb.off[e_ok]);
    const int b1 = __builtin_amdgcn_readfirstlane(tb.off[e_ok + 1]);
    const int sl = __builtin_amdgcn_readfirstlane(tb.slot[e_ok]);
    it.shared = shared;
    it.begin = routed ? b0 : 0;
    it.ne = routed ? b1 - b0 : (shared ? a.T : 0);
    it.slot_index = routed ? sl : (shared ? -2 : -1);
    const uint8_t* slot = routed ? (sl >= 0 ? a.bank + (size_t)sl * a.slot_bytes : nullptr) : (shared ? a.shared : nullptr);
    it.sres = make_rsrc(slot != nullptr ? slot : a.bank, slot != nullptr ? (uint32_t)a.slot_bytes : 0u);
    const bool has_col = c < it.ne;
    const int as = tb.sorted[it.begin + (routed && has_col ? c : 0)];
    const float ws = tb.w[routed && has_col ? as : 0];
    it.tok = !has_col ? -1 : (routed ? as / a.k : c);
    it.prow = !has_col ? 0 : (routed ? as : a.T * a.k + c);
    it.wc = !has_col ? 0.0f : (routed ? ws : 1.0f);
    return it;
}

// Prologue shared by the decode kernels (NW waves per workgroup), in two
// parts so that a kernel can start its first weight loads in between.
// stage_tables issues the routing-table and activation loads in one batch
// (tables first, so waiting for them waits for nothing else), puts the
// tables in LDS and lists the experts that have assignments (ascending); it
// ends with a workgroup barrier and returns their number (wave-uniform).
// stage_x then writes every token's activations to LDS as fp16 times a
// per-token power of two (xsh); the caller synchronises before reading them.
template <int NW>
struct XRegs {
    static constexpr int XT = (kDecodeMaxT + NW - 1) / NW;  // token rows staged per wave
    static constexpr int XC = 2560 / 8 / kWave;             // 16-byte chunks of a token row per lane (H <= 2560)
    u32x4_t v[XT][XC];
};

template <int NW>
__device__ __forceinline__ int stage_tables(const DecArgs& a, Tables& tb, XRegs<NW>& xr, int tid, int lane,
                                            int wave) {
    constexpr int NT = NW * kWave;
    const int H = a.H, T = a.T, k = a.k, E = a.E, n = T * k;
    constexpr int R = (kMaxE + 1 + NT - 1) / NT;
    constexpr int RA = (kDecodeMaxAssign + NT - 1) / NT;
    uint32_t vo[R], vs[R], va[RA], vw[RA];
    {
        const rsrc_t ro = make_rsrc(a.offsets, (uint32_t)(E + 1) * 4);
        const rsrc_t rs = make_rsrc(a.slot_of_expert, (uint32_t)E * 4);
        const rsrc_t ra = make_rsrc(a.sorted_assign, (uint32_t)n * 4);
        const rsrc_t rw = make_rsrc(a.w, (uint32_t)n * 4);
        const rsrc_t rx = make_rsrc(a.x, (uint32_t)T * H * 2);
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int i = tid + NT * r;
            vo[r] = buf_load4(ro, i <= E ? 4 * i : kOob);
            vs[r] = buf_load4(rs, i < E ? 4 * i : kOob);
        }
#pragma unroll
        for (int r = 0; r < RA; ++r) {
            const int i = tid + NT * r;
            va[r] = buf_load4(ra, i < n ? 4 * i : kOob);
            vw[r] = buf_load4(rw, i < n ? 4 * i : kOob);
        }
#pragma unroll
        for (int p = 0; p < XRegs<NW>::XT; ++p) {  // wave w stages tokens w, w + NW, ...
            const int t = wave + NW * p;
#pragma unroll
            for (int i = 0; i < XRegs<NW>::XC; ++i) {
                const int ch = lane + kWave * i;
                xr.v[p][i] = buf_load16(rx, t < T && ch < H / 8 ? 2 * (t * H + 8 * ch) : kOob);
            }
        }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int i = tid + NT * r;
        if (i <= E) tb.off[i] = (int)vo[r];
        if (i < E) tb.slot[i] = slot_or_skip((int)vs[r], a.num_slots);
    }
#pragma unroll
    for (int r = 0; r < RA; ++r) {
        const int i = tid + NT * r;
        if (i < n) tb.sorted[i] = (int)va[r], tb.w[i] = __uint_as_float(vw[r]);
    }
    __syncthreads();
    if (wave == 0) {  // compaction of the experts with assignments, ascending
        const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        int base = 0;
        for (int e0 = 0; e0 < E; e0 += kWave) {
            const int e = e0 + lane;
            const bool act = e < E && tb.off[e + 1] > tb.off[e];
            const uint64_t m = __ballot(act);
            if (act) tb.act[base + __popcll(m & below)] = e;
            base += __popcll(m);
        }
        if (lane == 0) tb.n_act = base;
    }
    __syncthreads();
    return __builtin_amdgcn_readfirstlane(tb.n_act);
}

// The same prologue for a kernel that routes itself (E <= 256): wave w
// selects the top-k of tokens w and w + NW straight from the logits, then
// every assignment is ranked directly,
//   offsets[e] = #{b : e_b < e},  pos(a) = #{b : (e_b, b) < (e_a, a)},
// the same stable grouping the routing kernels produce (for one token, whose
// k experts are distinct, a single pass over the experts).  Workgroup
// a.route_wg writes the routing outputs.
// after_loads() runs once the slot-map and activation loads are issued, before
// the routing: a caller can start loads that need no routing there, behind the
// activations (which every path then finds issued before its weight loads).
template <int NW, class AfterLoads>
__device__ __forceinline__ int stage_route(const DecArgs& a, Tables& tb, XRegs<NW>& xr, int tid, int lane,
                                           int wave, AfterLoads&& after_loads) {
    constexpr int NT = NW * kWave;
    const int H = a.H, T = a.T, k = a.k, E = a.E, n = T * k;
    constexpr int R = (kMaxE + NT - 1) / NT;
    uint32_t vs[R];
    {
        const rsrc_t rs = make_rsrc(a.slot_of_expert, (uint32_t)E * 4);
        const rsrc_t rx = make_rsrc(a.x, (uint32_t)T * H * 2);
        // groups of loads that no lane needs are skipped (uniform conditions), so that the routing's logit
        // loads do not queue behind out-of-range ones in the address units
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int i = tid + NT * r;
            vs[r] = NT * r < E ? buf_load4(rs, i < E ? 4 * i : kOob) : 0u;
        }
#pragma unroll
        for (int p = 0; p < XRegs<NW>::XT; ++p) {
            const int t = wave + NW * p;
#pragma unroll
            for (int i = 0; i < XRegs<NW>::XC; ++i) {
                const int ch = lane + kWave * i;
                xr.v[p][i] = t < T ? buf_load16(rx, ch < H / 8 ? 2 * (t * H + 8 * ch) : kOob) : u32x4_t{0, 0, 0, 0};
            }
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    after_loads();
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int p = 0; p < (kDecodeMaxT + NW - 1) / NW; ++p) {  // wave w: tokens w, w + NW
        const int t = wave + NW * p;
        if (t < T)
            topk_one_token<kRouteInKernelMaxE / kWave>(a.logits + (size_t)t * E, E, k, tb.ids + t * k, tb.w + t * k,
                                                        lane);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int i = tid + NT * r;
        if (i < E) tb.slot[i] = slot_or_skip((int)vs[r], a.num_slots);
    }
    __syncthreads();
    const bool out = (int)blockIdx.x == a.route_wg;
    if (T == 1) {  // uniform.  One token's k experts are distinct: each expert's group holds at most one assignment,
                   // so one pass over the experts gives offsets, the active list and the permutation
        const int4* ids4 = reinterpret_cast<const int4*>(tb.ids);  // read four at a time; ids past k are not used
        for (int e = tid; e <= E; e += NT) {
            int lt = 0, at = -1;
#pragma unroll 2
            for (int b = 0; b < k; b += 4) {
                const int4 v = ids4[b / 4];
                const int eb[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const bool in = b + u < k;
                    lt += in && eb[u] < e ? 1 : 0;
                    at = in && eb[u] == e ? b + u : at;
                }
            }
            tb.off[e] = lt;
            if (at >= 0) tb.act[lt] = e, tb.sorted[lt] = at;
            if (out) {
                a.r_offsets[e] = lt;
                if (at >= 0) {
                    a.r_ids[at] = e;
                    a.r_w[at] = tb.w[at];
                    a.r_sorted[lt] = at;
                    a.r_pos[at] = lt;
                }
            }
        }
        __syncthreads();
        return k;
    }
    // P consecutive lanes (a power of two, up to 16) share one assignment's count
    int P = 1;
    while (P < 16 && 2 * P * n <= NT) P *= 2;
    for (int idx = tid; idx < n * P; idx += NT) {
        const int as = idx / P, part = idx % P;
        const int e = tb.ids[as];
        int pos = 0;
#pragma unroll 4
        for (int b = part; b < n; b += P) {
            const int eb = tb.ids[b];
            pos += (eb < e || (eb == e && b < as)) ? 1 : 0;
        }
        for (int o = 1; o < P; o <<= 1) pos += __shfl_xor(pos, o, kWave);
        if (part == 0) {
            tb.sorted[pos] = as;
            if (out) {
                a.r_ids[as] = e;
                a.r_w[as] = tb.w[as];
                a.r_sorted[pos] = as;
                a.r_pos[as] = pos;
            }
        }
    }
    __syncthreads();
    // offsets[e]: the first sorted position whose expert is >= e
    for (int e = tid; e <= E; e += NT) {
        int lo = 0, hi = n;
        while (lo < hi) {
            const int mid = (lo + hi) >> 1;
            if (tb.ids[tb.sorted[mid]] < e) lo = mid + 1;
            else hi = mid;
        }
        tb.off[e] = lo;
        if (out) a.r_offsets[e] = lo;
    }
    __syncthreads();
    if (wave == 0) {  // compaction of the experts with assignments, ascending
        const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
        int base = 0;
        for (int e0 = 0; e0 < E; e0 += kWave) {
            const int e = e0 + lane;
            const bool act = e < E && tb.off[e + 1] > tb.off[e];
            const uint64_t m = __ballot(act);
            if (act) tb.act[base + __popcll(m & below)] = e;
            base += __popcll(m);
        }
        if (lane == 0) tb.n_act = base;
    }
    __syncthreads();
    return __builtin_amdgcn_readfirstlane(tb.n_act);
}

// y_t = sum_j dg_j * (sum over slices of row j's partials) over the routed
// rows j of token t, plus sigmoid(x_t . w_g) * dg_sh * (shared partials), in a
// fixed order; dg_j are the down-row globals of row j's expert, found through
// the slot the forward kernel recorded for the row.  Workgroup: one token and 64 output columns; thread (q, cl)
// handles row q (q < k: assignment t*k + q; q == k: the shared expert) of
// columns [4 cl, 4 cl + 4).  The first pass issues all of its loads before
// the first add (rows and slices past the end read as zero).
// CS: slices per row loaded in the first pass, the smallest instantiated
// batch that covers nsl (out-of-range loads still take the address units).
template <int CS>
__global__ void __launch_bounds__(256) dcombine_kernel(DecArgs a, int nsl, int nch) {
    __shared__ f32x4_t rr[16][16], rsh[16][16];
    __shared__ float dots[4];
    const int t = blockIdx.x / nch, ch = blockIdx.x % nch;
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave, cl = tid & 15, q = tid >> 4;
    const int H = a.H, k = a.k, T = a.T;
    const int col = 64 * ch + 4 * cl;
    const bool has_shared = a.shared != nullptr;
    const int nrows = k + (has_shared ? 1 : 0);
    const rsrc_t pres = make_rsrc(a.part, (uint32_t)((size_t)(T * k + T) * nsl * H * 4));
    const rsrc_t dgres = make_rsrc(a.dgrow, (uint32_t)((size_t)(T * k + T) * H * 4));
    f32x4_t sr = {0.0f, 0.0f, 0.0f, 0.0f}, ss = {0.0f, 0.0f, 0.0f, 0.0f};
    float gd = 0.0f;
    // this thread's chunks (tid, tid + 256) of x_t and w_g for the shared gate, loaded first so that their
    // latency overlaps the partials' (H <= 2560: at most 320 chunks)
    u32x4_t gx[2], gw[2];
    {
        const rsrc_t xres = make_rsrc(a.x + (size_t)t * H, has_shared ? (uint32_t)H * 2 : 0u);
        const rsrc_t gres = make_rsrc(a.wg, has_shared ? (uint32_t)H * 2 : 0u);
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int vv = tid + 256 * r;
            gx[r] = buf_load16(xres, vv < H / 8 ? 16 * vv : kOob);
            gw[r] = buf_load16(gres, vv < H / 8 ? 16 * vv : kOob);
        }
    }
    for (int j = q; j < nrows; j += 16) {
        const int row = j < k ? t * k + j : T * k + t;
        f32x4_t v[CS];
#pragma unroll
        for (int i = 0; i < CS; ++i)
            v[i] = __builtin_bit_cast(f32x4_t, buf_load16(pres, i < nsl ? 4 * ((row * nsl + i) * H + col) : kOob));
        f32x4_t dg = {1.0f, 1.0f, 1.0f, 1.0f};
        if (a.no_glob) {  // uniform: nothing to scale
        } else if (a.dgrow != nullptr) {  // uniform: the rows' globals were copied by the item kernel
            dg = __builtin_bit_cast(f32x4_t, buf_load16(dgres, 4 * (row * H + col)));
        } else {
            // (an entry outside the bank or the shared marker is read as "left out": never an address)
            const int rs0 = a.rowslot[row];
            const int rs = rs0 == -2 ? -2 : slot_or_skip(rs0, a.num_slots);
            const uint8_t* slot = rs >= 0 ? a.bank + (size_t)rs * a.slot_bytes : (rs == -2 ? a.shared : a.bank);
            const rsrc_t gsr = make_rsrc(slot, rs == -1 || (rs == -2 && a.shared == nullptr) ? 0u : (uint32_t)a.slot_bytes);
            dg = __builtin_bit_cast(f32x4_t, buf_load16(gsr, a.dn_glob + 4 * col));
        }
        __builtin_amdgcn_sched_barrier(0);
        f32x4_t sum = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int i = 0; i < CS; ++i) sum += v[i];
        for (int i = CS; i < nsl; ++i)
            sum += __builtin_bit_cast(f32x4_t, buf_load16(pres, 4 * ((row * nsl + i) * H + col)));
        if (j < k) sr += sum * dg;
        else ss = sum * dg;
    }
    if (has_shared) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            if (tid + 256 * r >= H / 8) break;  // the chunks in order, as the sum always ran
            gd = dot2_bf16(as_bf16x2(gx[r].x), as_bf16x2(gw[r].x), gd);
            gd = dot2_bf16(as_bf16x2(gx[r].y), as_bf16x2(gw[r].y), gd);
            gd = dot2_bf16(as_bf16x2(gx[r].z), as_bf16x2(gw[r].z), gd);
            gd = dot2_bf16(as_bf16x2(gx[r].w), as_bf16x2(gw[r].w), gd);
        }
        gd = wave_sum(gd);
    }
    rr[q][cl] = sr;
    rsh[q][cl] = ss;
    if (lane == 0) dots[wave] = gd;
    __syncthreads();
    if (tid >= 16) return;
    f32x4_t tr = {0.0f, 0.0f, 0.0f, 0.0f}, ts = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int i = 0; i < 16; ++i) tr += rr[i][tid], ts += rsh[i][tid];
    f32x4_t out = tr;
    if (has_shared) out += sigmoidf_(((dots[0] + dots[1]) + dots[2]) + dots[3]) * ts;
    f32x4_t* yp = reinterpret_cast<f32x4_t*>(a.y + (size_t)t * H + 64 * ch + 4 * tid);
    if (a.accumulate) out += *yp;
    *yp = out;
}



}  // namespace
}  // namespace moe
