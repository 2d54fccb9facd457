/*
 * CPU oracle for the NVFP4 routed-MoE layer of an offloaded-MoE server.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the plain, slow, obviously-correct
 * definition that the HIP library is checked against.  Only the test suite,
 * the package smoke check and the CPU-baseline leg of the benchmark may load
 * it.  It shares no code, header, table or constant generator with the HIP
 * library, and the library never calls it.
 *
 * Sources (FreeToken pages): PR #385 "What this adds" (NVFP4 expert banks
 * with packed codes, 16-wide scale blocks and per-row globals; sliced along
 * the intermediate axis; combine routed + sigmoid(gate) * shared before one
 * reduction) and issue #62 "What it touches" (gate_up is [2I, H] with gate
 * rows [0, I) and up rows [I, 2I); down is [H, I]; a rank's slice is two
 * disjoint gate/up row ranges plus a down column slice), and the R9700
 * interim report on #62 (norm_topk_prob: the k selected weights are
 * renormalised; the router is replicated).  Number formats: E2M1 and E4M3FN
 * are the OCP 8-bit / microscaling element formats.
 *
 * Readings where the pages are silent (each one is listed in the design doc):
 *  - code nibble order: of two columns sharing a byte, the even one is the
 *    low nibble;
 *  - slot byte order: the library header's operand-order formulas (a storage
 *    choice; the pages fix no byte order), read here element by element;
 *  - scale blocks run along the contraction axis (H for gate_up, I for down);
 *  - dequant: W = f32( f32(e2m1 * e4m3) * global ), the inner product exact;
 *  - routing weights: softmax over the k selected logits (the same as a full
 *    softmax followed by renormalisation over the top k), ties in selection
 *    broken by the lower expert index;
 *  - activation: SwiGLU, silu(gate) * up, no clamp;
 *  - shared gate: s_t = sigmoid(x_t . w_g), applied after the shared expert;
 *  - the MXFP4 bank format (issue #62 "What it touches" names it, its
 *    transposed blocks_t [K//2, N] and its 32-wide fp4 scale blocks): E2M1
 *    elements times one OCP E8M0 scale per 32 consecutive elements along
 *    the contraction axis, no per-row global; the scales are stored
 *    transposed like the blocks, scales_t [K/32, N]; W = f32(e2m1 * e8m0).
 *
 * Arithmetic: fp32 dequant, double accumulation, one rounding to f32 at the
 * output.  Build: gcc -O2 -fno-fast-math -ffp-contract=off -fopenmp.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

/* ---------------------------------------------------------------- formats */

/* E2M1: sign bit, 2 exponent bits (bias 1), 1 mantissa bit; no inf/NaN.
 * Exponent field 0 is subnormal: value 0.5 * m. */
double oracle_e2m1(int code) {
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -mag : mag;
}

/* E4M3FN (OCP): sign, 4 exponent bits (bias 7), 3 mantissa bits; no inf;
 * S.1111.111 is NaN; exponent field 0 is subnormal: (m/8) * 2^-6. */
double oracle_e4m3(int byte) {
    int s = (byte >> 7) & 1, e = (byte >> 3) & 15, m = byte & 7;
    if (e == 15 && m == 7) return NAN;
    double mag = (e == 0) ? ldexp(m / 8.0, -6) : ldexp(1.0 + m / 8.0, e - 7);
    return s ? -mag : mag;
}

static double bf16_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* One dequantised row: out[c] = f32( f32(e2m1(code) * e4m3(scale)) * g ). */
static void dequant_row(const uint8_t* codes, const uint8_t* scales, float g, int K, float* out) {
    for (int c = 0; c < K; ++c) {
        int code = (codes[c / 2] >> (4 * (c & 1))) & 0xF;
        float q = (float)(oracle_e2m1(code) * oracle_e4m3(scales[c / 16]));
        out[c] = q * g;
    }
}

/* Dequantise a [rows, K] NVFP4 matrix into fp32. */
void oracle_dequant(const uint8_t* codes, const uint8_t* scales, const float* globals, int rows, int K,
                    float* out) {
    for (int r = 0; r < rows; ++r)
        dequant_row(codes + (size_t)r * (K / 2), scales + (size_t)r * (K / 16), globals[r], K,
                    out + (size_t)r * K);
}

/* ---------------------------------------------------------------- routing */

/* Top-k by (logit descending, expert index ascending); weights are the
 * softmax over the k chosen logits, in double, stored rounded to f32.
 * Returns 0, or -1 if a logit is NaN (a precondition violation). */
int oracle_route(const float* logits, int T, int E, int k, int32_t* ids, float* w) {
    char* taken = (char*)malloc((size_t)E);
    double* ex = (double*)malloc(sizeof(double) * (size_t)k);
    int rc = 0;
    for (int t = 0; t < T && rc == 0; ++t) {
        const float* l = logits + (size_t)t * E;
        memset(taken, 0, (size_t)E);
        for (int e = 0; e < E; ++e)
            if (isnan(l[e])) rc = -1;
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e]) continue;
                if (best < 0 || l[e] > l[best]) best = e; /* strict: the lower index wins ties */
            }
            taken[best] = 1;
            ids[(size_t)t * k + j] = best;
        }
        double m = l[ids[(size_t)t * k]];
        double sum = 0.0;
        for (int j = 0; j < k; ++j) {
            ex[j] = exp((double)l[ids[(size_t)t * k + j]] - m);
            sum += ex[j];
        }
        for (int j = 0; j < k; ++j) w[(size_t)t * k + j] = (float)(ex[j] / sum);
    }
    free(taken);
    free(ex);
    return rc;
}

/* Router projection (the replicated router of the R9700 interim report on
 * #62, whose outputs the top-k above selects from): logits[t, e] =
 * sum_h x[t, h] * w[e, h] over bf16 activations x [T, H] and bf16 router
 * weights w [E, H], accumulated in double and rounded to f32 once. */
void oracle_router_logits(const uint16_t* x, const uint16_t* w, int T, int H, int E, float* logits) {
    for (int t = 0; t < T; ++t)
        for (int e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int h = 0; h < H; ++h) acc += bf16_to_double(x[(size_t)t * H + h]) * bf16_to_double(w[(size_t)e * H + h]);
            logits[(size_t)t * E + e] = (float)acc;
        }
}

/* Counting sort of the T*k assignments by expert.  offsets[E+1] is the
 * exclusive scan of the per-expert counts; sorted_assign lists flat indices
 * t*k+j ordered by (expert, t, j); assign_pos is its inverse. */
void oracle_permute(const int32_t* ids, int T, int E, int k, int32_t* offsets, int32_t* sorted_assign,
                    int32_t* assign_pos) {
    int n = T * k;
    int32_t* fill = (int32_t*)calloc((size_t)E + 1, sizeof(int32_t));
    for (int e = 0; e <= E; ++e) offsets[e] = 0;
    for (int a = 0; a < n; ++a) offsets[ids[a] + 1] += 1;
    for (int e = 0; e < E; ++e) offsets[e + 1] += offsets[e];
    for (int a = 0; a < n; ++a) {
        int e = ids[a];
        int p = offsets[e] + fill[e]++;
        sorted_assign[p] = a;
        assign_pos[a] = p;
    }
    free(fill);
}

/* ---------------------------------------------------------------- layer */

/* Byte offset of code (r, c) and of scale (r, block b) of a matrix with N
 * rows, in the slot's operand order (see the library header):
 * gate_up keeps a 16-row x 128-column tile per 1 KiB, down a 64-row x
 * 32-column tile; inside a tile, lane record 16*g + i holds row i (of the
 * 16-row group) and columns [8g, 8g+8) of each 32-column chunk. */
static size_t gu_code_at(int N, int r, int c) {
    size_t q = c / 128, m = (c / 32) % 4, g = (c / 8) % 4, e = c % 8, t = r / 16, i = r % 16;
    return 16 * (64 * (q * (N / 16) + t) + 16 * g + i) + 4 * m + e / 2;
}
static size_t gu_scale_at(int N, int r, int b) {
    size_t q = b / 8, m = (b / 2) % 4, h = b % 2, t = r / 16, i = r % 16;
    return 4 * (16 * (2 * (q * (N / 16) + t) + h) + i) + m;
}
static size_t dn_code_at(int N, int r, int c) {
    size_t k = c / 32, g = (c / 8) % 4, e = c % 8, p = r / 64, j = (r / 16) % 4, i = r % 16;
    return 16 * (64 * (k * (N / 64) + p) + 16 * g + i) + 4 * j + e / 2;
}
static size_t dn_scale_at(int N, int r, int b) {
    size_t k = b / 2, h = b % 2, p = r / 64, j = (r / 16) % 4, i = r % 16;
    return 4 * (16 * (2 * (k * (N / 64) + p) + h) + i) + j;
}

/* One matrix of a slot: N rows of K columns. */
typedef struct {
    const uint8_t *codes, *scales;
    const float* glob;
    int N, K, down;
} mat_view;

/* Region order in a slot: gate_up codes, gate_up scales, gate_up globals,
 * down codes, down scales, down globals, without padding. */
static mat_view view_matrix(const uint8_t* slot, int H, int I, int down) {
    size_t gc = (size_t)2 * I * H / 2, gs = (size_t)2 * I * H / 16, gg = (size_t)2 * I * 4;
    size_t dc = (size_t)H * I / 2, ds = (size_t)H * I / 16;
    mat_view v;
    if (!down) {
        v.codes = slot;
        v.scales = slot + gc;
        v.glob = (const float*)(slot + gc + gs);
        v.N = 2 * I, v.K = H;
    } else {
        v.codes = slot + gc + gs + gg;
        v.scales = v.codes + dc;
        v.glob = (const float*)(v.scales + ds);
        v.N = H, v.K = I;
    }
    v.down = down;
    return v;
}

static int code_of(const mat_view* v, int r, int c) {
    size_t o = v->down ? dn_code_at(v->N, r, c) : gu_code_at(v->N, r, c);
    return (v->codes[o] >> (4 * (c & 1))) & 0xF;
}

static int scale_of(const mat_view* v, int r, int b) {
    return v->scales[v->down ? dn_scale_at(v->N, r, b) : gu_scale_at(v->N, r, b)];
}

/* Row r of a slot matrix, dequantised: out[c] = f32( f32(e2m1 * e4m3) * g ). */
static void dequant_view_row(const mat_view* v, int r, float* out) {
    for (int c = 0; c < v->K; ++c) {
        float q = (float)(oracle_e2m1(code_of(v, r, c)) * oracle_e4m3(scale_of(v, r, c / 16)));
        out[c] = q * v->glob[r];
    }
}

int oracle_shape_ok(int H, int I) { return H > 0 && I > 0 && H % 128 == 0 && I % 32 == 0; }

size_t oracle_slot_bytes(int H, int I) {
    return (size_t)2 * I * H / 2 + (size_t)2 * I * H / 16 + (size_t)2 * I * 4 + (size_t)H * I / 2 +
           (size_t)H * I / 16 + (size_t)H * 4;
}

/* Dequantise matrix 0 (gate_up, [2I, H]) or 1 (down, [H, I]) of a slot. */
int oracle_dequant_slot(const uint8_t* slot, int H, int I, int matrix, float* out) {
    if (!oracle_shape_ok(H, I) || matrix < 0 || matrix > 1) return -1;
    mat_view v = view_matrix(slot, H, I, matrix);
    for (int r = 0; r < v.N; ++r) dequant_view_row(&v, r, out + (size_t)r * v.K);
    return 0;
}

/* Read matrix 0 or 1 of a slot back into row-major arrays: codes [N, K/2]
 * (even column in the low nibble), scales [N, K/16], globals [N]. */
int oracle_unpack_slot(const uint8_t* slot, int H, int I, int matrix, uint8_t* codes, uint8_t* scales,
                       float* globals) {
    if (!oracle_shape_ok(H, I) || matrix < 0 || matrix > 1) return -1;
    mat_view v = view_matrix(slot, H, I, matrix);
    for (int r = 0; r < v.N; ++r) {
        for (int c = 0; c < v.K; c += 2)
            codes[(size_t)r * (v.K / 2) + c / 2] = (uint8_t)(code_of(&v, r, c) | (code_of(&v, r, c + 1) << 4));
        for (int b = 0; b < v.K / 16; ++b) scales[(size_t)r * (v.K / 16) + b] = (uint8_t)scale_of(&v, r, b);
        globals[r] = v.glob[r];
    }
    return 0;
}

/* silu(z) * up with silu(z) = z / (1 + exp(-z)). */
static double swiglu(double gate, double up) { return gate / (1.0 + exp(-gate)) * up; }

/* Expert FFN for one token from the expert's dequantised matrices:
 * a = W_gu x; h = silu(a[:I]) * a[I:]; o = W_dn h, every sum in double in
 * column order. */
static void expert_ffn(const float* Wgu, const float* Wdn, int H, int I, const double* x, double* a, double* h,
                       double* o) {
    for (int r = 0; r < 2 * I; ++r) {
        const float* row = Wgu + (size_t)r * H;
        double acc = 0.0;
        for (int c = 0; c < H; ++c) acc += (double)row[c] * x[c];
        a[r] = acc;
    }
    for (int i = 0; i < I; ++i) h[i] = swiglu(a[i], a[I + i]);
    for (int r = 0; r < H; ++r) {
        const float* row = Wdn + (size_t)r * I;
        double acc = 0.0;
        for (int c = 0; c < I; ++c) acc += (double)row[c] * h[c];
        o[r] = acc;
    }
}

/* Shared-expert gate: s_t = 1 / (1 + exp(-(x_t . w_g))), dot in double. */
void oracle_shared_gate(const uint16_t* x, int T, int H, const uint16_t* wg, double* s) {
    for (int t = 0; t < T; ++t) {
        double g = 0.0;
        for (int c = 0; c < H; ++c) g += bf16_to_double(x[(size_t)t * H + c]) * bf16_to_double(wg[c]);
        s[t] = 1.0 / (1.0 + exp(-g));
    }
}

static int cmp_long(const void* a, const void* b) {
    long x = *(const long*)a, y = *(const long*)b;
    return (x > y) - (x < y);
}

/* y_t = sum_j w_tj * FFN_{ids[t,j]}(x_t) + s_t * FFN_shared(x_t), in double,
 * rounded once to f32.  Experts are found through slot_of_expert in the
 * bank (slot index, or -1 to leave that expert out); shared_slot < 0 means
 * no shared term.  Computes the n_tokens rows listed in tokens (all T when
 * tokens is NULL), y laid out in list order.  Returns 0 or -1 on bad input.
 *
 * Each slot that some listed token uses is dequantised once into dense fp32
 * matrices (the definition of the weights), every (token, expert) output
 * o_tj is formed from them and kept in double, and each token's outputs are
 * then added in the order j = 0..k-1, shared last. */
/* Dequantises both matrices of a slot: Wgu [2I, H] and Wdn [H, I], fp32 row-major. */
typedef void (*slot_dequant_fn)(const uint8_t* slot, int H, int I, float* Wgu, float* Wdn);

static void nvfp4_slot_dequant(const uint8_t* slot, int H, int I, float* Wgu, float* Wdn) {
    mat_view gu = view_matrix(slot, H, I, 0), dn = view_matrix(slot, H, I, 1);
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
    for (int r = 0; r < 2 * I + H; ++r) {
        if (r < 2 * I) dequant_view_row(&gu, r, Wgu + (size_t)r * H);
        else dequant_view_row(&dn, r - 2 * I, Wdn + (size_t)(r - 2 * I) * I);
    }
}

static int forward_core(int H, int I, int E, int k, const uint8_t* bank, size_t slot_bytes,
                        const int32_t* slot_of_expert, long shared_slot, const uint16_t* wg, const uint16_t* x, int T,
                        const int32_t* ids, const float* w, const int32_t* tokens, int n_tokens, float* y,
                        int nthreads, slot_dequant_fn dequant_slot_matrices);

int oracle_forward(int H, int I, int E, int k, const uint8_t* bank, size_t slot_bytes, const int32_t* slot_of_expert,
                   long shared_slot, const uint16_t* wg, const uint16_t* x, int T, const int32_t* ids, const float* w,
                   const int32_t* tokens, int n_tokens, float* y, int nthreads) {
    if (!oracle_shape_ok(H, I) || slot_bytes != oracle_slot_bytes(H, I)) return -1;
    return forward_core(H, I, E, k, bank, slot_bytes, slot_of_expert, shared_slot, wg, x, T, ids, w, tokens, n_tokens,
                        y, nthreads, nvfp4_slot_dequant);
}

static int forward_core(int H, int I, int E, int k, const uint8_t* bank, size_t slot_bytes,
                        const int32_t* slot_of_expert, long shared_slot, const uint16_t* wg, const uint16_t* x, int T,
                        const int32_t* ids, const float* w, const int32_t* tokens, int n_tokens, float* y,
                        int nthreads, slot_dequant_fn dequant_slot_matrices) {
    if (tokens == NULL) n_tokens = T;
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
#else
    (void)nthreads;
#endif
    const int K1 = k + 1; /* per token: k routed outputs, then the shared one */
    /* the slot of each (listed token, j) pair, -1 if it contributes nothing */
    long* use = (long*)malloc(sizeof(long) * (size_t)n_tokens * K1);
    for (int n = 0; n < n_tokens; ++n) {
        int t = tokens ? tokens[n] : n;
        if (t < 0 || t >= T) { free(use); return -1; }
        for (int j = 0; j < k; ++j) {
            int e = ids[(size_t)t * k + j];
            if (e < 0 || e >= E) { free(use); return -1; }
            use[(size_t)n * K1 + j] = slot_of_expert[e];
        }
        use[(size_t)n * K1 + k] = shared_slot >= 0 ? shared_slot : -1;
    }
    /* the distinct slots used, ascending */
    size_t npairs = (size_t)n_tokens * K1, nd = 0;
    long* slots = (long*)malloc(sizeof(long) * (npairs + 1));
    for (size_t i = 0; i < npairs; ++i)
        if (use[i] >= 0) slots[nd++] = use[i];
    qsort(slots, nd, sizeof(long), cmp_long);
    size_t nu = 0;
    for (size_t i = 0; i < nd; ++i)
        if (nu == 0 || slots[i] != slots[nu - 1]) slots[nu++] = slots[i];

    double* out = (double*)calloc(npairs * (size_t)H, sizeof(double)); /* o_tj for every used pair */
    float* Wgu = (float*)malloc(sizeof(float) * (size_t)2 * I * H);
    float* Wdn = (float*)malloc(sizeof(float) * (size_t)H * I);
    for (size_t u = 0; u < nu; ++u) {
        dequant_slot_matrices(bank + (size_t)slots[u] * slot_bytes, H, I, Wgu, Wdn);
#ifdef _OPENMP
#pragma omp parallel
#endif
        {
            double* xd = (double*)malloc(sizeof(double) * (size_t)H);
            double* a = (double*)malloc(sizeof(double) * (size_t)2 * I);
            double* h = (double*)malloc(sizeof(double) * (size_t)I);
#ifdef _OPENMP
#pragma omp for schedule(dynamic, 1)
#endif
            for (long i = 0; i < (long)npairs; ++i) {
                if (use[i] != slots[u]) continue;
                int n = (int)(i / K1), t = tokens ? tokens[n] : n;
                for (int c = 0; c < H; ++c) xd[c] = bf16_to_double(x[(size_t)t * H + c]);
                expert_ffn(Wgu, Wdn, H, I, xd, a, h, out + (size_t)i * H);
            }
            free(xd); free(a); free(h);
        }
    }
    for (int n = 0; n < n_tokens; ++n) {
        int t = tokens ? tokens[n] : n;
        double* acc = (double*)calloc((size_t)H, sizeof(double));
        for (int j = 0; j < k; ++j) {
            if (use[(size_t)n * K1 + j] < 0) continue;
            double wj = (double)w[(size_t)t * k + j];
            const double* o = out + ((size_t)n * K1 + j) * H;
            for (int c = 0; c < H; ++c) acc[c] += wj * o[c];
        }
        if (shared_slot >= 0) {
            double g = 0.0;
            for (int c = 0; c < H; ++c) g += bf16_to_double(x[(size_t)t * H + c]) * bf16_to_double(wg[c]);
            double st = 1.0 / (1.0 + exp(-g));
            const double* o = out + ((size_t)n * K1 + k) * H;
            for (int c = 0; c < H; ++c) acc[c] += st * o[c];
        }
        for (int c = 0; c < H; ++c) y[(size_t)n * H + c] = (float)acc[c];
        free(acc);
    }
    free(use); free(slots); free(out); free(Wgu); free(Wdn);
    return 0;
}

/* ---------------------------------------------------------------- MXFP4 */

/* The second fp4 bank format of issue #62 "What it touches": OCP MX FP4,
 * E2M1 elements with one shared E8M0 scale per 32 consecutive elements along
 * the contraction axis (the fp4 scale-block size of that section) and no
 * per-row global.  E8M0: 8 exponent bits, bias 127, no sign or mantissa;
 * 0xFF is NaN. */
double oracle_e8m0(int byte) { return (byte & 0xFF) == 0xFF ? NAN : ldexp(1.0, (byte & 0xFF) - 127); }

/* An MXFP4 matrix W [N, K] as its checkpoints store it, transposed
 * (issue #62 "What it touches": blocks_t [K//2, N]): byte (j, n) of
 * blocks_t holds W[n, 2j] in its low nibble and W[n, 2j+1] in its high
 * nibble; the scales are transposed the same way, scales_t [K/32, N].
 *     W[n, c] = f32( e2m1(code(n, c)) * e8m0(scales_t[c/32, n]) )
 * (the product is exact in double; one rounding to f32). */
void oracle_mx_dequant_t(const uint8_t* blocks_t, const uint8_t* scales_t, int N, int K, float* out) {
    for (int n = 0; n < N; ++n)
        for (int c = 0; c < K; ++c) {
            int code = (blocks_t[(size_t)(c / 2) * N + n] >> (4 * (c & 1))) & 0xF;
            out[(size_t)n * K + c] = (float)(oracle_e2m1(code) * oracle_e8m0(scales_t[(size_t)(c / 32) * N + n]));
        }
}

/* Byte offsets in an MXFP4 slot (the library header's formulas):
 * gate_up [2I, H] keeps a 16-row x 128-column tile per 1 KiB, lane record
 * 16*a + i holding row i and the 32 columns [32a, 32a+32) of the tile; its
 * scales are one byte per (row, 32-column block), the byte of lane record
 * 16*a + i in a 64-byte record per tile.  down [H, I] keeps a 64-row x
 * 32-column tile per 1 KiB exactly like the NVFP4 down matrix; its scales
 * are 64 bytes per tile, byte 4*i + j for row 16*j + i of the tile. */
static size_t mx_gu_code_at(int N, int r, int c) {
    size_t q = c / 128, a = (c / 32) % 4, e = c % 32, t = r / 16, i = r % 16;
    return 16 * (64 * (q * (N / 16) + t) + 16 * a + i) + e / 2;
}
static size_t mx_gu_scale_at(int N, int r, int b) {
    size_t q = b / 4, a = b % 4, t = r / 16, i = r % 16;
    return 64 * (q * (N / 16) + t) + 16 * a + i;
}
static size_t mx_dn_code_at(int N, int r, int c) {
    size_t kc = c / 32, g = (c / 8) % 4, e = c % 8, p = r / 64, j = (r / 16) % 4, i = r % 16;
    return 16 * (64 * (kc * (N / 64) + p) + 16 * g + i) + 4 * j + e / 2;
}
static size_t mx_dn_scale_at(int N, int r, int b) {
    size_t p = r / 64, j = (r / 16) % 4, i = r % 16;
    return 64 * ((size_t)b * (N / 64) + p) + 4 * i + j;
}

/* Region order in an MXFP4 slot: gate_up codes, gate_up scales, down
 * codes, down scales, without padding. */
size_t oracle_mx_slot_bytes(int H, int I) {
    return (size_t)2 * I * H / 2 + (size_t)2 * I * H / 32 + (size_t)H * I / 2 + (size_t)H * I / 32;
}

typedef struct {
    const uint8_t *codes, *scales;
    int N, K, down;
} mx_view;

static mx_view mx_view_matrix(const uint8_t* slot, int H, int I, int down) {
    size_t gc = (size_t)2 * I * H / 2, gs = (size_t)2 * I * H / 32, dc = (size_t)H * I / 2;
    mx_view v;
    if (!down) {
        v.codes = slot;
        v.scales = slot + gc;
        v.N = 2 * I, v.K = H;
    } else {
        v.codes = slot + gc + gs;
        v.scales = v.codes + dc;
        v.N = H, v.K = I;
    }
    v.down = down;
    return v;
}

static int mx_code_of(const mx_view* v, int r, int c) {
    size_t o = v->down ? mx_dn_code_at(v->N, r, c) : mx_gu_code_at(v->N, r, c);
    return (v->codes[o] >> (4 * (c & 1))) & 0xF;
}

static int mx_scale_of(const mx_view* v, int r, int b) {
    return v->scales[v->down ? mx_dn_scale_at(v->N, r, b) : mx_gu_scale_at(v->N, r, b)];
}

/* Row r of an MXFP4 slot matrix, dequantised: out[c] = f32(e2m1 * e8m0). */
static void mx_dequant_view_row(const mx_view* v, int r, float* out) {
    for (int c = 0; c < v->K; ++c)
        out[c] = (float)(oracle_e2m1(mx_code_of(v, r, c)) * oracle_e8m0(mx_scale_of(v, r, c / 32)));
}

/* Dequantise matrix 0 (gate_up, [2I, H]) or 1 (down, [H, I]) of an MXFP4 slot. */
int oracle_mx_dequant_slot(const uint8_t* slot, int H, int I, int matrix, float* out) {
    if (!oracle_shape_ok(H, I) || matrix < 0 || matrix > 1) return -1;
    mx_view v = mx_view_matrix(slot, H, I, matrix);
    for (int r = 0; r < v.N; ++r) mx_dequant_view_row(&v, r, out + (size_t)r * v.K);
    return 0;
}

/* Read matrix 0 or 1 of an MXFP4 slot back into the checkpoints' transposed
 * tensors: blocks_t [K/2, N] and scales_t [K/32, N]. */
int oracle_mx_unpack_slot(const uint8_t* slot, int H, int I, int matrix, uint8_t* blocks_t, uint8_t* scales_t) {
    if (!oracle_shape_ok(H, I) || matrix < 0 || matrix > 1) return -1;
    mx_view v = mx_view_matrix(slot, H, I, matrix);
    for (int r = 0; r < v.N; ++r) {
        for (int c = 0; c < v.K; c += 2)
            blocks_t[(size_t)(c / 2) * v.N + r] = (uint8_t)(mx_code_of(&v, r, c) | (mx_code_of(&v, r, c + 1) << 4));
        for (int b = 0; b < v.K / 32; ++b) scales_t[(size_t)b * v.N + r] = (uint8_t)mx_scale_of(&v, r, b);
    }
    return 0;
}

/* Slice r of n along the intermediate axis of an MXFP4 slot, I_l = I / n.
 * In the checkpoints' transposed tensors this is (issue #62 "What it
 * touches": mxfp4's slice runs along N and its scales slice differently):
 * gate_up blocks_t [H/2, 2I] and scales_t [H/32, 2I] keep the columns
 * [r*I_l, (r+1)*I_l) and [I + r*I_l, I + (r+1)*I_l); down blocks_t [I/2, H]
 * keeps the rows [r*I_l/2, (r+1)*I_l/2) and scales_t [I/32, H] the rows
 * [r*I_l/32, (r+1)*I_l/32).  Written element by element through the byte
 * formulas.  Returns 0, or -1 unless I_l is a multiple of 32. */
int oracle_mx_slice_slot(const uint8_t* src, int H, int I, int r, int n, uint8_t* dst) {
    if (n <= 0 || r < 0 || r >= n || I % n || !oracle_shape_ok(H, I)) return -1;
    int Il = I / n;
    if (!oracle_shape_ok(H, Il)) return -1;
    memset(dst, 0, oracle_mx_slot_bytes(H, Il));
    mx_view sg = mx_view_matrix(src, H, I, 0), sd = mx_view_matrix(src, H, I, 1);
    mx_view dg = mx_view_matrix(dst, H, Il, 0), dd = mx_view_matrix(dst, H, Il, 1);
    uint8_t *dgc = (uint8_t*)dg.codes, *dgs = (uint8_t*)dg.scales, *ddc = (uint8_t*)dd.codes,
            *dds = (uint8_t*)dd.scales;
    for (int rr = 0; rr < 2 * Il; ++rr) {
        int from = rr < Il ? r * Il + rr : I + r * Il + (rr - Il);
        for (int c = 0; c < H; ++c) dgc[mx_gu_code_at(2 * Il, rr, c)] |= (uint8_t)(mx_code_of(&sg, from, c) << (4 * (c & 1)));
        for (int b = 0; b < H / 32; ++b) dgs[mx_gu_scale_at(2 * Il, rr, b)] = (uint8_t)mx_scale_of(&sg, from, b);
    }
    for (int row = 0; row < H; ++row) {
        for (int c = 0; c < Il; ++c)
            ddc[mx_dn_code_at(H, row, c)] |= (uint8_t)(mx_code_of(&sd, row, r * Il + c) << (4 * (c & 1)));
        for (int b = 0; b < Il / 32; ++b) dds[mx_dn_scale_at(H, row, b)] = (uint8_t)mx_scale_of(&sd, row, r * Il / 32 + b);
    }
    return 0;
}

static void mxfp4_slot_dequant(const uint8_t* slot, int H, int I, float* Wgu, float* Wdn) {
    mx_view gu = mx_view_matrix(slot, H, I, 0), dn = mx_view_matrix(slot, H, I, 1);
#ifdef _OPENMP
#pragma omp parallel for schedule(static)
#endif
    for (int r = 0; r < 2 * I + H; ++r) {
        if (r < 2 * I) mx_dequant_view_row(&gu, r, Wgu + (size_t)r * H);
        else mx_dequant_view_row(&dn, r - 2 * I, Wdn + (size_t)(r - 2 * I) * I);
    }
}

/* The layer of oracle_forward with MXFP4 expert slots (same routing,
 * shared expert, SwiGLU and combine; only the weight decode differs). */
int oracle_mx_forward(int H, int I, int E, int k, const uint8_t* bank, size_t slot_bytes,
                      const int32_t* slot_of_expert, long shared_slot, const uint16_t* wg, const uint16_t* x, int T,
                      const int32_t* ids, const float* w, const int32_t* tokens, int n_tokens, float* y, int nthreads) {
    if (!oracle_shape_ok(H, I) || slot_bytes != oracle_mx_slot_bytes(H, I)) return -1;
    return forward_core(H, I, E, k, bank, slot_bytes, slot_of_expert, shared_slot, wg, x, T, ids, w, tokens, n_tokens,
                        y, nthreads, mxfp4_slot_dequant);
}

/* ---------------------------------------------------------------- slicing */

/* Slice r of n along the intermediate axis, I_l = I / n: the gate_up of
 * the result has gate rows [r*I_l, (r+1)*I_l) followed by up rows
 * [I + r*I_l, I + (r+1)*I_l), each with its codes, scales and global; its
 * down has columns [r*I_l, (r+1)*I_l) of every one of the H rows, with the
 * matching scale blocks and all H globals.  dst is a slot of shape (H, I_l),
 * written element by element through the format's byte formulas.  Returns 0,
 * or -1 if the slice is not a valid slot shape (I_l % 32 != 0). */
int oracle_slice_slot(const uint8_t* src, int H, int I, int r, int n, uint8_t* dst) {
    if (n <= 0 || r < 0 || r >= n || I % n || !oracle_shape_ok(H, I)) return -1;
    int Il = I / n;
    if (!oracle_shape_ok(H, Il)) return -1;
    memset(dst, 0, oracle_slot_bytes(H, Il));
    mat_view sg = view_matrix(src, H, I, 0), sd = view_matrix(src, H, I, 1);
    mat_view dg = view_matrix(dst, H, Il, 0), dd = view_matrix(dst, H, Il, 1);
    uint8_t *dgc = (uint8_t*)dg.codes, *dgs = (uint8_t*)dg.scales, *ddc = (uint8_t*)dd.codes,
            *dds = (uint8_t*)dd.scales;
    float *dgg = (float*)dg.glob, *ddg = (float*)dd.glob;
    for (int rr = 0; rr < 2 * Il; ++rr) {
        int from = rr < Il ? r * Il + rr : I + r * Il + (rr - Il);
        for (int c = 0; c < H; ++c) dgc[gu_code_at(2 * Il, rr, c)] |= (uint8_t)(code_of(&sg, from, c) << (4 * (c & 1)));
        for (int b = 0; b < H / 16; ++b) dgs[gu_scale_at(2 * Il, rr, b)] = (uint8_t)scale_of(&sg, from, b);
        dgg[rr] = sg.glob[from];
    }
    for (int row = 0; row < H; ++row) {
        for (int c = 0; c < Il; ++c)
            ddc[dn_code_at(H, row, c)] |= (uint8_t)(code_of(&sd, row, r * Il + c) << (4 * (c & 1)));
        for (int b = 0; b < Il / 16; ++b) dds[dn_scale_at(H, row, b)] = (uint8_t)scale_of(&sd, row, r * Il / 16 + b);
        ddg[row] = sd.glob[row];
    }
    return 0;
}

/* ---------------------------------------------------------------- LRU model */

/* One global pool of C cache slots shared by every (layer, expert), cold
 * at the start.  For each step and each layer in order: take the distinct
 * routed experts in ascending order; first mark the ones already cached as
 * most recently used (ascending order), then give each missing one, in
 * ascending order, the lowest free slot or else the slot of the least
 * recently used entry, which is evicted.
 *
 * ids: [steps][L][T*k] routed expert ids.  Outputs per (step, layer):
 * hits and misses counts; slot_map [steps][L][E] (cache slot of each routed
 * expert after the fill, -1 for experts not routed); miss_slots
 * [steps][L][T*k] lists, in ascending expert order, the slot each miss was
 * put in (unused entries -1).  Returns 0, or -1 if C is smaller than the
 * number of distinct experts one layer-step needs. */
int oracle_lru_run(int L, int E, int C, int steps, int T, int k, const int32_t* ids, int32_t* hits, int32_t* misses,
                   int32_t* slot_map, int32_t* miss_slots) {
    int n = T * k;
    int32_t* where = (int32_t*)malloc(sizeof(int32_t) * (size_t)L * E); /* (l,e) -> slot or -1 */
    int32_t* owner = (int32_t*)malloc(sizeof(int32_t) * (size_t)C);     /* slot -> l*E+e or -1 */
    int32_t* prev = (int32_t*)malloc(sizeof(int32_t) * (size_t)C);      /* recency list over slots */
    int32_t* next = (int32_t*)malloc(sizeof(int32_t) * (size_t)C);
    char* routed = (char*)malloc((size_t)E);
    int head = -1, tail = -1; /* head = least recently used, tail = most recently used */
    int rc = 0;
    for (size_t i = 0; i < (size_t)L * E; ++i) where[i] = -1;
    for (int c = 0; c < C; ++c) owner[c] = -1, prev[c] = next[c] = -1;
#define UNLINK(c)                                   \
    do {                                            \
        if (prev[c] >= 0) next[prev[c]] = next[c];  \
        else head = next[c];                        \
        if (next[c] >= 0) prev[next[c]] = prev[c];  \
        else tail = prev[c];                        \
        prev[c] = next[c] = -1;                     \
    } while (0)
#define PUSH_MRU(c)                                 \
    do {                                            \
        prev[c] = tail; next[c] = -1;               \
        if (tail >= 0) next[tail] = c; else head = c; \
        tail = c;                                   \
    } while (0)
    int n_free_next = 0; /* slots [n_free_next, C) have never been used */
    for (int st = 0; st < steps && rc == 0; ++st) {
        for (int l = 0; l < L; ++l) {
            size_t sl = (size_t)st * L + l;
            const int32_t* id = ids + sl * n;
            memset(routed, 0, (size_t)E);
            int distinct = 0;
            for (int a = 0; a < n; ++a)
                if (!routed[id[a]]) routed[id[a]] = 1, distinct++;
            if (distinct > C) { rc = -1; break; }
            int h = 0, m = 0;
            for (int e = 0; e < E; ++e) {
                if (!routed[e]) continue;
                int c = where[(size_t)l * E + e];
                if (c >= 0) { UNLINK(c); PUSH_MRU(c); h++; }
            }
            int32_t* ms = miss_slots ? miss_slots + sl * n : NULL;
            if (ms) for (int a = 0; a < n; ++a) ms[a] = -1;
            for (int e = 0; e < E; ++e) {
                if (!routed[e] || where[(size_t)l * E + e] >= 0) continue;
                int c;
                if (n_free_next < C) c = n_free_next++;
                else {
                    c = head;
                    UNLINK(c);
                    where[owner[c]] = -1;
                }
                owner[c] = l * E + e;
                where[(size_t)l * E + e] = c;
                PUSH_MRU(c);
                if (ms) ms[m] = c;
                m++;
            }
            hits[sl] = h;
            misses[sl] = m;
            if (slot_map)
                for (int e = 0; e < E; ++e) slot_map[sl * E + e] = routed[e] ? where[(size_t)l * E + e] : -1;
        }
    }
#undef UNLINK
#undef PUSH_MRU
    free(where); free(owner); free(prev); free(next); free(routed);
    return rc;
}
