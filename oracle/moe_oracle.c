/*
 * moe_oracle.c -- plain CPU oracle for the four steps of MoE dispatch/combine.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the CPU
 * baseline of the benchmark; never by the product path.  It shares no code with
 * the HIP library.  Written for a reader checking it against the pages by eye:
 * straight loops, no blocking, no fusion, one rounding per written operation.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fno-fast-math -shared -fPIC
 * (no contraction: every fused multiply-add below is an explicit fmaf).
 *
 * Precision: where a floating-point value decides an integer (which experts are
 * chosen, which FP8 code is written) the oracle computes it in fp32, the
 * precision the kernels decide in.  The combine, whose result has a plain
 * definition, is summed in double and rounded once to bf16.
 */
#include "moe_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* exp recipe.  The pages do not say how scores are exponentiated; bit-exact  */
/* top-k across CPU and GPU needs one fixed fp32 recipe, so both sides follow */
/* the same written one: Cody-Waite reduction by ln 2 split into a 17-bit     */
/* high part and a low part, then the degree-7 Taylor polynomial of e^r      */
/* (coefficients 1/i! rounded to fp32) by Horner's rule with fma, then an     */
/* exact scaling by 2^n.  The +-80 clamp keeps every result normal.          */
/* ------------------------------------------------------------------------ */
float orc_exp_r(float z)
{
    if (z >= 80.0f) return INFINITY;
    if (z <= -80.0f) return 0.0f;
    const float n = rintf(z * 1.44269504f);          /* nearest integer to z/ln2 */
    float r = fmaf(-n, 0.693145751953125f, z);       /* z - n*ln2_hi, exact      */
    r = fmaf(-n, 1.4286068e-6f, r);                  /* - n*ln2_lo               */
    const float c2 = 0x1.0p-1f;         /* 1/2!  */
    const float c3 = 0x1.555556p-3f;    /* 1/3!  */
    const float c4 = 0x1.555556p-5f;    /* 1/4!  */
    const float c5 = 0x1.111112p-7f;    /* 1/5!  */
    const float c6 = 0x1.6c16c2p-10f;   /* 1/6!  */
    const float c7 = 0x1.a01a02p-13f;   /* 1/7!  */
    float p = c7;
    p = fmaf(p, r, c6);
    p = fmaf(p, r, c5);
    p = fmaf(p, r, c4);
    p = fmaf(p, r, c3);
    p = fmaf(p, r, c2);
    p = fmaf(p, r, 1.0f);
    p = fmaf(p, r, 1.0f);
    return ldexpf(p, (int)n);
}

/* Sigmoid score (DeepSeek-V3-shaped router): 1 / (1 + e^-x). */
float orc_sigmoid(float x)
{
    const float e = orc_exp_r(-x);
    return 1.0f / (1.0f + e);
}

void orc_exp_r_array(const float* z, float* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_exp_r(z[i]);
}

void orc_sigmoid_array(const float* x, float* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_sigmoid(x[i]);
}

/* ------------------------------------------------------------------------ */
/* OCP E4M3FN: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; no     */
/* infinities; 0x7F/0xFF are NaN; largest finite magnitude 0x7E = 448;        */
/* subnormals are m * 2^-9.                                                   */
/* ------------------------------------------------------------------------ */
double orc_e4m3_value(uint8_t code)
{
    const int sign = code >> 7;
    const int e = (code >> 3) & 15;
    const int m = code & 7;
    if (e == 15 && m == 7) return NAN;
    double v;
    if (e == 0) v = ldexp((double)m, -9);
    else v = ldexp(1.0 + m / 8.0, e - 7);
    return sign ? -v : v;
}

/* Nearest code by definition: the largest non-negative code whose value does
   not exceed |y|, compared with the midpoint to the next code; an exact tie
   goes to the even code.  Magnitudes at or above 448 give 448 (saturation).
   The sign bit is copied from y, so -0 and negatives that round to zero give
   0x80.  All comparisons are exact in double. */
static double e4m3_table[127];      /* values of the non-negative finite codes */

__attribute__((constructor)) static void fill_e4m3_table(void)
{
    for (int c = 0; c < 127; ++c) e4m3_table[c] = orc_e4m3_value((uint8_t)c);
}

uint8_t orc_e4m3_from_f32(float y)
{
    const double* table = e4m3_table;
    const uint8_t sign = signbit(y) ? 0x80 : 0x00;
    const double a = fabs((double)y);
    if (isnan(y)) return (uint8_t)(sign | 0x7F);
    if (a >= 448.0) return (uint8_t)(sign | 0x7E);
    int lo = 0, hi = 126;          /* table[lo] <= a < table[hi] */
    while (hi - lo > 1) {
        const int mid = (lo + hi) / 2;
        if (table[mid] <= a) lo = mid; else hi = mid;
    }
    const double midpoint = (table[lo] + table[hi]) / 2.0;
    int c;
    if (a < midpoint) c = lo;
    else if (a > midpoint) c = hi;
    else c = (lo % 2 == 0) ? lo : hi;
    return (uint8_t)(sign | c);
}

void orc_e4m3_from_f32_array(const float* y, uint8_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_from_f32(y[i]);
}

/* bf16 has 8 significant bits and fp32's exponent range (smallest normal
   2^-126, subnormal quantum 2^-133).  Round |v| to a multiple of its quantum,
   ties to even (nearbyint in the default rounding mode), then take the upper
   16 bits of the exact fp32 image. */
uint16_t orc_bf16_from_f64(double v)
{
    if (isnan(v)) return 0x7FC0;
    const int neg = signbit(v) ? 1 : 0;
    const double a = fabs(v);
    if (a == 0.0) return neg ? 0x8000 : 0x0000;
    int e;
    frexp(a, &e);                       /* a in [2^(e-1), 2^e) */
    int qexp = (e - 1) - 7;
    if (qexp < -133) qexp = -133;
    const double q = ldexp(1.0, qexp);
    const double r = nearbyint(a / q) * q;
    uint32_t bits;
    if (r >= ldexp(1.0, 128)) {
        bits = 0x7F800000u;
    } else {
        const float f = (float)r;       /* exact */
        memcpy(&bits, &f, 4);
    }
    return (uint16_t)((bits >> 16) | (neg ? 0x8000u : 0u));
}

void orc_bf16_from_f64_array(const double* v, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_from_f64(v[i]);
}

static float bf16_to_f32(uint16_t h)
{
    const uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, 4);
    return f;
}

/* ------------------------------------------------------------------------ */
/* Step 1: group-limited top-k routing.                                       */
/* The router output is a score per expert; each token keeps its best        */
/* topk_group groups (a group's score is the sum of its group_topn largest   */
/* expert scores) and then its topk best experts inside the kept groups;     */
/* weights are the selected scores divided by their sum.                     */
/* Readings: experts are contiguous per group; ties between equal scores go  */
/* to the lower expert (or group) index and -0 equals +0 (plain float        */
/* comparison); slots are filled in descending score order; sums are taken  */
/* left to right in that order.  Softmax selects on the raw logits (softmax  */
/* is strictly increasing) and renormalised weights are                      */
/* exp(l_j - l_0) / sum_i exp(l_i - l_0) over the selected slots.            */
/* ------------------------------------------------------------------------ */
static int ahead(float a, int ia, float b, int ib)
{
    if (a > b) return 1;
    if (a < b) return 0;
    return ia < ib;
}

int orc_route(int T, int E, int G, int g, int k, int group_topn, int score_fn,
              int renormalize, const float* logits, int32_t* idx, float* w)
{
    if (T < 0 || E <= 0 || G <= 0 || E % G != 0 || g < 1 || g > G || k < 1) return -1;
    const int Eg = E / G;
    if (k > g * Eg) return -1;
    int n = group_topn > 0 ? group_topn : k / g;
    if (n < 1) n = 1;
    if (n > Eg) return -1;
    if (score_fn != 0 && score_fn != 1) return -1;

    float* s = (float*)malloc(sizeof(float) * (size_t)E);
    float* gs = (float*)malloc(sizeof(float) * (size_t)G);
    char* taken = (char*)malloc((size_t)E);
    char* gkept = (char*)malloc((size_t)G);
    int* sel = (int*)malloc(sizeof(int) * (size_t)k);

    for (int t = 0; t < T; ++t) {
        const float* l = logits + (size_t)t * E;
        for (int e = 0; e < E; ++e) s[e] = (score_fn == 0) ? orc_sigmoid(l[e]) : l[e];

        /* group scores and group selection */
        if (G > 1) {
            for (int gr = 0; gr < G; ++gr) {
                memset(taken, 0, (size_t)E);
                float sum = 0.0f;
                for (int i = 0; i < n; ++i) {
                    int best = -1;
                    for (int e = gr * Eg; e < (gr + 1) * Eg; ++e) {
                        if (taken[e]) continue;
                        if (best < 0 || ahead(s[e], e, s[best], best)) best = e;
                    }
                    taken[best] = 1;
                    sum = (i == 0) ? s[best] : sum + s[best];
                }
                gs[gr] = sum;
            }
            memset(gkept, 0, (size_t)G);
            for (int i = 0; i < g; ++i) {
                int best = -1;
                for (int gr = 0; gr < G; ++gr) {
                    if (gkept[gr]) continue;
                    if (best < 0 || ahead(gs[gr], gr, gs[best], best)) best = gr;
                }
                gkept[best] = 1;
            }
        } else {
            gkept[0] = 1;
        }

        /* expert selection inside the kept groups */
        memset(taken, 0, (size_t)E);
        for (int j = 0; j < k; ++j) {
            int best = -1;
            for (int e = 0; e < E; ++e) {
                if (taken[e] || !gkept[e / Eg]) continue;
                if (best < 0 || ahead(s[e], e, s[best], best)) best = e;
            }
            taken[best] = 1;
            sel[j] = best;
        }

        /* weights */
        for (int j = 0; j < k; ++j) idx[(size_t)t * k + j] = sel[j];
        float* wt = w + (size_t)t * k;
        if (score_fn == 0) {
            if (renormalize) {
                float den = s[sel[0]];
                for (int j = 1; j < k; ++j) den = den + s[sel[j]];
                for (int j = 0; j < k; ++j) wt[j] = (den > 0.0f) ? s[sel[j]] / den : 0.0f;
            } else {
                for (int j = 0; j < k; ++j) wt[j] = s[sel[j]];
            }
        } else {
            if (renormalize) {
                const float l0 = l[sel[0]];
                float u[64];
                float* uu = (k <= 64) ? u : (float*)malloc(sizeof(float) * (size_t)k);
                for (int j = 0; j < k; ++j) uu[j] = orc_exp_r(l[sel[j]] - l0);
                float den = uu[0];
                for (int j = 1; j < k; ++j) den = den + uu[j];
                for (int j = 0; j < k; ++j) wt[j] = uu[j] / den;
                if (uu != u) free(uu);
            } else {
                /* full softmax probability of each selected expert */
                float lmax = l[0];
                for (int e = 1; e < E; ++e) if (l[e] > lmax) lmax = l[e];
                float den = orc_exp_r(l[0] - lmax);
                for (int e = 1; e < E; ++e) den = den + orc_exp_r(l[e] - lmax);
                for (int j = 0; j < k; ++j) wt[j] = orc_exp_r(l[sel[j]] - lmax) / den;
            }
        }
    }
    free(s); free(gs); free(taken); free(gkept); free(sel);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Step 2: routing layout, a stable counting sort of the (token, slot) pairs */
/* by expert.  Counts per expert feed the grouped GEMM; every pair gets a    */
/* unique receive row without any coordination; the receive row remembers    */
/* its source (token*k + slot) for the combine.                              */
/* Readings: inside an expert's region rows follow ascending source token;   */
/* ranks own contiguous blocks of E/R experts; cnt_r counts distinct tokens  */
/* with at least one expert on the rank; off_r[r] = off_e[r*E/R] counts      */
/* (token, expert) pairs.  Padded mode: expert e owns rows e*C .. e*C+C-1,   */
/* pairs beyond C are dropped (pos -1) and bit 0 of *flags is set; empty     */
/* rows keep recv_src -1.  Bit 1 of *flags marks an expert index outside     */
/* [0,E) or repeated inside one token (the outputs are then unspecified).    */
/* ------------------------------------------------------------------------ */
int orc_layout(int T, int E, int k, int R, int C, int A, const int32_t* idx,
               int32_t* cnt_e, int32_t* cnt_r, int32_t* off_e, int32_t* off_r,
               int32_t* pos, int32_t* recv_src, int32_t* flags)
{
    if (T < 0 || E <= 0 || k < 1 || R <= 0 || E % R != 0 || C < 0 || A < 0) return -1;
    if (A > 1 && C > 0) return -1;
    const int Er = E / R;
    const int64_t N = (C > 0) ? (int64_t)E * C
                              : (int64_t)T * k + (A > 1 ? (int64_t)E * (A - 1) : 0);
    *flags = 0;

    for (int t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            const int e = idx[(size_t)t * k + j];
            if (e < 0 || e >= E) *flags |= 2;
            for (int i = 0; i < j; ++i)
                if (idx[(size_t)t * k + i] == e) *flags |= 2;
        }
    if (*flags & 2) return 0;

    for (int e = 0; e < E; ++e) cnt_e[e] = 0;
    for (int r = 0; r < R; ++r) cnt_r[r] = 0;
    char* hit = (char*)malloc((size_t)R);
    for (int t = 0; t < T; ++t) {
        memset(hit, 0, (size_t)R);
        for (int j = 0; j < k; ++j) {
            const int e = idx[(size_t)t * k + j];
            cnt_e[e] += 1;
            hit[e / Er] = 1;
        }
        for (int r = 0; r < R; ++r) cnt_r[r] += hit[r];
    }
    free(hit);

    /* Reading for the aligned variant (the pages mention a GEMM-friendly
       receive layout without describing it): every expert region starts on a
       multiple of A rows. */
    off_e[0] = 0;
    for (int e = 0; e < E; ++e) {
        int span = cnt_e[e];
        if (A > 1) span = (span + A - 1) / A * A;
        off_e[e + 1] = off_e[e] + span;
    }
    for (int r = 0; r <= R; ++r) off_r[r] = off_e[r * Er];

    if (C > 0 || A > 1)
        for (int64_t i = 0; i < N; ++i) recv_src[i] = -1;

    int32_t* seen = (int32_t*)calloc((size_t)E, sizeof(int32_t));
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            const int e = idx[(size_t)t * k + j];
            const int rank = seen[e]++;
            int32_t p;
            if (C == 0) {
                p = off_e[e] + rank;
            } else if (rank < C) {
                p = e * C + rank;
            } else {
                p = -1;
                *flags |= 1;
            }
            pos[(size_t)t * k + j] = p;
            if (p >= 0) recv_src[p] = t * k + j;
        }
    free(seen);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Step 3: dispatch.  Each token row goes to each of its receive rows, in    */
/* FP8 with block scaling factors (or verbatim in BF16).                     */
/* Readings: OCP E4M3FN; one fp32 scale per 128 consecutive channels;        */
/* a = max(amax, 2^-100); scale = a / 448 and inv = 448 / a (fp32, correctly */
/* rounded); code = nearest E4M3FN of the fp32 product x * inv; the scales   */
/* are a separate row-aligned [N, H/128] fp32 tensor.  dtype 2 takes the      */
/* power-of-two scale below instead, and dtype 3 stores that scale 2^e as    */
/* the one byte e + 127 (E8M0), the grouped-GEMM-friendly form.             */
/* ------------------------------------------------------------------------ */
/* One block of 128 fp32 values -> E4M3FN codes with a power-of-two scale:
   a = max(max |v|, 2^-100); scale = 2^e, the smallest power of two with
   a <= 448 * 2^e; code i = nearest E4M3FN of the exactly scaled v[i] * 2^-e.
   Returns the scale. */
static float quant_block_pow2(const float* v, uint8_t* q)
{
    float amax = 0.0f;
    for (int i = 0; i < 128; ++i)
        if (fabsf(v[i]) > amax) amax = fabsf(v[i]);
    const float a = (amax > 0x1.0p-100f) ? amax : 0x1.0p-100f;
    int e = ilogbf(a) - 9;
    while (ldexp(448.0, e) < (double)a) ++e;
    for (int i = 0; i < 128; ++i) q[i] = orc_e4m3_from_f32(ldexpf(v[i], -e));
    return ldexpf(1.0f, e);
}

int orc_dispatch(int T, int H, int k, int N, int dtype, const uint16_t* x,
                 const int32_t* pos, void* recv_x, void* recv_scales)
{
    if (T < 0 || H <= 0 || k < 1 || N < 0) return -1;
    if (dtype == 1) {
        uint16_t* out = (uint16_t*)recv_x;
        for (int t = 0; t < T; ++t)
            for (int j = 0; j < k; ++j) {
                const int p = pos[(size_t)t * k + j];
                if (p < 0) continue;
                if (p >= N) return -1;
                for (int c = 0; c < H; ++c)
                    out[(size_t)p * H + c] = x[(size_t)t * H + c];
            }
        return 0;
    }
    if ((dtype != 0 && dtype != 2 && dtype != 3) || H % 128 != 0) return -1;
    const int S = H / 128;
    uint8_t* out = (uint8_t*)recv_x;
    uint8_t q[128];
    for (int t = 0; t < T; ++t)
        for (int b = 0; b < S; ++b) {
            const uint16_t* xb = x + (size_t)t * H + (size_t)b * 128;
            float amax = 0.0f;
            for (int i = 0; i < 128; ++i) {
                const float v = fabsf(bf16_to_f32(xb[i]));
                if (v > amax) amax = v;
            }
            const float a = (amax > 0x1.0p-100f) ? amax : 0x1.0p-100f;
            float scale;
            if (dtype == 0) {
                scale = a / 448.0f;
                const float inv = 448.0f / a;
                for (int i = 0; i < 128; ++i) {
                    const float prod = bf16_to_f32(xb[i]) * inv;
                    q[i] = orc_e4m3_from_f32(prod);
                }
            } else {
                float v[128];
                for (int i = 0; i < 128; ++i) v[i] = bf16_to_f32(xb[i]);
                scale = quant_block_pow2(v, q);
            }
            for (int j = 0; j < k; ++j) {
                const int p = pos[(size_t)t * k + j];
                if (p < 0) continue;
                if (p >= N) return -1;
                memcpy(out + (size_t)p * H + (size_t)b * 128, q, 128);
                if (dtype == 3)     /* E8M0: the power of two 2^e as the byte e + 127 */
                    ((uint8_t*)recv_scales)[(size_t)p * S + b] = (uint8_t)(ilogbf(scale) + 127);
                else
                    ((float*)recv_scales)[(size_t)p * S + b] = scale;
            }
        }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Step 4: combine.  out[t] = sum_j w[t,j] * y[pos[t,j]], the router-weighted */
/* sum of the token's expert outputs, rounded once to bf16.                   */
/* ------------------------------------------------------------------------ */
int orc_combine(int T, int H, int k, int N, const uint16_t* y, const int32_t* pos,
                const float* w, uint16_t* out)
{
    if (T < 0 || H <= 0 || k < 1 || N < 0) return -1;
    for (int t = 0; t < T; ++t)
        for (int c = 0; c < H; ++c) {
            double acc = 0.0;
            for (int j = 0; j < k; ++j) {
                const int p = pos[(size_t)t * k + j];
                if (p < 0) continue;
                if (p >= N) return -1;
                acc += (double)w[(size_t)t * k + j] * (double)bf16_to_f32(y[(size_t)p * H + c]);
            }
            out[(size_t)t * H + c] = orc_bf16_from_f64(acc);
        }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Backward pair.  The pages state that dispatch's backward is carried out    */
/* by a combine and combine's backward by a dispatch (DeepEP V2 digest,      */
/* section "training/prefill/decoding usage").  Through the FP8 rounding the  */
/* gradient passes straight (the quantiser is treated as identity).          */
/* ------------------------------------------------------------------------ */
int orc_dispatch_backward(int T, int H, int k, int N, const uint16_t* grad_recv,
                          const int32_t* pos, uint16_t* grad_x)
{
    if (T < 0 || H <= 0 || k < 1 || N < 0) return -1;
    for (int t = 0; t < T; ++t)
        for (int c = 0; c < H; ++c) {
            double acc = 0.0;
            for (int j = 0; j < k; ++j) {
                const int p = pos[(size_t)t * k + j];
                if (p < 0) continue;
                if (p >= N) return -1;
                acc += (double)bf16_to_f32(grad_recv[(size_t)p * H + c]);
            }
            grad_x[(size_t)t * H + c] = orc_bf16_from_f64(acc);
        }
    return 0;
}

int orc_combine_backward(int T, int H, int k, int N, const uint16_t* grad_out,
                         const uint16_t* y, const int32_t* pos, const float* w,
                         uint16_t* grad_y, float* grad_w)
{
    if (T < 0 || H <= 0 || k < 1 || N < 0) return -1;
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            const int p = pos[(size_t)t * k + j];
            if (p < 0) {
                grad_w[(size_t)t * k + j] = 0.0f;
                continue;
            }
            if (p >= N) return -1;
            const double wj = (double)w[(size_t)t * k + j];
            double dot = 0.0;
            for (int c = 0; c < H; ++c) {
                const double g = (double)bf16_to_f32(grad_out[(size_t)t * H + c]);
                grad_y[(size_t)p * H + c] = orc_bf16_from_f64(wj * g);
                dot += g * (double)bf16_to_f32(y[(size_t)p * H + c]);
            }
            grad_w[(size_t)t * k + j] = (float)dot;
        }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Expert MLP on the receive buffer: the two linear layers and the SwiGLU    */
/* between dispatch and combine (Mega MoE news page: the MoE layer runs      */
/* dispatch, a first linear layer, SwiGLU, a second linear layer and         */
/* combine; TileKernels news page, "functions": SwiGLU fused with the FP8    */
/* quantisation).  Operands are FP8 E4M3FN with power-of-two block scales:   */
/* activations one scale per row and 128 columns, weights one per 128x128    */
/* block.  Every product and sum is taken in double on the dequantised       */
/* operands (code value times scale, exact), in index order.                 */
/* ------------------------------------------------------------------------ */
static int expert_of_row(int E, const int32_t* start, const int32_t* count, int p)
{
    for (int e = 0; e < E; ++e)
        if (p >= start[e] && p < start[e] + count[e]) return e;
    return -1;
}

/* Visits the rows to compute: the list if given, else every expert's range. */
static int mlp_rows(int N, int E, const int32_t* start, const int32_t* count, int nrows,
                    const int32_t* rows, int (*fn)(void*, int, int), void* ctx)
{
    if (rows) {
        for (int i = 0; i < nrows; ++i) {
            const int p = rows[i];
            if (p < 0 || p >= N) return -1;
            const int e = expert_of_row(E, start, count, p);
            if (e < 0) return -1;
            if (fn(ctx, p, e)) return -1;
        }
        return 0;
    }
    for (int e = 0; e < E; ++e) {
        if (count[e] < 0 || start[e] < 0 || (int64_t)start[e] + count[e] > N) return -1;
        for (int p = start[e]; p < start[e] + count[e]; ++p)
            if (fn(ctx, p, e)) return -1;
    }
    return 0;
}

struct up_ctx {
    int H, I;
    const uint8_t *x, *w1;
    const float *xs, *w1s;
    uint8_t* act;
    float* act_s;
    double* act_f64;
};

static int up_row(void* vc, int p, int e)
{
    const struct up_ctx* c = (const struct up_ctx*)vc;
    const int H = c->H, I = c->I, SH = H / 128, S2I = 2 * I / 128;
    double* xv = (double*)malloc(sizeof(double) * H);
    double* h = (double*)malloc(sizeof(double) * 2 * I);
    float* a32 = (float*)malloc(sizeof(float) * I);
    if (!xv || !h || !a32) { free(xv); free(h); free(a32); return -1; }
    for (int k = 0; k < H; ++k)
        xv[k] = orc_e4m3_value(c->x[(size_t)p * H + k]) * (double)c->xs[(size_t)p * SH + k / 128];
    for (int n = 0; n < 2 * I; ++n) {
        const uint8_t* wr = c->w1 + ((size_t)e * 2 * I + n) * H;
        const float* ws = c->w1s + ((size_t)e * S2I + n / 128) * SH;
        double acc = 0.0;
        for (int k = 0; k < H; ++k) acc += xv[k] * (orc_e4m3_value(wr[k]) * (double)ws[k / 128]);
        h[n] = acc;
    }
    for (int j = 0; j < I; ++j) {
        const double g = h[j], u = h[I + j];
        const double a = g / (1.0 + exp(-g)) * u;   /* SwiGLU: silu(gate) * up */
        if (c->act_f64) c->act_f64[(size_t)p * I + j] = a;
        a32[j] = (float)a;
    }
    for (int b = 0; b < I / 128; ++b)
        c->act_s[(size_t)p * (I / 128) + b] =
            quant_block_pow2(a32 + (size_t)b * 128, c->act + (size_t)p * I + (size_t)b * 128);
    free(xv); free(h); free(a32);
    return 0;
}

int orc_mlp_up(int N, int H, int I, int E, const int32_t* start, const int32_t* count, int nrows,
               const int32_t* rows, const uint8_t* x, const float* xs, const uint8_t* w1,
               const float* w1s, uint8_t* act, float* act_s, double* act_f64)
{
    if (N < 0 || H <= 0 || I <= 0 || E < 1 || H % 128 || I % 128) return -1;
    struct up_ctx c = {H, I, x, w1, xs, w1s, act, act_s, act_f64};
    return mlp_rows(N, E, start, count, nrows, rows, up_row, &c);
}

struct down_ctx {
    int H, I;
    const uint8_t *act, *w2;
    const float *as, *w2s;
    uint16_t* y;
};

static int down_row(void* vc, int p, int e)
{
    const struct down_ctx* c = (const struct down_ctx*)vc;
    const int H = c->H, I = c->I, SI = I / 128;
    double* av = (double*)malloc(sizeof(double) * I);
    if (!av) return -1;
    for (int k = 0; k < I; ++k)
        av[k] = orc_e4m3_value(c->act[(size_t)p * I + k]) * (double)c->as[(size_t)p * SI + k / 128];
    for (int n = 0; n < H; ++n) {
        const uint8_t* wr = c->w2 + ((size_t)e * H + n) * I;
        const float* ws = c->w2s + ((size_t)e * (H / 128) + n / 128) * SI;
        double acc = 0.0;
        for (int k = 0; k < I; ++k) acc += av[k] * (orc_e4m3_value(wr[k]) * (double)ws[k / 128]);
        c->y[(size_t)p * H + n] = orc_bf16_from_f64(acc);
    }
    free(av);
    return 0;
}

int orc_mlp_down(int N, int H, int I, int E, const int32_t* start, const int32_t* count, int nrows,
                 const int32_t* rows, const uint8_t* act, const float* act_s, const uint8_t* w2,
                 const float* w2s, uint16_t* y)
{
    if (N < 0 || H <= 0 || I <= 0 || E < 1 || H % 128 || I % 128) return -1;
    struct down_ctx c = {H, I, act, w2, act_s, w2s, y};
    return mlp_rows(N, E, start, count, nrows, rows, down_row, &c);
}
