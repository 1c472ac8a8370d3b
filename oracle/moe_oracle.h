/*
 * moe_oracle.h -- plain, slow, single-threaded CPU oracle for MoE dispatch/combine.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
 * leg of the benchmark may load this library.  The product path never calls it,
 * and it shares no source, header, table or helper with the HIP library.
 *
 * Every function is the plain definition (or the written recipe) of one step:
 *   - route:    "Efficient and Portable Mixture-of-Experts Communication"
 *               (Perplexity), section "Introduction" (router -> probability
 *               distribution -> top-K experts -> weighted sum), and
 *               "DeepSeek, DeepEP open-sourced" (GeekNews 19421), topic body
 *               (group-limited gating; top-4 groups then top-8 experts in the
 *               "Performance > Normal kernels" workload).
 *   - layout:   Perplexity page, sections "Portable kernels" and "Dispatch"
 *               (per-expert counts; unique receive addresses; source index kept
 *               for combine), DeepEP V2 digest, section "training/prefill/decoding
 *               usage" (per-expert token counts for the GEMM).
 *   - dispatch: Perplexity page, section "Dispatch" (tokens plus block scaling
 *               factors into contiguous per-expert buffers); FP8 dispatch of the
 *               DeepEP V1/V2 performance workloads.
 *   - combine:  Perplexity page, section "Combine" (weighted average of the expert
 *               contributions, 16-bit activations).
 *
 * Readings where the pages are silent (group score, tie-breaks, slot order, exp
 * recipe, scale definition, receive order, ...) are the ones listed in the design
 * notes; each function below states the reading it applies.
 *
 * Conventions: all arrays row-major, caller-owned; bf16 values travel as uint16
 * bit patterns; return 0 on success, -1 on an invalid argument.
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* exp recipe (Cody-Waite reduction + degree-7 Taylor), fp32. */
float orc_exp_r(float z);
/* 1 / (1 + exp_r(-x)), fp32, correctly rounded division. */
float orc_sigmoid(float x);
void orc_exp_r_array(const float* z, float* out, int64_t n);
void orc_sigmoid_array(const float* x, float* out, int64_t n);

/* OCP E4M3FN: value of a code (NaN for 0x7F/0xFF). */
double orc_e4m3_value(uint8_t code);
/* nearest E4M3FN code, ties to even, magnitudes above 448 saturate, sign kept. */
uint8_t orc_e4m3_from_f32(float y);
void orc_e4m3_from_f32_array(const float* y, uint8_t* out, int64_t n);
/* bf16 nearest-even of a double (single rounding). */
uint16_t orc_bf16_from_f64(double v);
void orc_bf16_from_f64_array(const double* v, uint16_t* out, int64_t n);

/* score_fn: 0 = sigmoid, 1 = softmax.  group_topn: experts summed per group score
   (0 selects topk / topk_group).  Outputs idx [T,k] int32, w [T,k] fp32. */
int orc_route(int T, int E, int G, int g, int k, int group_topn, int score_fn,
              int renormalize, const float* logits, int32_t* idx, float* w);

/* capacity C = 0: compact receive buffer, N = T*k rows.
   capacity C > 0: padded, N = E*C rows, expert e owns rows [e*C, e*C + C).
   align A > 1 (compact only): each expert's region starts at a multiple of A
   rows (off_e = scan of counts rounded up to A); N = T*k + E*(A-1) rows, the
   rows no pair fills hold recv_src -1.
   Outputs: cnt_e[E], cnt_r[R], off_e[E+1], off_r[R+1], pos[T,k], recv_src[N],
   overflow[1]. */
int orc_layout(int T, int E, int k, int R, int C, int A, const int32_t* idx,
               int32_t* cnt_e, int32_t* cnt_r, int32_t* off_e, int32_t* off_r,
               int32_t* pos, int32_t* recv_src, int32_t* overflow);

/* dtype 0: FP8 E4M3FN with one fp32 scale per 128 channels (recv_x bytes [N,H],
   recv_scales [N,H/128]); dtype 1: BF16 copy (recv_x as uint16 [N,H]);
   dtype 2: FP8 E4M3FN with power-of-two scales (the smallest 2^e with
   amax <= 448 * 2^e; codes of x / 2^e, exact scaling).
   dtype 3: the codes of dtype 2, each scale 2^e stored as the byte e + 127
   (E8M0), recv_scales uint8 [N, H/128].
   Rows whose pos is -1 are skipped; rows never addressed are left untouched. */
int orc_dispatch(int T, int H, int k, int N, int dtype, const uint16_t* x,
                 const int32_t* pos, void* recv_x, void* recv_scales);

/* out[t,c] = bf16( sum_j w[t,j] * y[pos[t,j], c] ), sum in double; pos -1
   contributes nothing. */
int orc_combine(int T, int H, int k, int N, const uint16_t* y, const int32_t* pos,
                const float* w, uint16_t* out);

/* Backward of dispatch (gradients flow straight through the FP8 rounding):
   grad_x[t,c] = bf16( sum_j grad_recv[pos[t,j], c] ), sum in double. */
int orc_dispatch_backward(int T, int H, int k, int N, const uint16_t* grad_recv,
                          const int32_t* pos, uint16_t* grad_x);

/* Backward of combine: grad_y[pos[t,j], c] = bf16(w[t,j] * grad_out[t,c])
   (exact product, one rounding); grad_w[t,j] = fp32( sum_c grad_out[t,c] *
   y[pos[t,j], c] ), sum in double.  Rows of grad_y no pair addresses are not
   written; dropped pairs (pos -1) get grad_w 0. */
int orc_combine_backward(int T, int H, int k, int N, const uint16_t* grad_out,
                         const uint16_t* y, const int32_t* pos, const float* w,
                         uint16_t* grad_y, float* grad_w);

/* Expert MLP (between dispatch and combine).  Expert e owns receive rows
   [start[e], start[e] + count[e]).  rows: the rows to compute (nrows of them,
   each inside some expert's range), or NULL for every row of every expert.
   Operands: x codes [N,H] with power-of-two scales xs [N,H/128]; w1 codes
   [E,2I,H] with scales w1s [E,2I/128,H/128] (rows 0..I-1 gate, I..2I-1 up);
   act codes [N,I] with scales [N,I/128]; w2 codes [E,H,I] with scales
   [E,H/128,I/128]; y bf16 [N,H].
   up:   h[p,n] = sum_k x(p,k) w1(e,n,k)  (double, dequantised operands);
         act[p,j] = silu(h[p,j]) * h[p,I+j], silu(g) = g/(1+exp(-g))  (double);
         then rounded to fp32 and quantised per 128 columns (power-of-two scale,
         as dispatch's FP8_E4M3_POW2); act_f64 (optional) receives the doubles.
   down: y[p,n] = bf16( sum_k act(p,k) w2(e,n,k) )  (double, one rounding).
   Rows not computed are left untouched. */
int orc_mlp_up(int N, int H, int I, int E, const int32_t* start, const int32_t* count, int nrows,
               const int32_t* rows, const uint8_t* x, const float* xs, const uint8_t* w1,
               const float* w1s, uint8_t* act, float* act_s, double* act_f64);
int orc_mlp_down(int N, int H, int I, int E, const int32_t* start, const int32_t* count, int nrows,
                 const int32_t* rows, const uint8_t* act, const float* act_s, const uint8_t* w2,
                 const float* w2s, uint16_t* y);

#ifdef __cplusplus
}
#endif
#endif
