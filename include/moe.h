/*
 * moe.h -- C ABI of the MI355X (gfx950) MoE dispatch/combine library.
 *
 * The library runs, on one GPU, one rank's share of the token exchange of a
 * Mixture-of-Experts layer, in four calls that follow the pages' statement of
 * the problem:
 *
 *   moe_route_topk  router scores -> group-limited top-k experts and weights
 *   moe_get_layout  per-expert / per-rank counts, offsets, and every
 *                   (token, slot) pair's receive row (the "handle")
 *   moe_dispatch    copy each token into its k receive rows of an
 *                   expert-contiguous buffer, FP8-quantised with per-128-
 *                   channel scales (or verbatim BF16)
 *   moe_combine     out[t] = sum_j w[t,j] * y[pos[t,j]]  (BF16 in and out)
 *
 * Conventions for every call:
 *   - All array pointers are DEVICE pointers owned by the caller; arrays are
 *     dense and row-major.  bf16 values are passed as uint16_t bit patterns.
 *   - The library never allocates or frees memory in these calls and keeps no
 *     data between them; it only remembers per-device facts it looked up once
 *     (occupancy figures, the address of moe_get_layout_noalloc's table).
 *   - Every call is asynchronous: it validates its arguments on the host,
 *     enqueues kernels on `stream` (a hipStream_t; NULL = the null stream)
 *     and returns without synchronising.
 *   - Host-side validation failures return MOE_ERR_INVALID and enqueue nothing.
 *     Launch failures return MOE_ERR_HIP.  moe_last_error() then describes the
 *     failure (per thread).
 *   - num_tokens == 0 is valid: route, dispatch and combine do nothing;
 *     moe_get_layout writes zero counts and offsets (and -1 to every padded
 *     recv_src row).
 *   - Pointers to 16-bit and FP8 row data must be 16-byte aligned.
 *   - Device-side data that is out of range (an expert index outside [0,E), a
 *     receive row outside [0,N)) never causes an out-of-bounds access: the
 *     offending pair is skipped and, in moe_get_layout, reported in *flags.
 *   - Results are deterministic: every output element is written by exactly
 *     one lane and no global atomics take part in any result.
 */
#ifndef CGL_MOE_H
#define CGL_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID = 1,     /* bad shape, null pointer, or inconsistent sizes */
    MOE_ERR_WORKSPACE = 2,   /* workspace missing or smaller than required */
    MOE_ERR_UNSUPPORTED = 4, /* valid request the library does not implement */
    MOE_ERR_HIP = 5          /* a HIP runtime call or kernel launch failed */
} moe_status;

typedef enum { MOE_SCORE_SIGMOID = 0, MOE_SCORE_SOFTMAX = 1 } moe_score_fn;
typedef enum {
    MOE_DISPATCH_FP8_E4M3 = 0,      /* fp32 scale = amax / 448 per 128 channels */
    MOE_DISPATCH_BF16 = 1,          /* verbatim copy */
    MOE_DISPATCH_FP8_E4M3_POW2 = 2, /* power-of-two scale per 128 channels */
    MOE_DISPATCH_FP8_E4M3_UE8M0 = 3 /* the same scale as one E8M0 byte */
} moe_dispatch_dtype;

/* Bits of the *flags word written by moe_get_layout. */
#define MOE_FLAG_CAPACITY_OVERFLOW 1  /* padded mode: some expert got more than C pairs */
#define MOE_FLAG_BAD_INDEX 2          /* an index outside [0,E) or repeated in a token */
#define MOE_FLAG_BAD_SCALE 8          /* moe_check_pow2_scales: a scale that is not a  */
                                      /* positive normal power of two                   */
#define MOE_FLAG_INCOMPLETE 4         /* moe_route_dispatch only: the launch did not   */
                                      /* complete (barrier give-up; see there)          */

/* ------------------------------------------------------------------------ */
/* moe_route_topk -- group-limited top-k gating.                            */
/*                                                                          */
/* Follows "Efficient and Portable Mixture-of-Experts Communication"        */
/* (Perplexity), section "Introduction": the router gives each token a      */
/* score distribution over experts, the token goes to its top-K experts and */
/* the outputs are summed with the router weights; and "DeepSeek, DeepEP    */
/* open-sourced" (GeekNews 19421), topic body and "Performance > Normal     */
/* kernels": group-limited gating, top-4 groups then top-8 experts.         */
/*                                                                          */
/* For each token t (logits row l = logits[t, 0..E-1]):                     */
/*  1. score s_e = 1/(1+exp(-l_e)) (SIGMOID) or s_e = l_e (SOFTMAX: softmax */
/*     is increasing, so selection on the logits is selection on the        */
/*     probabilities);                                                      */
/*  2. if num_groups G > 1: group gamma (experts gamma*E/G .. +E/G-1) scores */
/*     the sum of its group_topn largest s_e (0 = topk/topk_group, at least */
/*     1), added in descending order; keep the topk_group best groups;      */
/*  3. take the topk best experts of the kept groups, slots in descending   */
/*     score; equal scores go to the lower index (-0 equals +0);            */
/*  4. weights: renormalize=1: SIGMOID w_j = s_j / (s_0+...+s_{k-1}),       */
/*     SOFTMAX w_j = exp(l_j - l_0) / sum_i exp(l_i - l_0); renormalize=0:  */
/*     SIGMOID w_j = s_j, SOFTMAX w_j = full softmax probability.           */
/*  exp is a fixed fp32 recipe (Cody-Waite reduction by ln 2, degree-7      */
/*  Taylor polynomial by fma, exact 2^n scaling, clamped at |z| >= 80), so   */
/*  indices and weights are reproducible bit for bit.                       */
/*                                                                          */
/* logits   fp32  [T, E]   in                                               */
/* topk_idx int32 [T, k]   out, expert ids                                  */
/* topk_w   fp32  [T, k]   out, weights                                     */
/* Limits: 1 <= E <= 512, 1 <= G <= 64, E % G == 0, 1 <= topk_group <= G,  */
/*         1 <= k <= min(64, topk_group*E/G), 0 <= group_topn <= E/G.       */
/* ------------------------------------------------------------------------ */
typedef struct {
    int32_t num_tokens;   /* T */
    int32_t num_experts;  /* E */
    int32_t num_groups;   /* G (1 = no group limit) */
    int32_t topk_group;   /* groups kept per token */
    int32_t topk;         /* k */
    int32_t group_topn;   /* experts summed per group score; 0 = topk/topk_group */
    int32_t score_fn;     /* moe_score_fn */
    int32_t renormalize;  /* 0 or 1 */
} moe_route_cfg;

moe_status moe_route_topk(const moe_route_cfg* cfg, const float* logits, int32_t* topk_idx,
                          float* topk_w, void* stream);

/* ------------------------------------------------------------------------ */
/* moe_get_layout -- routing layout (the dispatch "handle").                */
/*                                                                          */
/* Follows the Perplexity page, sections "Portable kernels" (a fixed        */
/* per-expert capacity lets every sender derive a unique destination        */
/* address with no synchronisation) and "Dispatch" (per-expert token counts;*/
/* the receiver keeps source, expert and token index for the combine), and  */
/* the DeepEP V2 digest, section "training/prefill/decoding usage" (the     */
/* handle carries the per-expert token counts for the grouped GEMM).        */
/*                                                                          */
/* A stable counting sort of the T*k (token, slot) pairs by expert:         */
/*   cnt_e[e]   = #pairs routed to e                         int32 [E]      */
/*   cnt_r[r]   = #tokens with >= 1 expert on virtual rank r int32 [R]      */
/*                (rank r owns experts r*E/R .. r*E/R + E/R - 1)            */
/*   off_e[e]   = cnt_e[0] + ... + cnt_e[e-1]                int32 [E+1]    */
/*   off_r[r]   = off_e[r*E/R]  (pairs before rank r)        int32 [R+1]    */
/*   pos[t,j]   = receive row of pair (t,j)                  int32 [T,k]    */
/*       compact (capacity 0): off_e[e] + #{t' < t routed to e}; N = T*k    */
/*       padded  (capacity C): e*C + #{t' < t routed to e}, or -1 when that */
/*                is >= C (dropped; MOE_FLAG_CAPACITY_OVERFLOW); N = E*C    */
/*       aligned (capacity 0, align_rows A > 1): every expert region starts  */
/*                on a multiple of A rows: off_e is the exclusive scan of    */
/*                cnt_e rounded up to A, pos = off_e[e] + rank; N = T*k +    */
/*                E*(A-1) rows (an upper bound; off_e[E] rows are used).     */
/*                A grouped-GEMM-friendly variant of the receive layout.     */
/*   recv_src[p] = t*k + j for p = pos[t,j]; -1 for empty padded rows       */
/*                                                           int32 [N]      */
/*   flags[0]   = MOE_FLAG_* bits (0 = all good)             int32 [1]      */
/* Counts are never clamped.  If MOE_FLAG_BAD_INDEX is set the other        */
/* outputs are unspecified (but every write stays in bounds).               */
/* workspace: device memory of at least moe_layout_workspace_bytes(cfg),    */
/* 16-byte aligned; its contents need no initialisation.                    */
/* Limits: 1 <= E <= 512, 1 <= k <= 64, 1 <= R <= E, E % R == 0,          */
/*         T*k < 2^31, E*C < 2^31.                                          */
/* ------------------------------------------------------------------------ */
typedef struct {
    int32_t num_tokens;   /* T */
    int32_t num_experts;  /* E */
    int32_t topk;         /* k */
    int32_t num_ranks;    /* R */
    int32_t capacity;     /* 0 = compact; C > 0 = padded slots per expert */
    int32_t align_rows;   /* compact only: 0 or 1 = packed; A > 1 = regions start on multiples of A */
} moe_layout_cfg;

size_t moe_layout_workspace_bytes(const moe_layout_cfg* cfg);

moe_status moe_get_layout(const moe_layout_cfg* cfg, const int32_t* topk_idx, int32_t* cnt_e,
                          int32_t* cnt_r, int32_t* off_e, int32_t* off_r, int32_t* pos,
                          int32_t* recv_src, int32_t* flags, void* workspace,
                          size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* moe_get_layout_noalloc -- moe_get_layout with no workspace argument, for  */
/* callers that cannot allocate device memory (code under HIP graph capture,*/
/* serving loops and harnesses that forbid allocation).                     */
/*                                                                          */
/* Same arguments (less the workspace), outputs, limits and errors as       */
/* moe_get_layout.  The count table lives in a device array the library     */
/* owns: MOE_LAYOUT_NOALLOC_MAX_BYTES per GPU, held from the first call on   */
/* that GPU until the process ends.  Shapes whose                           */
/* moe_layout_workspace_bytes(cfg) exceeds it return MOE_ERR_WORKSPACE       */
/* before anything is enqueued (at E = 256, R = 32: above 231 936 tokens). */
/* The call allocates and frees nothing; the stream must belong to the      */
/* current device.  Every call on one GPU shares that GPU's array, so calls */
/* that may overlap on one GPU (different streams, or host threads) race    */
/* and give wrong results: serialise them, or use moe_get_layout with       */
/* separate workspaces.  Nothing in the array needs clearing between calls. */
/* ------------------------------------------------------------------------ */
#define MOE_LAYOUT_NOALLOC_MAX_BYTES 1048576

moe_status moe_get_layout_noalloc(const moe_layout_cfg* cfg, const int32_t* topk_idx, int32_t* cnt_e,
                                  int32_t* cnt_r, int32_t* off_e, int32_t* off_r, int32_t* pos,
                                  int32_t* recv_src, int32_t* flags, void* stream);

/* ------------------------------------------------------------------------ */
/* moe_dispatch -- scatter tokens into the expert-contiguous receive buffer. */
/*                                                                          */
/* Follows the Perplexity page, section "Dispatch": tokens are sent with    */
/* their block scaling factors and land in contiguous per-expert tensors    */
/* for the grouped GEMM; FP8 dispatch as in the DeepEP performance          */
/* workloads (GeekNews 19421, "Performance > Normal kernels").              */
/*                                                                          */
/* For every pair (t,j) with p = pos[t,j] in [0, N):                        */
/*  FP8_E4M3: for each block b of 128 channels, a = max(max_i |x[t,i]|,     */
/*    2^-100), scale = a/448, inv = 448/a (fp32, correctly rounded),        */
/*    recv_x[p, 128b+i] = E4M3FN nearest-even of the fp32 product           */
/*    x[t,128b+i]*inv (OCP E4M3FN: max 448, sign kept), recv_scales[p,b] =  */
/*    scale.  Dequantise as code * scale.                                    */
/*  FP8_E4M3_POW2: as FP8_E4M3 but scale = 2^e, the smallest power of two   */
/*    with a <= 448 * 2^e, and codes of the exactly scaled x * 2^-e (scales  */
/*    that a GEMM can apply as exponent shifts).                            */
/*  FP8_E4M3_UE8M0: the codes of FP8_E4M3_POW2, each scale 2^e stored as    */
/*    one byte, e + 127 (the E8M0 encoding: the scale's biased fp32         */
/*    exponent), a quarter of the scale bytes; the grouped-GEMM-friendly    */
/*    form of the DeepEP V2 digest, "V2 release main changes" ("a new GEMM  */
/*    layout").                                                             */
/*  BF16: recv_x[p, :] = x[t, :] bit for bit.                               */
/* Rows no pair addresses are not written.  pos of -1 (dropped) is skipped. */
/*                                                                          */
/* x           bf16 [T, H]                in                                */
/* pos         int32 [T, k]               in (from moe_get_layout)          */
/* recv_x      uint8 [N, H] (FP8) or bf16 [N, H]                 out        */
/* recv_scales fp32 [N, H/128] (FP8_E4M3, FP8_E4M3_POW2; 4-byte aligned),   */
/*             uint8 [N, H/128] (FP8_E4M3_UE8M0), NULL for BF16   out        */
/* Limits: H % 128 == 0 (FP8 dtypes) or H % 8 == 0 (BF16); 1 <= k <= 64.    */
/* ------------------------------------------------------------------------ */
typedef struct {
    int32_t num_tokens;     /* T */
    int32_t hidden;         /* H */
    int32_t topk;           /* k */
    int32_t num_recv_rows;  /* N */
    int32_t dtype;          /* moe_dispatch_dtype */
    int32_t units_per_wave; /* launch-shape override, 512-channel units per wave
                               (1, 2, 4, 7, 8 or 14); 0 = library choice.  Like
                               the num_sms override of the DeepEP V2 digest,
                               section "ElasticBuffer interface", it changes
                               speed only, never results. */
} moe_dispatch_cfg;

moe_status moe_dispatch(const moe_dispatch_cfg* cfg, const uint16_t* x, const int32_t* pos,
                        void* recv_x, void* recv_scales, void* stream);

/* ------------------------------------------------------------------------ */
/* moe_combine -- top-k weighted gather-reduce back into token order.       */
/*                                                                          */
/* Follows the Perplexity page, section "Combine": the receiver reads each  */
/* expert's 16-bit output for the token, picks buffer and weight from the   */
/* routing table, forms the weighted sum and writes it to a caller-         */
/* allocated tensor.                                                        */
/*                                                                          */
/* out[t, c] = bf16_rne( fma chain over j = 0..k-1 of w[t,j] * y[pos[t,j],c]*/
/*             in fp32, starting from 0 );  pairs with pos outside [0, N)    */
/*             contribute nothing.                                          */
/* y      bf16 [N, H]   in (expert outputs, rows in receive order)          */
/* pos    int32 [T, k]  in                                                  */
/* topk_w fp32 [T, k]   in                                                  */
/* out    bf16 [T, H]   out (must not alias y)                              */
/* Limits: H % 8 == 0; 1 <= k <= 64.                                        */
/* ------------------------------------------------------------------------ */
typedef struct {
    int32_t num_tokens;     /* T */
    int32_t hidden;         /* H */
    int32_t topk;           /* k */
    int32_t num_recv_rows;  /* N */
    int32_t units_per_wave; /* launch-shape override (1, 2, 4 or 7); 0 = library choice */
} moe_combine_cfg;

moe_status moe_combine(const moe_combine_cfg* cfg, const uint16_t* y, const int32_t* pos,
                       const float* topk_w, uint16_t* out, void* stream);

/* ------------------------------------------------------------------------ */
/* Backward pair.  The DeepEP V2 digest, section "training/prefill/decoding */
/* usage", states that dispatch's backward is carried out by a combine and  */
/* combine's backward by a dispatch.  Gradients pass straight through the   */
/* FP8 rounding (the quantiser is treated as identity).  Both take          */
/* moe_combine_cfg (units_per_wave: 1, 2, 4 or 7 for combine_backward).     */
/*                                                                          */
/* moe_dispatch_backward:                                                   */
/*   grad_x[t, c] = bf16_rne( fp32 sum over j of grad_recv[pos[t,j], c] )   */
/*   grad_recv bf16 [N,H] in, pos int32 [T,k] in, grad_x bf16 [T,H] out.   */
/*   (the combine kernel with every weight 1)                               */
/* moe_combine_backward:                                                    */
/*   grad_y[pos[t,j], c] = bf16_rne(w[t,j] * grad_out[t,c])  (exact product,*/
/*                         rounded once)                                    */
/*   grad_w[t, j]        = fp32 dot of grad_out[t, :] and y[pos[t,j], :]    */
/*   grad_out bf16 [T,H], y bf16 [N,H], pos int32 [T,k], topk_w fp32 [T,k]  */
/*   in; grad_y bf16 [N,H], grad_w fp32 [T,k] out.  Rows of grad_y that no  */
/*   pair addresses are not written; a pair with pos outside [0,N) gets     */
/*   grad_w 0.                                                              */
/* Limits: H % 8 == 0; 1 <= k <= 64.                                        */
/* ------------------------------------------------------------------------ */
moe_status moe_dispatch_backward(const moe_combine_cfg* cfg, const uint16_t* grad_recv, const int32_t* pos,
                                 uint16_t* grad_x, void* stream);

moe_status moe_combine_backward(const moe_combine_cfg* cfg, const uint16_t* grad_out, const uint16_t* y,
                                const int32_t* pos, const float* topk_w, uint16_t* grad_y, float* grad_w,
                                void* stream);

/* ------------------------------------------------------------------------ */
/* moe_route_dispatch -- decode path: route, layout and dispatch of a small  */
/* batch in ONE kernel launch.                                              */
/*                                                                          */
/* Follows the DeepEP V2 digest (GeekNews 19438), section "training/prefill/*/
/* decoding usage" (at decode, routing metadata should not cost a layout    */
/* recomputation and a CPU synchronisation), and "DeepSeek, DeepEP          */
/* open-sourced" (GeekNews 19421), "Performance > Low-latency kernels"      */
/* (decode batches of 128 tokens per rank, judged by latency).             */
/*                                                                          */
/* Computes exactly what moe_route_topk(route) -> moe_get_layout(layout) -> */
/* moe_dispatch(dispatch) compute, with every output of the three calls     */
/* (bit for bit), in one launch whose blocks meet once at a grid-wide       */
/* barrier after routing.  For inputs with MOE_FLAG_BAD_INDEX unset; on top */
/* of moe_get_layout it also writes -1 to compact rows no pair fills.       */
/* The three configurations must agree: the same num_tokens, num_experts    */
/* and topk; dispatch num_recv_rows equal to the layout's N;               */
/* dispatch units_per_wave 0.                                               */
/*                                                                          */
/* logits fp32 [T,E] and x bf16 [T,H] in; topk_idx, topk_w, cnt_e, cnt_r,   */
/* off_e, off_r, pos, recv_src, flags, recv_x, recv_scales out, with the    */
/* shapes and meanings of the three calls above.                            */
/* workspace: at least moe_route_dispatch_workspace_bytes() of device       */
/* memory, 16-byte aligned, ZEROED BEFORE ITS FIRST USE (e.g. hipMemset     */
/* once).  It holds the barrier's arrival counters and generation flags;    */
/* every call leaves the counters at zero, so it needs no clearing between  */
/* calls.                                                                   */
/* Calls that may run at the same time (different streams) need different   */
/* workspaces.  Its third 32-bit word (word 2) counts blocks that stopped   */
/* waiting at the barrier after about a second, which only happens if the  */
/* GPU cannot hold the whole grid at once.  It stays 0 in normal use.  Once */
/* it is nonzero the library never clears it: that call and every later    */
/* call on the workspace write MOE_FLAG_INCOMPLETE into flags[0] and leave  */
/* the other outputs incomplete (a refused call does not wait or count at   */
/* the barrier, so stray counts a give-up left behind are never used),      */
/* until the caller zeroes the workspace again.                             */
/* Limits: those of the three calls, and T <= 1024 with                     */
/*   8*ceil(T/64)*(E+R) + 4*(2E + 1 + T*k + 2048) <= 64512 bytes of LDS;     */
/*   larger shapes return MOE_ERR_UNSUPPORTED (use the three calls).        */
/* ------------------------------------------------------------------------ */
size_t moe_route_dispatch_workspace_bytes(void);

moe_status moe_route_dispatch(const moe_route_cfg* route, const moe_layout_cfg* layout,
                              const moe_dispatch_cfg* dispatch, const float* logits,
                              const uint16_t* x, int32_t* topk_idx, float* topk_w, int32_t* cnt_e,
                              int32_t* cnt_r, int32_t* off_e, int32_t* off_r, int32_t* pos,
                              int32_t* recv_src, int32_t* flags, void* recv_x, void* recv_scales,
                              void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Expert MLP on the receive buffer: the two linear layers of every routed   */
/* expert, between moe_dispatch and moe_combine.                            */
/*                                                                          */
/* Follows the Mega MoE news page (the MoE layer runs dispatch, a first     */
/* linear layer, SwiGLU, a second linear layer and combine) and the         */
/* TileKernels news page, "functions" (SwiGLU fused with the FP8            */
/* quantisation): moe_expert_up computes the first layer and applies SwiGLU */
/* and the FP8 requantisation in its epilogue, so the 2I-wide               */
/* pre-activation never reaches memory; moe_expert_down computes the second */
/* layer into the bf16 rows moe_combine reads.                              */
/*                                                                          */
/* Expert e owns receive rows [s_e, s_e + n_e): capacity 0: s_e = off_e[e], */
/* n_e = cnt_e[e]; capacity C > 0: s_e = e*C, n_e = min(cnt_e[e], C) (the   */
/* arrays moe_get_layout writes).  Rows outside every range are not         */
/* written.  A layout whose ranges leave [0, N) makes that expert skipped.  */
/* All operands are OCP E4M3FN codes with POWER-OF-TWO fp32 block scales    */
/* (the matrix cores take only the exponent bits, so a scale that is not a  */
/* positive normal power of two gives wrong results and is NOT checked here:*/
/* run moe_check_pow2_scales on the weight scales once when they are        */
/* loaded; activation scales that moe_dispatch(MOE_DISPATCH_FP8_E4M3_POW2)  */
/* or moe_expert_up wrote are powers of two by construction): activations  */
/* one scale per row and 128 columns; weights one per 128x128 block.        */
/* Accumulation is fp32 on the matrix cores.                                */
/*                                                                          */
/* moe_expert_up:                                                           */
/*   h[p, n]   = sum_k x(p,k) * w1(e,n,k), n < 2I (rows 0..I-1 gate, I..2I-1 */
/*               up), x(p,k) = code * x_scales[p, k/128], w1 likewise with  */
/*               w1_scales[e, n/128, k/128];                                */
/*   a[p, j]   = silu(h[p,j]) * h[p, I+j], silu(g) = g / (1 + exp(-g));      */
/*   act, act_scales = FP8 with power-of-two scales per 128 columns of a, by */
/*               the FP8_E4M3_POW2 recipe of moe_dispatch.                  */
/*   x uint8 [N,H], x_scales fp32 [N,H/128], w1 uint8 [E,2I,H], w1_scales   */
/*   fp32 [E,2I/128,H/128] in; act uint8 [N,I], act_scales fp32 [N,I/128]   */
/*   out.                                                                   */
/* moe_expert_down:                                                         */
/*   y[p, n]   = bf16_rne( sum_k act(p,k) * w2(e,n,k) ), n < H.             */
/*   act uint8 [N,I], act_scales fp32 [N,I/128], w2 uint8 [E,H,I],           */
/*   w2_scales fp32 [E,H/128,I/128] in; y bf16 [N,H] out.                   */
/* Limits: H and I multiples of 128, H <= 8192 for up, I <= 8192,           */
/* 1 <= E <= 512 (MOE_ERR_INVALID otherwise); N*H (up) and N*I (down) at    */
/* most 2^32, so that a row offset fits in 32 bits (MOE_ERR_UNSUPPORTED     */
/* otherwise).  Code arrays and y 16-byte aligned.                          */
/* ------------------------------------------------------------------------ */
typedef struct {
    int32_t num_rows;     /* N: rows of the receive buffer */
    int32_t hidden;       /* H */
    int32_t inter;        /* I: expert intermediate width */
    int32_t num_experts;  /* E */
    int32_t capacity;     /* 0: ranges from off_e/cnt_e; C > 0: padded ranges */
} moe_mlp_cfg;

moe_status moe_expert_up(const moe_mlp_cfg* cfg, const int32_t* cnt_e, const int32_t* off_e,
                         const uint8_t* x, const float* x_scales, const uint8_t* w1,
                         const float* w1_scales, uint8_t* act, float* act_scales, void* stream);

moe_status moe_expert_down(const moe_mlp_cfg* cfg, const int32_t* cnt_e, const int32_t* off_e,
                           const uint8_t* act, const float* act_scales, const uint8_t* w2,
                           const float* w2_scales, uint16_t* y, void* stream);

/* ------------------------------------------------------------------------ */
/* moe_layer_forward -- the MoE layer after routing in ONE kernel launch:    */
/* dispatch -> expert up -> expert down -> combine.                         */
/*                                                                          */
/* Follows the Mega MoE news page (dispatch, the first linear layer,        */
/* SwiGLU, the second linear layer and combine fused into one kernel).      */
/* Computes exactly, bit for bit, what this sequence computes and writes    */
/* every array it writes:                                                   */
/*   moe_dispatch(MOE_DISPATCH_FP8_E4M3_POW2; x, pos -> recv_x, recv_scales)*/
/*   moe_expert_up(cfg; recv_x, recv_scales, w1, w1_scales -> act,          */
/*                 act_scales)                                              */
/*   moe_expert_down(cfg; act, act_scales, w2, w2_scales -> y)              */
/*   moe_combine(y, pos, topk_w -> out)                                     */
/* with num_tokens T and topk k for dispatch and combine, num_recv_rows =   */
/* cfg->num_rows, hidden = cfg->hidden.  The blocks of the launch meet at   */
/* three grid-wide barriers; one block per compute unit, all resident.      */
/*                                                                          */
/* x bf16 [T,H], pos int32 [T,k], topk_w fp32 [T,k], cnt_e and off_e as for */
/* the expert MLP, w1/w1_scales/w2/w2_scales as for the expert MLP in;      */
/* recv_x uint8 [N,H], recv_scales fp32 [N,H/128], act uint8 [N,I],         */
/* act_scales fp32 [N,I/128], y bf16 [N,H] (the intermediate arrays, all    */
/* written), out bf16 [T,H] out.  All caller-allocated.                    */
/* workspace: at least moe_layer_workspace_bytes() of device memory,        */
/* 16-byte aligned, ZEROED BEFORE ITS FIRST USE; the barriers leave it at   */
/* rest after every call.  Calls that may run at the same time need         */
/* different workspaces.  Its third 32-bit word (word 2) counts blocks that */
/* stopped waiting at a barrier after about a second (only if the GPU       */
/* cannot hold the whole grid, e.g. while other kernels occupy it); it      */
/* stays 0 in normal use.  Once nonzero it is never cleared by the library: */
/* the outputs of that call and of every later call on the workspace are    */
/* incomplete (later calls are refused at the first barrier, so stray       */
/* counts a give-up left behind are never used) until the caller zeroes the */
/* workspace again.  Read word 2 after the call to know (e.g. the Python    */
/* binding's barrier_gave_up()).                                            */
/* Words 768..775 receive, as four 64-bit values (low word first), the     */
/* GPU's constant 100-MHz clock (s_memrealtime) read by block 0 at the      */
/* start and after each barrier: phase timings, for diagnostics only.       */
/* Limits: those of moe_dispatch, moe_expert_up, moe_expert_down and        */
/* moe_combine, 1 <= k <= 64 and T * ceil(H / 512) < 2^30 (MOE_ERR_INVALID  */
/* otherwise); a tile configuration with a one-launch kernel (256-row       */
/* tiles, or 128-row tiles with three stage buffers for both H and I, which */
/* every shape within these limits has), MOE_ERR_UNSUPPORTED otherwise (use */
/* the four calls).  Arrays of codes and bf16 rows 16-byte aligned, the     */
/* others 4-byte.                                                           */
/* ------------------------------------------------------------------------ */
size_t moe_layer_workspace_bytes(void);

moe_status moe_layer_forward(const moe_mlp_cfg* cfg, int num_tokens, int topk, const int32_t* pos,
                             const float* topk_w, const int32_t* cnt_e, const int32_t* off_e,
                             const uint16_t* x, const uint8_t* w1, const float* w1_scales,
                             const uint8_t* w2, const float* w2_scales, uint8_t* recv_x,
                             float* recv_scales, uint8_t* act, float* act_scales, uint16_t* y,
                             uint16_t* out, void* workspace, size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* moe_check_pow2_scales -- checks the precondition of the expert MLP and   */
/* the one-launch layer on their fp32 block scales: ORs MOE_FLAG_BAD_SCALE  */
/* into *status (device int32, never cleared by the library) if any of      */
/* scales[0..n) is not a positive normal power of two (sign 0, exponent     */
/* field 1..254, mantissa 0).  Asynchronous like every call: read *status   */
/* after the stream has reached it.  n >= 0; scales and status 4-byte       */
/* aligned device pointers.                                                 */
/* ------------------------------------------------------------------------ */
moe_status moe_check_pow2_scales(const float* scales, int64_t n, int32_t* status, void* stream);

/* ------------------------------------------------------------------------ */
/* moe_quantize_e4m3 -- the element conversion moe_dispatch uses, exposed   */
/* on its own: out[i] = E4M3FN nearest-even of in[i], magnitudes above 448  */
/* saturate to 448, sign kept (codes for NaN inputs are unspecified).       */
/* in fp32 [n], out uint8 [n]; n >= 0.                                      */
/* ------------------------------------------------------------------------ */
moe_status moe_quantize_e4m3(const float* in, uint8_t* out, int64_t n, void* stream);

const char* moe_status_string(moe_status status);
const char* moe_last_error(void);
/* moe_abi_version: 8 (adds the MOE_DISPATCH_FP8_E4M3_UE8M0 dispatch dtype */
/* to moe_dispatch and moe_route_dispatch, whose recv_scales became void*   */
/* for it; version 7 added moe_check_pow2_scales and MOE_FLAG_INCOMPLETE,   */
/* 6 moe_get_layout_noalloc, 5 moe_layer_forward and its workspace size).   */
int32_t moe_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* CGL_MOE_H */
