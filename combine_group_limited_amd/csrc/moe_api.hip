// moe_api.hip -- the C ABI declared in include/moe.h: argument validation on
// the host, then kernel launches on the caller's stream.  No allocation, no
// synchronisation, no state kept between calls (apart from the per-thread
// error message).
#include <stdarg.h>
#include <stdio.h>

#include "moe.h"
#include "moe_device.hpp"
#include "moe_internal.hpp"

namespace cgl {
namespace {

thread_local char g_err[512];

moe_status fail(moe_status st, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return st;
}

moe_status ok() {
    g_err[0] = 0;
    return MOE_OK;
}

moe_status hip_status(hipError_t e, const char* what) {
    if (e == hipSuccess) return ok();
    return fail(MOE_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

__host__ __device__ inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// out[i] = E4M3FN(in[i]); one thread converts four values (one 32-bit store).
__global__ __launch_bounds__(256) void quantize_e4m3_kernel(const float* in, uint8_t* out, int64_t n) {
    const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;  // quad index
    const int64_t i = q * 4;
    if (i + 3 < n) {
        const uint32_t w = pack_e4m3x4(in[i], in[i + 1], in[i + 2], in[i + 3]);
        if (aligned(out + i, 4)) {
            *(uint32_t*)(out + i) = w;
        } else {
            for (int b = 0; b < 4; ++b) out[i + b] = (uint8_t)(w >> (8 * b));
        }
    } else if (i < n) {
        float v[4] = {0.0f, 0.0f, 0.0f, 0.0f};
        for (int64_t b = 0; i + b < n; ++b) v[b] = in[i + b];
        const uint32_t w = pack_e4m3x4(v[0], v[1], v[2], v[3]);
        for (int64_t b = 0; i + b < n; ++b) out[i + b] = (uint8_t)(w >> (8 * b));
    }
}

// *status |= MOE_FLAG_BAD_SCALE if any s[i] is not a positive normal power
// of two (sign 0, exponent field 1..254, mantissa 0): one atomic per wave
// that saw one, none otherwise.
__global__ __launch_bounds__(256) void check_pow2_kernel(const float* s, int64_t n, int32_t* status) {
    bool bad = false;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
        const uint32_t b = __float_as_uint(s[i]);
        const uint32_t ex = (b >> 23) & 0xFFu;
        bad |= (b & 0x807FFFFFu) != 0u || ex == 0u || ex == 0xFFu;
    }
    const uint64_t any = __ballot(bad);  // every lane of the wave is active here
    if (any != 0u && (threadIdx.x & 63) == 0) atomicOr(status, MOE_FLAG_BAD_SCALE);
}

}  // namespace

hipError_t launch_check_pow2(const float* s, int64_t n, int32_t* status, hipStream_t stream) {
    const int64_t blocks = (n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024;
    hipLaunchKernelGGL(check_pow2_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, s, n, status);
    return hipGetLastError();
}

hipError_t launch_quantize_e4m3(const float* in, uint8_t* out, int64_t n, hipStream_t stream) {
    const int64_t quads = (n + 3) / 4;
    const int64_t blocks = (quads + 255) / 256;
    hipLaunchKernelGGL(quantize_e4m3_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, in, out, n);
    return hipGetLastError();
}

}  // namespace cgl

using namespace cgl;

extern "C" {

int32_t moe_abi_version(void) { return 8; }

const char* moe_last_error(void) { return g_err; }

const char* moe_status_string(moe_status s) {
    switch (s) {
        case MOE_OK: return "ok";
        case MOE_ERR_INVALID: return "invalid argument";
        case MOE_ERR_WORKSPACE: return "workspace too small";
        case MOE_ERR_UNSUPPORTED: return "unsupported";
        case MOE_ERR_HIP: return "HIP error";
    }
    return "unknown status";
}

// Validates a routing configuration; *n_out receives the group-score depth.
static moe_status check_route_cfg(const moe_route_cfg* c, int* n_out) {
    if (!c) return fail(MOE_ERR_INVALID, "route: cfg is NULL");
    const int T = c->num_tokens, E = c->num_experts, G = c->num_groups, g = c->topk_group, k = c->topk;
    if (T < 0) return fail(MOE_ERR_INVALID, "route: num_tokens %d < 0", T);
    if (E < 1 || E > 512) return fail(MOE_ERR_INVALID, "route: num_experts %d outside [1, 512]", E);
    if (G < 1 || G > 64 || E % G) return fail(MOE_ERR_INVALID, "route: num_groups %d must divide E and be <= 64", G);
    if (g < 1 || g > G) return fail(MOE_ERR_INVALID, "route: topk_group %d outside [1, %d]", g, G);
    const int Eg = E / G;
    if (k < 1 || k > 64 || k > g * Eg)
        return fail(MOE_ERR_INVALID, "route: topk %d outside [1, min(64, topk_group*E/G = %d)]", k, g * Eg);
    int n = c->group_topn > 0 ? c->group_topn : k / g;
    if (n < 1) n = 1;
    if (c->group_topn < 0 || n > Eg)
        return fail(MOE_ERR_INVALID, "route: group_topn %d outside [0, E/G = %d]", c->group_topn, Eg);
    if (c->score_fn != MOE_SCORE_SIGMOID && c->score_fn != MOE_SCORE_SOFTMAX)
        return fail(MOE_ERR_INVALID, "route: unknown score_fn %d", c->score_fn);
    if (c->renormalize != 0 && c->renormalize != 1)
        return fail(MOE_ERR_INVALID, "route: renormalize must be 0 or 1");
    *n_out = n;
    return MOE_OK;
}

moe_status moe_route_topk(const moe_route_cfg* c, const float* logits, int32_t* topk_idx, float* topk_w,
                          void* stream) {
    int n = 0;
    const moe_status st = check_route_cfg(c, &n);
    if (st != MOE_OK) return st;
    const int T = c->num_tokens;
    if (T == 0) return ok();
    if (!logits || !topk_idx || !topk_w) return fail(MOE_ERR_INVALID, "route: NULL array");
    if (!aligned(logits, 4) || !aligned(topk_idx, 4) || !aligned(topk_w, 4))
        return fail(MOE_ERR_INVALID, "route: arrays must be 4-byte aligned");
    return hip_status(launch_route(logits, topk_idx, topk_w, T, c->num_experts, c->num_groups, c->topk_group,
                                   c->topk, n, c->score_fn, c->renormalize, (hipStream_t)stream),
                      "route launch");
}

static moe_status check_layout_cfg(const moe_layout_cfg* c) {
    if (!c) return fail(MOE_ERR_INVALID, "layout: cfg is NULL");
    const int T = c->num_tokens, E = c->num_experts, k = c->topk, R = c->num_ranks, C = c->capacity;
    if (T < 0) return fail(MOE_ERR_INVALID, "layout: num_tokens %d < 0", T);
    if (E < 1 || E > 512) return fail(MOE_ERR_INVALID, "layout: num_experts %d outside [1, 512]", E);
    if (k < 1 || k > 64) return fail(MOE_ERR_INVALID, "layout: topk %d outside [1, 64]", k);
    if (R < 1 || R > E || E % R) return fail(MOE_ERR_INVALID, "layout: num_ranks %d must divide E", R);
    if (C < 0) return fail(MOE_ERR_INVALID, "layout: capacity %d < 0", C);
    const int A = c->align_rows;
    if (A < 0 || A > 4096) return fail(MOE_ERR_INVALID, "layout: align_rows %d outside [0, 4096]", A);
    if (A > 1 && C > 0) return fail(MOE_ERR_INVALID, "layout: align_rows needs the compact layout (capacity 0)");
    if (A > 1 && (int64_t)T * k + (int64_t)E * (A - 1) >= (1ll << 31))
        return fail(MOE_ERR_INVALID, "layout: T*k + E*(align_rows-1) too large");
    if ((int64_t)T * k >= (1ll << 31)) return fail(MOE_ERR_INVALID, "layout: T*k too large");
    if ((int64_t)E * C >= (1ll << 31)) return fail(MOE_ERR_INVALID, "layout: E*C too large");
    return MOE_OK;
}

size_t moe_layout_workspace_bytes(const moe_layout_cfg* c) {
    if (check_layout_cfg(c) != MOE_OK) return 0;
    return layout_workspace_bytes(c->num_tokens, c->num_experts, c->num_ranks);
}

// Checks moe_get_layout's arrays (everything but the workspace).
static_assert(kLayoutScratchBytes == MOE_LAYOUT_NOALLOC_MAX_BYTES, "header and library disagree");

static moe_status check_layout_arrays(const moe_layout_cfg* c, const int32_t* topk_idx, const int32_t* cnt_e,
                                      const int32_t* cnt_r, const int32_t* off_e, const int32_t* off_r,
                                      const int32_t* pos, const int32_t* recv_src, const int32_t* flags) {
    const int T = c->num_tokens;
    if (!cnt_e || !cnt_r || !off_e || !off_r || !flags)
        return fail(MOE_ERR_INVALID, "layout: NULL output array");
    if (T > 0 && (!topk_idx || !pos)) return fail(MOE_ERR_INVALID, "layout: NULL topk_idx or pos");
    const int64_t N = c->capacity > 0 ? (int64_t)c->num_experts * c->capacity
                      : (int64_t)T * c->topk + (c->align_rows > 1 ? (int64_t)c->num_experts * (c->align_rows - 1) : 0);
    if (N > 0 && !recv_src) return fail(MOE_ERR_INVALID, "layout: NULL recv_src");
    const void* ptrs[] = {topk_idx, cnt_e, cnt_r, off_e, off_r, pos, recv_src, flags};
    for (const void* p : ptrs)
        if (!aligned(p, 4)) return fail(MOE_ERR_INVALID, "layout: arrays must be 4-byte aligned");
    return MOE_OK;
}

moe_status moe_get_layout(const moe_layout_cfg* c, const int32_t* topk_idx, int32_t* cnt_e, int32_t* cnt_r,
                          int32_t* off_e, int32_t* off_r, int32_t* pos, int32_t* recv_src, int32_t* flags,
                          void* workspace, size_t workspace_bytes, void* stream) {
    moe_status st = check_layout_cfg(c);
    if (st != MOE_OK) return st;
    if ((st = check_layout_arrays(c, topk_idx, cnt_e, cnt_r, off_e, off_r, pos, recv_src, flags)) != MOE_OK)
        return st;
    const int T = c->num_tokens;
    const size_t need = layout_workspace_bytes(T, c->num_experts, c->num_ranks);
    if (!workspace || workspace_bytes < need)
        return fail(MOE_ERR_WORKSPACE, "layout: workspace needs %zu bytes, got %zu", need,
                    workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, 16)) return fail(MOE_ERR_INVALID, "layout: workspace must be 16-byte aligned");
    return hip_status(launch_layout(topk_idx, cnt_e, cnt_r, off_e, off_r, pos, recv_src, flags, workspace, T,
                                    c->num_experts, c->topk, c->num_ranks, c->capacity, c->align_rows,
                                    (hipStream_t)stream),
                      "layout launch");
}

moe_status moe_get_layout_noalloc(const moe_layout_cfg* c, const int32_t* topk_idx, int32_t* cnt_e,
                                  int32_t* cnt_r, int32_t* off_e, int32_t* off_r, int32_t* pos,
                                  int32_t* recv_src, int32_t* flags, void* stream) {
    moe_status st = check_layout_cfg(c);
    if (st != MOE_OK) return st;
    if ((st = check_layout_arrays(c, topk_idx, cnt_e, cnt_r, off_e, off_r, pos, recv_src, flags)) != MOE_OK)
        return st;
    const size_t need = layout_workspace_bytes(c->num_tokens, c->num_experts, c->num_ranks);
    if (need > kLayoutScratchBytes)
        return fail(MOE_ERR_WORKSPACE,
                    "layout_noalloc: this shape needs %zu bytes of count table, above the library's fixed %zu "
                    "(use moe_get_layout with a workspace)",
                    need, (size_t)kLayoutScratchBytes);
    void* ws = nullptr;  // the device address of this GPU's static count table
    const hipError_t e = layout_scratch(&ws);
    if (e != hipSuccess) return fail(MOE_ERR_HIP, "layout_noalloc: device scratch lookup: %s", hipGetErrorString(e));
    return hip_status(launch_layout(topk_idx, cnt_e, cnt_r, off_e, off_r, pos, recv_src, flags, ws,
                                    c->num_tokens, c->num_experts, c->topk, c->num_ranks, c->capacity,
                                    c->align_rows, (hipStream_t)stream),
                      "layout_noalloc launch");
}

static moe_status check_dispatch_cfg(const moe_dispatch_cfg* c) {
    if (!c) return fail(MOE_ERR_INVALID, "dispatch: cfg is NULL");
    const int T = c->num_tokens, H = c->hidden, k = c->topk, N = c->num_recv_rows;
    if (T < 0 || N < 0) return fail(MOE_ERR_INVALID, "dispatch: negative size");
    if (k < 1 || k > 64) return fail(MOE_ERR_INVALID, "dispatch: topk %d outside [1, 64]", k);
    const bool fp8 = c->dtype == MOE_DISPATCH_FP8_E4M3 || c->dtype == MOE_DISPATCH_FP8_E4M3_POW2 ||
                     c->dtype == MOE_DISPATCH_FP8_E4M3_UE8M0;
    if (!fp8 && c->dtype != MOE_DISPATCH_BF16) return fail(MOE_ERR_INVALID, "dispatch: unknown dtype %d", c->dtype);
    if (H < 1 || (fp8 && H % 128) || (!fp8 && H % 8))
        return fail(MOE_ERR_INVALID, "dispatch: hidden %d must be a positive multiple of %d", H, fp8 ? 128 : 8);
    const int upw = c->units_per_wave;
    if (!(upw == 0 || upw == 1 || upw == 2 || upw == 4 || upw == 7 || upw == 8 || upw == 14))
        return fail(MOE_ERR_INVALID, "dispatch: units_per_wave %d not in {0,1,2,4,7,8,14}", upw);
    return MOE_OK;
}

moe_status moe_dispatch(const moe_dispatch_cfg* c, const uint16_t* x, const int32_t* pos, void* recv_x,
                        void* recv_scales, void* stream) {
    const moe_status st = check_dispatch_cfg(c);
    if (st != MOE_OK) return st;
    const int T = c->num_tokens, H = c->hidden, k = c->topk, N = c->num_recv_rows;
    const bool fp8 = c->dtype != MOE_DISPATCH_BF16;
    if (T == 0) return ok();
    if (!x || !pos || (N > 0 && !recv_x) || (fp8 && N > 0 && !recv_scales))
        return fail(MOE_ERR_INVALID, "dispatch: NULL array");
    const size_t sc_align = c->dtype == MOE_DISPATCH_FP8_E4M3_UE8M0 ? 1 : 4;
    if (!aligned(x, 16) || !aligned(recv_x, 16) || !aligned(pos, 4) || !aligned(recv_scales, sc_align))
        return fail(MOE_ERR_INVALID, "dispatch: x/recv_x must be 16-byte aligned, pos and fp32 scales 4-byte");
    if (N == 0) return ok();
    return hip_status(launch_dispatch(x, pos, recv_x, recv_scales, T, H, k, N, c->dtype, c->units_per_wave,
                                      (hipStream_t)stream),
                      "dispatch launch");
}

size_t moe_route_dispatch_workspace_bytes(void) { return 4096; }

moe_status moe_route_dispatch(const moe_route_cfg* rc, const moe_layout_cfg* lc, const moe_dispatch_cfg* dc,
                              const float* logits, const uint16_t* x, int32_t* topk_idx, float* topk_w,
                              int32_t* cnt_e, int32_t* cnt_r, int32_t* off_e, int32_t* off_r, int32_t* pos,
                              int32_t* recv_src, int32_t* flags, void* recv_x, void* recv_scales, void* workspace,
                              size_t workspace_bytes, void* stream) {
    int n = 0;
    moe_status st = check_route_cfg(rc, &n);
    if (st != MOE_OK) return st;
    if ((st = check_layout_cfg(lc)) != MOE_OK) return st;
    if ((st = check_dispatch_cfg(dc)) != MOE_OK) return st;
    const int T = rc->num_tokens, E = rc->num_experts, k = rc->topk, R = lc->num_ranks, C = lc->capacity;
    const int A = lc->align_rows > 1 ? lc->align_rows : 0;
    if (lc->num_tokens != T || dc->num_tokens != T)
        return fail(MOE_ERR_INVALID, "route_dispatch: num_tokens differ (%d, %d, %d)", T, lc->num_tokens,
                    dc->num_tokens);
    if (lc->num_experts != E) return fail(MOE_ERR_INVALID, "route_dispatch: num_experts differ");
    if (lc->topk != k || dc->topk != k) return fail(MOE_ERR_INVALID, "route_dispatch: topk differs");
    const int64_t N = C > 0 ? (int64_t)E * C : (int64_t)T * k + (A > 1 ? (int64_t)E * (A - 1) : 0);
    if (dc->num_recv_rows != N)
        return fail(MOE_ERR_INVALID, "route_dispatch: num_recv_rows %d, the layout has %lld", dc->num_recv_rows,
                    (long long)N);
    if (dc->units_per_wave != 0) return fail(MOE_ERR_INVALID, "route_dispatch: units_per_wave must be 0");
    if (T > kFusedMaxTokens)
        return fail(MOE_ERR_UNSUPPORTED, "route_dispatch: num_tokens %d above %d", T, kFusedMaxTokens);
    const size_t lds = fused_decode_lds_bytes(T, E, k, R);
    if (lds > kFusedMaxLds)
        return fail(MOE_ERR_UNSUPPORTED, "route_dispatch: shape needs %zu bytes of LDS, above %zu", lds,
                    (size_t)kFusedMaxLds);
    const bool fp8 = dc->dtype != MOE_DISPATCH_BF16;
    if (!cnt_e || !cnt_r || !off_e || !off_r || !flags) return fail(MOE_ERR_INVALID, "route_dispatch: NULL array");
    if (T > 0 && (!logits || !x || !topk_idx || !topk_w || !pos))
        return fail(MOE_ERR_INVALID, "route_dispatch: NULL array");
    if (N > 0 && (!recv_src || !recv_x || (fp8 && !recv_scales)))
        return fail(MOE_ERR_INVALID, "route_dispatch: NULL receive array");
    const void* p4[] = {logits, topk_idx, topk_w, cnt_e, cnt_r, off_e, off_r, pos, recv_src, flags,
                        dc->dtype == MOE_DISPATCH_FP8_E4M3_UE8M0 ? nullptr : recv_scales};
    for (const void* p : p4)
        if (!aligned(p, 4)) return fail(MOE_ERR_INVALID, "route_dispatch: arrays must be 4-byte aligned");
    if (!aligned(x, 16) || !aligned(recv_x, 16))
        return fail(MOE_ERR_INVALID, "route_dispatch: x and recv_x must be 16-byte aligned");
    if (!workspace || workspace_bytes < moe_route_dispatch_workspace_bytes())
        return fail(MOE_ERR_WORKSPACE, "route_dispatch: workspace needs %zu bytes, got %zu",
                    moe_route_dispatch_workspace_bytes(), workspace ? workspace_bytes : (size_t)0);
    if (!aligned(workspace, 16)) return fail(MOE_ERR_INVALID, "route_dispatch: workspace must be 16-byte aligned");
    return hip_status(launch_fused_decode(logits, x, topk_idx, topk_w, cnt_e, cnt_r, off_e, off_r, pos, recv_src,
                                          flags, recv_x, recv_scales, (uint32_t*)workspace, T, E, rc->num_groups,
                                          rc->topk_group, k, n, rc->score_fn, rc->renormalize, R, C, A, (int)N,
                                          dc->hidden, dc->dtype, (hipStream_t)stream),
                      "route_dispatch launch");
}

moe_status moe_combine(const moe_combine_cfg* c, const uint16_t* y, const int32_t* pos, const float* topk_w,
                       uint16_t* out, void* stream) {
    if (!c) return fail(MOE_ERR_INVALID, "combine: cfg is NULL");
    const int T = c->num_tokens, H = c->hidden, k = c->topk, N = c->num_recv_rows;
    if (T < 0 || N < 0) return fail(MOE_ERR_INVALID, "combine: negative size");
    if (k < 1 || k > 64) return fail(MOE_ERR_INVALID, "combine: topk %d outside [1, 64]", k);
    if (H < 1 || H % 8) return fail(MOE_ERR_INVALID, "combine: hidden %d must be a positive multiple of 8", H);
    const int upw = c->units_per_wave;
    if (!(upw == 0 || upw == 1 || upw == 2 || upw == 4 || upw == 7))
        return fail(MOE_ERR_INVALID, "combine: units_per_wave %d not in {0,1,2,4,7}", upw);
    if (T == 0) return ok();
    if (!pos || !topk_w || !out || (N > 0 && !y)) return fail(MOE_ERR_INVALID, "combine: NULL array");
    if (!aligned(y, 16) || !aligned(out, 16) || !aligned(pos, 4) || !aligned(topk_w, 4))
        return fail(MOE_ERR_INVALID, "combine: y/out must be 16-byte aligned, pos/w 4-byte");
    return hip_status(launch_combine(y, pos, topk_w, out, T, H, k, N, upw, (hipStream_t)stream),
                      "combine launch");
}

static moe_status check_combine_cfg(const moe_combine_cfg* c, const char* who, bool backward) {
    if (!c) return fail(MOE_ERR_INVALID, "%s: cfg is NULL", who);
    const int T = c->num_tokens, H = c->hidden, k = c->topk, N = c->num_recv_rows;
    if (T < 0 || N < 0) return fail(MOE_ERR_INVALID, "%s: negative size", who);
    if (k < 1 || k > 64) return fail(MOE_ERR_INVALID, "%s: topk %d outside [1, 64]", who, k);
    if (H < 1 || H % 8) return fail(MOE_ERR_INVALID, "%s: hidden %d must be a positive multiple of 8", who, H);
    const int upw = c->units_per_wave;
    if (!(upw == 0 || upw == 1 || upw == 2 || upw == 4 || upw == 7))
        return fail(MOE_ERR_INVALID, "%s: units_per_wave %d not in {0,1,2,4,7}", who, upw);
    (void)backward;
    return MOE_OK;
}

moe_status moe_dispatch_backward(const moe_combine_cfg* c, const uint16_t* grad_recv, const int32_t* pos,
                                 uint16_t* grad_x, void* stream) {
    moe_status st = check_combine_cfg(c, "dispatch_backward", false);
    if (st != MOE_OK) return st;
    const int T = c->num_tokens, N = c->num_recv_rows;
    if (T == 0) return ok();
    if (!pos || !grad_x || (N > 0 && !grad_recv)) return fail(MOE_ERR_INVALID, "dispatch_backward: NULL array");
    if (!aligned(grad_recv, 16) || !aligned(grad_x, 16) || !aligned(pos, 4))
        return fail(MOE_ERR_INVALID, "dispatch_backward: grad_recv/grad_x must be 16-byte aligned, pos 4-byte");
    return hip_status(launch_combine(grad_recv, pos, nullptr, grad_x, T, c->hidden, c->topk, N, c->units_per_wave,
                                     (hipStream_t)stream),
                      "dispatch_backward launch");
}

moe_status moe_combine_backward(const moe_combine_cfg* c, const uint16_t* grad_out, const uint16_t* y,
                                const int32_t* pos, const float* topk_w, uint16_t* grad_y, float* grad_w,
                                void* stream) {
    moe_status st = check_combine_cfg(c, "combine_backward", true);
    if (st != MOE_OK) return st;
    const int T = c->num_tokens, N = c->num_recv_rows;
    if (T == 0) return ok();
    if (!grad_out || !pos || !topk_w || !grad_w || (N > 0 && (!y || !grad_y)))
        return fail(MOE_ERR_INVALID, "combine_backward: NULL array");
    if (!aligned(grad_out, 16) || !aligned(y, 16) || !aligned(grad_y, 16) || !aligned(pos, 4) ||
        !aligned(topk_w, 4) || !aligned(grad_w, 4))
        return fail(MOE_ERR_INVALID, "combine_backward: row data must be 16-byte aligned, pos/w 4-byte");
    return hip_status(launch_combine_backward(grad_out, y, pos, topk_w, grad_y, grad_w, T, c->hidden, c->topk, N,
                                              c->units_per_wave, (hipStream_t)stream),
                      "combine_backward launch");
}

static moe_status check_mlp_cfg(const moe_mlp_cfg* c, const char* who) {
    if (!c) return fail(MOE_ERR_INVALID, "%s: cfg is NULL", who);
    const int N = c->num_rows, H = c->hidden, I = c->inter, E = c->num_experts, C = c->capacity;
    if (N < 0) return fail(MOE_ERR_INVALID, "%s: num_rows %d < 0", who, N);
    if (H < 128 || H % 128 || H > 65536) return fail(MOE_ERR_INVALID, "%s: hidden %d must be a multiple of 128 in [128, 65536]", who, H);
    if (I < 128 || I % 128 || I > 8192) return fail(MOE_ERR_INVALID, "%s: inter %d must be a multiple of 128 in [128, 8192]", who, I);
    if (E < 1 || E > 512) return fail(MOE_ERR_INVALID, "%s: num_experts %d outside [1, 512]", who, E);
    if (C < 0) return fail(MOE_ERR_INVALID, "%s: capacity %d < 0", who, C);
    if ((int64_t)N * H >= (1ll << 40)) return fail(MOE_ERR_INVALID, "%s: N*H too large", who);
    return MOE_OK;
}

moe_status moe_expert_up(const moe_mlp_cfg* c, const int32_t* cnt_e, const int32_t* off_e, const uint8_t* x,
                         const float* x_scales, const uint8_t* w1, const float* w1_scales, uint8_t* act,
                         float* act_scales, void* stream) {
    const moe_status st = check_mlp_cfg(c, "expert_up");
    if (st != MOE_OK) return st;
    if (c->hidden > 8192) return fail(MOE_ERR_INVALID, "expert_up: hidden %d above 8192", c->hidden);
    if ((int64_t)c->num_rows * c->hidden > (1ll << 32))
        return fail(MOE_ERR_UNSUPPORTED, "expert_up: num_rows*hidden above 2^32");
    if (c->num_rows == 0) return ok();
    if (!cnt_e || (c->capacity == 0 && !off_e) || !x || !x_scales || !w1 || !w1_scales || !act || !act_scales)
        return fail(MOE_ERR_INVALID, "expert_up: NULL array");
    if (!aligned(x, 16) || !aligned(w1, 16) || !aligned(act, 16) || !aligned(x_scales, 4) ||
        !aligned(w1_scales, 4) || !aligned(act_scales, 4) || !aligned(cnt_e, 4) || !aligned(off_e, 4))
        return fail(MOE_ERR_INVALID, "expert_up: code arrays must be 16-byte aligned, the others 4-byte");
    const hipError_t pe = prepare_expert_mlp(true, c->num_rows, c->hidden, c->num_experts);
    if (pe != hipSuccess)
        return fail(MOE_ERR_HIP, "expert_up: setting %zu bytes of LDS: %s",
                    expert_mlp_lds_bytes(c->num_rows, c->hidden, c->num_experts), hipGetErrorString(pe));
    return hip_status(launch_expert_up(cnt_e, off_e, x, x_scales, w1, w1_scales, act, act_scales, c->num_rows,
                                       c->hidden, c->inter, c->num_experts, c->capacity, (hipStream_t)stream),
                      "expert_up launch");
}

moe_status moe_expert_down(const moe_mlp_cfg* c, const int32_t* cnt_e, const int32_t* off_e, const uint8_t* act,
                           const float* act_scales, const uint8_t* w2, const float* w2_scales, uint16_t* y,
                           void* stream) {
    const moe_status st = check_mlp_cfg(c, "expert_down");
    if (st != MOE_OK) return st;
    if ((int64_t)c->num_rows * c->inter > (1ll << 32))
        return fail(MOE_ERR_UNSUPPORTED, "expert_down: num_rows*inter above 2^32");
    if (c->num_rows == 0) return ok();
    if (!cnt_e || (c->capacity == 0 && !off_e) || !act || !act_scales || !w2 || !w2_scales || !y)
        return fail(MOE_ERR_INVALID, "expert_down: NULL array");
    if (!aligned(act, 16) || !aligned(w2, 16) || !aligned(y, 16) || !aligned(act_scales, 4) ||
        !aligned(w2_scales, 4) || !aligned(cnt_e, 4) || !aligned(off_e, 4))
        return fail(MOE_ERR_INVALID, "expert_down: code and output arrays must be 16-byte aligned, the others 4-byte");
    const hipError_t pe = prepare_expert_mlp(false, c->num_rows, c->inter, c->num_experts);
    if (pe != hipSuccess)
        return fail(MOE_ERR_HIP, "expert_down: setting %zu bytes of LDS: %s",
                    expert_mlp_lds_bytes(c->num_rows, c->inter, c->num_experts), hipGetErrorString(pe));
    return hip_status(launch_expert_down(cnt_e, off_e, act, act_scales, w2, w2_scales, y, c->num_rows, c->hidden,
                                         c->inter, c->num_experts, c->capacity, (hipStream_t)stream),
                      "expert_down launch");
}

size_t moe_layer_workspace_bytes(void) { return 4096; }

moe_status moe_layer_forward(const moe_mlp_cfg* c, int num_tokens, int topk, const int32_t* pos,
                             const float* topk_w, const int32_t* cnt_e, const int32_t* off_e, const uint16_t* x,
                             const uint8_t* w1, const float* w1_scales, const uint8_t* w2, const float* w2_scales,
                             uint8_t* recv_x, float* recv_scales, uint8_t* act, float* act_scales, uint16_t* y,
                             uint16_t* out, void* workspace, size_t workspace_bytes, void* stream) {
    const moe_status st = check_mlp_cfg(c, "layer_forward");
    if (st != MOE_OK) return st;
    const int T = num_tokens, k = topk, N = c->num_rows, H = c->hidden, I = c->inter, E = c->num_experts;
    if (T < 0) return fail(MOE_ERR_INVALID, "layer_forward: num_tokens %d < 0", T);
    if (k < 1 || k > 64) return fail(MOE_ERR_INVALID, "layer_forward: topk %d outside [1, 64]", k);
    if (H > 8192) return fail(MOE_ERR_INVALID, "layer_forward: hidden %d above 8192", H);
    if ((int64_t)N * H > (1ll << 32) || (int64_t)N * I > (1ll << 32))
        return fail(MOE_ERR_UNSUPPORTED, "layer_forward: num_rows*hidden or num_rows*inter above 2^32");
    // T*k, and T times the 512-channel units of a row (the item index of the
    // dispatch and combine phases, plus two grid strides), fit 32 bits
    if ((int64_t)T * H >= (1ll << 40) || (int64_t)T * k >= (1ll << 31) || (int64_t)T * ((H + 511) / 512) >= (1ll << 30))
        return fail(MOE_ERR_INVALID, "layer_forward: num_tokens too large");
    if (T == 0 || N == 0) return ok();
    if (!pos || !topk_w || !cnt_e || (c->capacity == 0 && !off_e) || !x || !w1 || !w1_scales || !w2 ||
        !w2_scales || !recv_x || !recv_scales || !act || !act_scales || !y || !out)
        return fail(MOE_ERR_INVALID, "layer_forward: NULL array");
    if (!aligned(x, 16) || !aligned(w1, 16) || !aligned(w2, 16) || !aligned(recv_x, 16) || !aligned(act, 16) ||
        !aligned(y, 16) || !aligned(out, 16) || !aligned(pos, 4) || !aligned(topk_w, 4) || !aligned(cnt_e, 4) ||
        !aligned(off_e, 4) || !aligned(w1_scales, 4) || !aligned(w2_scales, 4) || !aligned(recv_scales, 4) ||
        !aligned(act_scales, 4))
        return fail(MOE_ERR_INVALID, "layer_forward: code and row arrays must be 16-byte aligned, the others 4-byte");
    if (!workspace || workspace_bytes < moe_layer_workspace_bytes() || !aligned(workspace, 16))
        return fail(MOE_ERR_WORKSPACE, "layer_forward: workspace must be %zu bytes, 16-byte aligned (got %zu)",
                    moe_layer_workspace_bytes(), workspace ? workspace_bytes : (size_t)0);
    int supported = 0;
    const size_t lds = layer_lds_bytes(N, H, I, E, &supported);
    if (!supported || lds > 160 * 1024)
        return fail(MOE_ERR_UNSUPPORTED,
                    "layer_forward: no one-launch kernel for this tile configuration (use the four calls)");
    return hip_status(launch_layer(x, pos, topk_w, cnt_e, off_e, w1, w1_scales, w2, w2_scales, recv_x, recv_scales,
                                   act, act_scales, y, out, (uint32_t*)workspace, T, k, N, H, I, E, c->capacity,
                                   (hipStream_t)stream),
                      "layer_forward launch");
}

moe_status moe_check_pow2_scales(const float* scales, int64_t n, int32_t* status, void* stream) {
    if (n < 0) return fail(MOE_ERR_INVALID, "check_pow2_scales: n < 0");
    if (!status) return fail(MOE_ERR_INVALID, "check_pow2_scales: NULL status");
    if (!aligned(status, 4)) return fail(MOE_ERR_INVALID, "check_pow2_scales: status must be 4-byte aligned");
    if (n == 0) return ok();
    if (!scales || !aligned(scales, 4)) return fail(MOE_ERR_INVALID, "check_pow2_scales: scales NULL or unaligned");
    return hip_status(launch_check_pow2(scales, n, status, (hipStream_t)stream), "check_pow2_scales launch");
}

moe_status moe_quantize_e4m3(const float* in, uint8_t* out, int64_t n, void* stream) {
    if (n < 0) return fail(MOE_ERR_INVALID, "quantize: n < 0");
    if (n == 0) return ok();
    if (!in || !out) return fail(MOE_ERR_INVALID, "quantize: NULL array");
    if (!aligned(in, 4)) return fail(MOE_ERR_INVALID, "quantize: input must be 4-byte aligned");
    if ((n + 3) / 4 / 256 >= (1ll << 31)) return fail(MOE_ERR_INVALID, "quantize: n too large");
    return hip_status(launch_quantize_e4m3(in, out, n, (hipStream_t)stream), "quantize launch");
}

}  // extern "C"
