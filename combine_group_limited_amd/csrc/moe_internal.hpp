// moe_internal.hpp -- launchers behind the C ABI (host side).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace cgl {

hipError_t launch_route(const float* logits, int32_t* idx, float* w, int T, int E, int G, int g, int k,
                        int n, int score_fn, int renorm, hipStream_t stream);

size_t layout_workspace_bytes(int T, int E, int R);
// moe_get_layout_noalloc's count table: a static device array of this size per
// GPU; layout_scratch returns its address on the current device.
constexpr size_t kLayoutScratchBytes = (size_t)1 << 20;
hipError_t layout_scratch(void** ptr);
size_t layout_lds_bytes_host(int E, int R);
hipError_t launch_layout(const int32_t* idx, int32_t* cnt_e, int32_t* cnt_r, int32_t* off_e, int32_t* off_r,
                         int32_t* pos, int32_t* recv_src, int32_t* flags, void* workspace, int T, int E,
                         int k, int R, int C, int A, hipStream_t stream);

// upw: 512-channel units per wave (0 = the library's choice for the shape)
int dispatch_units_per_wave(int T, int H);
// dtype: 0 FP8 (amax/448 scales), 1 BF16, 2 FP8 with power-of-two scales, 3 the same
// with one E8M0 exponent byte per scale
hipError_t launch_dispatch(const uint16_t* x, const int32_t* pos, void* recv_x, void* recv_scales, int T,
                           int H, int k, int N, int dtype, int upw, hipStream_t stream);

int combine_units_per_wave(int T, int H);
hipError_t launch_combine(const uint16_t* y, const int32_t* pos, const float* w, uint16_t* out, int T, int H,
                          int k, int N, int upw, hipStream_t stream);

hipError_t launch_combine_backward(const uint16_t* grad_out, const uint16_t* y, const int32_t* pos, const float* w,
                                   uint16_t* grad_y, float* grad_w, int T, int H, int k, int N, int upw,
                                   hipStream_t stream);

// Fused decode path (route + layout + dispatch in one launch), for small T.
constexpr int kFusedMaxTokens = 1024;
constexpr size_t kFusedMaxLds = 64512;  // 64 KiB of dynamic LDS less 1 KiB for static
size_t fused_decode_lds_bytes(int T, int E, int k, int R);
hipError_t launch_fused_decode(const float* logits, const uint16_t* x, int32_t* idx, float* w, int32_t* cnt_e,
                               int32_t* cnt_r, int32_t* off_e, int32_t* off_r, int32_t* pos, int32_t* recv_src,
                               int32_t* flags, void* recv_x, void* recv_scales, uint32_t* barrier, int T, int E,
                               int G, int g, int k, int n, int score_fn, int renorm, int R, int C, int A, int N,
                               int H, int dtype, hipStream_t stream);

// The MoE layer after routing in one launch (dispatch -> up -> down -> combine).
size_t layer_lds_bytes(int N, int H, int I, int E, int* supported);
hipError_t launch_layer(const uint16_t* x, const int32_t* pos, const float* topk_w, const int32_t* cnt_e,
                        const int32_t* off_e, const uint8_t* w1, const float* w1s, const uint8_t* w2,
                        const float* w2s, uint8_t* recv_x, float* recv_s, uint8_t* act, float* act_s, uint16_t* y,
                        uint16_t* out, uint32_t* barrier, int T, int k, int N, int H, int I, int E, int C,
                        hipStream_t stream);

// Expert MLP (grouped FP8 GEMMs with power-of-two block scales).
size_t expert_mlp_lds_bytes(int N, int K, int E);
hipError_t prepare_expert_mlp(bool up, int N, int K, int E);
hipError_t launch_expert_up(const int32_t* cnt_e, const int32_t* off_e, const uint8_t* x, const float* xs,
                            const uint8_t* w1, const float* w1s, uint8_t* act, float* act_s, int N, int H, int I,
                            int E, int C, hipStream_t stream);
hipError_t launch_expert_down(const int32_t* cnt_e, const int32_t* off_e, const uint8_t* act, const float* act_s,
                              const uint8_t* w2, const float* w2s, uint16_t* y, int N, int H, int I, int E, int C,
                              hipStream_t stream);

hipError_t launch_quantize_e4m3(const float* in, uint8_t* out, int64_t n, hipStream_t stream);
hipError_t launch_check_pow2(const float* s, int64_t n, int32_t* status, hipStream_t stream);

}  // namespace cgl
