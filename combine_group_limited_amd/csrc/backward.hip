// backward.hip -- backward of the combine: the gradient of each expert output
// row and of each router weight.
//
// The pages state that combine's backward is carried out by a dispatch and
// dispatch's backward by a combine (DeepEP V2 digest, section
// "training/prefill/decoding usage").  For out[t] = sum_j w[t,j] y[pos[t,j]]:
//     grad_y[pos[t,j]] = w[t,j] * grad_out[t]     (a dispatch of grad_out,
//                                                  scaled per slot)
//     grad_w[t,j]      = <grad_out[t], y[pos[t,j]]>
// (dispatch's backward is the combine kernel with unit weights.)
//
// grad_y is rounded to bf16 once from the exact product: the fp32 product p
// and its fma residual decide the rare case where p sits exactly on a bf16
// rounding midpoint.  grad_y rows are written with streaming stores.
#include "moe_device.hpp"
#include "moe_internal.hpp"

namespace cgl {
namespace {

constexpr int kUnit = 512;

// cache policy of the grad_y writes: streaming (measured: 4 us faster here and
// 10 us in the following kernel, whose reads the plain stores would evict)
constexpr int kBwdStoreNT = 1;

struct CombineBwdArgs {
    const uint16_t* grad_out;
    const uint16_t* y;
    const int32_t* pos;
    const float* w;
    uint16_t* grad_y;
    float* grad_w;
    int T, H, k, N, units;
};

// bf16 nearest-even of the exact product w*g (g a bf16 value).
__device__ __forceinline__ uint32_t bf16_of_product(float w, float g) {
    const float p = w * g;
    const float r = __builtin_fmaf(w, g, -p);  // w*g - p, exact
    const uint32_t b = __float_as_uint(p);
    uint32_t h = (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
    if ((b & 0xFFFFu) == 0x8000u && r != 0.0f) {
        // p is a bf16 midpoint: the exact value lies on r's side of it
        const bool away = (r > 0.0f) == (p > 0.0f);
        h = away ? (b >> 16) + 1u : (b >> 16);
    }
    return h;
}

__device__ __forceinline__ uint32_t pack2(float w, uint32_t gw) {
    return bf16_of_product(w, bf16_lo(gw)) | (bf16_of_product(w, bf16_hi(gw)) << 16);
}

// Sum of one float per lane over the wave, the same in every lane: DPP
// butterflies inside rows of 16 (pairs always add the same two values), then
// the four row sums in a fixed order.
__device__ __forceinline__ float wave_sum(float v) {
    v = v + dppf<0xB1>(v);
    v = v + dppf<0x4E>(v);
    v = v + dppf<0x141>(v);
    v = v + dppf<0x140>(v);
    const float a = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 0));
    const float b = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 16));
    const float c = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 32));
    const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 48));
    return ((a + b) + c) + d;
}

// One wave per token.  The wave walks the row in chunks of U 512-channel
// units; for each chunk it loads grad_out's U KiB once and then, slot by
// slot, gathers the matching U KiB of y[pos], writes U KiB of grad_y and
// folds grad_out * y into that slot's per-lane fp32 partial dot product (each
// lane adds its channels in row order, whatever U is), which a fixed
// DPP/readlane tree sums at the end.  With k a compile-time constant (KC =
// 8, 4 or 2) the slots' partial sums stay in registers; any other k walks
// slot by slot and re-reads grad_out's chunk per slot.  Measured on MI355X,
// spreading a token over several waves with per-unit sums in LDS is slower,
// and re-reading grad_out per slot fetches it from beyond L2 about six times
// over (the streams of y and grad_y evict it).
constexpr int kBwdThreads = 256;

template <int U>
__device__ __forceinline__ void bwd_chunk(const u32x4 (&gv)[U], const uint16_t* yrow, uint16_t* dyrow, float wj, int u0,
                                          int lane, const CombineBwdArgs& a, float& dot) {
    u32x4 yv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c = min((u0 + u) * kUnit + lane * 8, a.H - 8);
        yv[u] = load_stream<1>((const u32x4*)(yrow + c));
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c = (u0 + u) * kUnit + lane * 8;
        if (u0 + u < a.units && c < a.H) {
            u32x4 o;
            o.x = pack2(wj, gv[u].x);
            o.y = pack2(wj, gv[u].y);
            o.z = pack2(wj, gv[u].z);
            o.w = pack2(wj, gv[u].w);
            store_stream<kBwdStoreNT>(o, (u32x4*)(dyrow + c));
            dot = __builtin_fmaf(bf16_lo(gv[u].x), bf16_lo(yv[u].x), dot);
            dot = __builtin_fmaf(bf16_hi(gv[u].x), bf16_hi(yv[u].x), dot);
            dot = __builtin_fmaf(bf16_lo(gv[u].y), bf16_lo(yv[u].y), dot);
            dot = __builtin_fmaf(bf16_hi(gv[u].y), bf16_hi(yv[u].y), dot);
            dot = __builtin_fmaf(bf16_lo(gv[u].z), bf16_lo(yv[u].z), dot);
            dot = __builtin_fmaf(bf16_hi(gv[u].z), bf16_hi(yv[u].z), dot);
            dot = __builtin_fmaf(bf16_lo(gv[u].w), bf16_lo(yv[u].w), dot);
            dot = __builtin_fmaf(bf16_hi(gv[u].w), bf16_hi(yv[u].w), dot);
        }
    }
}

template <int U>
__device__ __forceinline__ void load_chunk(u32x4 (&gv)[U], const uint16_t* grow, int u0, int lane, int H) {
#pragma unroll
    for (int u = 0; u < U; ++u) gv[u] = *(const u32x4*)(grow + min((u0 + u) * kUnit + lane * 8, H - 8));
}

template <int U, int KC>
__global__ __launch_bounds__(kBwdThreads) void combine_backward_kernel(CombineBwdArgs a) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * (kBwdThreads / kWave) + wave_in_block();
    if (t >= a.T) return;  // wave-uniform
    const int k = KC > 0 ? KC : a.k;
    int pv = (lane < k) ? a.pos[(size_t)t * k + lane] : -1;
    if (pv >= a.N) pv = -1;
    const float wv = (lane < k) ? a.w[(size_t)t * k + lane] : 0.0f;
    const uint16_t* grow = a.grad_out + (size_t)t * a.H;
    float gw_out = 0.0f;  // lane j ends with grad_w[t, j]

    if constexpr (KC > 0) {
        float dot[KC];
#pragma unroll
        for (int j = 0; j < KC; ++j) dot[j] = 0.0f;
        for (int u0 = 0; u0 < a.units; u0 += U) {
            u32x4 gv[U];
            load_chunk<U>(gv, grow, u0, lane, a.H);
#pragma unroll
            for (int j = 0; j < KC; ++j) {
                const int p = __builtin_amdgcn_readlane(pv, j);
                if (p < 0) continue;  // dropped pair (wave-uniform): grad_w stays 0
                const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wv), j));
                bwd_chunk<U>(gv, a.y + (size_t)p * a.H, a.grad_y + (size_t)p * a.H, wj, u0, lane, a, dot[j]);
            }
        }
#pragma unroll
        for (int j = 0; j < KC; ++j) {
            const float total = wave_sum(dot[j]);
            gw_out = (lane == j) ? total : gw_out;
        }
    } else {
        for (int j = 0; j < k; ++j) {
            const int p = __builtin_amdgcn_readlane(pv, j);
            if (p < 0) continue;
            const float wj = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wv), j));
            float dot = 0.0f;
            for (int u0 = 0; u0 < a.units; u0 += U) {
                u32x4 gv[U];
                load_chunk<U>(gv, grow, u0, lane, a.H);
                bwd_chunk<U>(gv, a.y + (size_t)p * a.H, a.grad_y + (size_t)p * a.H, wj, u0, lane, a, dot);
            }
            const float total = wave_sum(dot);
            gw_out = (lane == j) ? total : gw_out;
        }
    }
    if (lane < k) a.grad_w[(size_t)t * k + lane] = gw_out;
}

template <int U>
hipError_t launch_u(const CombineBwdArgs& a, hipStream_t s) {
    const unsigned blocks = (unsigned)((a.T + (kBwdThreads / kWave) - 1) / (kBwdThreads / kWave));
    switch (a.k) {
        case 8: hipLaunchKernelGGL((combine_backward_kernel<U, 8>), dim3(blocks), dim3(kBwdThreads), 0, s, a); break;
        case 4: hipLaunchKernelGGL((combine_backward_kernel<U, 4>), dim3(blocks), dim3(kBwdThreads), 0, s, a); break;
        case 2: hipLaunchKernelGGL((combine_backward_kernel<U, 2>), dim3(blocks), dim3(kBwdThreads), 0, s, a); break;
        default: hipLaunchKernelGGL((combine_backward_kernel<U, 0>), dim3(blocks), dim3(kBwdThreads), 0, s, a); break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_combine_backward(const uint16_t* grad_out, const uint16_t* y, const int32_t* pos, const float* w,
                                   uint16_t* grad_y, float* grad_w, int T, int H, int k, int N, int upw,
                                   hipStream_t stream) {
    CombineBwdArgs a{grad_out, y, pos, w, grad_y, grad_w, T, H, k, N, (H + kUnit - 1) / kUnit};
    // one unit per chunk: measured fastest at 4096 x 7168 top-8 (191 us against
    // 195 for 2 and 4 and 213 for 7), the smallest register footprint
    if (upw <= 0) upw = 1;
    switch (upw) {
        case 7: return launch_u<7>(a, stream);
        case 4: return launch_u<4>(a, stream);
        case 2: return launch_u<2>(a, stream);
        default: return launch_u<1>(a, stream);
    }
}

}  // namespace cgl
