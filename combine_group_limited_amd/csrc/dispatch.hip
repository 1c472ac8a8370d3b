// dispatch.hip -- scatter each token into its k receive rows, FP8-quantised
// with one scale per 128 channels (or verbatim BF16).
//
// Follows "Efficient and Portable Mixture-of-Experts Communication"
// (Perplexity), section "Dispatch": tokens travel with their block scaling
// factors and are unpacked into contiguous per-expert tensors for the grouped
// GEMM; FP8 dispatch as in the DeepEP workloads ("DeepSeek, DeepEP
// open-sourced", GeekNews 19421, "Performance > Normal kernels").
//
// Work unit: 512 channels of one token = one 16-byte load per lane of a wave
// (lane l holds channels 8l .. 8l+7, so a wave load is 1 KiB contiguous).  A
// 128-channel scale block is then exactly one 16-lane DPP row, and its absmax
// is a 4-step row reduction of integer magnitudes (|bf16| bit patterns order
// like their values).  A wave takes U consecutive units of one token, reads
// them once, quantises them once, and writes the codes (8 bytes per lane, a
// 512-byte contiguous store per unit) and the scales to each of the token's k
// receive rows.  Every output byte is written by exactly one lane.
#include "dispatch_impl.hpp"
#include "moe_device.hpp"
#include "moe_internal.hpp"

namespace cgl {
namespace {

template <int U, int MODE>
__global__ __launch_bounds__(kDispatchThreads) void dispatch_fp8_kernel(DispatchArgs a) {
    dispatch_fp8_wave<U, MODE>(a, blockIdx.x * (kDispatchThreads / kWave) + wave_in_block());
}

template <int U>
__global__ __launch_bounds__(kDispatchThreads) void dispatch_bf16_kernel(DispatchArgs a) {
    dispatch_bf16_wave<U>(a, blockIdx.x * (kDispatchThreads / kWave) + wave_in_block());
}

template <int U>
hipError_t launch_u(DispatchArgs a, int dtype, hipStream_t s) {
    a.chunks = (a.units + U - 1) / U;
    const long long waves = (long long)a.T * a.chunks;
    a.drain = waves >= kDrainWaves ? 1 : 0;
    const int wpb = kDispatchThreads / kWave;
    const unsigned blocks = (unsigned)((waves + wpb - 1) / wpb);
    if (dtype == 0)
        hipLaunchKernelGGL((dispatch_fp8_kernel<U, kScaleF32>), dim3(blocks), dim3(kDispatchThreads), 0, s, a);
    else if (dtype == 2)
        hipLaunchKernelGGL((dispatch_fp8_kernel<U, kScalePow2>), dim3(blocks), dim3(kDispatchThreads), 0, s, a);
    else if (dtype == 3)
        hipLaunchKernelGGL((dispatch_fp8_kernel<U, kScaleUE8M0>), dim3(blocks), dim3(kDispatchThreads), 0, s, a);
    else
        hipLaunchKernelGGL((dispatch_bf16_kernel<U>), dim3(blocks), dim3(kDispatchThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

int dispatch_units_per_wave(int T, int H) {
    const int units = (H + kDispatchUnit - 1) / kDispatchUnit;
    // enough waves to fill 256 CUs several times over, otherwise fewer loads
    // per wave; U must divide the unit count to avoid idle lanes
    static const int choices[] = {14, 8, 7, 4, 2, 1};
    for (int u : choices) {
        if (u > units || units % u) continue;
        if ((long long)T * (units / u) >= 4096 || u == 1) return u;
    }
    return 1;
}

hipError_t launch_dispatch(const uint16_t* x, const int32_t* pos, void* recv_x, void* recv_scales, int T,
                           int H, int k, int N, int dtype, int upw, hipStream_t stream) {
    DispatchArgs a{};
    a.x = x;
    a.pos = pos;
    a.recv_x = recv_x;
    a.recv_scales = recv_scales;
    a.T = T;
    a.H = H;
    a.k = k;
    a.N = N;
    a.S = H / 128;
    a.units = (H + kDispatchUnit - 1) / kDispatchUnit;
    if (upw <= 0) upw = dispatch_units_per_wave(T, H);
    switch (upw) {
        case 14: return launch_u<14>(a, dtype, stream);
        case 8: return launch_u<8>(a, dtype, stream);
        case 7: return launch_u<7>(a, dtype, stream);
        case 4: return launch_u<4>(a, dtype, stream);
        case 2: return launch_u<2>(a, dtype, stream);
        default: return launch_u<1>(a, dtype, stream);
    }
}

}  // namespace cgl
