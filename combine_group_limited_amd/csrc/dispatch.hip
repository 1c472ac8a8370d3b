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
#include "moe_device.hpp"
#include "moe_internal.hpp"

namespace cgl {
namespace {

constexpr int kUnit = 512;             // channels per wave-wide 16-byte load
#ifndef CGL_DISPATCH_THREADS
#define CGL_DISPATCH_THREADS 256
#endif
// LDS bytes requested per block only to cap how many blocks share a CU
// (0 = no cap)
#ifndef CGL_DISPATCH_LDS_CAP
#define CGL_DISPATCH_LDS_CAP 0
#endif
constexpr int kDispatchThreads = CGL_DISPATCH_THREADS;  // waves per block = threads / 64
constexpr long long kDrainWaves = 2048;

// cache policy of the x reads and the receive-buffer writes (1 = streaming).
// Measured on MI355X at 4096 x 7168 top-8: streaming loads with ordinary
// stores are fastest in the dispatch -> combine sequence.
#ifndef CGL_DISPATCH_LOAD_NT
#define CGL_DISPATCH_LOAD_NT 1
#endif
#ifndef CGL_DISPATCH_STORE_NT
#define CGL_DISPATCH_STORE_NT 0
#endif
// 1: wait until a destination row's stores have completed before starting
// the next row (fewer rows open at once across the chip) when the grid has
// at least kDrainWaves waves; smaller grids leave every row in flight.
// Measured on MI355X: 48.9 vs 52.6 us at 4096 tokens (4 096 waves), but
// 4.6 vs 3.8 us at 128 tokens (1 792 waves).
#ifndef CGL_DISPATCH_DRAIN
#define CGL_DISPATCH_DRAIN 1
#endif

struct DispatchArgs {
    const uint16_t* x;
    const int32_t* pos;
    void* recv_x;
    float* recv_scales;
    int T, H, k, N, S;
    int units;   // ceil(H / 512)
    int chunks;  // ceil(units / U): waves per token
    int drain;   // wait for each row's stores before the next
};

__device__ __forceinline__ u32x4 load16(const uint16_t* p) {
    return load_stream<CGL_DISPATCH_LOAD_NT>((const u32x4*)p);
}

template <int U, bool POW2>
__global__ __launch_bounds__(kDispatchThreads) void dispatch_fp8_kernel(DispatchArgs a) {
    const int lane = threadIdx.x & 63;
    const int wave = blockIdx.x * (kDispatchThreads / kWave) + wave_in_block();
    const int t = wave / a.chunks;
    if (t >= a.T) return;  // wave-uniform
    const int u0 = (wave - t * a.chunks) * U;
    const uint16_t* xrow = a.x + (size_t)t * a.H;
    // the token's k receive rows, one per lane, read once up front so the
    // store loop below issues no loads (a load there would make the wave wait
    // for its outstanding stores too)
    const int pv = (lane < a.k) ? a.pos[(size_t)t * a.k + lane] : -1;

    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c = (u0 + u) * kUnit + lane * 8;
        v[u] = (c < a.H) ? load16(xrow + c) : u32x4{0u, 0u, 0u, 0u};
    }

    u32x2 code[U];
    float scale[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        code[u] = quantize_unit<POW2>(v[u], scale[u]);
    }

    uint8_t* rx = (uint8_t*)a.recv_x;
    for (int j = 0; j < a.k; ++j) {
        const int p = __builtin_amdgcn_readlane(pv, j);
        if (p < 0 || p >= a.N) continue;  // dropped pair (wave-uniform)
        uint8_t* dst = rx + (size_t)p * a.H;
        float* sdst = a.recv_scales + (size_t)p * a.S;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = (u0 + u) * kUnit + lane * 8;
            if (c < a.H) {
                store_stream<CGL_DISPATCH_STORE_NT>(code[u], (u32x2*)(dst + c));
                if ((lane & 15) == 0) sdst[c >> 7] = scale[u];
            }
        }
        if (CGL_DISPATCH_DRAIN && a.drain) __builtin_amdgcn_s_waitcnt(kWaitStores);
    }
}

template <int U>
__global__ __launch_bounds__(kDispatchThreads) void dispatch_bf16_kernel(DispatchArgs a) {
    const int lane = threadIdx.x & 63;
    const int wave = blockIdx.x * (kDispatchThreads / kWave) + wave_in_block();
    const int t = wave / a.chunks;
    if (t >= a.T) return;
    const int u0 = (wave - t * a.chunks) * U;
    const uint16_t* xrow = a.x + (size_t)t * a.H;
    const int pv = (lane < a.k) ? a.pos[(size_t)t * a.k + lane] : -1;
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c = (u0 + u) * kUnit + lane * 8;
        v[u] = (c < a.H) ? load16(xrow + c) : u32x4{0u, 0u, 0u, 0u};
    }
    uint16_t* rx = (uint16_t*)a.recv_x;
    for (int j = 0; j < a.k; ++j) {
        const int p = __builtin_amdgcn_readlane(pv, j);
        if (p < 0 || p >= a.N) continue;
        uint16_t* dst = rx + (size_t)p * a.H;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = (u0 + u) * kUnit + lane * 8;
            if (c < a.H) store_stream<CGL_DISPATCH_STORE_NT>(v[u], (u32x4*)(dst + c));
        }
        if (CGL_DISPATCH_DRAIN && a.drain) __builtin_amdgcn_s_waitcnt(kWaitStores);
    }
}

template <int U>
hipError_t launch_u(DispatchArgs a, int dtype, hipStream_t s) {
    a.chunks = (a.units + U - 1) / U;
    const long long waves = (long long)a.T * a.chunks;
    a.drain = waves >= kDrainWaves ? 1 : 0;
    const int wpb = kDispatchThreads / kWave;
    const unsigned blocks = (unsigned)((waves + wpb - 1) / wpb);
    if (dtype == 0)
        hipLaunchKernelGGL((dispatch_fp8_kernel<U, false>), dim3(blocks), dim3(kDispatchThreads), CGL_DISPATCH_LDS_CAP,
                           s, a);
    else if (dtype == 2)
        hipLaunchKernelGGL((dispatch_fp8_kernel<U, true>), dim3(blocks), dim3(kDispatchThreads), CGL_DISPATCH_LDS_CAP,
                           s, a);
    else
        hipLaunchKernelGGL((dispatch_bf16_kernel<U>), dim3(blocks), dim3(kDispatchThreads), CGL_DISPATCH_LDS_CAP, s, a);
    return hipGetLastError();
}

}  // namespace

int dispatch_units_per_wave(int T, int H) {
    const int units = (H + kUnit - 1) / kUnit;
    // enough waves to fill 256 CUs several times over, otherwise fewer loads
    // per wave; U must divide the unit count to avoid idle lanes
    static const int choices[] = {14, 8, 7, 4, 2, 1};
    for (int u : choices) {
        if (u > units || units % u) continue;
        if ((long long)T * (units / u) >= 4096 || u == 1) return u;
    }
    return 1;
}

hipError_t launch_dispatch(const uint16_t* x, const int32_t* pos, void* recv_x, float* recv_scales, int T,
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
    a.units = (H + kUnit - 1) / kUnit;
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
