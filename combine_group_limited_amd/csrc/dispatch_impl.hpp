// dispatch_impl.hpp -- the per-wave bodies of the dispatch (FP8 and BF16),
// shared by the standalone dispatch launch (dispatch.hip) and the one-launch
// MoE layer (layer.hip).  See dispatch.hip for the pages it follows and how
// the work is laid out.
#pragma once
#include "moe_device.hpp"

namespace cgl {
namespace {

constexpr int kDispatchUnit = 512;             // channels per wave-wide 16-byte load
constexpr int kDispatchThreads = 256;          // waves per block = threads / 64
constexpr long long kDrainWaves = 2048;

// Cache policy of the x reads and the receive-buffer writes (1 = streaming).
// Measured on MI355X at 4096 x 7168 top-8: streaming loads with ordinary
// stores are fastest in the dispatch -> combine sequence (48 us against
// 57-59 us with streaming stores).
constexpr int kDispatchLoadNT = 1;
constexpr int kDispatchStoreNT = 0;
// Grids of at least kDrainWaves waves wait until a destination row's stores
// have completed before starting the next row (fewer rows open at once across
// the chip); smaller grids leave every row in flight.  Measured on MI355X:
// 48.9 vs 52.6 us at 4096 tokens (4 096 waves), but 4.6 vs 3.8 us at 128
// tokens (1 792 waves).

struct DispatchArgs {
    const uint16_t* x;
    const int32_t* pos;
    void* recv_x;
    void* recv_scales;  // fp32 [N, S], or uint8 [N, S] E8M0 exponent bytes
    int T, H, k, N, S;
    int units;   // ceil(H / 512)
    int chunks;  // ceil(units / U): waves per token
    int drain;   // wait for each row's stores before the next
};

__device__ __forceinline__ u32x4 load16(const uint16_t* p) {
    return load_stream<kDispatchLoadNT>((const u32x4*)p);
}

// Scale formats of the FP8 dispatch: amax/448 in fp32, a power of two in
// fp32, or the same power of two as one E8M0 byte (its biased exponent).
enum { kScaleF32 = 0, kScalePow2 = 2, kScaleUE8M0 = 3 };

__device__ __forceinline__ uint8_t e8m0_byte(float pow2_scale) {
    return (uint8_t)((__float_as_uint(pow2_scale) >> 23) & 0xFFu);
}

template <int MODE>
__device__ __forceinline__ void store_scale(void* scales, size_t i, float scale) {
    if constexpr (MODE == kScaleUE8M0)
        ((uint8_t*)scales)[i] = e8m0_byte(scale);
    else
        ((float*)scales)[i] = scale;
}

template <int U, int MODE>
__device__ __forceinline__ void dispatch_fp8_wave(const DispatchArgs& a, int wave) {
    const int lane = threadIdx.x & 63;
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
        const int c = (u0 + u) * kDispatchUnit + lane * 8;
        v[u] = (c < a.H) ? load16(xrow + c) : u32x4{0u, 0u, 0u, 0u};
    }

    u32x2 code[U];
    float scale[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        code[u] = quantize_unit<MODE != kScaleF32>(v[u], scale[u]);
    }

    uint8_t* rx = (uint8_t*)a.recv_x;
    for (int j = 0; j < a.k; ++j) {
        const int p = __builtin_amdgcn_readlane(pv, j);
        if (p < 0 || p >= a.N) continue;  // dropped pair (wave-uniform)
        uint8_t* dst = rx + (size_t)p * a.H;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = (u0 + u) * kDispatchUnit + lane * 8;
            if (c < a.H) {
                store_stream<kDispatchStoreNT>(code[u], (u32x2*)(dst + c));
                if ((lane & 15) == 0) store_scale<MODE>(a.recv_scales, (size_t)p * a.S + (c >> 7), scale[u]);
            }
        }
        if (a.drain) __builtin_amdgcn_s_waitcnt(kWaitStores);
    }
}

template <int U>
__device__ __forceinline__ void dispatch_bf16_wave(const DispatchArgs& a, int wave) {
    const int lane = threadIdx.x & 63;
    const int t = wave / a.chunks;
    if (t >= a.T) return;
    const int u0 = (wave - t * a.chunks) * U;
    const uint16_t* xrow = a.x + (size_t)t * a.H;
    const int pv = (lane < a.k) ? a.pos[(size_t)t * a.k + lane] : -1;
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c = (u0 + u) * kDispatchUnit + lane * 8;
        v[u] = (c < a.H) ? load16(xrow + c) : u32x4{0u, 0u, 0u, 0u};
    }
    uint16_t* rx = (uint16_t*)a.recv_x;
    for (int j = 0; j < a.k; ++j) {
        const int p = __builtin_amdgcn_readlane(pv, j);
        if (p < 0 || p >= a.N) continue;
        uint16_t* dst = rx + (size_t)p * a.H;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = (u0 + u) * kDispatchUnit + lane * 8;
            if (c < a.H) store_stream<kDispatchStoreNT>(v[u], (u32x4*)(dst + c));
        }
        if (a.drain) __builtin_amdgcn_s_waitcnt(kWaitStores);
    }
}

}  // namespace
}  // namespace cgl
