// combine.hip -- top-k weighted gather-reduce of BF16 expert outputs back
// into token order.
//
// Follows "Efficient and Portable Mixture-of-Experts Communication"
// (Perplexity), section "Combine": the receiver reads every expert's 16-bit
// output for a token, the routing table says which row to read and which
// weight to apply, and the weighted sum goes to a caller-allocated tensor.
//
// Same unit as dispatch: 512 channels of one token per 16-byte-per-lane wave
// load.  A wave takes U units of one token and, for each slot j in order,
// gathers the U 1 KiB pieces of row pos[t,j] (issued together) and folds them
// into fp32 accumulators with one fma per element; the result is rounded to
// bf16 once (v_cvt_pk_bf16_f32, nearest-even) and stored with 16-byte writes.
#include "moe_device.hpp"
#include "moe_internal.hpp"

namespace cgl {
namespace {

constexpr int kUnit = 512;
constexpr int kCombineThreads = 256;

struct CombineArgs {
    const uint16_t* y;
    const int32_t* pos;
    const float* w;
    uint16_t* out;
    int T, H, k, N;
    int units, chunks;
};

template <int U>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(CombineArgs a) {
    const int lane = threadIdx.x & 63;
    const int wave = blockIdx.x * (kCombineThreads / kWave) + (threadIdx.x >> 6);
    const int t = wave / a.chunks;
    if (t >= a.T) return;  // wave-uniform
    const int u0 = (wave - t * a.chunks) * U;

    float acc[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[u][i] = 0.0f;

    const int32_t* prow = a.pos + (size_t)t * a.k;
    const float* wrow = a.w + (size_t)t * a.k;
    for (int j = 0; j < a.k; ++j) {
        const int p = prow[j];
        if (p < 0 || p >= a.N) continue;  // dropped pair (wave-uniform)
        const float wj = wrow[j];
        const uint16_t* src = a.y + (size_t)p * a.H;
        u32x4 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = (u0 + u) * kUnit + lane * 8;
            v[u] = (c < a.H) ? __builtin_nontemporal_load((const u32x4*)(src + c)) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            acc[u][0] = __builtin_fmaf(wj, bf16_lo(v[u].x), acc[u][0]);
            acc[u][1] = __builtin_fmaf(wj, bf16_hi(v[u].x), acc[u][1]);
            acc[u][2] = __builtin_fmaf(wj, bf16_lo(v[u].y), acc[u][2]);
            acc[u][3] = __builtin_fmaf(wj, bf16_hi(v[u].y), acc[u][3]);
            acc[u][4] = __builtin_fmaf(wj, bf16_lo(v[u].z), acc[u][4]);
            acc[u][5] = __builtin_fmaf(wj, bf16_hi(v[u].z), acc[u][5]);
            acc[u][6] = __builtin_fmaf(wj, bf16_lo(v[u].w), acc[u][6]);
            acc[u][7] = __builtin_fmaf(wj, bf16_hi(v[u].w), acc[u][7]);
        }
    }

    uint16_t* orow = a.out + (size_t)t * a.H;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c = (u0 + u) * kUnit + lane * 8;
        if (c < a.H) {
            u32x4 o;
            o.x = pack_bf16x2(acc[u][0], acc[u][1]);
            o.y = pack_bf16x2(acc[u][2], acc[u][3]);
            o.z = pack_bf16x2(acc[u][4], acc[u][5]);
            o.w = pack_bf16x2(acc[u][6], acc[u][7]);
            __builtin_nontemporal_store(o, (u32x4*)(orow + c));
        }
    }
}

template <int U>
hipError_t launch_u(CombineArgs a, hipStream_t s) {
    a.chunks = (a.units + U - 1) / U;
    const long long waves = (long long)a.T * a.chunks;
    const int wpb = kCombineThreads / kWave;
    const unsigned blocks = (unsigned)((waves + wpb - 1) / wpb);
    hipLaunchKernelGGL((combine_kernel<U>), dim3(blocks), dim3(kCombineThreads), 0, s, a);
    return hipGetLastError();
}

}  // namespace

int combine_units_per_wave(int T, int H) {
    const int units = (H + kUnit - 1) / kUnit;
    static const int choices[] = {7, 4, 2, 1};
    for (int u : choices) {
        if (u > units || units % u) continue;
        if ((long long)T * (units / u) >= 4096 || u == 1) return u;
    }
    return 1;
}

hipError_t launch_combine(const uint16_t* y, const int32_t* pos, const float* w, uint16_t* out, int T, int H,
                          int k, int N, int upw, hipStream_t stream) {
    CombineArgs a{};
    a.y = y;
    a.pos = pos;
    a.w = w;
    a.out = out;
    a.T = T;
    a.H = H;
    a.k = k;
    a.N = N;
    a.units = (H + kUnit - 1) / kUnit;
    if (upw <= 0) upw = combine_units_per_wave(T, H);
    switch (upw) {
        case 7: return launch_u<7>(a, stream);
        case 4: return launch_u<4>(a, stream);
        case 2: return launch_u<2>(a, stream);
        default: return launch_u<1>(a, stream);
    }
}

}  // namespace cgl
