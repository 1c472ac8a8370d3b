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
#include "combine_impl.hpp"
#include "moe_device.hpp"
#include "moe_internal.hpp"

namespace cgl {
namespace {

template <int U, int KC, bool ALL = false>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(CombineArgs a) {
    combine_wave<U, KC, ALL>(a, blockIdx.x * (kCombineThreads / kWave) + wave_in_block());
}

// Grids below this many waves issue all k slots' gathers at once (k = 8, 4 or
// 2, one unit per wave): decode-sized batches.
constexpr long long kAllSlotsWaves = 2048;

template <int U>
hipError_t launch_u(CombineArgs a, hipStream_t s) {
    a.chunks = (a.units + U - 1) / U;
    const long long waves = (long long)a.T * a.chunks;
    const int wpb = kCombineThreads / kWave;
    const unsigned blocks = (unsigned)((waves + wpb - 1) / wpb);
    if constexpr (U == 1) {
        if (waves < kAllSlotsWaves) switch (a.k) {
            case 8: hipLaunchKernelGGL((combine_kernel<U, 8, true>), dim3(blocks), dim3(kCombineThreads), 0, s, a);
                return hipGetLastError();
            case 4: hipLaunchKernelGGL((combine_kernel<U, 4, true>), dim3(blocks), dim3(kCombineThreads), 0, s, a);
                return hipGetLastError();
            case 2: hipLaunchKernelGGL((combine_kernel<U, 2, true>), dim3(blocks), dim3(kCombineThreads), 0, s, a);
                return hipGetLastError();
            default: break;
        }
    }
    switch (a.k) {
        case 8: hipLaunchKernelGGL((combine_kernel<U, 8>), dim3(blocks), dim3(kCombineThreads), 0, s, a); break;
        case 4: hipLaunchKernelGGL((combine_kernel<U, 4>), dim3(blocks), dim3(kCombineThreads), 0, s, a); break;
        case 2: hipLaunchKernelGGL((combine_kernel<U, 2>), dim3(blocks), dim3(kCombineThreads), 0, s, a); break;
        default: hipLaunchKernelGGL((combine_kernel<U, 0>), dim3(blocks), dim3(kCombineThreads), 0, s, a); break;
    }
    return hipGetLastError();
}

}  // namespace

int combine_units_per_wave(int T, int H) {
    const int units = (H + kCombineUnit - 1) / kCombineUnit;
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
    a.units = (H + kCombineUnit - 1) / kCombineUnit;
    if (upw <= 0) upw = combine_units_per_wave(T, H);
    switch (upw) {
        case 7: return launch_u<7>(a, stream);
        case 4: return launch_u<4>(a, stream);
        case 2: return launch_u<2>(a, stream);
        default: return launch_u<1>(a, stream);
    }
}

}  // namespace cgl
