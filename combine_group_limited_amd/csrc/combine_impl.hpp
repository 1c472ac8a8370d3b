// combine_impl.hpp -- the per-wave body of the top-k weighted combine,
// shared by the standalone combine launch (combine.hip) and the one-launch
// MoE layer (layer.hip).  See combine.hip for the pages it follows and how
// the work is laid out.
#pragma once
#include "moe_device.hpp"

namespace cgl {
namespace {

constexpr int kCombineUnit = 512;
constexpr int kCombineThreads = 256;  // waves per block = threads / 64
// Cache policy of the y gathers and the output writes: both streaming.
// Measured on MI355X at 4096 x 7168 top-8: plain loads 109 us against 88 us.
constexpr int kCombineLoadNT = 1;
constexpr int kCombineStoreNT = 1;

struct CombineArgs {
    const uint16_t* y;
    const int32_t* pos;
    const float* w;
    uint16_t* out;
    int T, H, k, N;
    int units, chunks;
};

// Gathers U 16-byte pieces of one row.  Loads are unconditional (a lane past
// the end of the row reads the row's last piece instead; its result is never
// stored), so no branch separates the loads and the compiler can overlap them
// with the folds of the previous slot.
template <int U>
__device__ __forceinline__ void gather_row(u32x4 (&v)[U], const uint16_t* src, int u0, int lane, int H) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c = min((u0 + u) * kCombineUnit + lane * 8, H - 8);
        v[u] = load_stream<kCombineLoadNT>((const u32x4*)(src + c));
    }
}

template <int U>
__device__ __forceinline__ void fold_row(float (&acc)[U][8], const u32x4 (&v)[U], float wj) {
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

__device__ __forceinline__ float lane_float(float v, int j) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), j));
}

// The token's k receive rows and weights are read once, one per lane, and
// broadcast with readlane, so the slot loop issues only the row gathers, one
// slot at a time, folded in slot order (issuing the next slot's gathers while
// folding the current one measured slower on large batches: 92-102 against
// 88 us at 4096 tokens).  ALL (small grids, compile-time k): the gathers of
// all k slots are issued together before the folds, which still run in slot
// order: a decode-sized batch is bound by the latency of each gather round,
// not by bandwidth.
template <int U, int KC, bool ALL = false>
__device__ __forceinline__ void combine_wave(const CombineArgs& a, int wave) {
    const int lane = threadIdx.x & 63;
    const int t = wave / a.chunks;
    if (t >= a.T) return;  // wave-uniform
    const int u0 = (wave - t * a.chunks) * U;
    const int k = KC > 0 ? KC : a.k;

    int pv = (lane < k) ? a.pos[(size_t)t * k + lane] : -1;
    if (pv >= a.N) pv = -1;                     // out of range: contributes nothing
    // no weights (the backward of dispatch): every slot weighs 1
    const float wv = (lane < k) ? (a.w ? a.w[(size_t)t * k + lane] : 1.0f) : 0.0f;

    float acc[U][8];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[u][i] = 0.0f;

    if constexpr (ALL && KC > 0) {
        u32x4 v[KC][U];
#pragma unroll
        for (int j = 0; j < KC; ++j) {
            const int p = __builtin_amdgcn_readlane(pv, j);
            if (p >= 0) gather_row<U>(v[j], a.y + (size_t)p * a.H, u0, lane, a.H);  // wave-uniform
        }
#pragma unroll
        for (int j = 0; j < KC; ++j)
            if (__builtin_amdgcn_readlane(pv, j) >= 0) fold_row<U>(acc, v[j], lane_float(wv, j));
    } else {
        for (int j = 0; j < k; ++j) {
            const int p = __builtin_amdgcn_readlane(pv, j);
            if (p < 0) continue;  // wave-uniform
            u32x4 v[U];
            gather_row<U>(v, a.y + (size_t)p * a.H, u0, lane, a.H);
            fold_row<U>(acc, v, lane_float(wv, j));
        }
    }

    uint16_t* orow = a.out + (size_t)t * a.H;
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int c = (u0 + u) * kCombineUnit + lane * 8;
        if (c < a.H) {
            u32x4 o;
            o.x = pack_bf16x2(acc[u][0], acc[u][1]);
            o.y = pack_bf16x2(acc[u][2], acc[u][3]);
            o.z = pack_bf16x2(acc[u][4], acc[u][5]);
            o.w = pack_bf16x2(acc[u][6], acc[u][7]);
            store_stream<kCombineStoreNT>(o, (u32x4*)(orow + c));
        }
    }
}

}  // namespace
}  // namespace cgl
