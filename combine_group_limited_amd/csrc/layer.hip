// layer.hip -- a whole MoE layer after routing in ONE launch: dispatch (FP8
// with power-of-two scales) -> expert up (SwiGLU, FP8 requantisation) ->
// expert down -> top-k weighted combine.
//
// Follows the Mega MoE news page: a MoE layer runs dispatch, a first linear
// layer, SwiGLU, a second linear layer and combine, and fusing the steps into
// one kernel removes the launch boundaries between them.  On one GPU there is
// no transport to overlap with the GEMMs, so what the single launch removes is
// three kernel boundaries and their launch overhead.
//
// The grid is persistent: one block per compute unit (the expert-MLP tiles
// fill a CU's LDS), all resident, meeting at grid-wide barriers between the
// phases.  The expert-MLP phases run the standalone kernels' block code
// (mlp_impl.hpp) over their block indices; the dispatch and combine phases
// run the standalone arithmetic (quantize_unit, the slot-ordered fma folds,
// one bf16 rounding) in loops pipelined for a grid of four waves per CU.  So
// every output is bit for bit what moe_dispatch -> moe_expert_up ->
// moe_expert_down -> moe_combine write.  The phases hand their results to
// blocks on other XCDs through ordinary stores, so the barriers release and
// acquire at agent scope (one L2 write-back and one L1/L2 invalidation per
// block), as a kernel boundary would.
#include "combine_impl.hpp"
#include "dispatch_impl.hpp"
#include "grid_barrier.hpp"
#include "mlp_impl.hpp"
#include "moe_device.hpp"
#include "moe_internal.hpp"

namespace cgl {
namespace {

constexpr int kLayerThreads = 256;  // the expert-MLP block shape
// 512-channel units per wave item in the dispatch and combine phases (any
// count is exact: units past the row end are skipped).  The grid has only
// four waves per CU, so each wave keeps many 1-KiB pieces in flight and
// issues the next item's loads before the current item's stores: vmcnt
// retires loads and stores in issue order, so a load issued after a store
// would also wait for the store.
constexpr int kLayerUnits = 14;        // dispatch: a whole 7168-wide row per item
constexpr int kLayerCombineUnits = 7;  // combine: two buffers of gathers and the sums

// FP8 (power-of-two) dispatch of items w0, w0 + stride, ... (item = U units of
// one token), the arithmetic of dispatch_fp8_wave.
template <int U>
__device__ __forceinline__ void layer_dispatch(const DispatchArgs& a, int w0, int stride) {
    const int lane = threadIdx.x & 63;
    const int items = a.T * a.chunks;
    if (w0 >= items) return;  // wave-uniform
    auto load_item = [&](int w, u32x4 (&v)[U], int& pv) {
        const int t = w / a.chunks, u0 = (w - t * a.chunks) * U;
        const uint16_t* xrow = a.x + (size_t)t * a.H;
        pv = (lane < a.k) ? a.pos[(size_t)t * a.k + lane] : -1;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int c = (u0 + u) * kDispatchUnit + lane * 8;
            v[u] = (c < a.H) ? load16(xrow + c) : u32x4{0u, 0u, 0u, 0u};
        }
    };
    // two items ahead: v (item w), n1 (w + stride), n2 loaded for w + 2 stride
    // (past the end, loads re-read the last item: they stay unconditional)
    auto clampi = [&](int w) { return w < items ? w : items - 1; };
    u32x4 v[U], n1[U];
    int pv, p1;
    load_item(w0, v, pv);
    load_item(clampi(w0 + stride), n1, p1);
    for (int w = w0; w < items; w += stride) {
        u32x4 n2[U];
        int p2;
        load_item(clampi(w + 2 * stride), n2, p2);
        const int t = w / a.chunks, u0 = (w - t * a.chunks) * U;
        u32x2 code[U];
        float scale[U];
#pragma unroll
        for (int u = 0; u < U; ++u) code[u] = quantize_unit<true>(v[u], scale[u]);
        uint8_t* rx = (uint8_t*)a.recv_x;
        for (int j = 0; j < a.k; ++j) {
            const int p = __builtin_amdgcn_readlane(pv, j);
            if (p < 0 || p >= a.N) continue;  // dropped pair (wave-uniform)
            uint8_t* dst = rx + (size_t)p * a.H;
            float* sdst = (float*)a.recv_scales + (size_t)p * a.S;
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = (u0 + u) * kDispatchUnit + lane * 8;
                if (c < a.H) {
                    store_stream<kDispatchStoreNT>(code[u], (u32x2*)(dst + c));
                    if ((lane & 15) == 0) sdst[c >> 7] = scale[u];
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            v[u] = n1[u];
            n1[u] = n2[u];
        }
        pv = p1;
        p1 = p2;
    }
}

// Combine of items w0, w0 + stride, ... (item = U units of one token), the
// arithmetic of combine_wave: slots folded in order with one fma per element,
// dropped slots skipped, one bf16 rounding.  Slot j+1's gathers (or the next
// item's first slot) are in flight while slot j is folded, and the next
// item's routing row is read at the start of the current item.
template <int U>
__device__ __forceinline__ void layer_combine(const CombineArgs& a, int w0, int stride) {
    const int lane = threadIdx.x & 63;
    const int items = a.T * a.chunks;
    if (w0 >= items) return;  // wave-uniform
    const int k = a.k;
    auto meta = [&](int w, int& pv, float& wv) {
        const int t = w / a.chunks;
        pv = (lane < k) ? a.pos[(size_t)t * k + lane] : -1;
        if (pv >= a.N) pv = -1;  // out of range: contributes nothing
        wv = (lane < k) ? (a.w ? a.w[(size_t)t * k + lane] : 1.0f) : 0.0f;
    };
    // slot row p of item w (a dropped slot gathers row 0 and is not folded)
    auto gather = [&](u32x4 (&g)[U], int w, int p) {
        const int t = w / a.chunks, u0 = (w - t * a.chunks) * U;
        gather_row<U>(g, a.y + (size_t)(p < 0 ? 0 : p) * a.H, u0, lane, a.H);
    };
    int pvn;
    float wvn;
    meta(w0, pvn, wvn);
    u32x4 cur[U];
    gather(cur, w0, __builtin_amdgcn_readlane(pvn, 0));
    for (int w = w0; w < items; w += stride) {
        const int pv = pvn;
        const float wv = wvn;
        const int wn = w + stride < items ? w + stride : w;
        meta(wn, pvn, wvn);
        float acc[U][8];
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[u][i] = 0.0f;
        for (int j = 0; j < k; ++j) {
            u32x4 nxt[U];
            if (j + 1 < k) gather(nxt, w, __builtin_amdgcn_readlane(pv, j + 1));
            else gather(nxt, wn, __builtin_amdgcn_readlane(pvn, 0));
            if (__builtin_amdgcn_readlane(pv, j) >= 0) fold_row<U>(acc, cur, lane_float(wv, j));
#pragma unroll
            for (int u = 0; u < U; ++u) cur[u] = nxt[u];
        }
        const int t = w / a.chunks, u0 = (w - t * a.chunks) * U;
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
}
static_assert(kLayerThreads == kThreads, "the expert-MLP block body assumes its own block shape");

struct LayerArgs {
    DispatchArgs d;            // FP8 power-of-two dispatch, kLayerUnits units per wave item
    MlpArgs up, down;          // tile grids filled as for the standalone launches
    CombineArgs c;             // kLayerCombineUnits units per wave item
    unsigned up_blocks, down_blocks;
    uint32_t* bar;             // barrier workspace; word 2: blocks that gave up
};

// Workspace words from here on: block 0's 100-MHz real-time clock (64 bits)
// at the start and after each of the three barriers, for phase timings.
constexpr int kStampWord = 768;  // the barrier uses words 0..575 of the 1024

__device__ __forceinline__ void stamp(uint32_t* ws, int i) {
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        const uint64_t t = __builtin_amdgcn_s_memrealtime();
        ws[kStampWord + 2 * i] = (uint32_t)t;
        ws[kStampWord + 2 * i + 1] = (uint32_t)(t >> 32);
    }
}

template <int TM, int NRU, int NRD>
__global__ __launch_bounds__(kLayerThreads) void layer_kernel(LayerArgs a) {
    const int waves = gridDim.x * (kLayerThreads / kWave);
    const int w0 = blockIdx.x * (kLayerThreads / kWave) + wave_in_block();
    // a workspace an earlier launch gave up on is refused at the first barrier
    const bool refused = threadIdx.x == 0 && barrier_gave_up(a.bar);
    stamp(a.bar, 0);

    layer_dispatch<kLayerUnits>(a.d, w0, waves);
    if (!grid_barrier<true>(a.bar, refused)) return;  // block-uniform
    stamp(a.bar, 1);

    for (unsigned b = blockIdx.x; b < a.up_blocks; b += gridDim.x) {
        mlp_block<true, TM, NRU, true>(a.up, (int)b);
        __syncthreads();  // the next tile rewrites the LDS this one read last
    }
    if (!grid_barrier<true>(a.bar, false)) return;
    stamp(a.bar, 2);

    for (unsigned b = blockIdx.x; b < a.down_blocks; b += gridDim.x) {
        mlp_block<false, TM, NRD, true>(a.down, (int)b);
        __syncthreads();
    }
    if (!grid_barrier<true>(a.bar, false)) return;
    stamp(a.bar, 3);

    layer_combine<kLayerCombineUnits>(a.c, w0, waves);
}

template <int TM, int NRU, int NRD>
hipError_t launch_layer_tm(LayerArgs& a, size_t lds, hipStream_t s) {
    const auto kern = layer_kernel<TM, NRU, NRD>;
    hipError_t err = hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    int dev = 0, cus = 0, per_cu = 0;
    if (err == hipSuccess) err = hipGetDevice(&dev);
    if (err == hipSuccess) err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (err == hipSuccess) err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kLayerThreads, lds);
    if (err != hipSuccess) return err;
    if (per_cu < 1 || cus < 8) return hipErrorInvalidConfiguration;
    // one block per CU, a multiple of 8 so that block b + i*grid stays on the
    // XCD of block b and the expert-MLP tile order keeps its rectangles
    const unsigned blocks = (unsigned)(cus / 8 * 8);
    hipLaunchKernelGGL(kern, dim3(blocks), dim3(kLayerThreads), lds, s, a);
    return hipGetLastError();
}

}  // namespace

// 0 when the shape's tile configuration has a one-launch kernel, else the
// reason it does not (the caller returns MOE_ERR_UNSUPPORTED).
size_t layer_lds_bytes(int N, int H, int I, int E, int* supported) {
    const int tm = pick_tm(N, E), nru = pick_nr(tm, H, E), nrd = pick_nr(tm, I, E);
    *supported = (tm == 4 && nru == 2 && nrd == 2) || (tm == 2 && nru == 3 && nrd == 3);
    const size_t lu = tm == 4 ? lds_bytes_for<4>(H, E, nru) : lds_bytes_for<2>(H, E, nru);
    const size_t ld = tm == 4 ? lds_bytes_for<4>(I, E, nrd) : lds_bytes_for<2>(I, E, nrd);
    return lu > ld ? lu : ld;
}

hipError_t launch_layer(const uint16_t* x, const int32_t* pos, const float* topk_w, const int32_t* cnt_e,
                        const int32_t* off_e, const uint8_t* w1, const float* w1s, const uint8_t* w2,
                        const float* w2s, uint8_t* recv_x, float* recv_s, uint8_t* act, float* act_s, uint16_t* y,
                        uint16_t* out, uint32_t* barrier, int T, int k, int N, int H, int I, int E, int C,
                        hipStream_t stream) {
    LayerArgs a{};
    a.d.x = x;
    a.d.pos = pos;
    a.d.recv_x = recv_x;
    a.d.recv_scales = recv_s;
    a.d.T = T;
    a.d.H = H;
    a.d.k = k;
    a.d.N = N;
    a.d.S = H / 128;
    a.d.units = (H + kDispatchUnit - 1) / kDispatchUnit;
    a.d.chunks = (a.d.units + kLayerUnits - 1) / kLayerUnits;
    a.d.drain = 0;

    MlpArgs& u = a.up;
    u.a = recv_x;
    u.as = recv_s;
    u.w = w1;
    u.ws = w1s;
    u.cnt_e = cnt_e;
    u.off_e = off_e;
    u.act = act;
    u.act_s = act_s;
    u.N = N;
    u.K = H;
    u.WR = 2 * I;
    u.E = E;
    u.C = C;
    u.I = I;
    MlpArgs& dn = a.down;
    dn.a = act;
    dn.as = act_s;
    dn.w = w2;
    dn.ws = w2s;
    dn.cnt_e = cnt_e;
    dn.off_e = off_e;
    dn.y = y;
    dn.N = N;
    dn.K = I;
    dn.WR = H;
    dn.E = E;
    dn.C = C;
    dn.I = I;

    a.c.y = y;
    a.c.pos = pos;
    a.c.w = topk_w;
    a.c.out = out;
    a.c.T = T;
    a.c.H = H;
    a.c.k = k;
    a.c.N = N;
    a.c.units = (H + kCombineUnit - 1) / kCombineUnit;
    a.c.chunks = (a.c.units + kLayerCombineUnits - 1) / kLayerCombineUnits;
    a.bar = barrier;

    int supported = 0;
    const size_t lds = layer_lds_bytes(N, H, I, E, &supported);
    if (!supported) return hipErrorNotSupported;
    if (pick_tm(N, E) == 4) {
        a.up_blocks = mlp_grid<true, 4>(a.up);
        a.down_blocks = mlp_grid<false, 4>(a.down);
        return launch_layer_tm<4, 2, 2>(a, lds, stream);
    }
    a.up_blocks = mlp_grid<true, 2>(a.up);
    a.down_blocks = mlp_grid<false, 2>(a.down);
    return launch_layer_tm<2, 3, 3>(a, lds, stream);
}

}  // namespace cgl
