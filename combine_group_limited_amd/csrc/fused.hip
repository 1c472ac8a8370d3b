// fused.hip -- the decode path in one launch: group-limited top-k routing,
// the routing layout and the FP8 (or BF16) dispatch of a small batch.
//
// Follows the DeepEP V2 digest, section "training/prefill/decoding usage",
// and "DeepSeek, DeepEP open-sourced" (GeekNews 19421), "Performance >
// Low-latency kernels": at decode the batch per rank is small and the cost is
// latency, so the layout pass and its host round trip should not stand
// between the router and the send.  The result is identical to
// moe_route_topk -> moe_get_layout -> moe_dispatch; only the launch structure
// differs.
//
// One launch of 256-thread blocks, all resident at once (the host sizes the
// grid from the occupancy of this kernel, with a factor-two margin):
//   1. waves 0..T-1 route token = wave index (route_impl.hpp);
//   2. a grid-wide barrier (below);
//   3. every wave loads its first 512-channel unit of x, and while those loads
//      are in flight every block rebuilds the whole layout of the batch in LDS
//      (T <= 1024: a 64-bit token mask per expert and 64-token chunk, popcount
//      ranks, a block-wide scan), which is cheaper than a second barrier;
//   4. every wave stores its unit(s) into the token's k receive rows;
//   5. the layout outputs are split between blocks so that every element is
//      written by exactly one block (block 0: counts, offsets and flags;
//      block b: a slice of pos and whole 2048-row slices of recv_src, built in
//      LDS, -1 for empty rows).
//
// The only data that crosses blocks inside the launch is topk_idx.  It is
// written and read with device-scope atomic stores and loads, which the
// gfx950 memory model performs at the device coherence point (past the
// per-XCD L2s), and every wave waits for its stores to complete before its
// block arrives.  Device-scope release/acquire fences would instead write back
// and invalidate each XCD's whole L2 once per block: measured on MI355X at
// 128 tokens, they cost 11 us of a 17 us launch.
#include <mutex>
#include <vector>

#include "dispatch_impl.hpp"
#include "grid_barrier.hpp"
#include "moe_internal.hpp"
#include "route_impl.hpp"

namespace cgl {
namespace {

constexpr int kFusedThreads = 256;
constexpr int kFusedWaves = kFusedThreads / kWave;
constexpr int kUnitChannels = 512;  // one 16-byte load per lane
constexpr int kSliceRows = 2048;    // recv_src rows per LDS slice
constexpr int kFlagIncomplete = 4;  // MOE_FLAG_INCOMPLETE

struct FusedArgs {
    RouteArgs r;  // logits -> idx [T,k], w [T,k]; T, E, G, g, k, n, score_fn, renorm
    int32_t *cnt_e, *cnt_r, *off_e, *off_r, *pos, *recv_src, *flags;
    const uint16_t* x;
    void* recv_x;
    void* recv_scales;
    uint32_t* bar;  // barrier workspace (see grid_barrier); word 2: blocks that gave up
    int R, C, A, N;
    int H, S, units, dtype;
    int nch;  // ceil(T / 64)
};

__device__ __forceinline__ u32x4 load_unit(const FusedArgs& a, int item, int lane) {
    const int t = item / a.units;
    const int c = (item - t * a.units) * kUnitChannels + lane * 8;
    if (c >= a.H) return u32x4{0u, 0u, 0u, 0u};
    return __builtin_nontemporal_load((const u32x4*)(a.x + (size_t)t * a.H + c));
}

// Stores one unit of token t into its k receive rows (rows from LDS posl).
// At decode sizes the rows' stores are left in flight together: waiting for
// each row (which pays at 4096 tokens) costs 1 us here.
__device__ __forceinline__ void store_unit(const FusedArgs& a, const int32_t* posl, int item, int lane,
                                           const u32x4& v, const u32x2& code, float scale) {
    const int t = item / a.units;
    const int c = (item - t * a.units) * kUnitChannels + lane * 8;
    const int k = a.r.k;
    const int pv = (lane < k) ? posl[t * k + lane] : -1;
    for (int j = 0; j < k; ++j) {
        const int p = __builtin_amdgcn_readlane(pv, j);
        if (p < 0 || p >= a.N) continue;  // dropped pair (wave-uniform)
        if (c < a.H) {
            if (a.dtype == 1) {
                *(u32x4*)((uint16_t*)a.recv_x + (size_t)p * a.H + c) = v;
            } else {
                *(u32x2*)((uint8_t*)a.recv_x + (size_t)p * a.H + c) = code;
                if ((lane & 15) == 0) {
                    if (a.dtype == 3)
                        store_scale<kScaleUE8M0>(a.recv_scales, (size_t)p * a.S + (c >> 7), scale);
                    else
                        store_scale<kScaleF32>(a.recv_scales, (size_t)p * a.S + (c >> 7), scale);
                }
            }
        }
    }
}

__device__ __forceinline__ u32x2 quantize(const FusedArgs& a, const u32x4& v, float& scale) {
    if (a.dtype >= 2) return quantize_unit<true>(v, scale);
    return quantize_unit<false>(v, scale);  // also run for BF16, result unused
}


template <int EPL, int LPG>
__global__ __launch_bounds__(kFusedThreads) void fused_decode_kernel(FusedArgs a) {
    extern __shared__ uint64_t lds[];
    const int T = a.r.T, E = a.r.E, k = a.r.k, R = a.R;
    uint64_t* emask = lds;                                   // [nch][E]
    uint64_t* rmask = emask + (size_t)a.nch * E;             // [nch][R]
    int32_t* tot = (int32_t*)(rmask + (size_t)a.nch * R);    // [E]
    int32_t* off = tot + E;                                  // [E+1]
    int32_t* posl = off + E + 1;                             // [T*k] indices, then rows
    int32_t* slice = posl + T * k;                           // [kSliceRows]

    const int tid = threadIdx.x, lane = tid & 63;
    const int gw = blockIdx.x * kFusedWaves + wave_in_block();
    const int nw = gridDim.x * kFusedWaves;
    const int items = T * a.units;

    // a workspace an earlier launch gave up on is refused at the barrier
    const bool refused = tid == 0 && barrier_gave_up(a.bar);

    // ---- 1. routing ------------------------------------------------------------
    for (int t = gw; t < T; t += nw) route_token<EPL, LPG, true>(a.r, t);

    // ---- 2. every token routed ---------------------------------------------
    if (!grid_barrier<false>(a.bar, refused)) {  // block-uniform
        // block 0 writes the flags only here or at its end, never both
        if (blockIdx.x == 0 && tid == 0) a.flags[0] = kFlagIncomplete;
        return;
    }
    // a block of this launch that stopped waiting as the barrier opened
    const bool gave_up = blockIdx.x == 0 && tid == 0 && barrier_gave_up(a.bar);

    // first unit of x, in flight while the layout is built
    u32x4 v0 = u32x4{0u, 0u, 0u, 0u};
    if (gw < items) v0 = load_unit(a, gw, lane);

    // ---- 3. the layout of the whole batch, in LDS ----------------------------
    for (int i = tid; i < a.nch * E; i += kFusedThreads) emask[i] = 0;
    for (int i = tid; i < a.nch * R; i += kFusedThreads) rmask[i] = 0;
    __syncthreads();
    const int Er = E / R;
    int bad = 0;
    // four consecutive pairs per thread, their device-scope loads all issued
    // before the first is used (one load in flight per slot costs 1.3 us)
    for (int i0 = 4 * tid; i0 < T * k; i0 += 4 * kFusedThreads) {
        int ev[4];
#pragma unroll
        for (int c = 0; c < 4; ++c)
            ev[c] = i0 + c < T * k ? __hip_atomic_load(&a.r.idx[i0 + c], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                   : 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const int i = i0 + c;
            if (i >= T * k) break;
            const int t = i / k, e = ev[c];
            const uint64_t bit = 1ull << (t & 63);
            const int ch = t >> 6;
            posl[i] = e;
            if (e < 0 || e >= E) {
                bad = 1;
                continue;
            }
            const uint64_t old = atomicOr((unsigned long long*)&emask[ch * E + e], (unsigned long long)bit);
            if (old & bit) bad = 1;
            atomicOr((unsigned long long*)&rmask[ch * R + e / Er], (unsigned long long)bit);
        }
    }
    const int any_bad = __syncthreads_or(bad);
    for (int e = tid; e < E; e += kFusedThreads) {
        int c = 0;
        for (int ch = 0; ch < a.nch; ++ch) c += __popcll(emask[ch * E + e]);
        tot[e] = c;
    }
    __syncthreads();
    block_exclusive_scan<kFusedThreads>(tot, off, E, a.A);  // ends with a barrier
    for (int i = tid; i < T * k; i += kFusedThreads) {
        const int t = i / k, ch = t >> 6;
        const int e = posl[i];
        int p = -1;
        if (e >= 0 && e < E) {
            int rank = __popcll(emask[ch * E + e] & ((1ull << (t & 63)) - 1ull));
            for (int cc = 0; cc < ch; ++cc) rank += __popcll(emask[cc * E + e]);
            if (a.C == 0)
                p = off[e] + rank;
            else if (rank < a.C)
                p = e * a.C + rank;
        }
        posl[i] = p;
    }
    __syncthreads();

    // ---- 4. dispatch ----------------------------------------------------------
    float s0 = 0.0f;
    const u32x2 q0 = quantize(a, v0, s0);
    if (gw < items) store_unit(a, posl, gw, lane, v0, q0, s0);
    for (int item = gw + nw; item < items; item += nw) {
        const u32x4 v = load_unit(a, item, lane);
        float s = 0.0f;
        const u32x2 q = quantize(a, v, s);
        store_unit(a, posl, item, lane, v, q, s);
    }

    // ---- 5. layout outputs, each element by one block -------------------------
    if (blockIdx.x == 0) {
        for (int e = tid; e < E; e += kFusedThreads) a.cnt_e[e] = tot[e];
        for (int e = tid; e <= E; e += kFusedThreads) a.off_e[e] = off[e];
        for (int r = tid; r < R; r += kFusedThreads) {
            int c = 0;
            for (int ch = 0; ch < a.nch; ++ch) c += __popcll(rmask[ch * R + r]);
            a.cnt_r[r] = c;
        }
        for (int r = tid; r <= R; r += kFusedThreads) a.off_r[r] = off[r * Er];
        int over = 0;
        if (a.C > 0)
            for (int e = tid; e < E; e += kFusedThreads) over |= tot[e] > a.C;
        const int any_over = __syncthreads_or(over);
        if (tid == 0) a.flags[0] = (any_over ? 1 : 0) | (any_bad ? 2 : 0) | (gave_up ? kFlagIncomplete : 0);
    }
    const int pairs = T * k;
    const int per = (pairs + gridDim.x - 1) / gridDim.x;
    const int p0 = min(pairs, (int)blockIdx.x * per), p1 = min(pairs, p0 + per);
    for (int i = p0 + tid; i < p1; i += kFusedThreads) a.pos[i] = posl[i];
    const int nslices = (a.N + kSliceRows - 1) / kSliceRows;
    for (int sl = blockIdx.x; sl < nslices; sl += gridDim.x) {
        const int r0 = sl * kSliceRows, len = min(kSliceRows, a.N - r0);
        for (int i = tid; i < len; i += kFusedThreads) slice[i] = -1;
        __syncthreads();
        for (int i = tid; i < pairs; i += kFusedThreads) {
            const int p = posl[i] - r0;
            if (p >= 0 && p < len) slice[p] = i;
        }
        __syncthreads();
        for (int i = tid; i < len; i += kFusedThreads) a.recv_src[r0 + i] = slice[i];
        __syncthreads();
    }
}

size_t fused_lds_bytes(int T, int E, int k, int R) {
    const size_t nch = (size_t)(T + 63) / 64;
    return 8 * nch * (E + R) + 4 * ((size_t)E + E + 1 + (size_t)T * k + kSliceRows);
}

// Blocks of a kernel that the current device holds at once with the given
// dynamic LDS: asked of the runtime once per (device, kernel, LDS size) and
// then kept, since a decode loop calls this path every step and the query
// costs host time of the order of the kernel itself.
template <class K>
hipError_t resident_blocks(K kern, size_t lds, long long* out) {
    struct Entry {
        int dev;
        const void* kern;
        size_t lds;
        long long blocks;
    };
    static std::mutex mu;
    static std::vector<Entry> cache;
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    {
        std::lock_guard<std::mutex> g(mu);
        for (const Entry& e : cache)
            if (e.dev == dev && e.kern == (const void*)kern && e.lds == lds) {
                *out = e.blocks;
                return hipSuccess;
            }
    }
    int cus = 0, per_cu = 0;
    err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (err == hipSuccess) err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kFusedThreads, lds);
    if (err != hipSuccess) return err;
    *out = (long long)per_cu * cus;
    std::lock_guard<std::mutex> g(mu);
    if (cache.size() < 256) cache.push_back(Entry{dev, (const void*)kern, lds, *out});
    return hipSuccess;
}

struct FusedLaunch {
    const FusedArgs& a;
    hipStream_t s;
    template <int EPL, int LPG>
    hipError_t run() {
        const auto kern = fused_decode_kernel<EPL, LPG>;
        const size_t lds = fused_lds_bytes(a.r.T, a.r.E, a.r.k, a.R);
        long long fits = 0;
        const hipError_t err = resident_blocks(kern, lds, &fits);
        if (err != hipSuccess) return err;
        // at most half of what the GPU can hold at once: every block must be
        // resident for the barrier, with margin for anything else running
        const long long resident = fits / 2;
        if (resident < 1) return hipErrorInvalidConfiguration;
        const long long items = (long long)a.r.T * a.units;
        long long want = (items + kFusedWaves - 1) / kFusedWaves;
        want = want < 1 ? 1 : want;
        const unsigned blocks = (unsigned)(want < resident ? want : resident);
        hipLaunchKernelGGL(kern, dim3(blocks), dim3(kFusedThreads), lds, s, a);
        return hipGetLastError();
    }
};

}  // namespace

size_t fused_decode_lds_bytes(int T, int E, int k, int R) { return fused_lds_bytes(T, E, k, R); }

hipError_t launch_fused_decode(const float* logits, const uint16_t* x, int32_t* idx, float* w, int32_t* cnt_e,
                               int32_t* cnt_r, int32_t* off_e, int32_t* off_r, int32_t* pos, int32_t* recv_src,
                               int32_t* flags, void* recv_x, void* recv_scales, uint32_t* barrier, int T, int E,
                               int G, int g, int k, int n, int score_fn, int renorm, int R, int C, int A, int N,
                               int H, int dtype, hipStream_t stream) {
    FusedArgs a{};
    a.r = RouteArgs{logits, idx, w, T, E, G, g, k, n, score_fn, renorm};
    a.cnt_e = cnt_e;
    a.cnt_r = cnt_r;
    a.off_e = off_e;
    a.off_r = off_r;
    a.pos = pos;
    a.recv_src = recv_src;
    a.flags = flags;
    a.x = x;
    a.recv_x = recv_x;
    a.recv_scales = recv_scales;
    a.bar = barrier;
    a.R = R;
    a.C = C;
    a.A = A;
    a.N = N;
    a.H = H;
    a.S = H / 128;
    a.units = (H + kUnitChannels - 1) / kUnitChannels;
    a.dtype = dtype;
    a.nch = (T + 63) / 64;
    FusedLaunch f{a, stream};
    return with_route_shape(E, G, f);
}

}  // namespace cgl
