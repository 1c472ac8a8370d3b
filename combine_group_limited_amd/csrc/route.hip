// route.hip -- group-limited top-k gating, one wave64 per token.
//
// Follows "Efficient and Portable Mixture-of-Experts Communication"
// (Perplexity), section "Introduction" (router scores -> top-K experts ->
// weighted sum), and "DeepSeek, DeepEP open-sourced" (GeekNews 19421), topic
// body and "Performance > Normal kernels" (group-limited gating: top-4 groups,
// then top-8 experts).
//
// Lane l holds experts l*EPL .. l*EPL+EPL-1 (EPL = ceil(E/64), at most 8), so
// a 256-expert row is one coalesced 1 KiB read.  Every selection is a max over
// 64-bit keys (score order, then lower index), which makes the choice unique
// and equal to the host's.  With contiguous groups whose size is a multiple of
// EPL, a group occupies an aligned power-of-two run of lanes and all group
// scores come out of one segmented DPP reduction per round; other shapes fall
// back to one full-wave reduction per group and round.
#include "moe_device.hpp"
#include "moe_internal.hpp"

namespace cgl {
namespace {

struct RouteArgs {
    const float* logits;
    int32_t* idx;
    float* w;
    int T, E, G, g, k, n, score_fn, renorm;
};

constexpr int kTokensPerBlock = 4;  // one wave per token, 256 threads

// Group scores with groups aligned to LPG-lane segments.  Returns, in lane
// gamma (< G), the score of group gamma.
template <int EPL, int LPG>
__device__ __forceinline__ float group_scores_segmented(const uint64_t (&key)[EPL], int n, int lane) {
    uint32_t taken = 0;
    float sum = 0.0f;
    for (int r = 0; r < n; ++r) {
        uint64_t best = 0;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if (!(taken & (1u << i))) best = umax64(best, key[i]);
        best = seg_max64<LPG>(best);
        const float v = key_value(best);
        sum = (r == 0) ? v : sum + v;
        const uint32_t e = key_index(best);  // 0xFFFFFFFF when the segment is empty
        if (e / EPL == (uint32_t)lane) taken |= 1u << (e % EPL);
    }
    // segment gamma starts at lane gamma*LPG; move its sum to lane gamma
    const int src = (lane * LPG) & 63;
    return __uint_as_float(bperm32(__float_as_uint(sum), src));
}

// General group scores: G * n full-wave reductions.
template <int EPL>
__device__ __forceinline__ float group_scores_general(const uint64_t (&key)[EPL], int E, int G, int n,
                                                      int lane) {
    const int Eg = E / G;
    float mine = 0.0f;
    for (int gr = 0; gr < G; ++gr) {
        uint32_t taken = 0;
        float sum = 0.0f;
        for (int r = 0; r < n; ++r) {
            uint64_t best = 0;
#pragma unroll
            for (int i = 0; i < EPL; ++i) {
                const int e = lane * EPL + i;
                if (e < E && e / Eg == gr && !(taken & (1u << i))) best = umax64(best, key[i]);
            }
            best = wave_max64(best);
            const float v = key_value(best);
            sum = (r == 0) ? v : sum + v;
            const uint32_t e = key_index(best);
            if (e / EPL == (uint32_t)lane) taken |= 1u << (e % EPL);
        }
        if (lane == gr) mine = sum;
    }
    return mine;
}

template <int EPL, int LPG>
__global__ __launch_bounds__(256) void route_kernel(RouteArgs a) {
    const int lane = threadIdx.x & 63;
    const int t = blockIdx.x * kTokensPerBlock + (threadIdx.x >> 6);
    if (t >= a.T) return;  // wave-uniform
    const int E = a.E;
    const float* row = a.logits + (size_t)t * E;

    float l[EPL];
    uint64_t key[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane * EPL + i;
        l[i] = (e < E) ? row[e] : 0.0f;
        const float s = (a.score_fn == 0) ? sigmoid_fixed(l[i]) : l[i];
        key[i] = (e < E) ? make_key(s, (uint32_t)e) : 0ull;
    }

    // ---- group limit: keep the a.g best groups --------------------------
    if (a.G > 1) {
        float gs;
        if constexpr (LPG > 0)
            gs = group_scores_segmented<EPL, LPG>(key, a.n, lane);
        else
            gs = group_scores_general<EPL>(key, E, a.G, a.n, lane);
        uint64_t gkey = (lane < a.G) ? make_key(gs, (uint32_t)lane) : 0ull;
        uint64_t kept = 0;  // bit gamma set: group gamma kept
        for (int r = 0; r < a.g; ++r) {
            const uint64_t best = wave_max64(gkey);
            const int gr = (int)key_index(best);
            kept |= 1ull << gr;
            if (lane == gr) gkey = 0;
        }
        const int Eg = E / a.G;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = lane * EPL + i;
            if (e < E && !((kept >> (e / Eg)) & 1ull)) key[i] = 0;
        }
    }

    // ---- top-k experts; lane j keeps slot j -------------------------------
    int my_e = 0;
    float my_v = 0.0f;   // score (sigmoid) or logit (softmax) of slot j
    float my_u = 0.0f;   // softmax numerator exp(l_j - l_0)
    float den = 0.0f;
    float l0 = 0.0f;
    for (int j = 0; j < a.k; ++j) {
        uint64_t best = 0;
#pragma unroll
        for (int i = 0; i < EPL; ++i) best = umax64(best, key[i]);
        best = wave_max64(best);
        const uint32_t e = key_index(best);
        const float v = key_value(best);
        if (e / EPL == (uint32_t)lane) {
#pragma unroll
            for (int i = 0; i < EPL; ++i)
                if ((uint32_t)i == e % EPL) key[i] = 0;
        }
        if (a.score_fn == 0) {
            den = (j == 0) ? v : den + v;
        } else {
            if (j == 0) l0 = v;
            const float u = exp_fixed(v - l0);
            den = (j == 0) ? u : den + u;
            if (lane == j) my_u = u;
        }
        if (lane == j) {
            my_e = (int)e;
            my_v = v;
        }
    }

    float wgt;
    if (a.score_fn == 0) {
        if (a.renorm)
            wgt = (den > 0.0f) ? my_v / den : 0.0f;
        else
            wgt = my_v;
    } else if (a.renorm) {
        wgt = my_u / den;
    } else {
        // full softmax probability: max and sum over all E logits, the sum
        // taken in expert order (a sequential chain, as the host does)
        uint32_t mo = 0;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if (lane * EPL + i < E) mo = max(mo, float_order(l[i]));
        uint64_t mk = wave_max64((uint64_t)mo << 32);
        const float lmax = order_float((uint32_t)(mk >> 32));
        float sum = 0.0f;
        for (int src = 0; src < 64; ++src) {
#pragma unroll
            for (int i = 0; i < EPL; ++i) {
                const int e = src * EPL + i;
                if (e < E) {
                    const float le = __uint_as_float(
                        (uint32_t)__builtin_amdgcn_readlane((int)__float_as_uint(l[i]), src));
                    const float u = exp_fixed(le - lmax);
                    sum = (e == 0) ? u : sum + u;
                }
            }
        }
        wgt = exp_fixed(my_v - lmax) / sum;
    }
    if (lane < a.k) {
        a.idx[(size_t)t * a.k + lane] = my_e;
        a.w[(size_t)t * a.k + lane] = wgt;
    }
}

template <int EPL, int LPG>
hipError_t launch(const RouteArgs& a, hipStream_t s) {
    const int blocks = (a.T + kTokensPerBlock - 1) / kTokensPerBlock;
    hipLaunchKernelGGL((route_kernel<EPL, LPG>), dim3(blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

template <int EPL>
hipError_t pick_lpg(const RouteArgs& a, hipStream_t s) {
    const int Eg = a.E / a.G;
    int lpg = 0;  // 0: general path
    if (a.G > 1 && Eg % EPL == 0 && a.G <= 64) {
        const int l = Eg / EPL;
        if ((l & (l - 1)) == 0 && l <= 64) lpg = l;
    }
    switch (lpg) {
        case 1: return launch<EPL, 1>(a, s);
        case 2: return launch<EPL, 2>(a, s);
        case 4: return launch<EPL, 4>(a, s);
        case 8: return launch<EPL, 8>(a, s);
        case 16: return launch<EPL, 16>(a, s);
        case 32: return launch<EPL, 32>(a, s);
        case 64: return launch<EPL, 64>(a, s);
        default: return launch<EPL, 0>(a, s);
    }
}

}  // namespace

hipError_t launch_route(const float* logits, int32_t* idx, float* w, int T, int E, int G, int g,
                        int k, int n, int score_fn, int renorm, hipStream_t stream) {
    RouteArgs a{logits, idx, w, T, E, G, g, k, n, score_fn, renorm};
    const int epl = (E + 63) / 64;
    if (epl <= 1) return pick_lpg<1>(a, stream);
    if (epl <= 2) return pick_lpg<2>(a, stream);
    if (epl <= 4) return pick_lpg<4>(a, stream);
    return pick_lpg<8>(a, stream);
}

}  // namespace cgl
