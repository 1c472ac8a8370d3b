// route_impl.hpp -- group-limited top-k gating of one token by one wave64.
//
// Follows "Efficient and Portable Mixture-of-Experts Communication"
// (Perplexity), section "Introduction" (router scores -> top-K experts ->
// weighted sum), and "DeepSeek, DeepEP open-sourced" (GeekNews 19421), topic
// body and "Performance > Normal kernels" (group-limited gating: top-4 groups,
// then top-8 experts).
//
// Lane l holds experts l*EPL .. l*EPL+EPL-1 (EPL = ceil(E/64), at most 8), so
// a 256-expert row is one coalesced 1 KiB read.  Scores are mapped once to
// order-preserving 32-bit keys (-0 folded onto +0; 0 marks a removed or
// excluded expert), so every max and min below is an integer op that fuses
// with its DPP operand.  Each selection round is a wave max (DPP inside rows
// of 16, the four row results on the scalar unit) followed by a ballot that
// picks, among the lanes holding that maximum, the lowest expert index -- the
// order "higher score first, equal scores by lower index", the same order the
// host uses.  With contiguous groups whose size is a multiple of EPL, a group
// occupies an aligned power-of-two run of lanes and all group scores come out
// of segmented DPP reductions; other shapes reduce once per group.  Group
// selection ranks each group against all others in one pass.
//
// Included by the stand-alone routing kernel and by the fused decode kernel.
#pragma once

#include "moe_device.hpp"

namespace cgl {
namespace {

struct RouteArgs {
    const float* logits;
    int32_t* idx;
    float* w;
    int T, E, G, g, k, n, score_fn, renorm;
};

// Index (0..EPL-1) of the first of a lane's keys equal to m, or EPL.
template <int EPL>
__device__ __forceinline__ uint32_t first_equal(const uint32_t (&v)[EPL], uint32_t m) {
    uint32_t c = EPL;
#pragma unroll
    for (int i = EPL - 1; i >= 0; --i) c = (v[i] == m) ? (uint32_t)i : c;
    return c;
}

// Removes expert e (sets its key to 0) if this lane holds it; branch-free.
template <int EPL>
__device__ __forceinline__ void drop(uint32_t (&v)[EPL], uint32_t e, int lane) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) v[i] = (e == (uint32_t)(lane * EPL + i)) ? 0u : v[i];
}

template <int EPL>
__device__ __forceinline__ uint32_t lane_max(const uint32_t (&v)[EPL]) {
    uint32_t m = v[0];
#pragma unroll
    for (int i = 1; i < EPL; ++i) m = max(m, v[i]);
    return m;
}

// A lane's keys as a list in descending order, ties by ascending index: an
// adjacent-compare (insertion) network that swaps only strict inversions is
// stable, so equal keys keep their index order.  idx holds the local index.
template <int EPL>
__device__ __forceinline__ void sort_lane(uint32_t (&k)[EPL], uint32_t (&idx)[EPL]) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) idx[i] = (uint32_t)i;
#pragma unroll
    for (int i = 1; i < EPL; ++i)
#pragma unroll
        for (int j = i; j > 0; --j) {
            const bool sw = k[j] > k[j - 1];
            const uint32_t a = k[j - 1], b = k[j], ia = idx[j - 1], ib = idx[j];
            k[j - 1] = sw ? b : a;
            k[j] = sw ? a : b;
            idx[j - 1] = sw ? ib : ia;
            idx[j] = sw ? ia : ib;
        }
}

// Pops the head of a lane's sorted list when adv is set (shift left, 0 in).
template <int EPL>
__device__ __forceinline__ void pop_head(uint32_t (&k)[EPL], uint32_t (&idx)[EPL], bool adv) {
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        k[i] = adv ? ((i + 1 < EPL) ? k[i + 1] : 0u) : k[i];
        idx[i] = adv ? ((i + 1 < EPL) ? idx[i + 1] : 0u) : idx[i];
    }
}

// Group score (sum of the n largest scores) of every group, groups aligned to
// LPG-lane segments: every lane of segment gamma receives group gamma's score.
template <int EPL, int LPG>
__device__ __forceinline__ float group_scores_segmented(const uint32_t (&key)[EPL], int n, int lane) {
    uint32_t v[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) v[i] = key[i];
    float sum = 0.0f;
    for (int r = 0; r < n; ++r) {
        const uint32_t m = seg_maxu<LPG>(lane_max<EPL>(v));
        const float sv = order_float(m);
        sum = (r == 0) ? sv : sum + sv;
        // lowest expert of the segment holding the maximum
        const uint32_t c = first_equal<EPL>(v, m);
        const uint32_t e = (c < EPL) ? (uint32_t)lane * EPL + c : 0xFFFFFFFFu;
        drop<EPL>(v, seg_minu<LPG>(e), lane);
    }
    return sum;
}

// Same, from sorted lane lists: each round compares list heads only; the
// lowest lane holding the maximum pops its head.
template <int EPL, int LPG>
__device__ __forceinline__ float group_scores_sorted(const uint32_t (&sk)[EPL], const uint32_t (&si)[EPL], int n,
                                                     int lane) {
    uint32_t k2[EPL], i2[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        k2[i] = sk[i];
        i2[i] = si[i];
    }
    float sum = 0.0f;
    for (int r = 0; r < n; ++r) {
        const uint32_t m = seg_maxu<LPG>(k2[0]);
        const float sv = order_float(m);
        sum = (r == 0) ? sv : sum + sv;
        const uint32_t winner = seg_minu<LPG>((k2[0] == m) ? (uint32_t)lane : 0xFFFFFFFFu);
        pop_head<EPL>(k2, i2, winner == (uint32_t)lane);
    }
    return sum;
}

// Group scores for any contiguous grouping: G * n full-wave rounds.  Returns
// in lane gamma (< G) the score of group gamma.
template <int EPL>
__device__ __forceinline__ float group_scores_general(const uint32_t (&key)[EPL], int E, int G, int n, int lane) {
    const int Eg = E / G;
    float mine = 0.0f;
    for (int gr = 0; gr < G; ++gr) {
        uint32_t v[EPL];
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const int e = lane * EPL + i;
            v[i] = (e < E && e / Eg == gr) ? key[i] : 0u;
        }
        float sum = 0.0f;
        for (int r = 0; r < n; ++r) {
            const uint32_t m = wave_maxu(lane_max<EPL>(v));
            const float sv = order_float(m);
            sum = (r == 0) ? sv : sum + sv;
            const uint32_t c = first_equal<EPL>(v, m);
            const uint64_t bal = __ballot(c < EPL);
            const int src = __builtin_ctzll(bal);
            const int ci = __builtin_amdgcn_readlane((int)c, src);
            drop<EPL>(v, (uint32_t)(src * EPL + ci), lane);
        }
        if (lane == gr) mine = sum;
    }
    return mine;
}

// Routes token t: writes idx[t, 0..k-1] and w[t, 0..k-1] (slot j from lane
// j).  LPG > 0: groups aligned to LPG-lane runs; LPG == 0: any contiguous
// grouping (general path); LPG < 0: no groups.  Sorted lane lists are used
// whenever a lane's experts all share one group (LPG != 0).  Called by a
// whole wave with a wave-uniform t < T; uses no LDS and no block barrier.
// DEVICE_IDX: write idx with device-scope atomic stores, so that other blocks
// of the same launch can read it with device-scope atomic loads.
template <int EPL, int LPG, bool DEVICE_IDX = false>
__device__ __forceinline__ void route_token(const RouteArgs& a, const int t) {
    constexpr bool kSorted = LPG != 0;
    const int lane = threadIdx.x & 63;
    const int E = a.E;
    const float* row = a.logits + (size_t)t * E;

    // all EPL loads are issued before any is used (clamped index, no branch)
    float l[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) l[i] = row[min(lane * EPL + i, E - 1)];
    uint32_t key[EPL], kidx[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane * EPL + i;
        if (e >= E) l[i] = 0.0f;
        const float sc = (a.score_fn == 0) ? sigmoid_fixed(l[i]) : l[i];
        key[i] = (e < E) ? float_order(sc) : 0u;
    }
    if constexpr (kSorted) sort_lane<EPL>(key, kidx);

    // ---- group limit: keep the a.g best groups ----------------------------
    if (LPG >= 0 && a.G > 1) {
        const int Eg = E / a.G;
        float gs;      // in lane gamma (< G): score of group gamma
        if constexpr (LPG > 0) {
            const float seg = group_scores_sorted<EPL, (LPG > 0 ? LPG : 1)>(key, kidx, a.n, lane);
            gs = __int_as_float(__builtin_amdgcn_ds_bpermute(((lane * LPG) & 63) << 2, __float_as_int(seg)));
        } else {
            gs = group_scores_general<EPL>(key, E, a.G, a.n, lane);
        }
        // rank of each group among all groups (higher score first, then lower
        // index); a group is kept when its rank is below topk_group
        const uint32_t gk = float_order(gs);
        int rank = 0;
        for (int q = 0; q < a.G; ++q) {
            const uint32_t o = (uint32_t)__builtin_amdgcn_readlane((int)gk, q);
            rank += (o > gk || (o == gk && q < lane)) ? 1 : 0;
        }
        const uint64_t kept = __ballot(lane < a.G && rank < a.g);
        if constexpr (kSorted) {
            // all of a lane's experts are in one group: keep or clear the list
            const bool keep = lane * EPL < E && ((kept >> ((lane * EPL) / Eg)) & 1ull);
#pragma unroll
            for (int i = 0; i < EPL; ++i) key[i] = keep ? key[i] : 0u;
        } else {
#pragma unroll
            for (int i = 0; i < EPL; ++i) {
                const int e = lane * EPL + i;
                key[i] = (e < E && ((kept >> (e / Eg)) & 1ull)) ? key[i] : 0u;
            }
        }
    }

    // ---- top-k experts; lane j keeps slot j --------------------------------
    int my_e = 0;
    float my_v = 0.0f;   // score (sigmoid) or logit (softmax) of slot j
    float my_u = 0.0f;   // softmax numerator exp(l_j - l_0)
    float den = 0.0f;
    float l0 = 0.0f;
    for (int j = 0; j < a.k; ++j) {
        int e;
        uint32_t m;
        if constexpr (kSorted) {
            m = wave_maxu(key[0]);
            const uint64_t bal = __ballot(key[0] == m);
            const int src = __builtin_ctzll(bal);
            e = src * EPL + __builtin_amdgcn_readlane((int)kidx[0], src);
            pop_head<EPL>(key, kidx, lane == src);
        } else {
            m = wave_maxu(lane_max<EPL>(key));
            const uint32_t c = first_equal<EPL>(key, m);
            const uint64_t bal = __ballot(c < EPL);
            const int src = __builtin_ctzll(bal);
            e = src * EPL + __builtin_amdgcn_readlane((int)c, src);
            drop<EPL>(key, (uint32_t)e, lane);
        }
        const float v = order_float(m);
        if (a.score_fn == 0) {
            den = (j == 0) ? v : den + v;
        } else {
            if (j == 0) l0 = v;
            const float u = exp_fixed(v - l0);
            den = (j == 0) ? u : den + u;
            my_u = (lane == j) ? u : my_u;
        }
        my_e = (lane == j) ? e : my_e;
        my_v = (lane == j) ? v : my_v;
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
        const float lmax = order_float(wave_maxu(mo));
        float sum = 0.0f;
        for (int src = 0; src < 64; ++src) {
#pragma unroll
            for (int i = 0; i < EPL; ++i) {
                const int e = src * EPL + i;
                if (e < E) {
                    const float le = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(l[i]), src));
                    const float u = exp_fixed(le - lmax);
                    sum = (e == 0) ? u : sum + u;
                }
            }
        }
        wgt = exp_fixed(my_v - lmax) / sum;
    }
    if (lane < a.k) {
        if constexpr (DEVICE_IDX)
            __hip_atomic_store(&a.idx[(size_t)t * a.k + lane], my_e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
            a.idx[(size_t)t * a.k + lane] = my_e;
        a.w[(size_t)t * a.k + lane] = wgt;
    }
}

// Calls f.template run<EPL, LPG>() with the compile-time shape that serves
// (E, G): EPL = experts per lane, LPG = lanes per group (see route_token).
template <int EPL, class F>
hipError_t with_lpg(int E, int G, F& f) {
    const int Eg = E / G;
    if (G == 1) return f.template run<EPL, -1>();
    int lpg = 0;  // 0: general path
    if (Eg % EPL == 0) {
        const int l = Eg / EPL;
        if ((l & (l - 1)) == 0 && l <= 64) lpg = l;
    }
    switch (lpg) {
        case 1: return f.template run<EPL, 1>();
        case 2: return f.template run<EPL, 2>();
        case 4: return f.template run<EPL, 4>();
        case 8: return f.template run<EPL, 8>();
        case 16: return f.template run<EPL, 16>();
        case 32: return f.template run<EPL, 32>();
        case 64: return f.template run<EPL, 64>();
        default: return f.template run<EPL, 0>();
    }
}

template <class F>
hipError_t with_route_shape(int E, int G, F& f) {
    const int epl = (E + 63) / 64;
    if (epl <= 1) return with_lpg<1>(E, G, f);
    if (epl <= 2) return with_lpg<2>(E, G, f);
    if (epl <= 4) return with_lpg<4>(E, G, f);
    return with_lpg<8>(E, G, f);
}

}  // namespace
}  // namespace cgl
