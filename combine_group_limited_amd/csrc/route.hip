// route.hip -- group-limited top-k gating: one wave64 per token, four tokens
// per 256-thread block.  The per-token algorithm is route_token in
// route_impl.hpp; see there for the pages it follows and how it works.
#include "moe_internal.hpp"
#include "route_impl.hpp"

namespace cgl {
namespace {

constexpr int kTokensPerBlock = 4;  // one wave per token, 256 threads

template <int EPL, int LPG>
__global__ __launch_bounds__(256) void route_kernel(RouteArgs a) {
    const int t = blockIdx.x * kTokensPerBlock + wave_in_block();
    if (t >= a.T) return;  // wave-uniform
    route_token<EPL, LPG>(a, t);
}

// ---------------------------------------------------------------------------
// Row routing for large batches: four tokens per wave, one DPP row of 16 lanes
// per token, EPL = E/16 experts per lane (lane r of a row holds experts
// r*EPL .. r*EPL+EPL-1), groups of LPG = 16/G lanes.  Every reduction is a
// DPP step inside the row, so a wave routes four tokens with about the
// instructions one token costs the one-token-per-wave kernel; large batches
// are bound by that instruction count (four such waves per SIMD at 4096
// tokens), small ones by latency, which the one-token kernel keeps lower.
// Same selection order and arithmetic as route_token: scores by the fixed
// sigmoid recipe, order keys with -0 folded onto +0, group score = the sum of
// the group's n largest scores in descending order, groups ranked by (score,
// lower index), experts by (score, lower index), weights as route_token.
constexpr int kRowTokensPerBlock = 16;   // 256 threads
constexpr int kRowMinTokens = 2048;      // below this the one-token kernel is faster

// DPP row_ror:N (rotate right by N lanes inside each row of 16)
template <int N>
__device__ __forceinline__ uint32_t row_ror(uint32_t v) {
    return dpp32<0x120 + N>(v);
}

// The first of a lane's keys equal to m removed (set to 0) when `mine`.
template <int EPL>
__device__ __forceinline__ void drop_first_equal(uint32_t (&v)[EPL], uint32_t m, bool mine) {
    bool done = !mine;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const bool hit = !done && v[i] == m;
        v[i] = hit ? 0u : v[i];
        done = done || hit;
    }
}

template <int EPL, int LPG>
__global__ __launch_bounds__(256) void route_rows_kernel(RouteArgs a) {
    const int lane = threadIdx.x & 63, r = lane & 15;
    const int t = blockIdx.x * kRowTokensPerBlock + (int)(threadIdx.x >> 4);
    const int E = a.E;
    const int tc = t < a.T ? t : a.T - 1;  // rows past the end compute on the last token and store nothing
    const float* src = a.logits + (size_t)tc * E + r * EPL;

    float l[EPL];
    if constexpr (EPL % 4 == 0) {
#pragma unroll
        for (int i = 0; i < EPL; i += 4) {
            const float4 q = *(const float4*)(src + i);
            l[i] = q.x; l[i + 1] = q.y; l[i + 2] = q.z; l[i + 3] = q.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < EPL; ++i) l[i] = src[i];
    }
    uint32_t key[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) key[i] = float_order(a.score_fn == 0 ? sigmoid_fixed(l[i]) : l[i]);

    // ---- group limit (G = 16 / LPG groups of LPG lanes) --------------------
    if constexpr (LPG < 16) {
        constexpr int G = 16 / LPG;
        uint32_t v[EPL];
#pragma unroll
        for (int i = 0; i < EPL; ++i) v[i] = key[i];
        float gs = 0.0f;
        for (int rr = 0; rr < a.n; ++rr) {
            const uint32_t lm = lane_max<EPL>(v);
            const uint32_t m = seg_maxu<LPG>(lm);
            const float sv = order_float(m);
            gs = (rr == 0) ? sv : gs + sv;
            const uint32_t owner = seg_minu<LPG>(lm == m ? (uint32_t)r : 16u);
            drop_first_equal<EPL>(v, m, owner == (uint32_t)r);
        }
        // rank of this lane's group among the G groups of the row
        const uint32_t gk = float_order(gs);
        const uint32_t gid = (uint32_t)(r / LPG);
        uint32_t ok = gk, og = gid;
        int rank = 0;
#pragma unroll
        for (int q = 1; q < G; ++q) {
            ok = row_ror<LPG>(ok);
            og = row_ror<LPG>(og);
            rank += (ok > gk || (ok == gk && og < gid)) ? 1 : 0;
        }
        const bool keep = rank < a.g;
#pragma unroll
        for (int i = 0; i < EPL; ++i) key[i] = keep ? key[i] : 0u;
    }

    // ---- top-k experts; lane j of the row keeps slot j ------------------------
    int my_e = 0;
    float my_v = 0.0f, my_u = 0.0f, den = 0.0f, l0 = 0.0f;
    for (int j = 0; j < a.k; ++j) {
        const uint32_t lm = lane_max<EPL>(key);
        const uint32_t m = seg_maxu<16>(lm);
        const uint32_t c = first_equal<EPL>(key, m);
        const uint32_t e = seg_minu<16>(lm == m ? (uint32_t)(r * EPL) + c : 0xFFFFu);
#pragma unroll
        for (int i = 0; i < EPL; ++i) key[i] = ((uint32_t)(r * EPL + i) == e) ? 0u : key[i];
        const float v = order_float(m);
        if (a.score_fn == 0) {
            den = (j == 0) ? v : den + v;
        } else {
            if (j == 0) l0 = v;
            const float u = exp_fixed(v - l0);
            den = (j == 0) ? u : den + u;
            my_u = (r == j) ? u : my_u;
        }
        my_e = (r == j) ? (int)e : my_e;
        my_v = (r == j) ? v : my_v;
    }

    float wgt;
    if (a.score_fn == 0) {
        wgt = a.renorm ? ((den > 0.0f) ? my_v / den : 0.0f) : my_v;
    } else if (a.renorm) {
        wgt = my_u / den;
    } else {
        // full softmax probability: the row's largest logit, then the sum of
        // exp(l - max) over all E experts in expert order, a sequential chain
        // passed from lane to lane along the row
        uint32_t mo = 0;
#pragma unroll
        for (int i = 0; i < EPL; ++i) mo = max(mo, float_order(l[i]));
        const float lmax = order_float(seg_maxu<16>(mo));
        float u[EPL];
#pragma unroll
        for (int i = 0; i < EPL; ++i) u[i] = exp_fixed(l[i] - lmax);
        float run = 0.0f, sum = 0.0f;
        for (int rr = 0; rr < 16; ++rr) {
            float s_ = run;
#pragma unroll
            for (int i = 0; i < EPL; ++i) s_ = s_ + u[i];
            sum = s_;  // lane 15's value after its own step is the total
            const float nxt = __uint_as_float(dpp32<0x111>(__float_as_uint(s_)));  // row_shr:1
            run = (r == rr + 1) ? nxt : run;
        }
        const float total = __shfl(sum, (lane & ~15) + 15, 64);
        wgt = exp_fixed(my_v - lmax) / total;
    }
    if (t < a.T && r < a.k) {
        a.idx[(size_t)t * a.k + r] = my_e;
        a.w[(size_t)t * a.k + r] = wgt;
    }
}

struct RowLaunch {
    const RouteArgs& a;
    hipStream_t s;
    template <int EPL, int LPG>
    hipError_t run() {
        const int blocks = (a.T + kRowTokensPerBlock - 1) / kRowTokensPerBlock;
        hipLaunchKernelGGL((route_rows_kernel<EPL, LPG>), dim3(blocks), dim3(256), 0, s, a);
        return hipGetLastError();
    }
};

// The row kernel serves E in {16, 32, 64, 128, 256} with G dividing 16 and
// k <= 16 (slot j is kept by lane j of the row), logits 16-byte aligned.
template <class F>
hipError_t with_row_shape(int E, int G, F& f) {
    switch (G) {
#define CGL_ROW_G(GG)                                          \
    case GG:                                                   \
        switch (E) {                                           \
            case 16: return f.template run<1, 16 / GG>();      \
            case 32: return f.template run<2, 16 / GG>();      \
            case 64: return f.template run<4, 16 / GG>();      \
            case 128: return f.template run<8, 16 / GG>();     \
            case 256: return f.template run<16, 16 / GG>();    \
        }                                                      \
        break;
        CGL_ROW_G(1)
        CGL_ROW_G(2)
        CGL_ROW_G(4)
        CGL_ROW_G(8)
        CGL_ROW_G(16)
#undef CGL_ROW_G
    }
    return hipErrorNotSupported;
}

bool row_shape_ok(const float* logits, int T, int E, int G, int k) {
    return T >= kRowMinTokens && (E == 16 || E == 32 || E == 64 || E == 128 || E == 256) && 16 % G == 0 &&
           k <= 16 && ((uintptr_t)logits & 15) == 0;
}

struct RouteLaunch {
    const RouteArgs& a;
    hipStream_t s;
    template <int EPL, int LPG>
    hipError_t run() {
        const int blocks = (a.T + kTokensPerBlock - 1) / kTokensPerBlock;
        hipLaunchKernelGGL((route_kernel<EPL, LPG>), dim3(blocks), dim3(256), 0, s, a);
        return hipGetLastError();
    }
};

}  // namespace

hipError_t launch_route(const float* logits, int32_t* idx, float* w, int T, int E, int G, int g, int k, int n,
                        int score_fn, int renorm, hipStream_t stream) {
    RouteArgs a{logits, idx, w, T, E, G, g, k, n, score_fn, renorm};
    if (row_shape_ok(logits, T, E, G, k)) {
        RowLaunch f{a, stream};
        return with_row_shape(E, G, f);
    }
    RouteLaunch f{a, stream};
    return with_route_shape(E, G, f);
}

}  // namespace cgl
