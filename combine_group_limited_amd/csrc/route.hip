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
    RouteLaunch f{a, stream};
    return with_route_shape(E, G, f);
}

}  // namespace cgl
