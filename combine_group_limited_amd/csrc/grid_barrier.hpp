// grid_barrier.hpp -- a grid-wide barrier for launches whose blocks are all
// resident (the caller sizes the grid from the occupancy API), shared by the
// one-launch decode path (fused.hip) and the one-launch MoE layer (layer.hip).
// The arrival and wait protocol, its workspace words and what a give-up
// leaves behind are in barrier_protocol.hpp.
#pragma once
#include "barrier_protocol.hpp"
#include "moe_device.hpp"

namespace cgl {
namespace {

constexpr uint32_t kSpinLimit = 1u << 22;  // barrier polls before a block gives up (seconds)

struct AgentAtomics {
    __device__ uint32_t load(uint32_t* p) const {
        return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __device__ void store(uint32_t* p, uint32_t v) const {
        __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __device__ uint32_t fetch_add(uint32_t* p, uint32_t v) const {
        return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __device__ void pause() const { __builtin_amdgcn_s_sleep(2); }
};

// Grid-wide barrier (a two-level tree of arrival counters, so a single
// counter's queue of atomics is avoided: one counter costs 10 us at 448
// blocks, the tree 3 us).  Returns true in every thread of a block that got
// through, false in every thread of a block that stopped waiting or found the
// workspace refused (see barrier_protocol.hpp); the caller then returns.
// Counters and flags only order control: with FENCE = false the data they
// guard must travel by device-scope atomics; with FENCE = true the block's
// ordinary stores are released at agent scope before it arrives and acquired
// after the barrier, so plain loads after the barrier see plain stores made
// before it by blocks on any XCD.  One wave does both for its block: once
// every wave has waited for its own stores and the block has met, those
// stores sit in the XCD's L2, which the release writes back whole; after the
// barrier the same wave's acquire invalidates the CU's L1 and the XCD's L2,
// and only then does the closing block barrier let the other waves load.  (A
// release and an acquire in every wave cost four whole-L2 write-backs and
// invalidations per block.)
// `refused` is read in thread 0 only: barrier_gave_up() as that thread read
// it at the start of the launch, for the launch's first barrier; false for
// the others.
template <bool FENCE>
__device__ bool grid_barrier(uint32_t* ws, bool refused) {
    __shared__ int passed;
    __builtin_amdgcn_s_waitcnt(kWaitStores);  // this wave's stores have completed
    __syncthreads();
    if (threadIdx.x == 0) {
        if (FENCE) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        const bool ok =
            barrier_arrive_wait(AgentAtomics{}, ws, (int)blockIdx.x, (int)gridDim.x, kSpinLimit, refused);
        if (FENCE) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        passed = ok ? 1 : 0;
    }
    __syncthreads();
    return passed != 0;
}

// Word 2 of the barrier workspace: nonzero once any block of this or an
// earlier launch on the workspace stopped waiting.
__device__ __forceinline__ bool barrier_gave_up(uint32_t* ws) { return barrier_refused(AgentAtomics{}, ws); }

}  // namespace
}  // namespace cgl
