// grid_barrier.hpp -- a grid-wide barrier for launches whose blocks are all
// resident (the caller sizes the grid from the occupancy API), shared by the
// one-launch decode path (fused.hip) and the one-launch MoE layer (layer.hip).
#pragma once
#include "moe_device.hpp"

namespace cgl {
namespace {

constexpr int kSpinLimit = 1 << 22;  // barrier polls before a block gives up (seconds)

// Grid-wide barrier, a two-level tree of arrival counters: block b arrives
// at the counter of group b % 8 (each counter and flag on its own 256-byte
// line of the workspace), the last block of a group at the top counter, and
// the last block overall resets the counters and publishes the next
// generation to every group's flag, which the group's other blocks poll.  So
// no more than ceil(blocks / 8) atomics queue on one address (a single
// counter costs 10 us at 448 blocks, the tree 3 us).  Polls are bounded; a
// block that gives up (only possible if the grid is not resident) counts
// itself in word 2 and returns false in all its threads.  Counters and flags
// only order control: with FENCE = false the data they guard must travel by
// device-scope atomics; with FENCE = true the block's ordinary stores are
// released at agent scope before it arrives and acquired after the barrier,
// so plain loads after the barrier see plain stores made before it by blocks
// on any XCD.  One wave does both for its block: once every wave has waited
// for its own stores and the block has met, those stores sit in the XCD's L2,
// which the release writes back whole; after the barrier the same wave's
// acquire invalidates the CU's L1 and the XCD's L2, and only then does the
// closing block barrier let the other waves load.  (A release and an acquire
// in every wave cost four whole-L2 write-backs and invalidations per block.)
constexpr int kGroups = 8;
constexpr int kGroupStride = 64;  // 32-bit words: 256 bytes per group

template <bool FENCE>
__device__ bool grid_barrier(uint32_t* ws) {
    __shared__ int gave_up;
    __builtin_amdgcn_s_waitcnt(kWaitStores);  // this wave's stores have completed
    __syncthreads();
    if (threadIdx.x == 0) {
        if (FENCE) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        const int nb = gridDim.x, c = blockIdx.x % kGroups;
        const int in_group = (nb - c + kGroups - 1) / kGroups;
        const int groups = nb < kGroups ? nb : kGroups;
        uint32_t* counter = ws + kGroupStride * (1 + c);
        uint32_t* flag = counter + 1;
        const uint32_t gen = __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        bool last = false;
        if (__hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
            (uint32_t)(in_group - 1)) {
            __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (__hip_atomic_fetch_add(&ws[0], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                (uint32_t)(groups - 1)) {
                __hip_atomic_store(&ws[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                for (int q = 0; q < groups; ++q)
                    __hip_atomic_store(ws + kGroupStride * (1 + q) + 1, gen + 1u, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
                last = true;
            }
        }
        int fail = 0;
        if (!last) {
            int spins = 0;
            while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gen) {
                if (++spins > kSpinLimit) {
                    fail = 1;
                    __hip_atomic_fetch_add(&ws[2], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
            }
        }
        if (FENCE) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        gave_up = fail;
    }
    __syncthreads();
    return gave_up == 0;
}

}  // namespace
}  // namespace cgl
