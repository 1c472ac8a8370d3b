// barrier_protocol.hpp -- the arrival and wait protocol of the grid-wide
// barrier, written once for the GPU (grid_barrier.hpp, with agent-scope
// atomics) and for a host test that runs it with threads as blocks.
//
// Workspace words (32-bit): 0 the top arrival counter; 2 the give-up count;
// 64*(1+c) and 64*(1+c)+1 the arrival counter and generation flag of group c
// (block b belongs to group b % 8), each group on its own 256-byte line.
//
// A block arrives at its group's counter; the last block of a group arrives
// at the top counter, and the last block overall resets both counters it
// used and publishes the next generation to every group's flag, which the
// other blocks of the group poll.  So no more than ceil(blocks / 8) atomics
// queue on one address.  Polls are bounded; a block that stops waiting counts
// itself in word 2.  Word 2 is sticky: the library never clears it.  A block
// that finds it nonzero -- before arriving or while waiting -- stops at once,
// so after a give-up the counters, which may then hold stray arrivals, are
// never used again: every later launch on the workspace refuses to wait at
// all until the caller zeroes the workspace.
#pragma once

#include <stdint.h>

#ifdef __HIPCC__
#define CGL_HD __host__ __device__
#else
#define CGL_HD
#endif

namespace cgl {

constexpr int kBarrierGroups = 8;
constexpr int kBarrierGroupStride = 64;  // 32-bit words: 256 bytes per group
constexpr int kBarrierGiveUpWord = 2;

// Ops supplies load(p), store(p, v), fetch_add(p, v) (all atomic, returning
// the old value for fetch_add) and pause().
template <class Ops>
CGL_HD inline bool barrier_refused(const Ops& op, uint32_t* ws) {
    return op.load(ws + kBarrierGiveUpWord) != 0u;
}

// Arrival and wait of block `block` of `nb`; true once every block has
// arrived, false if the block stopped waiting (then counted in word 2).
// `refused` is barrier_refused() as the block read it when its launch
// started (read early so that its latency stays off the barrier's path); a
// refused block neither arrives nor waits.  Only the first barrier of a
// launch needs it: within a launch a give-up leaves the later barriers
// incomplete, and their waiters stop as soon as they see word 2.
template <class Ops>
CGL_HD inline bool barrier_arrive_wait(const Ops& op, uint32_t* ws, int block, int nb, uint32_t spin_limit,
                                       bool refused) {
    if (refused) return false;
    const int c = block % kBarrierGroups;
    const int in_group = (nb - c + kBarrierGroups - 1) / kBarrierGroups;
    const int groups = nb < kBarrierGroups ? nb : kBarrierGroups;
    uint32_t* counter = ws + kBarrierGroupStride * (1 + c);
    uint32_t* flag = counter + 1;
    const uint32_t gen = op.load(flag);
    if (op.fetch_add(counter, 1u) == (uint32_t)(in_group - 1)) {
        op.store(counter, 0u);
        if (op.fetch_add(ws, 1u) == (uint32_t)(groups - 1)) {
            op.store(ws, 0u);
            for (int q = 0; q < groups; ++q) op.store(ws + kBarrierGroupStride * (1 + q) + 1, gen + 1u);
            return true;
        }
    }
    for (uint32_t spins = 0; op.load(flag) == gen; ++spins) {
        if (spins >= spin_limit || barrier_refused(op, ws)) {
            op.fetch_add(ws + kBarrierGiveUpWord, 1u);
            return false;
        }
        op.pause();
    }
    return true;
}

}  // namespace cgl
