// grid_exchange.hpp -- level (4) of the reduction ladder for rows split over G workgroups.
//
// The QuACK article (无需CUDA代码，给H100加速33%-50%), section 硬件感知的归约策略 part 4
// and the section 内存吞吐量, lets up to 16 blocks of a cluster reduce one row through
// distributed shared memory, so that rows too large for one SM are still read from
// HBM only once (instead of an online algorithm that reads twice, or register
// spills).  gfx950 has no clusters, so the G workgroups of a row meet in a small
// global workspace instead:
//
//  * every workgroup k of a row group publishes its partial result in slot k as
//    64-bit words (epoch << 32) | float_bits, written and read with agent-scope
//    relaxed atomics.  The epoch (row iteration + 1) travels in the same word as the
//    value, so a reader that sees the right epoch has the right value: no fences,
//    no separate flag, no cache write-back or invalidate;
//  * slots come in kSlotSets = 4 sets, used in turn by the row iterations.  A
//    workgroup may publish iteration k before it waits for iteration k - 1 (the
//    deferred exchange of the split-row kernels); it has then finished waiting for
//    k - 2, so every peer has published k - 2, which a peer does only after it
//    finished reading k - 4: the set of k - 4, which k overwrites, is free;
//  * wave 0 polls the G slots (one lane per slot), then merges the partials in slot
//    order, so every workgroup of the row computes the same bits;
//  * each poll loop is bounded by `spin_limit`; a workgroup that gives up sets the
//    workspace error word, takes NaN as the row's merged result (so its share of the
//    row is written as NaN, never as a wrong number) and carries on, so a kernel
//    always finishes.  Later waits of that workgroup poll once: a row whose peers
//    have all published is still exact, any other row is NaN;
//  * after its last row every workgroup increments the group's departure counter;
//    the last one to leave zeroes the group's slots and the counter, so the
//    workspace is all zero again for the next launch.
//
// Membership by block id.  Row group g is the G consecutive blocks gG .. gG + G - 1,
// and block b is member b % G.  Blocks go to the eight XCDs in turn (block b to XCD
// b mod 8), and each XCD starts its blocks in the order of their ids; so the members
// of every group that has not finished are either running or next in line on their
// XCD, and a grid larger than the device holds at once (other work holding slots, or
// a test override) still drains when each XCD can hold ceil(G / 8) workgroups of the
// kernel: the lowest unfinished group's members on an XCD come right after the
// blocks of finished groups there.  The planner sizes the grid from the occupancy
// query, so normally all of it runs at once.  Past that, the bounded wait ends a wait
// that cannot be met.  Which chunks of a row each member holds: row_io.hpp, lane_of.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "configs.hpp"
#include "reduce.hpp"

namespace rr {

struct GroupRef {
    uint32_t *depart;  // departure counter
    uint64_t *slots;   // [kSlotSets][G][2]
    uint32_t *error;   // workspace error word
};

template <int G>
__device__ __forceinline__ GroupRef group_ref(uint8_t *ws, int group) {
    uint8_t *rec = ws + kWsHeader + (size_t)group * group_stride_for(G);
    return {reinterpret_cast<uint32_t *>(rec), reinterpret_cast<uint64_t *>(rec + 64),
            reinterpret_cast<uint32_t *>(ws)};
}

__device__ __forceinline__ uint64_t tag(uint32_t epoch, float v) {
    return ((uint64_t)epoch << 32) | __float_as_uint(v);
}

__device__ __forceinline__ void atomic_put(uint64_t *p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t atomic_get(const uint64_t *p) {
    return __hip_atomic_load(const_cast<uint64_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Publishes (a, b) for member k at iteration `it` (thread 0 writes; the values are
// the same in every thread).
template <int G>
__device__ __forceinline__ void publish_pair(GroupRef g, int k, int it, float a, float b) {
    if (threadIdx.x == 0) {
        uint64_t *slot = g.slots + (size_t)(it & (kSlotSets - 1)) * G * 2;
        const uint32_t epoch = (uint32_t)it + 1u;
        atomic_put(slot + 2 * k, tag(epoch, a));
        atomic_put(slot + 2 * k + 1, tag(epoch, b));
    }
}

// Waits until all G members have published iteration `it` and leaves the G pairs
// merged in bcast[0..1] (the same bits for the whole workgroup, and in every member:
// the merge order is fixed).  Called by every thread; uses one barrier.  Lane l of
// wave 0 polls the slots of members l, l + 64, l + 128 and l + 192 (those below G),
// merges them in that order, and
// the wave merges its lanes' pairs with the butterfly of reduce.hpp (`Merge::lanes`;
// lanes with no member hold the empty pair), log2 G steps on every lane at once.
// Merging one member after the other from lane 0 instead kept all G pairs in
// registers at once (12 more VGPRs at G = 16).  A wait that gives up (after
// `spin_limit` polls; at once if spin_limit <= 0) leaves NaN in bcast[0..1], which
// every op's epilogue carries into each value it writes for the row, and lowers
// `spin_limit` to 1 so that the rest of the launch does not wait long again (a limit
// of 0, which only a test sets, stays 0: every wait of the launch gives up).
template <int G, class Merge>
__device__ __forceinline__ void wait_pairs(GroupRef g, int it, int &spin_limit, float *bcast,
                                           Merge merge2) {
    static_assert(G >= 1 && G <= 256, "one wave polls at most four slots per lane");
    constexpr int kPer = (G + 63) / 64;
    const int tid = threadIdx.x;
    const uint32_t epoch = (uint32_t)it + 1u;
    const uint64_t *slot = g.slots + (size_t)(it & (kSlotSets - 1)) * G * 2;
    if (tid < 64) {
        const int lane = tid;
        uint64_t wa[kPer], wb[kPer];
#pragma unroll
        for (int s = 0; s < kPer; ++s) wa[s] = wb[s] = 0;
        bool all_in = false;
        int spins = 0;
        while (true) {
            bool mine = true;
#pragma unroll
            for (int s = 0; s < kPer; ++s) {
                const int m = lane + 64 * s;
                if (m < G) {
                    wa[s] = atomic_get(slot + 2 * m);
                    wb[s] = atomic_get(slot + 2 * m + 1);
                    mine = mine && (uint32_t)(wa[s] >> 32) == epoch &&
                           (uint32_t)(wb[s] >> 32) == epoch;
                }
            }
            all_in = __all(mine);
            if (all_in || ++spins >= spin_limit) break;
            __builtin_amdgcn_s_sleep(1);
        }
        all_in = all_in && spin_limit > 0;
        if (!all_in && lane == 0) {
            __hip_atomic_store(g.error, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            bcast[2] = 1.0f;
        }
        float acc_a = Merge::kEmptyA, acc_b = Merge::kEmptyB;
        if (lane < G) {
            acc_a = __uint_as_float((uint32_t)wa[0]);
            acc_b = __uint_as_float((uint32_t)wb[0]);
        }
#pragma unroll
        for (int s = 1; s < kPer; ++s) {
            if (lane + 64 * s < G)
                merge2(acc_a, acc_b, __uint_as_float((uint32_t)wa[s]),
                       __uint_as_float((uint32_t)wb[s]));
        }
        constexpr int W = G >= 64 ? 64 : G > 32 ? 64 : G > 16 ? 32 : G > 8 ? 16 : G > 4 ? 8
                                                                              : G > 2 ? 4 : 2;
        Merge::template lanes<W>(acc_a, acc_b);
        if (lane == 0) {
            bcast[0] = all_in ? acc_a : __builtin_nanf("");
            bcast[1] = all_in ? acc_b : __builtin_nanf("");
        }
    }
    __syncthreads();
    if (bcast[2] != 0.0f && spin_limit > 1) spin_limit = 1;
}

// Publish, then wait for the same iteration.
template <int G, class Merge>
__device__ __forceinline__ void exchange_pairs(GroupRef g, int k, int it, float a, float b,
                                               int &spin_limit, float *bcast, Merge merge2) {
    publish_pair<G>(g, k, it, a, b);
    wait_pairs<G>(g, it, spin_limit, bcast, merge2);
}

// Called once per workgroup after its last row (only if it processed any row).
template <int G>
__device__ __forceinline__ void depart_group(GroupRef g) {
    if (threadIdx.x == 0) {
        uint32_t before =
            __hip_atomic_fetch_add(g.depart, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (before == (uint32_t)G - 1u) {
            for (int i = 0; i < kSlotSets * G * 2; ++i) atomic_put(g.slots + i, 0ull);
            __hip_atomic_store(g.depart, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// Which row group and member this workgroup is (see the membership note above).
template <int G>
__device__ __forceinline__ void member_of(int *group, int *member) {
    *group = (int)(blockIdx.x / G);
    *member = (int)(blockIdx.x % G);
}

}  // namespace rr
