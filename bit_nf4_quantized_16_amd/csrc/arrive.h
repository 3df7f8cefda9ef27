// Counting the workgroups of a launch done, for launches that a HIP graph
// may replay with the same token (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlnf4 {

// ---------------------------------------------------------------------------
// A captured launch replays with its token and tag, so words it hands from
// one workgroup to another must be cleared by its last workgroup before the
// next replay. The kArriveWords counters of such a launch are zeroed by a
// small fill kernel recorded right before it (in the launch's source file),
// so each arrival is one fetch-and-add: workgroup i of `total` adds one to
// counter i % kArriveSub, and the last arrival on that counter adds one to
// the top counter (atomics on one word are served one after another, so one
// counter for all would queue them). Called by one thread once the
// workgroup's accesses to the words have completed (vmcnt); those, and what
// the last arrival does next, are agent-scope atomics performed at the
// device's coherence point, so relaxed ordering suffices. Returns true for
// the last of all `total` arrivals. (A compare-and-swap count that needs no
// zeroing, token-tagged, cost 24 us per decode call in a graph: its retries
// queue.)
// ---------------------------------------------------------------------------
constexpr int kArriveSub = 32;
constexpr int kArriveWords = kArriveSub + 1;

__device__ __forceinline__ bool count_arrival(uint64_t* counters, int i, int total) {
    const int k = i % kArriveSub, groups = total < kArriveSub ? total : kArriveSub;
    const int in_k = total / kArriveSub + (k < total % kArriveSub ? 1 : 0);  // arrivals on counter k
    if (static_cast<int>(__hip_atomic_fetch_add(counters + k, uint64_t{1}, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT)) + 1 != in_k)
        return false;
    return static_cast<int>(__hip_atomic_fetch_add(counters + kArriveSub, uint64_t{1}, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT)) + 1 == groups;
}

// Up to four blocks of kArriveWords counters (null: none), for the fill
// kernel of a launch that serves several weights.
struct CounterSet {
    uint64_t* c[4];
};

}  // namespace qlnf4
