// Counting the workgroups of a launch done, for launches that a HIP graph may
// replay with the same token (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlnf4 {

// ---------------------------------------------------------------------------
// Counting workgroups done inside a launch (for the launches that a graph
// may replay with the same token). A counter holds token << 24 | count; one
// holding another token counts as zero, and each counter's last arrival
// leaves it at zero (compare-and-swap), so nothing needs resetting before a
// launch. Workgroup i of `total` counts on counter i % kArriveSub, the last
// arrival on each of those on counter kArriveSub (atomics on one word are
// served one after another). Called by one thread; returns true for the
// last of all `total` arrivals. The caller has completed (vmcnt) the memory
// accesses the count stands for; those, and what the last arrival does
// next, are agent-scope atomics performed at the device's coherence point,
// so relaxed ordering suffices.
// ---------------------------------------------------------------------------
constexpr int kArriveSub = 32;

__device__ __forceinline__ bool tagged_arrive_one(uint64_t* c, uint64_t token, int n) {
    uint64_t old = __hip_atomic_load(c, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int arrived;
    uint64_t nv;
    do {
        arrived = static_cast<int>((old >> 24) == token ? (old & 0xFFFFFFu) : 0u) + 1;
        nv = (token << 24) | static_cast<uint64_t>(arrived == n ? 0 : arrived);
    } while (!__hip_atomic_compare_exchange_strong(c, &old, nv, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                  __HIP_MEMORY_SCOPE_AGENT));
    return arrived == n;
}

// counters: kArriveSub + 1 words; token: at most 40 bits
__device__ __forceinline__ bool tagged_arrive(uint64_t* counters, uint64_t token, int i, int total) {
    const int k = i % kArriveSub, groups = total < kArriveSub ? total : kArriveSub;
    const int in_k = total / kArriveSub + (k < total % kArriveSub ? 1 : 0);  // arrivals on counter k
    return tagged_arrive_one(counters + k, token, in_k) && tagged_arrive_one(counters + kArriveSub, token, groups);
}

}  // namespace qlnf4
