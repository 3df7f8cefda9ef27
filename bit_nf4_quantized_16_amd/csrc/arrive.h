// Tags of the words one workgroup hands to another inside a launch, for
// launches that a HIP graph may replay (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace qlnf4 {

// ---------------------------------------------------------------------------
// Words handed from one workgroup to another carry a tag of their launch, so
// a reader can tell this launch's words from those an earlier launch left in
// the workspace. An eager launch gets a fresh tag from the host. A captured
// launch is replayed with the tag it was captured with, so its tag also
// mixes in an epoch word of the workspace that a one-thread kernel recorded
// just before the launch advances at every replay: every workgroup reads the
// epoch (the advance completed before the launch started), and the words of
// the previous replay carry the previous epoch's tag. Nothing is counted or
// cleared. (Counting the workgroups done so that the last one clears the
// words cost more: a token-tagged compare-and-swap count 24 us per decode
// call, its retries queueing; zeroed counters with fetch-and-add, 1.3 us
// more than this.)
// ---------------------------------------------------------------------------

// The tag of a launch: its host tag alone, or mixed with the epoch (a
// captured launch); never zero, so a cleared word never passes.
__device__ __forceinline__ uint32_t launch_tag(uint32_t host_tag, const uint64_t* epoch) {
    if (epoch == nullptr) return host_tag;
    const uint64_t e = __hip_atomic_load(epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    uint64_t h = (e + 1) * 0x9E3779B97F4A7C15ull ^ (uint64_t{host_tag} << 17);
    h ^= h >> 29;
    h *= 0xBF58476D1CE4E5B9ull;
    h ^= h >> 32;
    const uint32_t t = static_cast<uint32_t>(h);
    return t != 0 ? t : 1u;
}

// Records the one-thread kernel that advances `epoch` (before a captured
// launch; defined with the decode GEMV).
void launch_advance_epoch(uint64_t* epoch, hipStream_t stream);

}  // namespace qlnf4
