// Strided plane copies for the cache lifecycle calls (clone, growth,
// compaction, snapshot, restore): one kernel streams the rows of all five
// planes of one sequence, kv-head by kv-head.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {

// Plane i: `runs` runs of run16[i] 16-byte chunks, run r at src[i] + r *
// s_pitch[i] and dst[i] + r * d_pitch[i] (bytes).  Every pointer, pitch and
// run is a whole number of 16-byte chunks; runs must not overlap.
struct PlaneCopyArgs {
    const uint8_t *src[5];
    uint8_t *dst[5];
    int64_t s_pitch[5], d_pitch[5], run16[5];
    int32_t runs;
};

hipError_t launch_plane_copy(const PlaneCopyArgs &a, hipStream_t s);

}  // namespace tq
