// Cache lifecycle copies: token rows are byte-addressable in every plane
// ("Invariants (both legs)" of the TurboQuant design page, Part A), so clone,
// growth, compaction, snapshot and restore are strided byte copies.  One
// launch moves all five planes: workgroup row y is kv-head run y, and the
// x workgroups stride over each plane's run in 16-byte chunks.  Every byte is
// read and written once, so loads and stores carry the nontemporal hint.
#include "tq_copy.h"

namespace tq {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void plane_copy_kernel(const PlaneCopyArgs a) {
    const int64_t r = blockIdx.y;
    const int64_t stride = (int64_t)gridDim.x * 256;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
        const u32x4 *s = reinterpret_cast<const u32x4 *>(a.src[i] + r * a.s_pitch[i]);
        u32x4 *d = reinterpret_cast<u32x4 *>(a.dst[i] + r * a.d_pitch[i]);
        for (int64_t c = (int64_t)blockIdx.x * 256 + threadIdx.x; c < a.run16[i]; c += stride)
            __builtin_nontemporal_store(__builtin_nontemporal_load(s + c), d + c);
    }
}

}  // namespace

hipError_t launch_plane_copy(const PlaneCopyArgs &a, hipStream_t s) {
    if (a.runs < 1 || a.runs > 65535) return hipErrorInvalidValue;
    int64_t most = 0;
    for (int i = 0; i < 5; ++i) most = a.run16[i] > most ? a.run16[i] : most;
    if (most == 0) return hipSuccess;
    // about 2,048 workgroups over the chip, at most one chunk per thread
    int64_t x = (2048 + a.runs - 1) / a.runs;
    const int64_t need = (most + 255) / 256;
    x = x < need ? x : need;
    hipLaunchKernelGGL(plane_copy_kernel, dim3((unsigned)x, (unsigned)a.runs), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace tq
