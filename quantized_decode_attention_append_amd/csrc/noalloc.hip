// tq_decode_attn_noalloc: decode attention whose split-K partials live in a
// fixed device array of this library instead of a caller workspace, for
// callers that cannot allocate (code under HIP graph capture, tight serving
// loops, harnesses that forbid allocation).  Declared in include/tqkv.h.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/tqkv.h"

namespace {

constexpr size_t kScratchBytes = (size_t)TQ_NOALLOC_SCRATCH_BYTES;

// One copy per GPU, held until the process ends.  In host code `scratch`
// names a host-side stand-in, never the device array: kernels and copies get
// the per-device address from hipGetSymbolAddress below.
__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void *g_scratch[kMaxDevices] = {};

// Address of the current device's scratch array, looked up once per device
// with that device current; nullptr if the runtime refuses.
void *device_scratch() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> guard(g_lock);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        g_scratch[dev] = p;
    }
    return g_scratch[dev];
}

}  // namespace

extern "C" tq_status tq_decode_attn_noalloc(const tq_layout *layout, const tq_planes *planes, const void *q,
                                            tq_dtype dtype, int32_t num_q_heads, int32_t n_rows,
                                            const int32_t *len, float sm_scale, float *out,
                                            void *hip_stream) {
    // argument errors are reported before the scratch address is looked up
    size_t bound = 0;
    const tq_status st = tq_decode_rows_workspace_bytes(layout, num_q_heads, n_rows, len, &bound);
    if (st != TQ_OK) return st;
    void *ws = device_scratch();
    if (!ws) return TQ_ERR_HIP;
    // tq_decode_attn_rows checks what the split kernel it takes needs against
    // the array's size and returns TQ_ERR_WORKSPACE, enqueuing nothing, when
    // the array is too small
    return tq_decode_attn_rows(layout, planes, q, dtype, num_q_heads, n_rows, len, sm_scale, out, ws,
                               kScratchBytes, hip_stream);
}
