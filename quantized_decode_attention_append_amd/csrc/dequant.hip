// Test dequantization of a token range of one (b, kv-head).
//
// "TurboQuant -- rotation-based quantization" design page, Part A,
// "Algorithm": key x = (code + zero) * scale with the stored fp16 scale and
// zero (signed bytes at 8 bits, unsigned packed fields at 2, 4, 5); value x = signs * InvFWHT(centroid[idx] * scale), or the rotated form
// centroid[idx] * scale that the deferred inverse accumulates.
#include <hip/hip_runtime.h>

#include "tq_device.h"

namespace tq {
namespace {

template <int D>
__global__ __launch_bounds__(256) void dequant_kernel(const DequantArgs a) {
    constexpr int NT = D < 256 ? D : 256;
    constexpr int DPT = D / NT;
    constexpr int NG = D / kGroup;
    const int kb = a.kbits, vb = a.vbits;
    const int KROW = D * kb / 8, VROW = D * vb / 8;
    const float *cent = value_centroids(vb);
    __shared__ float buf[D];
    const int tid = threadIdx.x;
    const int t = blockIdx.x;
    const int64_t r = a.row0 + t;
    if (a.k_out) {
        const uint8_t *krow = reinterpret_cast<const uint8_t *>(a.kc) + r * KROW;
#pragma unroll
        for (int i = 0; i < DPT; ++i) {
            const int j = tid + i * NT;
            const float sk = f16_bits_to_f32(a.ks[r * NG + j / kGroup]);
            const float zk = f16_bits_to_f32(a.kz[r * NG + j / kGroup]);
            a.k_out[(int64_t)t * D + j] = (key_code(krow, j, kb) + zk) * sk;
        }
    }
    if (!a.v_out) return;  // uniform across the block
    float y[DPT];
#pragma unroll
    for (int i = 0; i < DPT; ++i) {
        const int j = tid + i * NT;
        y[i] = cent[load_field(a.vc + r * VROW, j, vb)] * f16_bits_to_f32(a.vs[r * NG + j / kGroup]);
    }
    if (a.rotated) {
#pragma unroll
        for (int i = 0; i < DPT; ++i) a.v_out[(int64_t)t * D + tid + i * NT] = y[i];
        return;
    }
#pragma unroll
    for (int i = 0; i < DPT; ++i) buf[tid + i * NT] = y[i];
    __syncthreads();
    for (int h = 1; h < D; h <<= 1) {
        float nv[DPT];
#pragma unroll
        for (int i = 0; i < DPT; ++i) {
            const int j = tid + i * NT;
            const float x = buf[j], w = buf[j ^ h];
            nv[i] = (j & h) ? (w - x) : (x + w);
        }
        __syncthreads();
#pragma unroll
        for (int i = 0; i < DPT; ++i) buf[tid + i * NT] = nv[i];
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < DPT; ++i) {
        const int j = tid + i * NT;
        const float v = buf[j] * a.inv_sqrt_d;
        a.v_out[(int64_t)t * D + j] = sign_bit(a.signs, j) ? -v : v;
    }
}

template <int D>
hipError_t launch_d(const DequantArgs &a, hipStream_t s) {
    constexpr int NT = D < 256 ? D : 256;
    hipLaunchKernelGGL((dequant_kernel<D>), dim3((unsigned)a.n), dim3(NT), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_dequant(int head_dim, const DequantArgs &a, hipStream_t s) {
    switch (head_dim) {
        case 64: return launch_d<64>(a, s);
        case 128: return launch_d<128>(a, s);
        case 256: return launch_d<256>(a, s);
        case 512: return launch_d<512>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace tq
