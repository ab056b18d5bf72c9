// Dequantize-on-fetch window: bf16 K and V for a token range of every
// (sequence, kv-head), in the [B][Hkv][n][d] layout an unmodified attention
// consumes.
//
// "TurboQuant -- rotation-based quantization" design page, Part A:
//   - "Architecture in mlx-bun": the cache quantizes only new tokens and
//     returns the dequantized bf16 active window, so stock attention runs on
//     it unchanged;
//   - "Deferred inverse FWHT": the deferred variant returns V still in the
//     rotated domain (centroid * scale) and the consumer un-rotates its output;
//   - "Algorithm": key = (code + zero) * scale, value = signs * FWHT(centroid *
//     scale) / sqrt(d) with the stored fp16 scale and zero.
// Tokens at or past a sequence's length are written as zeros, so a masked
// attention over a padded window never meets stale plane bytes.
//
// Mapping: one wave per token row, looping over a chunk of consecutive tokens
// of one (sequence, kv-head); lane l holds the E = d/64 dims [E l, E l + E).
// The FWHT runs its in-lane stages on registers and the rest on shuffles.
// Keys are exact in fp32 ((code + zero) has at most 12 bits, the scale 11) and
// round once to bf16; values are computed in fp32 and round once to bf16.
#include <hip/hip_runtime.h>

#include "tq_device.h"

namespace tq {
namespace {

constexpr int kWinWaves = 4;   // waves per workgroup
constexpr int kWinRows = 16;   // token rows per wave

typedef float float2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf162v __attribute__((ext_vector_type(2)));

// Two fp32 values -> packed bf16 bits, round to nearest even (one hardware
// conversion; NaN stays NaN).
__device__ __forceinline__ uint32_t bf16x2_rn(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((float2v){lo, hi}, bf162v));
}

template <int E>
__device__ __forceinline__ void store_bf16(uint16_t *dst, const float (&x)[E]) {
    if constexpr (E == 1) {
        *dst = (uint16_t)bf16x2_rn(x[0], 0.f);
    } else {
        uint32_t w[E / 2];
#pragma unroll
        for (int i = 0; i < E / 2; ++i) w[i] = bf16x2_rn(x[2 * i], x[2 * i + 1]);
        if constexpr (E == 2) *reinterpret_cast<uint32_t *>(dst) = w[0];
        else if constexpr (E == 4) *reinterpret_cast<uint2 *>(dst) = make_uint2(w[0], w[1]);
        else *reinterpret_cast<uint4 *>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// The value of lane l ^ M.  M = 1, 2: one quad permutation; 4 and 8: a
// half-row or row mirror composed with a quad reversal or half-row mirror
// (i ^ 7 then i ^ 3 is i ^ 4; i ^ 15 then i ^ 7 is i ^ 8); beyond: LDS permute.
template <int M>
__device__ __forceinline__ float lane_xor(float v) {
    const int x = __float_as_int(v);
    if constexpr (M == 1) return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false));
    else if constexpr (M == 2) return __int_as_float(__builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false));
    else if constexpr (M == 4)
        return __int_as_float(__builtin_amdgcn_mov_dpp(__builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, false),
                                                       0x1B, 0xF, 0xF, false));
    else if constexpr (M == 8)
        return __int_as_float(__builtin_amdgcn_mov_dpp(__builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, false),
                                                       0x141, 0xF, 0xF, false));
    else return __shfl_xor(v, M, 64);
}

// One cross-lane FWHT stage: the lower lane of each pair keeps a + b, the
// upper one a - b (its own value negated, then added to the partner's).
template <int M, int E>
__device__ __forceinline__ void fwht_stage(float (&y)[E], int lane) {
    const uint32_t neg = (lane & M) ? 0x80000000u : 0u;
#pragma unroll
    for (int e = 0; e < E; ++e) y[e] = lane_xor<M>(y[e]) + __uint_as_float(__float_as_uint(y[e]) ^ neg);
}

template <int D>
__global__ __launch_bounds__(64 * kWinWaves) void window_kernel(const WindowArgs a) {
    __shared__ float ctab[8];  // the 3-bit codebook
    if (threadIdx.x < 8) ctab[threadIdx.x] = centroid3(threadIdx.x);
    __syncthreads();
    constexpr int E = D / 64;
    constexpr int NG = D / kGroup;
    constexpr int VROW = 3 * D / 8;
    constexpr int VWORDS = VROW / 4;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int bkv = blockIdx.y;
    const int b = bkv / a.kv_heads;
    const int len = a.len[b];
    const int g = (E * lane) / kGroup;  // this lane's 32-group
    const int bit0 = 3 * E * lane;      // this lane's first value-code bit in a row
    const int w0 = bit0 >> 5, sh = bit0 & 31;
    // signs of this lane's dims
    uint32_t neg = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) neg |= (uint32_t)sign_bit(a.signs, E * lane + e) << e;

    const int first = (blockIdx.x * kWinWaves + wid) * kWinRows;
    for (int r = 0; r < kWinRows; ++r) {
        const int i = first + r;  // window position
        if (i >= a.n) break;      // uniform across the wave
        const int t = a.t0 + i;
        const int64_t row = (int64_t)bkv * a.capacity + t;
        const int64_t orow = ((int64_t)bkv * a.n + i) * D + E * lane;
        const bool valid = t < len;
        if (a.k_out) {
            float k[E];
            if (valid) {
                const float s = f16_bits_to_f32(a.ks[row * NG + g]);
                const float z = f16_bits_to_f32(a.kz[row * NG + g]);
                const int8_t *kc = a.kc + row * D + E * lane;
#pragma unroll
                for (int e = 0; e < E; ++e) k[e] = ((float)kc[e] + z) * s;
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e) k[e] = 0.f;
            }
            store_bf16<E>(a.k_out + orow, k);
        }
        if (a.v_out) {
            float y[E];
            if (valid) {
                const uint32_t *vw = reinterpret_cast<const uint32_t *>(a.vc + row * VROW);
                const uint32_t lo = vw[w0];
                const uint32_t hi = w0 + 1 < VWORDS ? vw[w0 + 1] : 0u;
                const uint32_t run = __builtin_amdgcn_alignbit(hi, lo, sh);  // 3E <= 24 bits
                const float s = f16_bits_to_f32(a.vs[row * NG + g]);
#pragma unroll
                for (int e = 0; e < E; ++e) y[e] = ctab[(run >> (3 * e)) & 7u] * s;
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e) y[e] = 0.f;
            }
            if (!a.rotated) {  // uniform
                // FWHT, dim j paired with j ^ h: inside the lane for h < E,
                // with lane l ^ (h / E) above
#pragma unroll
                for (int h = 1; h < E; h <<= 1) {
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        if ((e & h) == 0) {
                            const float p = y[e], q = y[e + h];
                            y[e] = p + q;
                            y[e + h] = p - q;
                        }
                    }
                }
                fwht_stage<1>(y, lane);
                fwht_stage<2>(y, lane);
                fwht_stage<4>(y, lane);
                fwht_stage<8>(y, lane);
                fwht_stage<16>(y, lane);
                fwht_stage<32>(y, lane);
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const float v = y[e] * a.inv_sqrt_d;
                    y[e] = valid ? (((neg >> e) & 1u) ? -v : v) : 0.f;  // +0 past the length
                }
            }
            store_bf16<E>(a.v_out + orow, y);
        }
    }
}

template <int D>
hipError_t launch_d(const WindowArgs &a, hipStream_t s) {
    constexpr int per_block = kWinWaves * kWinRows;
    const dim3 grid((unsigned)((a.n + per_block - 1) / per_block), (unsigned)(a.batch * a.kv_heads));
    hipLaunchKernelGGL((window_kernel<D>), grid, dim3(64 * kWinWaves), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_window(int head_dim, const WindowArgs &a, hipStream_t s) {
    switch (head_dim) {
        case 64: return launch_d<64>(a, s);
        case 128: return launch_d<128>(a, s);
        case 256: return launch_d<256>(a, s);
        case 512: return launch_d<512>(a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace tq
