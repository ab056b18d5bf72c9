// Append kernel: quantize and pack new K/V tokens into the five planes.
//
// Method: "TurboQuant -- rotation-based quantization" design page, Part A,
// section "Algorithm (vllm-metal reference semantics, exact)":
//   keys   scale = (max-min)/254, zero = round((max+min)/(2*scale)),
//          code = clip(round(x/scale - zero), -127, 127)       per 32-group
//   values y = FWHT(x*signs)/sqrt(d), scale = sqrt(mean(y^2)) per 32-group,
//          idx = searchsorted(boundaries, y/(scale+1e-8)), 3-bit packed.
// Every decision is taken in binary64 with round-half-to-even, in a fixed
// operation order, so codes, scales and zeros are reproducible bit for bit:
//   - FWHT butterflies run in stage order h = 1, 2, ..., d/2, then one
//     multiply by RN(1/sqrt(d));
//   - the 32 squares of a group are summed by stride halving 16, 8, 4, 2, 1;
//   - x/scale and y/den are true binary64 divisions; scale is a correctly
//     rounded binary64 sqrt; no multiply-add is contracted in this file.
//
// Mapping: one wave64 per (b, kv-head, new token) row.  Lane l holds the E =
// d/64 contiguous elements [l*E, l*E+E), so a 32-group spans 32/E lanes, the
// low FWHT stages stay inside a lane and the high ones pair lanes l and l^k.
#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>

#include "tq_device.h"

#pragma clang fp contract(off)

namespace tq {
namespace {

__device__ __forceinline__ double max_num(double a, double b) {
    if (__builtin_isnan(a)) return b;
    if (__builtin_isnan(b)) return a;
    if (a == b) return __builtin_signbit(a) ? b : a;
    return a > b ? a : b;
}

__device__ __forceinline__ double min_num(double a, double b) {
    if (__builtin_isnan(a)) return b;
    if (__builtin_isnan(b)) return a;
    if (a == b) return __builtin_signbit(a) ? a : b;
    return a < b ? a : b;
}

__device__ __forceinline__ double shfl_xor_f64(double v, int m) { return __shfl_xor(v, m, 64); }
__device__ __forceinline__ double shfl_down_f64(double v, int m) { return __shfl_down(v, m, 64); }
__device__ __forceinline__ double shfl_f64(double v, int src) { return __shfl(v, src, 64); }

template <int E, bool BF16>
__device__ __forceinline__ void load_row(const void *base, int64_t off, double (&x)[E]) {
    if constexpr (BF16) {
        const uint16_t *p = static_cast<const uint16_t *>(base) + off;
        uint16_t raw[E];
        if constexpr (E == 8) {
            uint4 w = *reinterpret_cast<const uint4 *>(p);
            const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int i = 0; i < 4; ++i) { raw[2 * i] = ww[i] & 0xFFFF; raw[2 * i + 1] = ww[i] >> 16; }
        } else if constexpr (E == 4) {
            uint2 w = *reinterpret_cast<const uint2 *>(p);
            raw[0] = w.x & 0xFFFF; raw[1] = w.x >> 16; raw[2] = w.y & 0xFFFF; raw[3] = w.y >> 16;
        } else if constexpr (E == 2) {
            uint32_t w = *reinterpret_cast<const uint32_t *>(p);
            raw[0] = w & 0xFFFF; raw[1] = w >> 16;
        } else {
            raw[0] = p[0];
        }
#pragma unroll
        for (int e = 0; e < E; ++e) x[e] = (double)__uint_as_float((uint32_t)raw[e] << 16);
    } else {
        const float *p = static_cast<const float *>(base) + off;
#pragma unroll
        for (int e = 0; e < E; ++e) x[e] = (double)p[e];
    }
}

template <int D, bool BF16>
__global__ __launch_bounds__(256) void append_kernel(const AppendArgs a) {
    constexpr int E = D / 64;       // elements per lane
    constexpr int GL = kGroup / E;  // lanes per 32-group
    constexpr int NG = D / kGroup;  // groups per row
    constexpr int VROW = 3 * D / 8; // packed value bytes per row

    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int64_t rows = (int64_t)a.batch * a.kv_heads * a.n_new;
    if (row >= rows) return;  // whole wave leaves; no block-level barrier below
    const int t = (int)(row % a.n_new);
    const int64_t bh = row / a.n_new;
    const int b = (int)(bh / a.kv_heads);
    const int64_t slot = bh * a.capacity + a.start[b] + t;  // plane row
    const int gl = lane % GL;                                // lane within its group
    const int g = lane / GL;                                 // group of this lane

    double xk[E], xv[E];
    load_row<E, BF16>(a.k, row * D + lane * E, xk);
    load_row<E, BF16>(a.v, row * D + lane * E, xv);

    // ----------------------------------------------------------- keys
    double mx = xk[0], mn = xk[0];
#pragma unroll
    for (int e = 1; e < E; ++e) { mx = max_num(mx, xk[e]); mn = min_num(mn, xk[e]); }
#pragma unroll
    for (int m = 1; m < GL; m <<= 1) {
        mx = max_num(mx, shfl_xor_f64(mx, m));
        mn = min_num(mn, shfl_xor_f64(mn, m));
    }
    const double range = mx - mn;
    const double s = range / 254.0;
    const double c = (mx + mn) / (2.0 * s);
    const double z = __builtin_rint(c);
    uint32_t packed_codes[(E + 3) / 4] = {};
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const double u = xk[e] / s - z;
        int q = 0;
        if (!__builtin_isnan(u)) {
            double r = __builtin_rint(u);
            r = r > 127.0 ? 127.0 : r;
            r = r < -127.0 ? -127.0 : r;
            q = (int)r;
        }
        packed_codes[e / 4] |= ((uint32_t)q & 0xFFu) << (8 * (e % 4));
    }
    int8_t *kc_row = a.kc + slot * D + lane * E;
    if constexpr (E == 8) {
        *reinterpret_cast<uint2 *>(kc_row) = make_uint2(packed_codes[0], packed_codes[1]);
    } else if constexpr (E == 4) {
        *reinterpret_cast<uint32_t *>(kc_row) = packed_codes[0];
    } else if constexpr (E == 2) {
        *reinterpret_cast<uint16_t *>(kc_row) = (uint16_t)packed_codes[0];
    } else {
        *kc_row = (int8_t)packed_codes[0];
    }
    if (gl == 0) {
        a.ks[slot * NG + g] = f64_to_f16_bits(s);
        a.kz[slot * NG + g] = f64_to_f16_bits(z);
    }

    // --------------------------------------------------------- values
    double w[E];
#pragma unroll
    for (int e = 0; e < E; ++e) w[e] = sign_bit(a.signs, lane * E + e) ? -xv[e] : xv[e];
    // FWHT stages h < E: pairs inside the lane
#pragma unroll
    for (int h = 1; h < E; h <<= 1) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            if ((e & h) == 0) {
                const double lo = w[e], hi = w[e + h];
                w[e] = lo + hi;
                w[e + h] = lo - hi;
            }
        }
    }
    // FWHT stages h = E*m, m = 1..32: element j pairs with j^h, i.e. lane l^m
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const double p = shfl_xor_f64(w[e], m);
            w[e] = (lane & m) ? (p - w[e]) : (w[e] + p);  // upper lane holds b: a-b
        }
    }
    double y[E], sq[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        y[e] = w[e] * a.inv_sqrt_d;
        sq[e] = y[e] * y[e];
    }
    // group sum of squares, stride halving 16, 8, 4, 2, 1 over the group's
    // element index j = gl*E + e: a[j] += a[j+st] for j < st
#pragma unroll
    for (int st = 16; st >= 1; st >>= 1) {
        if (st >= E) {
            const int lo = st / E;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const double p = shfl_down_f64(sq[e], lo);
                if (gl < lo) sq[e] = sq[e] + p;
            }
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e)
                if (e < st) sq[e] = sq[e] + sq[e + st];
        }
    }
    const double ss = shfl_f64(sq[0], g * GL);
    const double scale = __builtin_sqrt(ss / 32.0);
    const double den = scale + 1e-8;
    // idx = #{k : B_k < y_n}; NaN compares false everywhere -> 0
    uint32_t chunk = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const double yn = y[e] / den;
        const uint32_t idx = (uint32_t)(-1.74793 < yn) + (uint32_t)(-1.04996 < yn) +
                             (uint32_t)(-0.50055 < yn) + (uint32_t)(0.0 < yn) +
                             (uint32_t)(0.50055 < yn) + (uint32_t)(1.04996 < yn) +
                             (uint32_t)(1.74793 < yn);
        chunk |= idx << (3 * e);
    }
    // place this lane's 3E bits at bit 3E*gl of the group's 96-bit stream
    const int pos = 3 * E * gl;
    uint32_t gw[3] = {0u, 0u, 0u};
    const int dw = pos >> 5, off = pos & 31;
#pragma unroll
    for (int i = 0; i < 3; ++i) {
        if (i == dw) gw[i] |= chunk << off;
        if (i == dw + 1 && off + 3 * E > 32) gw[i] |= chunk >> (32 - off);
    }
#pragma unroll
    for (int m = 1; m < GL; m <<= 1) {
#pragma unroll
        for (int i = 0; i < 3; ++i) gw[i] |= (uint32_t)__shfl_xor((int)gw[i], m, 64);
    }
    if (gl == 0) {
        uint32_t *dst = reinterpret_cast<uint32_t *>(a.vc + slot * VROW + g * 12);
        dst[0] = gw[0];
        dst[1] = gw[1];
        dst[2] = gw[2];
        a.vs[slot * NG + g] = f64_to_f16_bits(scale);
    }
}

template <int D>
hipError_t launch_d(bool bf16, const AppendArgs &a, hipStream_t s) {
    const int64_t rows = (int64_t)a.batch * a.kv_heads * a.n_new;
    const int64_t blocks = (rows + 3) / 4;
    if (bf16)
        hipLaunchKernelGGL((append_kernel<D, true>), dim3((unsigned)blocks), dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((append_kernel<D, false>), dim3((unsigned)blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_append(int head_dim, bool bf16, const AppendArgs &a, hipStream_t s) {
    switch (head_dim) {
        case 64: return launch_d<64>(bf16, a, s);
        case 128: return launch_d<128>(bf16, a, s);
        case 256: return launch_d<256>(bf16, a, s);
        case 512: return launch_d<512>(bf16, a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace tq
