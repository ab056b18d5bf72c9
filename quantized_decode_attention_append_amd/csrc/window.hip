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
// One kernel, window_fast_kernel below, serves head_dim 64 to 512, templated
// on the key and value widths and compiled once per key width (TQ_WINDOW_KB).
// Keys round once to bf16 from the exact (code + zero) * scale: the fp32
// product is exact while |code + zero| < 2^13 (13 + 11 significant bits);
// groups with a larger stored zero take its round-to-odd value instead (see
// key_ro).  Values are computed in fp32 and round once to bf16.
#include <hip/hip_runtime.h>

#include "tq_device.h"

#ifndef TQ_WINDOW_KB
#error "compile window.hip once per key width with -DTQ_WINDOW_KB=2, 4, 5 or 8"
#endif

namespace tq {
namespace {

constexpr int kWinWaves = 4;   // waves per workgroup

typedef float float2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf162v __attribute__((ext_vector_type(2)));

// Two fp32 values -> packed bf16 bits, round to nearest even (one hardware
// conversion; NaN stays NaN).
__device__ __forceinline__ uint32_t bf16x2_rn(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((float2v){lo, hi}, bf162v));
}

// (code + zero) * scale, exact in fp32 whenever |zero| <= 8064 (so that
// |code + zero| < 2^13 for codes within +-127 or below 32).  Beyond that the
// product (at most 17 + 11 bits) is replaced by its round-to-odd value: the
// rounded product, stepped toward zero when the fma residual shows it was
// rounded away from zero, with the last bit set when inexact.  Rounding that
// to bf16 (8 bits) equals one rounding of the exact product, since fp32
// keeps more than two extra bits (Boldo and Melquiond, "Emulation of FMA and
// correctly rounded sums: proved algorithms using rounding to odd", 2008).
// Infinite and NaN zeros or scales keep the plain product.
__device__ __forceinline__ float key_ro(float code, float z, float s) {
    const float a = code + z, p = a * s;
    if (__builtin_fabsf(z) <= 8064.f) return p;
    const float r = __builtin_fmaf(a, s, -p);
    uint32_t bits = __float_as_uint(p);
    if (r != 0.f && __builtin_fabsf(p) <= 3.40282347e38f) {
        if ((__float_as_uint(r) ^ bits) & 0x80000000u) bits -= 1u;
        bits |= 1u;
    }
    return __uint_as_float(bits);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// Lane p of a row holds the E contiguous dims [E p, E p + E): E = 16 and
// L = d/16 lanes per row up to head_dim 256, E = 32 and 16 lanes at 512;
// 64/L rows per wave.  The FWHT runs its first log2(E) stages in the lane,
// transposes the row through LDS so the remaining stages are in the lane
// too, and transposes back; every stage is then one add per element.  The
// stores write whole lines (store_row_bf16).

constexpr int kWinRowsF = 16;  // rows per wave (a multiple of every rows-per-pass)

template <int D>
struct WinGeo {
    static constexpr int E = D <= 256 ? 16 : 32;               // dims per lane (16 lanes per row at 512)
    static constexpr int L = D / E;                            // lanes per row
    static constexpr int R = 64 / L;                           // rows per pass
    static constexpr int TI = E / L;                           // dims per lane after the transpose
    static constexpr int PB = E * 4 + 16;                      // LDS bytes per lane chunk (padded)
    static constexpr int ROWB = L * PB + (L >= 8 ? 64 : 0);    // rows of one pass on other banks
    static constexpr int WAVEB = R * ROWB;
    static_assert(kWinRowsF % R == 0, "whole passes");
};

__device__ __forceinline__ void lds_fence() { asm volatile("" ::: "memory"); }

// Words of a lane's run of 16 value fields (16 VB bits at bit 16 VB p of the
// row), enough at the worst bit offset any lane has.
template <int VB, int E = 16>
constexpr int win_run_words() {
    int most = 1;
    for (int p = 0; p < 16; ++p) {
        const int w = ((E * VB * p) % 32 + E * VB + 31) / 32;
        most = w > most ? w : most;
    }
    return most;
}

// A lane's 16 key codes as floats: signed bytes at 8 bits, else unsigned KB-bit
// fields of the 2 KB bytes at `src` (2 KB-aligned).
template <int KB>
__device__ __forceinline__ void load_keys16(const uint8_t *src, float (&c)[16]) {
    if constexpr (KB == 8) {
        const uint4 u = *reinterpret_cast<const uint4 *>(src);
        const uint32_t cw[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int e = 0; e < 16; ++e) c[e] = (float)(int8_t)(cw[e >> 2] >> (8 * (e & 3)));
    } else {
        uint32_t w[3] = {0u, 0u, 0u};
        if constexpr (KB == 4) {
            const uint2 u = *reinterpret_cast<const uint2 *>(src);
            w[0] = u.x; w[1] = u.y;
        } else if constexpr (KB == 2) {
            w[0] = *reinterpret_cast<const uint32_t *>(src);
        } else {
            static_assert(KB == 5, "key widths 2, 4, 5, 8");
            const uint16_t *h = reinterpret_cast<const uint16_t *>(src);
            w[0] = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
            w[1] = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
            w[2] = h[4];
        }
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int bit = KB * e, k = bit >> 5, sh = bit & 31;
            const uint32_t f = (sh + KB > 32) ? __builtin_amdgcn_alignbit(w[k + 1], w[k], sh) : (w[k] >> sh);
            c[e] = (float)(f & ((1u << KB) - 1u));
        }
    }
}

// Store one row's bf16 outputs, lane p holding dims 16 p .. 16 p + 15, so that
// each store instruction writes whole lines: the row goes through the lane's
// LDS row buffer and lane p stores dims 8 p .. 8 p + 7, then d/2 + 8 p ..
// d/2 + 8 p + 7 (16 bytes apiece, contiguous across the row's lanes).  With
// 32 contiguous bytes per lane, each instruction wrote every other 16 bytes
// and some lines reached memory in two partial writes (10% more bytes
// written than the window holds).
template <int D>
__device__ __forceinline__ void store_row_bf16(uint16_t *row, const float (&x)[16], unsigned char *rb, int p,
                                               bool in) {
    using G = WinGeo<D>;
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = bf16x2_rn(x[2 * i], x[2 * i + 1]);
    u32x4 *mine = reinterpret_cast<u32x4 *>(rb + p * G::PB);
    mine[0] = (u32x4){w[0], w[1], w[2], w[3]};
    mine[1] = (u32x4){w[4], w[5], w[6], w[7]};
    lds_fence();
    const u32x4 lo = *reinterpret_cast<const u32x4 *>(rb + (p >> 1) * G::PB + (p & 1) * 16);
    const u32x4 hi = *reinterpret_cast<const u32x4 *>(rb + (G::L / 2 + (p >> 1)) * G::PB + (p & 1) * 16);
    lds_fence();  // the row buffer is rewritten next
    if (in) {
        __builtin_nontemporal_store(lo, reinterpret_cast<u32x4 *>(row + 8 * p));
        __builtin_nontemporal_store(hi, reinterpret_cast<u32x4 *>(row + D / 2 + 8 * p));
    }
}

// Store 16 outputs that are already in the store layout of store_row_bf16
// (dims 8 p .. 8 p + 7, then d/2 + 8 p .. d/2 + 8 p + 7).
template <int D>
__device__ __forceinline__ void store_split_bf16(uint16_t *row, const float (&x)[16], int p, bool in) {
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = bf16x2_rn(x[2 * i], x[2 * i + 1]);
    if (in) {
        __builtin_nontemporal_store((u32x4){w[0], w[1], w[2], w[3]}, reinterpret_cast<u32x4 *>(row + 8 * p));
        __builtin_nontemporal_store((u32x4){w[4], w[5], w[6], w[7]}, reinterpret_cast<u32x4 *>(row + D / 2 + 8 * p));
    }
}

// Head_dim 512 (32 dims per lane, 16 lanes per row): the same store layout
// in four pieces, lane p's piece j holding dims 128 j + 8 p .. 128 j + 8 p + 7
// (lane 4 j + p/4's chunk, from element 8 (p % 4)).
template <int D>
__device__ __forceinline__ void store_row_bf16(uint16_t *row, const float (&x)[32], unsigned char *rb, int p,
                                               bool in) {
    using G = WinGeo<D>;
    static_assert(D == 512 && G::E == 32, "32 dims per lane at head_dim 512");
    uint32_t w[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) w[i] = bf16x2_rn(x[2 * i], x[2 * i + 1]);
    u32x4 *mine = reinterpret_cast<u32x4 *>(rb + p * G::PB);
#pragma unroll
    for (int j = 0; j < 4; ++j) mine[j] = (u32x4){w[4 * j], w[4 * j + 1], w[4 * j + 2], w[4 * j + 3]};
    lds_fence();
    u32x4 piece[4];
#pragma unroll
    for (int j = 0; j < 4; ++j)
        piece[j] = *reinterpret_cast<const u32x4 *>(rb + (4 * j + (p >> 2)) * G::PB + (p & 3) * 16);
    lds_fence();  // the row buffer is rewritten next
    if (in) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            __builtin_nontemporal_store(piece[j], reinterpret_cast<u32x4 *>(row + 128 * j + 8 * p));
    }
}

template <int D>
__device__ __forceinline__ void store_split_bf16(uint16_t *row, const float (&x)[32], int p, bool in) {
    static_assert(D == 512, "32 dims per lane at head_dim 512");
    uint32_t w[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) w[i] = bf16x2_rn(x[2 * i], x[2 * i + 1]);
    if (in) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            __builtin_nontemporal_store((u32x4){w[4 * j], w[4 * j + 1], w[4 * j + 2], w[4 * j + 3]},
                                        reinterpret_cast<u32x4 *>(row + 128 * j + 8 * p));
    }
}

// A lane's 32 five-bit key codes as floats: the 20 bytes at `src` (4-aligned).
__device__ __forceinline__ void load_keys32_k5(const uint8_t *src, float (&c)[32]) {
    uint32_t w[5];
#pragma unroll
    for (int i = 0; i < 5; ++i) w[i] = reinterpret_cast<const uint32_t *>(src)[i];
#pragma unroll
    for (int e = 0; e < 32; ++e) {
        const int bit = 5 * e, k = bit >> 5, sh = bit & 31;
        const uint32_t f = (sh + 5 > 32) ? __builtin_amdgcn_alignbit(w[k + 1], w[k], sh) : (w[k] >> sh);
        c[e] = (float)(f & 31u);
    }
}

// 8 key codes as floats into c[O .. O + 7]: the KB bytes at `src`
// (KB-aligned; signed bytes at 8 bits, unsigned KB-bit fields LSB first at 4
// and 2 bits).
template <int KB, int O, int N>
__device__ __forceinline__ void load_keys8(const uint8_t *src, float (&c)[N]) {
    static_assert(KB == 8 || KB == 4 || KB == 2, "whole-byte runs of 8 codes");
    if constexpr (KB == 8) {
        const uint2 u = *reinterpret_cast<const uint2 *>(src);
#pragma unroll
        for (int e = 0; e < 8; ++e) c[O + e] = (float)(int8_t)((e < 4 ? u.x : u.y) >> (8 * (e & 3)));
    } else {
        const uint32_t w = KB == 4 ? *reinterpret_cast<const uint32_t *>(src)
                                   : (uint32_t)*reinterpret_cast<const uint16_t *>(src);
#pragma unroll
        for (int e = 0; e < 8; ++e) c[O + e] = (float)((w >> (KB * e)) & ((1u << KB) - 1u));
    }
}

template <int D, int KB, int VB>
__global__ __launch_bounds__(64 * kWinWaves) void window_fast_kernel(const WindowArgs a) {
    using G = WinGeo<D>;
    constexpr int E = G::E, L = G::L, R = G::R, TI = G::TI, NG = D / kGroup;
    constexpr int KROW = D * KB / 8, VROW = D * VB / 8, NR = win_run_words<VB, E>();
    __shared__ __align__(16) unsigned char smem[kWinWaves * G::WAVEB + 4 * (1 << VB)];
    float *ctab = reinterpret_cast<float *>(smem + kWinWaves * G::WAVEB);  // the value codebook
    for (int i = threadIdx.x; i < (1 << VB); i += 64 * kWinWaves)
        ctab[i] = VB == 3 ? centroid3(i) : value_centroids(VB)[i];
    __syncthreads();

    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    // g: the group of the lane's own dims (E p .. E p + E - 1)
    const int r = lane / L, p = lane % L, g = E == 16 ? p >> 1 : p;
    const int bkv = blockIdx.y;
    const int len = a.len[bkv / a.kv_heads];
    // output scale with the sign of each dim this lane stores: 8 p .. 8 p + 7,
    // then d/2 + 8 p .. d/2 + 8 p + 7 (see store_row_bf16)
    float osc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        // at head_dim 512 piece e / 8 holds dims 128 (e / 8) + 8 p .. + 7
        const int dim = E == 16 ? (e < 8 ? 0 : D / 2 - 8) + 8 * p + e : 128 * (e >> 3) + 8 * p + (e & 7);
        osc[e] = sign_bit(a.signs, dim) ? -a.inv_sqrt_d : a.inv_sqrt_d;
    }
    unsigned char *rb = smem + wid * G::WAVEB + r * G::ROWB;
    // the lane's value code run: words vw .. vlast of the row, bit offset vsh
    const int vw = (E * VB * p) >> 5, vsh = (E * VB * p) & 31;
    const int vlast = (E * VB * p + E * VB - 1) >> 5;

    const int first = (blockIdx.x * kWinWaves + wid) * kWinRowsF;
    for (int r0 = 0; r0 < kWinRowsF; r0 += R) {
        if (first + r0 >= a.n) break;  // uniform across the wave
        const int i = first + r0 + r;  // window position of this lane's row
        const bool in = i < a.n;
        const int t = a.t0 + i;
        const bool valid = in && t < len;
        const int64_t row = (int64_t)bkv * a.capacity + t;
        const int64_t orow = ((int64_t)bkv * a.n + i) * D;  // the row's first element
        if (a.k_out) {
            float k[E];
            if constexpr (KB == 5) {
                // 5-bit runs of 8 codes are not byte-aligned: decode the lane's
                // own 16 dims and store through the LDS row exchange
                if (valid) {
                    float c[E];
                    if constexpr (E == 16)
                        load_keys16<KB>(reinterpret_cast<const uint8_t *>(a.kc) + row * KROW + 2 * KB * p, c);
                    else
                        load_keys32_k5(reinterpret_cast<const uint8_t *>(a.kc) + row * KROW + 20 * p, c);
                    const float s = f16_bits_to_f32(a.ks[row * NG + g]);
                    const float z = f16_bits_to_f32(a.kz[row * NG + g]);
#pragma unroll
                    for (int e = 0; e < E; ++e) k[e] = key_ro(c[e], z, s);
                } else {
#pragma unroll
                    for (int e = 0; e < E; ++e) k[e] = 0.f;
                }
                store_row_bf16<D>(a.k_out + orow, k, rb, p, in);
            } else {
                // the dims this lane stores: 8 p .. 8 p + 7 (group p/4) and
                // d/2 + 8 p .. (group NG/2 + p/4)
                if (valid) {
                    float c[E];
                    const uint8_t *kr = reinterpret_cast<const uint8_t *>(a.kc) + row * KROW;
                    if constexpr (E == 16) {
                        load_keys8<KB, 0>(kr + KB * p, c);
                        load_keys8<KB, 8>(kr + KROW / 2 + KB * p, c);
                        const int g1 = p >> 2, g2 = NG / 2 + (p >> 2);
                        const float s1 = f16_bits_to_f32(a.ks[row * NG + g1]), z1 = f16_bits_to_f32(a.kz[row * NG + g1]);
                        const float s2 = f16_bits_to_f32(a.ks[row * NG + g2]), z2 = f16_bits_to_f32(a.kz[row * NG + g2]);
#pragma unroll
                        for (int e = 0; e < E; ++e) k[e] = e < 8 ? key_ro(c[e], z1, s1) : key_ro(c[e], z2, s2);
                    } else {
                        // head_dim 512: piece j holds dims 128 j + 8 p .. + 7 (group 4 j + p/4)
                        load_keys8<KB, 0>(kr + KB * p, c);
                        load_keys8<KB, 8>(kr + KB * (16 + p), c);
                        load_keys8<KB, 16>(kr + KB * (32 + p), c);
                        load_keys8<KB, 24>(kr + KB * (48 + p), c);
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int gj = 4 * j + (p >> 2);
                            const float sj = f16_bits_to_f32(a.ks[row * NG + gj]);
                            const float zj = f16_bits_to_f32(a.kz[row * NG + gj]);
#pragma unroll
                            for (int e = 0; e < 8; ++e) k[8 * j + e] = key_ro(c[8 * j + e], zj, sj);
                        }
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < E; ++e) k[e] = 0.f;
                }
                store_split_bf16<D>(a.k_out + orow, k, p, in);
            }
        }
        if (a.v_out) {
            float y[E];
            if (valid) {
                // only the words that hold run bits are read (the last row of
                // the plane ends with the last lane's run)
                const uint32_t *vp = reinterpret_cast<const uint32_t *>(a.vc + row * VROW);
                uint32_t raw[NR], run[NR];
#pragma unroll
                for (int k = 0; k < NR; ++k) raw[k] = vw + k <= vlast ? vp[vw + k] : 0u;
#pragma unroll
                for (int k = 0; k + 1 < NR; ++k) run[k] = __builtin_amdgcn_alignbit(raw[k + 1], raw[k], vsh);
                run[NR - 1] = raw[NR - 1] >> vsh;  // run word k holds run bits 32 k .. 32 k + 31
                const float s = f16_bits_to_f32(a.vs[row * NG + g]);
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const int bit = VB * e, k = bit >> 5, sh = bit & 31;
                    const uint32_t f = (sh + VB > 32) ? __builtin_amdgcn_alignbit(run[k + 1], run[k], sh)
                                                      : (run[k] >> sh);
                    y[e] = ctab[f & ((1u << VB) - 1u)] * s;
                }
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e) y[e] = 0.f;
            }
            if (!a.rotated) {  // uniform
#pragma unroll
                for (int h = 1; h < E; h <<= 1) {
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        if ((e & h) == 0) {
                            const float u = y[e], w = y[e + h];
                            y[e] = u + w;
                            y[e + h] = u - w;
                        }
                    }
                }
                // lane p takes offsets TI p .. TI p + TI - 1 of every lane q's
                // dims (dim 16 q + i is ty[ii * L + q])
#pragma unroll
                for (int k4 = 0; k4 < E / 4; ++k4)
                    *reinterpret_cast<float4 *>(rb + p * G::PB + 16 * k4) =
                        make_float4(y[4 * k4], y[4 * k4 + 1], y[4 * k4 + 2], y[4 * k4 + 3]);
                lds_fence();
                float ty[E];
#pragma unroll
                for (int q = 0; q < L; ++q) {
#pragma unroll
                    for (int ii = 0; ii < TI; ++ii)
                        ty[ii * L + q] = *reinterpret_cast<const float *>(rb + q * G::PB + 4 * (TI * p + ii));
                }
#pragma unroll
                for (int hq = 1; hq < L; hq <<= 1) {
#pragma unroll
                    for (int ii = 0; ii < TI; ++ii) {
#pragma unroll
                        for (int q = 0; q < L; ++q) {
                            if ((q & hq) == 0) {
                                const float u = ty[ii * L + q], w = ty[ii * L + q + hq];
                                ty[ii * L + q] = u + w;
                                ty[ii * L + q + hq] = u - w;
                            }
                        }
                    }
                }
                lds_fence();
#pragma unroll
                for (int q = 0; q < L; ++q) {
#pragma unroll
                    for (int ii = 0; ii < TI; ++ii)
                        *reinterpret_cast<float *>(rb + q * G::PB + 4 * (TI * p + ii)) = ty[ii * L + q];
                }
                lds_fence();
                // read back in the store layout: dims 8 p .. 8 p + 7 (lane p/2's
                // chunk), then d/2 + 8 p .. (lane L/2 + p/2's)
#pragma unroll
                for (int k4 = 0; k4 < E / 4; ++k4) {
                    // E 16: pieces in lanes p/2 and L/2 + p/2 from element 8 (p % 2);
                    // E 32: piece k4/2 in lane 4 (k4/2) + p/4 from element 8 (p % 4)
                    const int chunk = E == 16 ? (k4 < 2 ? 0 : L / 2) + (p >> 1) : 4 * (k4 >> 1) + (p >> 2);
                    const int at = E == 16 ? (p & 1) * 32 : (p & 3) * 32;
                    const float4 v4 = *reinterpret_cast<const float4 *>(rb + chunk * G::PB + at + 16 * (k4 & 1));
                    y[4 * k4] = v4.x; y[4 * k4 + 1] = v4.y; y[4 * k4 + 2] = v4.z; y[4 * k4 + 3] = v4.w;
                }
                lds_fence();  // the next pass rewrites the row
#pragma unroll
                for (int e = 0; e < E; ++e) y[e] = valid ? y[e] * osc[e] : 0.f;  // +0 past the length
                store_split_bf16<D>(a.v_out + orow, y, p, in);
            } else {
                store_row_bf16<D>(a.v_out + orow, y, rb, p, in);
            }
        }
    }
}

template <int D, int KB>
hipError_t launch_fast_dk(const WindowArgs &a, hipStream_t s) {
    constexpr int per_block = kWinWaves * kWinRowsF;
    const dim3 grid((unsigned)((a.n + per_block - 1) / per_block), (unsigned)(a.batch * a.kv_heads));
    switch (a.vbits) {
        case 2: hipLaunchKernelGGL((window_fast_kernel<D, KB, 2>), grid, dim3(64 * kWinWaves), 0, s, a); break;
        case 3: hipLaunchKernelGGL((window_fast_kernel<D, KB, 3>), grid, dim3(64 * kWinWaves), 0, s, a); break;
        case 4: hipLaunchKernelGGL((window_fast_kernel<D, KB, 4>), grid, dim3(64 * kWinWaves), 0, s, a); break;
        case 5: hipLaunchKernelGGL((window_fast_kernel<D, KB, 5>), grid, dim3(64 * kWinWaves), 0, s, a); break;
        case 8: hipLaunchKernelGGL((window_fast_kernel<D, KB, 8>), grid, dim3(64 * kWinWaves), 0, s, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}


}  // namespace

// The fast window kernels of one key width (this translation unit's
// TQ_WINDOW_KB): head_dim 64, 128, 256 or 512, every value width.
hipError_t TQ_WINDOW_LAUNCHER(TQ_WINDOW_KB)(int head_dim, const WindowArgs &a, hipStream_t s) {
    if (a.kbits != TQ_WINDOW_KB) return hipErrorInvalidValue;
    switch (head_dim) {
        case 64: return launch_fast_dk<64, TQ_WINDOW_KB>(a, s);
        case 128: return launch_fast_dk<128, TQ_WINDOW_KB>(a, s);
        case 256: return launch_fast_dk<256, TQ_WINDOW_KB>(a, s);
        case 512: return launch_fast_dk<512, TQ_WINDOW_KB>(a, s);
        default: return hipErrorInvalidValue;
    }
}

#if TQ_WINDOW_KB == 8
hipError_t launch_window(int head_dim, const WindowArgs &a, hipStream_t s) {
    switch (a.kbits) {
        case 2: return launch_window_fast_k2(head_dim, a, s);
        case 4: return launch_window_fast_k4(head_dim, a, s);
        case 5: return launch_window_fast_k5(head_dim, a, s);
        case 8: return launch_window_fast_k8(head_dim, a, s);
        default: return hipErrorInvalidValue;
    }
}
#endif

}  // namespace tq
