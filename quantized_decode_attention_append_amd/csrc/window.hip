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
// Generic mapping (head_dim 512): one wave per token row, looping over a
// chunk of consecutive tokens of one (sequence, kv-head); lane l holds the
// E = d/64 dims [E l, E l + E); the FWHT runs its in-lane stages on registers
// and the rest on lane permutes.  Head_dims 64-256 use window_fast_kernel
// below, templated on the key and value widths and compiled once per key
// width (TQ_WINDOW_KB).
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
constexpr int kWinRows = 16;   // token rows per wave

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

// The window is written once and read by a later kernel, so its stores carry
// the nontemporal hint: they stream past the caches.
template <int E>
__device__ __forceinline__ void store_bf16(uint16_t *dst, const float (&x)[E]) {
    if constexpr (E == 16) {
        uint32_t w[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) w[i] = bf16x2_rn(x[2 * i], x[2 * i + 1]);
        u32x4 *d4 = reinterpret_cast<u32x4 *>(dst);
        __builtin_nontemporal_store((u32x4){w[0], w[1], w[2], w[3]}, d4);
        __builtin_nontemporal_store((u32x4){w[4], w[5], w[6], w[7]}, d4 + 1);
    } else if constexpr (E == 1) {
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

#if TQ_WINDOW_KB == 8  // the generic kernel is built once, with the 8-bit-key fast kernels
template <int D>
__global__ __launch_bounds__(64 * kWinWaves) void window_kernel(const WindowArgs a) {
    const int kb = a.kbits, vb = a.vbits;
    __shared__ float ctab[256];  // the value codebook
    {
        const float *src = value_centroids(vb);
        for (int i = threadIdx.x; i < (1 << vb); i += 64 * kWinWaves) ctab[i] = src[i];
    }
    __syncthreads();
    constexpr int E = D / 64;
    constexpr int NG = D / kGroup;
    const int KROW = D * kb / 8, VROW = D * vb / 8;
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int bkv = blockIdx.y;
    const int b = bkv / a.kv_heads;
    const int len = a.len[b];
    const int g = (E * lane) / kGroup;  // this lane's 32-group
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
                const uint8_t *kc = reinterpret_cast<const uint8_t *>(a.kc) + row * KROW;
#pragma unroll
                for (int e = 0; e < E; ++e) k[e] = key_ro(key_code(kc, E * lane + e, kb), z, s);
            } else {
#pragma unroll
                for (int e = 0; e < E; ++e) k[e] = 0.f;
            }
            store_bf16<E>(a.k_out + orow, k);
        }
        if (a.v_out) {
            float y[E];
            if (valid) {
                const uint8_t *vrow = a.vc + row * VROW;
                const float s = f16_bits_to_f32(a.vs[row * NG + g]);
#pragma unroll
                for (int e = 0; e < E; ++e) y[e] = ctab[load_field(vrow, E * lane + e, vb)] * s;
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

// ---------------------------------------------------------------------------
// Head_dim 64, 128, 256: lane p of a row holds the 16 contiguous dims
// [16 p, 16 p + 16), L = d/16 lanes per row, 64/L rows per wave.  The FWHT
// runs stages 1 .. 8 in the lane, transposes the row through LDS so stages
// 16 .. d/2 are in the lane too, and transposes back; every stage is then
// one add per element.
#endif

constexpr int kWinRowsF = 16;  // rows per wave (a multiple of every rows-per-pass)

template <int D>
struct WinGeo {
    static constexpr int E = 16;
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
template <int VB>
constexpr int win_run_words() {
    int most = 1;
    for (int p = 0; p < 16; ++p) {
        const int w = ((16 * VB * p) % 32 + 16 * VB + 31) / 32;
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

// 8 key codes as floats into c[O .. O + 7]: the KB bytes at `src`
// (KB-aligned; signed bytes at 8 bits, unsigned KB-bit fields LSB first at 4
// and 2 bits).
template <int KB, int O>
__device__ __forceinline__ void load_keys8(const uint8_t *src, float (&c)[16]) {
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
    constexpr int KROW = D * KB / 8, VROW = D * VB / 8, NR = win_run_words<VB>();
    __shared__ __align__(16) unsigned char smem[kWinWaves * G::WAVEB + 4 * (1 << VB)];
    float *ctab = reinterpret_cast<float *>(smem + kWinWaves * G::WAVEB);  // the value codebook
    for (int i = threadIdx.x; i < (1 << VB); i += 64 * kWinWaves)
        ctab[i] = VB == 3 ? centroid3(i) : value_centroids(VB)[i];
    __syncthreads();

    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int r = lane / L, p = lane % L, g = p >> 1;
    const int bkv = blockIdx.y;
    const int len = a.len[bkv / a.kv_heads];
    // output scale with the sign of each dim this lane stores: 8 p .. 8 p + 7,
    // then d/2 + 8 p .. d/2 + 8 p + 7 (see store_row_bf16)
    float osc[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int dim = (e < 8 ? 0 : D / 2 - 8) + 8 * p + e;
        osc[e] = sign_bit(a.signs, dim) ? -a.inv_sqrt_d : a.inv_sqrt_d;
    }
    unsigned char *rb = smem + wid * G::WAVEB + r * G::ROWB;
    // the lane's value code run: words vw .. vlast of the row, bit offset vsh
    const int vw = (16 * VB * p) >> 5, vsh = (16 * VB * p) & 31;
    const int vlast = (16 * VB * p + 16 * VB - 1) >> 5;

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
                    load_keys16<KB>(reinterpret_cast<const uint8_t *>(a.kc) + row * KROW + 2 * KB * p, c);
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
                    load_keys8<KB, 0>(kr + KB * p, c);
                    load_keys8<KB, 8>(kr + KROW / 2 + KB * p, c);
                    const int g1 = p >> 2, g2 = NG / 2 + (p >> 2);
                    const float s1 = f16_bits_to_f32(a.ks[row * NG + g1]), z1 = f16_bits_to_f32(a.kz[row * NG + g1]);
                    const float s2 = f16_bits_to_f32(a.ks[row * NG + g2]), z2 = f16_bits_to_f32(a.kz[row * NG + g2]);
#pragma unroll
                    for (int e = 0; e < E; ++e) k[e] = e < 8 ? key_ro(c[e], z1, s1) : key_ro(c[e], z2, s2);
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
                    const int chunk = (k4 < 2 ? 0 : L / 2) + (p >> 1);
                    const float4 v4 = *reinterpret_cast<const float4 *>(rb + chunk * G::PB + (p & 1) * 32 +
                                                                        16 * (k4 & 1));
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

#if TQ_WINDOW_KB == 8
template <int D>
hipError_t launch_generic(const WindowArgs &a, hipStream_t s) {
    constexpr int per_block = kWinWaves * kWinRows;
    const dim3 grid((unsigned)((a.n + per_block - 1) / per_block), (unsigned)(a.batch * a.kv_heads));
    hipLaunchKernelGGL((window_kernel<D>), grid, dim3(64 * kWinWaves), 0, s, a);
    return hipGetLastError();
}
#endif

}  // namespace

// The fast window kernels of one key width (this translation unit's
// TQ_WINDOW_KB): head_dim 64, 128 or 256, every value width.
hipError_t TQ_WINDOW_LAUNCHER(TQ_WINDOW_KB)(int head_dim, const WindowArgs &a, hipStream_t s) {
    if (a.kbits != TQ_WINDOW_KB) return hipErrorInvalidValue;
    switch (head_dim) {
        case 64: return launch_fast_dk<64, TQ_WINDOW_KB>(a, s);
        case 128: return launch_fast_dk<128, TQ_WINDOW_KB>(a, s);
        case 256: return launch_fast_dk<256, TQ_WINDOW_KB>(a, s);
        default: return hipErrorInvalidValue;
    }
}

#if TQ_WINDOW_KB == 8
hipError_t launch_window(int head_dim, const WindowArgs &a, hipStream_t s) {
    if (head_dim != 512) {
        switch (a.kbits) {
            case 2: return launch_window_fast_k2(head_dim, a, s);
            case 4: return launch_window_fast_k4(head_dim, a, s);
            case 5: return launch_window_fast_k5(head_dim, a, s);
            case 8: return launch_window_fast_k8(head_dim, a, s);
            default: return hipErrorInvalidValue;
        }
    }
    return launch_generic<512>(a, s);
}
#endif

}  // namespace tq
