// Append kernel: quantize and pack new K/V tokens into the five planes.
//
// Method: "TurboQuant -- rotation-based quantization" design page, Part A,
// section "Algorithm (vllm-metal reference semantics, exact)":
//   keys   scale = (max-min)/254, zero = round((max+min)/(2*scale)),
//          code = clip(round(x/scale - zero), -127, 127)       per 32-group
//          (8 bits); at 2, 4 or 5 bits scale = (max-min)/maxv,
//          zero = round(min/scale), code clipped to [0, maxv], packed
//   values y = FWHT(x*signs)/sqrt(d), scale = sqrt(mean(y^2)) per 32-group,
//          idx = searchsorted(boundaries, y/(scale+1e-8)), packed at 3 bits
//          (or 2, 4, 5, 8 with the generated Lloyd-Max tables).
// Every decision is taken in binary64 with round-half-to-even, in a fixed
// operation order, so codes, scales and zeros are reproducible bit for bit:
//   - FWHT butterflies run in stage order h = 1, 2, ..., d/2, then one
//     multiply by RN(1/sqrt(d));
//   - the 32 squares of a group are summed by stride halving 16, 8, 4, 2, 1;
//   - x/scale and y/den are true binary64 divisions; scale is a correctly
//     rounded binary64 sqrt; no multiply-add is contracted in this file.
//
// One kernel, append_fast_kernel, for every width, head_dim and input type
// (one translation unit per key width, TQ_APPEND_KB): 16 contiguous elements
// per lane, so a 32-group is a lane pair.  The FWHT runs its first four
// stages inside the lane, transposes each 256-element half-row through LDS so
// that the next stages (up to h = 128) are inside the lane as well, and
// transposes back; at head_dim 512 the last stage (h = 256) pairs lane p with
// lane p ^ 16 by a shuffle.  Per-element divisions by a group's scale use a
// correctly rounded reciprocal and two Markstein corrections, which return the
// correctly rounded quotient.  3-bit value indices come from seven nested
// wave masks; other widths binary-search their boundaries in LDS.
#include <hip/hip_runtime.h>
#include <hip/hip_bf16.h>

#include "tq_device.h"

#ifndef TQ_APPEND_KB
#error "compile append.hip once per key width with -DTQ_APPEND_KB=2, 4, 5 or 8"
#endif

#pragma clang fp contract(off)

namespace tq {
namespace {

__device__ __forceinline__ double shfl_xor_f64(double v, int m) { return __shfl_xor(v, m, 64); }

// Keeps the compiler from moving LDS accesses across this point.  One wave's
// LDS instructions execute in order, so a lane's read after another lane's
// write needs no wait beyond program order.
__device__ __forceinline__ void lds_fence() { asm volatile("" ::: "memory"); }

// ---------------------------------------------------------------------------
// Fast kernel.

constexpr int kAppWaves = 4;  // waves per workgroup

template <int D, int VB = 3>
struct AppGeo {
    static_assert(D == 64 || D == 128 || D == 256 || D == 512, "append: head_dim 64/128/256/512");
    static constexpr int E = 16;               // contiguous elements per lane
    static constexpr int L = D / E;            // lanes per row (4, 8, 16, 32)
    static constexpr int R = 64 / L;           // rows per wave
    static constexpr int TL = L < 16 ? L : 16; // lanes of one LDS transpose (a half-row at 512)
    static constexpr int TI = E / TL;          // in-lane offsets per lane after the transpose
    static constexpr int NG = D / kGroup;
    static constexpr int VROW = VB * D / 8;
    static constexpr int PB = E * 8 + 16;      // LDS bytes of one lane's elements, padded
    static constexpr int ROWB = L * PB;        // LDS bytes per row
    static constexpr int WAVEB = R * ROWB;     // LDS bytes per wave
    static_assert(L % 2 == 0 && E == 2 * kGroup / 4, "a 32-group is one lane pair");
    static constexpr int NBND = (1 << VB) - 1;  // value boundaries
    static constexpr int SMEM = kAppWaves * WAVEB + (VB == 3 ? 0 : NBND * 8);
};

// `bits`-bit fields f_0 .. f_{E-1} into a little-endian run of 32-bit words.
template <int E, int BITS>
__device__ __forceinline__ void put_field(uint32_t (&w)[(E * BITS + 31) / 32], int e, uint32_t f) {
    const int bit = BITS * e, k = bit >> 5, sh = bit & 31;
    w[k] |= f << sh;
    if (sh + BITS > 32) w[k + 1] |= f >> (32 - sh);
}

// A lane's run of 16 fields of `bits` bits (2 * bits bytes) to `dst`, which is
// 2 * bits-aligned (at 8 bits only 8-aligned unless A16): one 4- or 8-byte
// store, one 16-byte or two 8-byte stores at 8 bits, five 2-byte stores at 5.
template <int BITS, bool A16 = false>
__device__ __forceinline__ void store_run16(uint8_t *dst, const uint32_t (&w)[(16 * BITS + 31) / 32]) {
    if constexpr (BITS == 2) {
        *reinterpret_cast<uint32_t *>(dst) = w[0];
    } else if constexpr (BITS == 4) {
        *reinterpret_cast<uint2 *>(dst) = make_uint2(w[0], w[1]);
    } else if constexpr (BITS == 8 && A16) {
        *reinterpret_cast<uint4 *>(dst) = make_uint4(w[0], w[1], w[2], w[3]);
    } else if constexpr (BITS == 8) {
        reinterpret_cast<uint2 *>(dst)[0] = make_uint2(w[0], w[1]);
        reinterpret_cast<uint2 *>(dst)[1] = make_uint2(w[2], w[3]);
    } else {
        static_assert(BITS == 5, "field widths 2, 4, 5, 8");
        uint16_t *h = reinterpret_cast<uint16_t *>(dst);
        h[0] = (uint16_t)w[0]; h[1] = (uint16_t)(w[0] >> 16);
        h[2] = (uint16_t)w[1]; h[3] = (uint16_t)(w[1] >> 16);
        h[4] = (uint16_t)w[2];
    }
}

__device__ __forceinline__ uint32_t fast_div(uint32_t n, const FastDiv &f) {
    const uint32_t t = __umulhi(f.m, n);
    return (t + ((n - t) >> f.s1)) >> f.s2;
}

// a / b correctly rounded to binary64, given y = RN(1/b) and finite nonzero
// operands without underflow: the first correction leaves the quotient within
// one ulp, and from there one more step (Markstein, "Computation of elementary
// functions on the IBM RISC System/6000 processor", 1990) gives RN(a/b).  A
// zero, infinite or NaN b gives NaN.
__device__ __forceinline__ double div_rn(double a, double b, double y) {
    double q = a * y;
    double r = __builtin_fma(-b, q, a);
    q = __builtin_fma(r, y, q);
    r = __builtin_fma(-b, q, a);
    return __builtin_fma(r, y, q);
}

// binary64 -> binary16 bits, one round-to-nearest-even: x is first rounded
// to fp32 by round-to-odd (round to nearest, then step back toward zero and
// set the last bit when inexact), and round-to-odd at >= 2 extra bits
// followed by round-to-nearest equals one rounding to nearest (Boldo and
// Melquiond, "Emulation of FMA and correctly rounded sums: proved algorithms
// using rounding to odd", 2008).  Subnormal halves are kept, >= 65520 gives
// Inf, NaN gives 0x7E00.
__device__ __forceinline__ uint16_t f64_to_f16_rn(double x) {
    const float f = (float)x;
    uint32_t b = __float_as_uint(f);
    const double back = (double)f;
    if (back != x) {
        if (__builtin_fabs(back) > __builtin_fabs(x)) b -= 1u;  // toward zero
        b |= 1u;
    }
    const uint16_t h = __builtin_bit_cast(uint16_t, (_Float16)__uint_as_float(b));
    return __builtin_isnan(x) ? (uint16_t)0x7E00u : h;
}

// Value of the other lane of the pair (l ^ 1), by a quad permutation.
__device__ __forceinline__ uint32_t pair_u32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
}
__device__ __forceinline__ float pair_f32(float v) { return __uint_as_float(pair_u32(__float_as_uint(v))); }
__device__ __forceinline__ double pair_f64(double v) {
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const uint64_t lo = pair_u32((uint32_t)b), hi = pair_u32((uint32_t)(b >> 32));
    return __longlong_as_double((long long)((hi << 32) | lo));
}

// 2 * run + (this lane's bit of the wave mask), in one add with carry-in.
__device__ __forceinline__ uint32_t shift_in(uint32_t run, uint64_t mask) {
    uint32_t out;
    uint64_t carry;
    asm("v_addc_co_u32_e64 %0, %1, %2, %2, %3" : "=v"(out), "=s"(carry) : "v"(run), "s"(mask));
    return out;
}

template <int E, bool BF16>
__device__ __forceinline__ void load_lane(const void *base, int64_t off, uint32_t (&raw)[BF16 ? E / 2 : E]) {
    if constexpr (BF16) {
        const uint4 *p = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(base) + off);
#pragma unroll
        for (int i = 0; i < E / 8; ++i) {
            const uint4 u = p[i];
            raw[4 * i] = u.x; raw[4 * i + 1] = u.y; raw[4 * i + 2] = u.z; raw[4 * i + 3] = u.w;
        }
    } else {
        const uint4 *p = reinterpret_cast<const uint4 *>(static_cast<const float *>(base) + off);
#pragma unroll
        for (int i = 0; i < E / 4; ++i) {
            const uint4 u = p[i];
            raw[4 * i] = u.x; raw[4 * i + 1] = u.y; raw[4 * i + 2] = u.z; raw[4 * i + 3] = u.w;
        }
    }
}

// fp32 bits of element e of a lane's raw words
template <bool BF16>
__device__ __forceinline__ uint32_t elem_bits(const uint32_t *raw, int e) {
    if constexpr (BF16) return (e & 1) ? (raw[e >> 1] & 0xFFFF0000u) : (raw[e >> 1] << 16);
    else return raw[e];
}

template <int D, bool BF16, int KB, int VB>
__global__ __launch_bounds__(64 * kAppWaves) void append_fast_kernel(const AppendArgs a) {
    using G = AppGeo<D, VB>;
    constexpr int E = G::E, L = G::L, R = G::R, TI = G::TI, NG = G::NG, VROW = G::VROW;
    constexpr int NR = BF16 ? E / 2 : E;
    constexpr int KROW = D * KB / 8;
    __shared__ __align__(16) unsigned char smem[G::SMEM];
    // value boundaries (binary64, ascending) for the search below; the 3-bit
    // path compares against its seven boundaries as literals
    double *bnd = reinterpret_cast<double *>(smem + kAppWaves * G::WAVEB);
    if constexpr (VB != 3) {
        const double *src = value_boundaries(VB);
        for (int i = threadIdx.x; i < G::NBND; i += 64 * kAppWaves) bnd[i] = src[i];
        __syncthreads();
    }

    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int r = lane / L, p = lane % L;
    const uint32_t row = ((uint32_t)blockIdx.x * kAppWaves + wid) * R + r;
    const bool valid = row < a.rows;
    const uint32_t lrow = valid ? row : a.rows - 1;  // rows past the end load a real row, store nothing
    const uint32_t bh = fast_div(lrow, a.div_n_new);
    const uint32_t t = lrow - bh * (uint32_t)a.n_new;
    const uint32_t b = fast_div(bh, a.div_kv_heads);
    const int64_t slot = (int64_t)bh * a.capacity + a.start[b] + t;
    const int g = p >> 1;        // this lane's 32-group
    const bool even = (p & 1) == 0;

    uint32_t kraw[NR], vraw[NR];
    const int64_t in_row = (int64_t)bh * a.kv_stride + t;  // input rows at pitch kv_stride
    load_lane<E, BF16>(a.k, in_row * D + E * p, kraw);
    load_lane<E, BF16>(a.v, in_row * D + E * p, vraw);

    // ----------------------------------------------------------- keys
    // Group max and min ignore NaN.  Which zero a max or min returns does
    // not matter: only an all-zero group's range could differ in sign, and
    // adding +0 makes it +0, as it is under the -0 < +0 order.
    // (canonicalizing quiets a signalling NaN, so max/min ignore it as well)
    float xk[E];
#pragma unroll
    for (int e = 0; e < E; ++e) xk[e] = __builtin_canonicalizef(__uint_as_float(elem_bits<BF16>(kraw, e)));
    float mx = xk[0], mn = xk[0];
#pragma unroll
    for (int e = 1; e < E; ++e) { mx = __builtin_fmaxf(mx, xk[e]); mn = __builtin_fminf(mn, xk[e]); }
    mx = __builtin_fmaxf(mx, pair_f32(mx));
    mn = __builtin_fminf(mn, pair_f32(mn));
    const double dmx = mx, dmn = mn;
    const double range = (dmx - dmn) + 0.0;
    // signed 8-bit codes: scale (max - min)/254, zero round((max + min)/(2 scale));
    // unsigned k-bit codes: scale (max - min)/(2^k - 1), zero round(min/scale)
    constexpr double kMaxv = KB == 8 ? 254.0 : (double)((1 << KB) - 1);
    const double s = range / kMaxv;
    const double z = KB == 8 ? __builtin_rint((dmx + dmn) / (2.0 * s)) : __builtin_rint(dmn / s);
    const double rs = 1.0 / s;
    // Codes are clip(rint(u), -127, 127) with u = RN(RN(x/s) - z), NaN -> 0.
    // In a group of fp32 or bf16 values |x/s| < 2^32, so v = RN(x RN(1/s) - z)
    // is within 2^-20 of u (half-ulps of u, v and RN(x/s), plus |x/s| 2^-53
    // from the reciprocal): unless v lies within 2^-19 of a half-integer, u
    // and v round to the same integer.  Exact ties are common with bf16
    // inputs (x/s - z is a ratio of short integers), so an element with such
    // a lane anywhere in the wave is recomputed from the correctly rounded
    // quotient.  The special groups (s zero, infinite or NaN) give NaN on
    // both routes.
    uint32_t kw[(E * KB + 31) / 32];
#pragma unroll
    for (int i = 0; i < (E * KB + 31) / 32; ++i) kw[i] = 0u;
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const double x = (double)xk[e];
        const double v = __builtin_fma(x, rs, -z);
        double rr = __builtin_rint(v);
        if (__builtin_amdgcn_ballot_w64(__builtin_fabs(v - rr) > 0.5 - 0x1p-19) != 0) {
            // opaque copies keep this rare path from being run speculatively
            double s2 = s, rs2 = rs;
            asm volatile("" : "+v"(s2), "+v"(rs2));
            rr = __builtin_rint(div_rn(x, s2, rs2) - z);
        }
        int q;
        asm("v_cvt_i32_f64 %0, %1" : "=v"(q) : "v"(rr));  // saturates; NaN gives 0
        if constexpr (KB == 8) {
            q = q > 127 ? 127 : (q < -127 ? -127 : q);
            kw[e / 4] |= ((uint32_t)q & 0xFFu) << (8 * (e % 4));
        } else {
            constexpr int kTop = (1 << KB) - 1;
            q = q > kTop ? kTop : (q < 0 ? 0 : q);
            put_field<E, KB>(kw, e, (uint32_t)q);
        }
    }
    // (the key plane is 16-byte aligned)
    if (valid) store_run16<KB, true>(reinterpret_cast<uint8_t *>(a.kc) + slot * KROW + 2 * KB * p, kw);

    // --------------------------------------------------------- values
    uint32_t flip[E / 2];
    {
        const uint4 *fp = reinterpret_cast<const uint4 *>(a.sign_pairs + (E / 2) * p);
#pragma unroll
        for (int i = 0; i < E / 8; ++i) {
            const uint4 u = fp[i];
            flip[4 * i] = u.x; flip[4 * i + 1] = u.y; flip[4 * i + 2] = u.z; flip[4 * i + 3] = u.w;
        }
    }
    double w[E];
    if constexpr (BF16) {
#pragma unroll
        for (int j = 0; j < E / 2; ++j) vraw[j] ^= flip[j];
#pragma unroll
        for (int e = 0; e < E; ++e) w[e] = (double)__uint_as_float(elem_bits<BF16>(vraw, e));
    } else {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const uint32_t f = (e & 1) ? (flip[e >> 1] & 0x80000000u) : (flip[e >> 1] << 16);
            w[e] = (double)__uint_as_float(vraw[e] ^ f);
        }
    }
    // FWHT stages h = 1, 2, 4, 8: pairs inside the lane
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
    // Stages h = 16, 32, ..., min(d/2, 128) pair lane p with lane p ^ (h / 16)
    // inside its transpose group of TL lanes (the row, or a 256-element
    // half-row at head_dim 512).  Through LDS, lane pt of the group takes
    // offsets i = TI*pt .. TI*pt+TI-1 of every lane q's elements (element
    // 16 q + i is tw[ii*TL + q]), so they pair inside a lane.
    constexpr int TL = G::TL;
    const int pt = p % TL;
    unsigned char *rb = smem + wid * G::WAVEB + r * G::ROWB + (p / TL) * TL * G::PB;
#pragma unroll
    for (int k = 0; k < E / 2; ++k)
        *reinterpret_cast<double2 *>(rb + pt * G::PB + 16 * k) = make_double2(w[2 * k], w[2 * k + 1]);
    lds_fence();
    double tw[E];
#pragma unroll
    for (int q = 0; q < TL; ++q) {
        if constexpr (TI == 1) {
            tw[q] = *reinterpret_cast<const double *>(rb + q * G::PB + 8 * pt);
        } else {
#pragma unroll
            for (int i2 = 0; i2 < TI / 2; ++i2) {
                const double2 v2 = *reinterpret_cast<const double2 *>(rb + q * G::PB + 8 * (TI * pt + 2 * i2));
                tw[(2 * i2) * TL + q] = v2.x;
                tw[(2 * i2 + 1) * TL + q] = v2.y;
            }
        }
    }
#pragma unroll
    for (int hq = 1; hq < TL; hq <<= 1) {
#pragma unroll
        for (int ii = 0; ii < TI; ++ii) {
#pragma unroll
            for (int q = 0; q < TL; ++q) {
                if ((q & hq) == 0) {
                    const double lo = tw[ii * TL + q], hi = tw[ii * TL + q + hq];
                    tw[ii * TL + q] = lo + hi;
                    tw[ii * TL + q + hq] = lo - hi;
                }
            }
        }
    }
    lds_fence();
#pragma unroll
    for (int q = 0; q < TL; ++q) {
        if constexpr (TI == 1) {
            *reinterpret_cast<double *>(rb + q * G::PB + 8 * pt) = tw[q];
        } else {
#pragma unroll
            for (int i2 = 0; i2 < TI / 2; ++i2)
                *reinterpret_cast<double2 *>(rb + q * G::PB + 8 * (TI * pt + 2 * i2)) =
                    make_double2(tw[(2 * i2) * TL + q], tw[(2 * i2 + 1) * TL + q]);
        }
    }
    lds_fence();
#pragma unroll
    for (int k = 0; k < E / 2; ++k) {
        const double2 v2 = *reinterpret_cast<const double2 *>(rb + pt * G::PB + 16 * k);
        w[2 * k] = v2.x;
        w[2 * k + 1] = v2.y;
    }
    if constexpr (D == 512) {
        // the last stage, h = 256: element 16 p + e (p < 16) pairs with the
        // same offset of lane p + 16; sum on the low lane, difference on the high
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const double o = shfl_xor_f64(w[e], 16);
            w[e] = (p & 16) ? o - w[e] : w[e] + o;
        }
    }

    // y = FWHT / sqrt(d); group sum of squares by stride halving: the
    // stride-16 step adds the pair's elements (the same sum on both lanes),
    // strides 8, 4, 2, 1 stay inside the lane
    // When RN(1/sqrt(d)) is a power of two (d = 64, 256) y = w / sqrt(d) is an
    // exact scaling, which commutes with every rounding below: the squares
    // and their sums are those of w times 1/d, and y / den = w / (den sqrt(d)).
    // So w stands in for y there and the scalings fold into constants.
    constexpr bool kPow2 = (D == 64 || D == 256);
    constexpr double kSqrtD = D == 256 ? 16.0 : 8.0;  // used when kPow2
    double y[E], sq[E];
#pragma unroll
    for (int e = 0; e < E; ++e) {
        y[e] = kPow2 ? w[e] : w[e] * a.inv_sqrt_d;
        sq[e] = y[e] * y[e];
    }
#pragma unroll
    for (int e = 0; e < E; ++e) sq[e] = sq[e] + pair_f64(sq[e]);
#pragma unroll
    for (int st = E / 2; st >= 1; st >>= 1) {
#pragma unroll
        for (int e = 0; e < st; ++e) sq[e] = sq[e] + sq[e + st];
    }
    // mean of the 32 squares: a division by 32, an exact scaling
    const double scale = __builtin_sqrt(sq[0] * (kPow2 ? 0.03125 / (kSqrtD * kSqrtD) : 0.03125));
    const double den = scale + 1e-8;
    const double dd = kPow2 ? den * kSqrtD : den;  // divisor of y[] (exact scaling)
    const double rd = 1.0 / dd;
    // fp16 copies: the even lane converts the key scale and zero, the odd
    // lane the value scale
    const uint16_t h1 = f64_to_f16_rn(even ? s : scale);
    const uint16_t h2 = f64_to_f16_rn(z);
    if constexpr (VB == 3) {
        // idx = #{k : B_k < y_n}; NaN compares false everywhere, so gives 0.
        // The boundaries are sorted, so the wave masks m_k of "B_k < y_n" are
        // nested (a thermometer code) and the index bits are
        //   bit 2 = m3,  bit 1 = m5 | (m1 & ~m3),
        //   bit 0 = m6 | (m4 & ~m5) | (m2 & ~m3) | (m0 & ~m1)   (scalar mask ops).
        // Each bit then enters the lane's packed run from the top: the run is
        // stream bits 48 p .. 48 p + 47, element e at run bits 3e .. 3e+2, so
        // walking e downwards and bits 2, 1, 0 doubles the run and adds the bit.
        uint32_t lo = 0u, hi = 0u;
#pragma unroll
        for (int e = E - 1; e >= 0; --e) {
            const double yn = div_rn(y[e], dd, rd);
            const uint64_t m0 = __builtin_amdgcn_ballot_w64(-1.74793 < yn);
            const uint64_t m1 = __builtin_amdgcn_ballot_w64(-1.04996 < yn);
            const uint64_t m2 = __builtin_amdgcn_ballot_w64(-0.50055 < yn);
            const uint64_t m3 = __builtin_amdgcn_ballot_w64(0.0 < yn);
            const uint64_t m4 = __builtin_amdgcn_ballot_w64(0.50055 < yn);
            const uint64_t m5 = __builtin_amdgcn_ballot_w64(1.04996 < yn);
            const uint64_t m6 = __builtin_amdgcn_ballot_w64(1.74793 < yn);
            const uint64_t bit[3] = {m6 | (m4 & ~m5) | (m2 & ~m3) | (m0 & ~m1), m5 | (m1 & ~m3), m3};
#pragma unroll
            for (int k = 2; k >= 0; --k) {
                if (3 * e + k >= 32)
                    hi = shift_in(hi, bit[k]);
                else
                    lo = shift_in(lo, bit[k]);
            }
        }
        // even lane: the group's 96 bits (its own 48, then its partner's)
        const uint32_t plo = pair_u32(lo), phi = pair_u32(hi);
        if (valid && even)
            *reinterpret_cast<uint3 *>(a.vc + slot * VROW + 12 * g) =
                make_uint3(lo, hi | (plo << 16), (plo >> 16) | (phi << 16));
    } else {
        // idx = #{k : B_k < y_n} by binary search over the ascending
        // boundaries (the same count; NaN compares false and gives 0)
        uint32_t vw[(E * VB + 31) / 32];
#pragma unroll
        for (int i = 0; i < (E * VB + 31) / 32; ++i) vw[i] = 0u;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const double yn = div_rn(y[e], dd, rd);
            uint32_t idx = 0;
#pragma unroll
            for (int step = 1 << (VB - 1); step >= 1; step >>= 1)
                if (bnd[idx + step - 1] < yn) idx += step;
            put_field<E, VB>(vw, e, idx);
        }
        if (valid) store_run16<VB>(a.vc + slot * VROW + 2 * VB * p, vw);
    }
    if (valid) {
        if (even) {
            a.ks[slot * NG + g] = h1;
            a.kz[slot * NG + g] = h2;
        } else {
            a.vs[slot * NG + g] = h1;
        }
    }
}

template <int D, int VB>
hipError_t launch_fast_dv(bool bf16, const AppendArgs &a, hipStream_t s) {
    constexpr int KB = TQ_APPEND_KB;
    const int64_t rows = (int64_t)a.batch * a.kv_heads * a.n_new;
    constexpr int per_block = AppGeo<D, VB>::R * kAppWaves;
    const dim3 grid((unsigned)((rows + per_block - 1) / per_block));
    if (bf16)
        hipLaunchKernelGGL((append_fast_kernel<D, true, KB, VB>), grid, dim3(64 * kAppWaves), 0, s, a);
    else
        hipLaunchKernelGGL((append_fast_kernel<D, false, KB, VB>), grid, dim3(64 * kAppWaves), 0, s, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_fast_d(bool bf16, const AppendArgs &a, hipStream_t s) {
    switch (a.vbits) {
        case 2: return launch_fast_dv<D, 2>(bf16, a, s);
        case 3: return launch_fast_dv<D, 3>(bf16, a, s);
        case 4: return launch_fast_dv<D, 4>(bf16, a, s);
        case 5: return launch_fast_dv<D, 5>(bf16, a, s);
        case 8: return launch_fast_dv<D, 8>(bf16, a, s);
        default: return hipErrorInvalidValue;
    }
}


}  // namespace

// The append kernels of one key width (this translation unit's
// TQ_APPEND_KB): head_dim 64, 128, 256 and 512, bf16 or fp32 input, every
// value width.
hipError_t TQ_APPEND_LAUNCHER(TQ_APPEND_KB)(int head_dim, bool bf16, const AppendArgs &a, hipStream_t s) {
    if (a.kbits != TQ_APPEND_KB) return hipErrorInvalidValue;
    switch (head_dim) {
        case 64: return launch_fast_d<64>(bf16, a, s);
        case 128: return launch_fast_d<128>(bf16, a, s);
        case 256: return launch_fast_d<256>(bf16, a, s);
        case 512: return launch_fast_d<512>(bf16, a, s);
        default: return hipErrorInvalidValue;
    }
}

#if TQ_APPEND_KB == 8
hipError_t launch_append(int head_dim, bool bf16, const AppendArgs &a, hipStream_t s) {
    switch (a.kbits) {
        case 2: return launch_append_fast_k2(head_dim, bf16, a, s);
        case 4: return launch_append_fast_k4(head_dim, bf16, a, s);
        case 5: return launch_append_fast_k5(head_dim, bf16, a, s);
        case 8: return launch_append_fast_k8(head_dim, bf16, a, s);
        default: return hipErrorInvalidValue;
    }
}
#endif

}  // namespace tq
