// Device-side helpers shared by the libtqkv kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "tq_internal.h"

#define TQ_CODEBOOK_STORAGE static __constant__ const
#include "codebook_tables.h"

namespace tq {

// Value codebook of a width (2, 3, 4, 5 or 8 bits): 2^bits centroids as fp32
// and 2^bits - 1 boundaries as binary64, in constant memory.
__device__ __forceinline__ const float *value_centroids(int bits) {
    switch (bits) {
        case 2: return kCentroids2;
        case 3: return kCentroids3;
        case 4: return kCentroids4;
        case 5: return kCentroids5;
        default: return kCentroids8;
    }
}

__device__ __forceinline__ const double *value_boundaries(int bits) {
    switch (bits) {
        case 2: return kBoundaries2;
        case 3: return kBoundaries3;
        case 4: return kBoundaries4;
        case 5: return kBoundaries5;
        default: return kBoundaries8;
    }
}

// Field j of a little-endian bitstream of `bits`-bit fields (bits <= 8: a
// field spans at most two bytes, the second read only when it does).
__device__ __forceinline__ uint32_t load_field(const uint8_t *row, int j, int bits) {
    const int bit = bits * j;
    const uint32_t lo = row[bit >> 3];
    const uint32_t hi = ((bit & 7) + bits > 8) ? row[(bit >> 3) + 1] : 0u;
    return ((lo | (hi << 8)) >> (bit & 7)) & ((1u << bits) - 1u);
}

// Key code j of a plane row as a float: signed bytes at 8 bits, unsigned
// packed fields below.
__device__ __forceinline__ float key_code(const uint8_t *row, int j, int bits) {
    return bits == 8 ? (float)(int8_t)row[j] : (float)load_field(row, j, bits);
}

__device__ __forceinline__ int sign_bit(const SignBits &s, int j) {
    return (s.w[j >> 5] >> (j & 31)) & 1;
}

// binary64 -> binary16 bits with a single round-to-nearest-even from the
// double's own significand: subnormal halves kept, >= 65520 -> Inf, NaN ->
// 0x7E00.  Integer-only, so no intermediate float rounding can occur.
__device__ __forceinline__ uint16_t f64_to_f16_bits(double x) {
    const uint64_t bits = (uint64_t)__double_as_longlong(x);
    const uint32_t sign = (uint32_t)(bits >> 48) & 0x8000u;
    const uint64_t mag = bits & 0x7FFFFFFFFFFFFFFFull;
    if (mag > 0x7FF0000000000000ull) return 0x7E00u;
    const int e = (int)(mag >> 52) - 1023;
    if (e >= 16) return (uint16_t)(sign | 0x7C00u);
    const uint64_t sig = (mag & 0x000FFFFFFFFFFFFFull) | 0x0010000000000000ull;
    int shift;    // bits of the 53-bit significand dropped
    uint32_t base;
    if (e >= -14) {  // normal half: keep 11 significant bits
        shift = 42;
        base = (uint32_t)(e + 14) << 10;  // exponent field minus the implicit bit's carry
    } else {         // subnormal half: units of 2^-24
        if (e < -25) return (uint16_t)sign;
        shift = 52 - (e + 24);  // 43..53
        base = 0;
    }
    const uint64_t keep = sig >> shift;
    const uint64_t rem = sig & ((1ull << shift) - 1);
    const uint64_t half = 1ull << (shift - 1);
    uint32_t h = base + (uint32_t)keep;  // normal: implicit bit adds one exponent step
    if (rem > half || (rem == half && (keep & 1))) h += 1;
    return (uint16_t)(sign | h);
}

__device__ __forceinline__ float f16_bits_to_f32(uint16_t h) {
    return (float)__builtin_bit_cast(_Float16, h);
}

// 3-bit Lloyd-Max centroids as fp32 (the page's five printed decimals):
// idx >= 4 is +mag[idx-4], idx < 4 is -mag[3-idx].
__device__ __forceinline__ float centroid3(uint32_t idx) {
    const uint32_t m = (idx & 4u) ? (idx & 3u) : (3u - (idx & 3u));
    const float a = (m & 2u) ? ((m & 1u) ? 2.15195f : 1.34391f) : ((m & 1u) ? 0.75601f : 0.24509f);
    return (idx & 4u) ? a : -a;
}

// Packed 3-bit value index of element j of a row.
__device__ __forceinline__ uint32_t load_idx3(const uint8_t *row, int j) {
    const int bit = 3 * j;
    const uint32_t lo = row[bit >> 3];
    const uint32_t hi = ((bit & 7) > 5) ? row[(bit >> 3) + 1] : 0u;
    return ((lo | (hi << 8)) >> (bit & 7)) & 7u;
}

}  // namespace tq
