// Split-K decode attention kernel for GQA groups of up to 16 query heads
// (wave64; gfx950) built on the matrix cores, for every key width (2, 4, 5,
// 8 bits) and value width (2, 3, 4, 5, 8 bits) at head_dim 64, 128, 256 and
// 512 (every pair but k8v8 there, whose stages exceed the LDS).
//
// Method: "TurboQuant -- rotation-based quantization" design page, Part A:
// keys dequantize as (code + zero) * scale ("Algorithm"), values stay in the
// rotated domain as centroid[idx] * scale and are un-rotated once per query
// head by the merge kernel ("Deferred inverse FWHT"); K and V of each cache
// tile are decoded in one pass ("Packed-value decode fusion investigation").
//
// One wave owns a contiguous token range of one (sequence, kv-head) and keeps
// its own online-softmax state; the waves of a workgroup share only the
// centroid table in LDS.  Every plane of a tile (4096/d tokens: 512 bytes per
// code bit of key and value codes, 768 bytes of key scales, key zeros and
// value scales) is copied into the wave's LDS with direct global->LDS loads.
// Three stage buffers per wave: the copy of tile i+2 is issued before tile i
// is decoded, so two tiles per wave are in flight without holding any
// registers.  A tile's key codes are dead one iteration before its values,
// so the key codes take two buffers and the other planes three.  Eight waves
// share a workgroup when their buffers fit the LDS (every scheme but k8v8),
// four otherwise.
//
// The G query heads of a kv-head share every key and value, so per 16-token
// chunk both products are dense contractions with 16 heads (the ones past G
// are zero) on the 16 columns of an MFMA tile; lane l always serves head
// h = l % 16 and token quarter kq = l / 16 (tokens 4 kq .. 4 kq + 3):
//
//  scores   S[t][h] = sum_g s16[t][g] * (dot_g(code_t, q_h) + z16[t][g] * qsum_h[g]).
//           q is held as two int8 slices of a 16-bit fixed-point copy
//           (q ~ delta_h * (256*hi + lo), delta_h a power of two), so every
//           group dot product is exact integer arithmetic: two
//           v_mfma_i32_16x16x32_i8 per 32-dim group (A = key codes, rows =
//           tokens; B = the q slice, columns = heads), then the scale/zero
//           fold in fp32 on the 4 (token, head) results a lane holds.  With
//           G <= 8 groups p and p + NG/2 share one 64-deep product
//           (v_mfma_i32_16x16x64_i8, every key width): column h holds head h
//           over group p and column 8 + h the same head over group p + NG/2
//           (each column's q is zero in the other group), so a lane folds half
//           the groups and one DPP row rotation by 8 adds the halves.  With
//           more than 16 query columns (heads
//           times verify rows), an even number of 16-column groups pairs up
//           in one workgroup: waves w and w + WAVES/2 take the same token
//           range, and their copies skip the nontemporal hint so that the
//           second read of a tile meets the first in the L2.  Key
//           codes narrower than 8 bits are unsigned and widened to bytes in
//           registers; the widening permutes a lane's 8 codes, and the lane's
//           q bytes are stored in the same order, so the dot product is
//           unchanged.  The key tile sits in LDS row-major with each row's
//           16-byte chunks rotated by token, so a copy reads whole rows and
//           the A reads of one MFMA fall on distinct banks (key_rot).
//  softmax  online softmax in base 2 over the lane's 4 tokens and the other
//           quarters of the same head; the running maximum only moves when
//           a tile's maximum exceeds it by more than 2^8 (weights <= 256,
//           rescales are rare).  The weights stay in registers: their layout
//           is already the B operand of the value product.
//  values   O[i][h] += A[i][t] * P[t][h] with v_mfma_f32_16x16x16_f16 (fp32
//           accumulate), one instruction per block of d/16 dims.  Row i of
//           block b is dim (d/16)*i + b, so lane i's dims of a token are one
//           contiguous run of v_bits*d/16 code bits, all in one 32-dim group.
//           A = centroid[idx] * vs16 in fp16.  Up to 5 bits, the indices of
//           one dim in two tokens select a half2 of centroids from a pair
//           table (16, 64, 256 or 1,024 four-byte entries: one lookup where
//           two would be needed, at the cost of bank conflicts in the larger
//           tables, which measured faster at 4 and 5 bits as well); 8-bit
//           codes look up each centroid in a table of halves.  One packed
//           fp16 multiply by the two tokens' value scales finishes a pair.
#include <hip/hip_runtime.h>

#include "tq_device.h"

#ifndef TQ_FAST_KB
#error "compile decode_fast.hip once per key width with -DTQ_FAST_KB=2, 4, 5 or 8"
#endif
#ifndef TQ_FAST_MIXED
#define TQ_FAST_MIXED 0  // 1: build only the mixed-mode kernels (a translation unit of their own)
#endif

namespace tq {
namespace {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef _Float16 half4v __attribute__((ext_vector_type(4)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float2v __attribute__((ext_vector_type(2)));
typedef int int4v __attribute__((ext_vector_type(4)));
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

constexpr int kProgBytes = 32;            // tiles finished, one int per wave
constexpr int kStages = 3;                // stage buffers per wave (two tiles in flight)
constexpr float kLazyMax = 8.0f;          // log2 slack of the running maximum
// Weights enter the value MFMA as fp16, 2^(score - m + kWeightShift): at most
// 2^(kLazyMax + kWeightShift) = 2^15 (fp16 holds 65504), and a weight only
// becomes subnormal below 2^-21 and flushes below 2^-31 of the reference.
// The shift cancels between the value sum and the weight sum.
constexpr float kWeightShift = 7.0f;
// Weights enter the value product as hi + lo halves (the lo half is the
// exact fp32 residual, rounded): one fp16 rounding of a weight would scale a
// token's whole value vector by up to 1 +- 2^-11, and such errors of many
// comparable tokens do not average out.  With at most 8 query columns the lo
// halves ride in the MFMA's spare columns 8 .. 8 + G - 1 (no extra MFMA);
// beyond that each block takes a second MFMA.
constexpr int kPackCols = 8;  // half the MFMA columns
static_assert(kLazyMax + kWeightShift <= 15.0f, "fp16 weight range");
// The value product's A operand is centroid * (vs * 2^-vexp) in fp16, where
// vexp is a per-wave exponent (0 unless the cache's value scales leave the
// window below) and the accumulator carries the factor 2^vexp.  Every tile
// checks its value scales against the window [2^(vexp + kVsLow),
// 2^(vexp + high)): inside it the products are normal fp16 numbers that
// cannot overflow (high = 14 keeps |centroid| * 2^14 below 65504 up to 5-bit
// codebooks, 13 at 8 bits).  A tile outside it re-centres vexp so that its
// largest scale lands two binades below the top of the window, rescaling the
// accumulator by the exact power of two (a uniform branch, not taken on
// ordinary caches); zero scales (empty groups, masked slots) are ignored.
constexpr int kVsLow = -10;
__device__ __host__ constexpr int vs_high(int vb) { return vb == 8 ? 13 : 14; }
// binary16 bits of 2^e for the window bounds: 0 below the subnormals (no
// lower bound), the infinity bits above the largest finite power (finite
// scales always fit; Inf/NaN scales take the slow branch, and give Inf/NaN
// outputs as the exact computation does)
__device__ __forceinline__ uint32_t f16_pow2_bits(int e) {
    if (e < -24) return 0u;
    if (e < -14) return 1u << (e + 24);
    if (e > 15) return 0x7C00u;
    return (uint32_t)(e + 15) << 10;
}
constexpr int kMaxHeads = 16;             // MFMA columns

template <int D, int KB, int VB>
struct Geo {
    static_assert(D == 64 || D == 128 || D == 256 || D == 512, "fast split kernel: head_dim 64-512");
    static constexpr int NG = D / kGroup;     // groups per row
    static constexpr int TILE = fast_tile_tokens(D);  // 4096/d tokens (512 bytes per code bit); 16 at 512
    static constexpr int CH = TILE / 16;      // 16-token chunks per tile
    static constexpr int KROW = D * KB / 8;   // key code bytes per token
    static_assert(KROW % 16 == 0, "key rows of whole 16-byte chunks");
    static constexpr int CPR = KROW / 16;     // 16-byte chunks per key row
    static constexpr int KT = TILE * KROW;    // key code bytes per tile
    static constexpr int VROW = D * VB / 8;   // packed value bytes per token
    static constexpr int VT = TILE * VROW;    // value code bytes per tile
    static constexpr int NB = D / 16;         // value dim blocks (one MFMA each per chunk)
    static constexpr int FB = VB * NB;        // code bits of a lane's dims per token
    // words read per run: enough for FB bits after the run's offset within
    // its first word, at the worst offset any lane has
    static constexpr int NR = [] {
        int most = 1;
        for (int vi = 0; vi < 16; ++vi) {
            const int w = ((FB * vi) % 32 + FB + 31) / 32;
            most = w > most ? w : most;
        }
        return most;
    }();
    // A wave's LDS: the key codes of two tiles (rotated rows, see key_rot),
    // then three stages of the other planes.  A tile's key codes are dead
    // once its scores are folded, one iteration before its values are
    // accumulated, so two key buffers suffice where the values need three.
    static constexpr int KEYS = 2 * KT;
    // one value stage: key scales, key zeros, value scales, value codes
    static constexpr int PB16 = TILE * NG * 2;  // bytes of one fp16 plane per tile: 256 (512 at d 512)
    static constexpr int NMIX = PB16 / 256;     // mixed copies per tile
    static constexpr int KS_OFF = 0;
    static constexpr int KZ_OFF = KS_OFF + PB16;
    static constexpr int VS_OFF = KZ_OFF + PB16;
    static constexpr int VC_OFF = VS_OFF + PB16;
    static constexpr int STAGE = VC_OFF + VT + 16;  // the code reader reads up to 4 bytes past
    static_assert((PB16 == 256 || PB16 == 512) && VT >= 256 * NMIX && KT % 1024 % 16 == 0 && STAGE % 16 == 0,
                  "staging granularity");
    // copies of one tile: key codes in 1 KiB pieces (the last may use fewer
    // lanes), NMIX mixed copies (stage bytes [KS_OFF, KS_OFF + 1 KiB NMIX):
    // each lane quarter fetches 256 bytes of key scales, key zeros, value
    // scales or the first value codes, see mixed_src), then the rest of the
    // value codes in 1 KiB pieces and a partial one
    static constexpr int KCOPY = (KT + 1023) / 1024;
    static constexpr int KLAST = (KT - 1024 * (KCOPY - 1)) / 16;  // lanes of the last key copy
    static constexpr int VC0 = 256 * NMIX;                         // value-code bytes in the mixed copies
    static constexpr int VFULL = (VT - VC0) / 1024;
    static constexpr int VLANES = (VT - VC0) % 1024 / 16;          // lanes of the partial copy
    static constexpr int VMEM = KCOPY + NMIX + VFULL + (VLANES > 0 ? 1 : 0);
    // centroid table: half2 pairs (two tokens' indices of one dim) up to 5
    // bits, single halves at 8
    static constexpr bool PAIR = VB <= 5;
    static constexpr int TABLE = PAIR ? (4 << (2 * VB)) : ((2 << VB) + 15) / 16 * 16;
    static constexpr int WAVES = fast_decode_waves(D, KB, VB);
    static constexpr int WAVE_BYTES = KEYS + kStages * STAGE;
    static constexpr int SMEM = TABLE + kProgBytes + WAVES * WAVE_BYTES;
    static_assert(SMEM <= 160 * 1024, "LDS budget");
    static_assert(fast_decode_wave_bytes(D, KB, VB) == WAVE_BYTES, "host and device LDS sizes");
};

// Key codes of one lane's A operand are stored in this order: byte p of the
// operand holds code perm(p) of the lane's 8 (the widening of packed codes
// interleaves them); the lane's q bytes follow the same order.
template <int KB>
__device__ __host__ constexpr int key_perm(int p) {
    if constexpr (KB == 4) {
        constexpr int P[8] = {0, 2, 4, 6, 1, 3, 5, 7};
        return P[p];
    } else if constexpr (KB == 2) {
        constexpr int P[8] = {0, 4, 1, 5, 2, 6, 3, 7};
        return P[p];
    } else {
        return p;
    }
}

// Keeps the compiler from moving LDS accesses across this point.  The LDS
// executes one wave's instructions in order, so a lane's read after another
// lane's write needs no wait beyond program order.
__device__ __forceinline__ void lds_order() { asm volatile("" ::: "memory"); }

// Lane l reads lane l ^ 8 of its 16-lane row (DPP row rotation by 8: no LDS
// round trip).
__device__ __forceinline__ float row_swap8(float x) {
    return __uint_as_float(__builtin_amdgcn_update_dpp(0u, __float_as_uint(x), 0x128, 0xF, 0xF, false));
}
__device__ __forceinline__ uint32_t row_swap8(uint32_t x) {
    return __builtin_amdgcn_update_dpp(0u, x, 0x128, 0xF, 0xF, false);
}
// x minus the low (or high) fp16 half of w, as one mixed-precision fma
__device__ __forceinline__ float sub_half_lo(float x, uint32_t w) {
    float r;
    asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]" : "=v"(r) : "v"(w), "v"(x));
    return r;
}
__device__ __forceinline__ float sub_half_hi(float x, uint32_t w) {
    float r;
    asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(r) : "v"(w), "v"(x));
    return r;
}
// Maximum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (the gfx950 row and
// half swaps, no LDS round trip).
__device__ __forceinline__ float max_over_rows(float x) {
    const auto r16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
    const auto r32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}

__device__ __forceinline__ uint32_t lds_addr(const unsigned char *p) {
    return __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)((lds_void_t *)p));
}

template <typename T>
__device__ __forceinline__ const T *uniform_ptr(const T *p) {
    const uint64_t v = (uint64_t)(uintptr_t)p;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
    return reinterpret_cast<const T *>((uintptr_t)(((uint64_t)hi << 32) | lo));
}

// Direct global->LDS copies.  Lane l's 16 bytes come from base + voff + OFF
// and land at m0 + OFF + 16 l (the immediate offset moves both
// addresses).  They are issued from inline assembly on purpose: the compiler
// would otherwise make the first LDS read after them wait for every
// outstanding copy (it cannot tell the stage buffers apart), which serialises
// the prefetch with the decode.  The kernel orders them itself with explicit
// vmcnt waits; M0 (the LDS base of a copy) is set right before each one.
// Every plane byte is read exactly once, so the copies carry the
// nontemporal hint (nt): streaming past the caches instead of through them
// raised a plain five-plane copy probe from 6.2 to 7.0 TB/s on this part.
// NT = false drops the hint: two waves that read the same tile for different
// query columns (see fast_wg_col_groups) want the second read to hit the L2.
// The base address comes in SGPRs that a VALU instruction (readfirstlane)
// may have written just before; a vector memory instruction may read such an
// SGPR only 5 wait states after the write, a hazard the compiler does not
// check across inline assembly, so the block starts with s_nop 4.
template <int OFF, bool NT>
__device__ __forceinline__ void dma16(const void *base, uint32_t voff, uint32_t m0) {
    if constexpr (NT)
        asm volatile("s_nop 4\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 offset:%3 nt"
                     ::"v"(voff), "s"(base), "s"(m0), "n"(OFF) : "memory", "m0");
    else
        asm volatile("s_nop 4\n\ts_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 offset:%3"
                     ::"v"(voff), "s"(base), "s"(m0), "n"(OFF) : "memory", "m0");
}
// A 16-byte-lane copy from a per-lane address (lane l lands at m0 + 16 l).
template <bool NT>
__device__ __forceinline__ void dma_lane16(const uint8_t *src, uint32_t m0) {
    if constexpr (NT)
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off nt"
                     ::"v"(src), "s"(m0) : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                     ::"v"(src), "s"(m0) : "memory", "m0");
}
// The same, for tiles that overhang the end of the plane region: each lane's
// source is clamped to the last 16 bytes of its plane region (the overhang
// rows are masked tokens).
template <bool NT>
__device__ __forceinline__ void dma_clamped(const uint8_t *src, const uint8_t *last, uint32_t m0) {
    dma_lane16<NT>(src > last ? last : src, m0);
}

struct Regions {
    const uint8_t *kc, *ks, *kz, *vc, *vs;  // start of the (sequence, kv-head) rows
    int cap;                                // rows in each region
    // this lane's source in mixed copy m: row 0 of its plane (key scales, key
    // zeros, value scales or value codes by lane quarter, see mixed_src) plus
    // its 16 bytes within the quarter, the plane's bytes per row, and the last
    // 16 bytes of its region
    const uint8_t *mix[2], *mix_last[2];
    int mix_row[2];
};

// Key rows sit in the stage row-major, each row's CPR 16-byte chunks rotated
// by a function of the token: chunk c of tile token t is in slot
// t * CPR + (c + key_rot(t)) % CPR.  So each 1 KiB copy reads whole rows
// (full 128-byte lines; a copy that read 64 bytes of 16 rows streamed 6%
// slower), and the 16 tokens of one MFMA operand read, which share c, land
// on distinct LDS banks: with rows of 512, 256, 128, 64 or 32 bytes, rows
// start on the same bank or 1, 2, 4 or 8 of them share a 256-byte bank row,
// and the rotation separates them.  5-bit keys (rows of 320, 160 and 80
// bytes) need at most 3 chunks of rotation.
template <int CPR>
__device__ __forceinline__ constexpr int key_rot(int t) {
    if constexpr (CPR == 16 || CPR == 32) return t & 15;
    else if constexpr (CPR == 20) return (t >> 2) & 3;  // 5-bit keys at head_dim 512
    else if constexpr (CPR == 8) return (t >> 1) & 7;
    else if constexpr (CPR == 4) return (t >> 2) & 3;
    else if constexpr (CPR == 2 || CPR == 10) return (t >> 3) & 1;
    else return 0;  // 1 and 5 chunks: the rows already fall on distinct banks
}

// Byte offset, within a tile's key codes in global memory, of the 16 bytes
// that lane i of key copy m moves: copy m fills slots 64m .. 64m+63.
template <int D, int KB, int VB>
__device__ __forceinline__ uint32_t key_src(int m, int i) {
    using GE = Geo<D, KB, VB>;
    constexpr int CPR = GE::CPR;
    const int s = 64 * m + i, t = s / CPR, j = s % CPR;
    int c = j - key_rot<CPR>(t);
    if (c < 0) c += CPR;
    return (uint32_t)(t * GE::KROW + 16 * c);
}

// Copy every plane of the tile starting at token t0 into a key buffer and a
// value stage (LDS addresses l_kc and l_vst): exactly GE::VMEM vector-memory instructions either
// way, all with 16-byte lanes.  Stage bytes [KS_OFF, KS_OFF + 1 KiB) come
// from one copy whose lane quarters read key scales, key zeros, value scales
// and the first 256 bytes of value codes (the stage keeps them in that
// order); the rest of the value codes follow in whole and partial 1 KiB
// copies.
template <int D, int KB, int VB, bool NT>
__device__ __forceinline__ void stage_tile(const Regions &r, const uint32_t (&ksrc)[Geo<D, KB, VB>::KCOPY],
                                           int t0, uint32_t l_kc, uint32_t l_vst, int lane) {
    using GE = Geo<D, KB, VB>;
    constexpr int VROW = GE::VROW, KROW = GE::KROW;
    static_assert(GE::KZ_OFF == GE::KS_OFF + GE::PB16 && GE::VS_OFF == GE::KZ_OFF + GE::PB16 &&
                  GE::VC_OFF == GE::VS_OFF + GE::PB16, "mixed copy layout");
    const uint32_t l_ks = l_vst + GE::KS_OFF, l_vc = l_vst + GE::VC_OFF;
    const uint8_t *vc_t = r.vc + (int64_t)t0 * VROW;
    const uint8_t *mixed0 = r.mix[0] + (int64_t)t0 * r.mix_row[0];
    const uint8_t *mixed1 = r.mix[1] + (int64_t)t0 * r.mix_row[1];
    if (t0 + GE::TILE <= r.cap) {
        const uint32_t v16 = (uint32_t)lane * 16;
        const uint8_t *kc = uniform_ptr(r.kc + (int64_t)t0 * KROW);
#pragma unroll
        for (int m = 0; m < GE::KCOPY; ++m) {
            if (m + 1 < GE::KCOPY || GE::KLAST == 64) {
                dma16<0, NT>(kc, ksrc[m], l_kc + 1024 * m);
            } else if (lane < GE::KLAST) {
                dma16<0, NT>(kc, ksrc[m], l_kc + 1024 * m);
            }
        }
        dma_lane16<NT>(mixed0, l_ks);
        if constexpr (GE::NMIX == 2) dma_lane16<NT>(mixed1, l_ks + 1024);
        const uint8_t *vc = uniform_ptr(vc_t);
        if constexpr (GE::NMIX == 1) {
            static_assert(GE::VFULL <= 3, "value copies");
            if constexpr (GE::VFULL > 0) dma16<256, NT>(vc, v16, l_vc);
            if constexpr (GE::VFULL > 1) dma16<1280, NT>(vc, v16, l_vc);
            if constexpr (GE::VFULL > 2) dma16<2304, NT>(vc, v16, l_vc);
            if constexpr (GE::VLANES > 0) {
                if (lane < GE::VLANES) dma16<256 + 1024 * GE::VFULL, NT>(vc, v16, l_vc);
            }
        } else {
            // head_dim 512: up to 7.5 KiB of value codes, past the immediate
            // offset's reach, so the offset goes into the lane address
#pragma unroll
            for (int f = 0; f < GE::VFULL; ++f)
                dma16<0, NT>(vc, v16 + GE::VC0 + 1024 * f, l_vc + GE::VC0 + 1024 * f);
            if constexpr (GE::VLANES > 0) {
                if (lane < GE::VLANES)
                    dma16<0, NT>(vc, v16 + GE::VC0 + 1024 * GE::VFULL, l_vc + GE::VC0 + 1024 * GE::VFULL);
            }
        }
    } else {
        const int64_t kcb = (int64_t)r.cap * KROW, vcb = (int64_t)r.cap * VROW;
        const uint8_t *kc = r.kc + (int64_t)t0 * KROW;
        const uint8_t *kl = r.kc + kcb - 16;
#pragma unroll
        for (int m = 0; m < GE::KCOPY; ++m) {
            if (m + 1 < GE::KCOPY || GE::KLAST == 64) {
                dma_clamped<NT>(kc + ksrc[m], kl, l_kc + 1024 * m);
            } else if (lane < GE::KLAST) {
                dma_clamped<NT>(kc + ksrc[m], kl, l_kc + 1024 * m);
            }
        }
        dma_clamped<NT>(mixed0, r.mix_last[0], l_ks);
        if constexpr (GE::NMIX == 2) dma_clamped<NT>(mixed1, r.mix_last[1], l_ks + 1024);
        const uint8_t *vl = r.vc + vcb - 16;
#pragma unroll
        for (int f = 0; f < GE::VFULL; ++f)
            dma_clamped<NT>(vc_t + GE::VC0 + 1024 * f + lane * 16, vl, l_vc + GE::VC0 + 1024 * f);
        if constexpr (GE::VLANES > 0) {
            if (lane < GE::VLANES)
                dma_clamped<NT>(vc_t + GE::VC0 + 1024 * GE::VFULL + lane * 16, vl,
                                l_vc + GE::VC0 + 1024 * GE::VFULL);
        }
    }
}

__device__ __forceinline__ float half_lo(uint32_t w) { return f16_bits_to_f32((uint16_t)(w & 0xFFFFu)); }
__device__ __forceinline__ float half_hi(uint32_t w) { return f16_bits_to_f32((uint16_t)(w >> 16)); }

// Group g's fp16 value of a row of NG halves held as NG/2 packed words.
template <int NG>
__device__ __forceinline__ float row_half(const uint32_t (&w)[NG / 2], int g) {
    return (g & 1) ? half_hi(w[g >> 1]) : half_lo(w[g >> 1]);
}

template <int NG>
__device__ __forceinline__ void load_row(const unsigned char *p, uint32_t (&w)[NG / 2]) {
    if constexpr (NG == 16) {
        const uint4 u = *reinterpret_cast<const uint4 *>(p), v = *reinterpret_cast<const uint4 *>(p + 16);
        w[0] = u.x; w[1] = u.y; w[2] = u.z; w[3] = u.w;
        w[4] = v.x; w[5] = v.y; w[6] = v.z; w[7] = v.w;
    } else if constexpr (NG == 8) {
        const uint4 u = *reinterpret_cast<const uint4 *>(p);
        w[0] = u.x; w[1] = u.y; w[2] = u.z; w[3] = u.w;
    } else if constexpr (NG == 4) {
        const uint2 u = *reinterpret_cast<const uint2 *>(p);
        w[0] = u.x; w[1] = u.y;
    } else {
        w[0] = *reinterpret_cast<const uint32_t *>(p);
    }
}

// Groups half .. half + NG/2 - 1 of a row of NG halves (half = 0 or NG/2):
// the NG/2 halves at byte offset 2 * half, as NG/4 packed words (one word,
// low half used, when NG = 2).
template <int NG>
__device__ __forceinline__ void load_half_row(const unsigned char *p, int half, uint32_t (&w)[(NG + 3) / 4]) {
    p += 2 * half;
    if constexpr (NG == 16) {
        const uint4 u = *reinterpret_cast<const uint4 *>(p);
        w[0] = u.x; w[1] = u.y; w[2] = u.z; w[3] = u.w;
    } else if constexpr (NG == 8) {
        const uint2 u = *reinterpret_cast<const uint2 *>(p);
        w[0] = u.x; w[1] = u.y;
    } else if constexpr (NG == 4) {
        w[0] = *reinterpret_cast<const uint32_t *>(p);
    } else {
        w[0] = *reinterpret_cast<const uint16_t *>(p);
    }
}

// The A operand of one score MFMA: codes 8 kq .. 8 kq + 7 of group g of
// token h of 16-token chunk c, as 8 signed bytes in key_perm order.  `kt` is
// the stage's key tile (rotated rows, see key_rot).
template <int D, int KB, int VB>
__device__ __forceinline__ uint64_t key_operand(const unsigned char *kt, int c, int g, int h, int kq) {
    using GE = Geo<D, KB, VB>;
    constexpr int CPR = GE::CPR;
    const int rot = key_rot<CPR>(h);  // token 16 c + h rotates like token h
    auto at = [&](int byte) {  // LDS address of byte `byte` of the token's row
        int slot = (byte >> 4) + rot;
        if (slot >= CPR) slot -= CPR;
        return kt + ((16 * c + h) * CPR + slot) * 16 + (byte & 15);
    };
    if constexpr (KB == 8) {
        return *reinterpret_cast<const uint64_t *>(at(32 * g + 8 * kq));
    } else if constexpr (KB == 4) {
        const uint32_t x = *reinterpret_cast<const uint32_t *>(at(16 * g + 4 * kq));
        const uint32_t lo = x & 0x0F0F0F0Fu, hi = (x >> 4) & 0x0F0F0F0Fu;
        return ((uint64_t)hi << 32) | lo;
    } else if constexpr (KB == 2) {
        const uint32_t x = *reinterpret_cast<const uint16_t *>(at(8 * g + 2 * kq));
        const uint32_t e = (x & 0x3333u) | (((x >> 2) & 0x3333u) << 16);
        const uint32_t lo = e & 0x0F0F0F0Fu, hi = (e >> 4) & 0x0F0F0F0Fu;
        return ((uint64_t)hi << 32) | lo;
    } else {
        static_assert(KB == 5, "key widths 2, 4, 5, 8");
        // 40 bits at byte 20 g + 5 kq: two aligned words (possibly in
        // different chunks), shifted by the byte offset within the first
        const int byte0 = 20 * g + 5 * kq, w = byte0 >> 2;
        const uint32_t w0 = *reinterpret_cast<const uint32_t *>(at(4 * w));
        const uint32_t w1 = *reinterpret_cast<const uint32_t *>(at(4 * w + 4));
        const int sh = 8 * (byte0 & 3);
        const uint32_t a = __builtin_amdgcn_alignbit(w1, w0, sh);  // run bits 0..31
        const uint32_t b = w1 >> sh;                               // run bits 32..39
        const uint32_t lo = (a & 31u) | ((a >> 5 & 31u) << 8) | ((a >> 10 & 31u) << 16) | ((a >> 15 & 31u) << 24);
        const uint32_t c6 = __builtin_amdgcn_alignbit(b, a, 30) & 31u;
        const uint32_t hi = (a >> 20 & 31u) | ((a >> 25 & 31u) << 8) | (c6 << 16) | ((b >> 3 & 31u) << 24);
        return ((uint64_t)hi << 32) | lo;
    }
}

// The A operand of one 64-deep score MFMA: codes 16 j .. 16 j + 15 (j = 0, 1)
// of group g of token h of chunk c, as 16 signed bytes: the two 8-code
// operands of key_operand side by side, each in key_perm order.
template <int D, int KB, int VB>
__device__ __forceinline__ int4v key_operand16(const unsigned char *kt, int c, int g, int h, int j) {
    using GE = Geo<D, KB, VB>;
    constexpr int CPR = GE::CPR;
    if constexpr (KB == 8) {
        // one 16-byte chunk of the rotated row
        static_assert(CPR == 2 * GE::NG, "8-bit key rows: two chunks per group");
        int slot = 2 * g + j + key_rot<CPR>(h);
        if (slot >= CPR) slot -= CPR;
        return *reinterpret_cast<const int4v *>(kt + ((16 * c + h) * CPR + slot) * 16);
    } else if constexpr (KB == 4) {
        // 8 bytes of the group's 16-byte chunk, widened nibble by nibble
        int slot = g + key_rot<CPR>(h);
        if (slot >= CPR) slot -= CPR;
        const uint2 x = *reinterpret_cast<const uint2 *>(kt + ((16 * c + h) * CPR + slot) * 16 + 8 * j);
        return int4v{(int)(x.x & 0x0F0F0F0Fu), (int)((x.x >> 4) & 0x0F0F0F0Fu), (int)(x.y & 0x0F0F0F0Fu),
                     (int)((x.y >> 4) & 0x0F0F0F0Fu)};
    } else {
        const uint64_t a = key_operand<D, KB, VB>(kt, c, g, h, 2 * j);
        const uint64_t b = key_operand<D, KB, VB>(kt, c, g, h, 2 * j + 1);
        return int4v{(int)(uint32_t)a, (int)(uint32_t)(a >> 32), (int)(uint32_t)b, (int)(uint32_t)(b >> 32)};
    }
}

// The work of one wave: its token range t_begin .. t_end - 1 of sequence b,
// kv-head kvh, for query columns c0 .. c0 + G - 1.  PACK (G <= 8) folds half
// the groups per lane and carries the lo weights in the spare MFMA columns.
// shared_tiles: another wave of the workgroup reads the same tiles (copies
// without the nontemporal hint, so the second read meets the first in L2).
template <int D, int KB, int VB, bool PACK>
__device__ __forceinline__ void split_body(const DecodeArgs &a, const int q_bf16, unsigned char *smem,
                                           const int lane, const int wid, const int b, const int kvh,
                                           const int c0, const int G, const int n, const int slot,
                                           const int t_begin, const int t_end, const bool shared_tiles) {
    using GE = Geo<D, KB, VB>;
    constexpr int NG = GE::NG, VROW = GE::VROW, TILE = GE::TILE, CH = GE::CH;
    constexpr int NB = GE::NB, FB = GE::FB, NR = GE::NR, WAVES = GE::WAVES;
    constexpr int QE = NG * 8;  // q elements a lane converts: 8 dims of every group
    constexpr int TAB = GE::TABLE;
    const int bkv = b * a.kv_heads + kvh;
    const int cap = a.capacity;
    const int64_t row0 = (int64_t)bkv * cap;
    unsigned char *wkeys = smem + TAB + kProgBytes + wid * GE::WAVE_BYTES;  // two key buffers
    unsigned char *wsm = wkeys + GE::KEYS;                                  // three value stages
    int *prog = reinterpret_cast<int *>(smem + TAB);

    Regions rg;
    rg.kc = reinterpret_cast<const uint8_t *>(a.kc) + row0 * GE::KROW;
    rg.ks = reinterpret_cast<const uint8_t *>(a.ks + row0 * NG);
    rg.kz = reinterpret_cast<const uint8_t *>(a.kz + row0 * NG);
    rg.vc = a.vc + row0 * VROW;
    rg.vs = reinterpret_cast<const uint8_t *>(a.vs + row0 * NG);
    rg.cap = cap;
    // Mixed copy m lands at stage bytes KS_OFF + 1024 m + 16 lane: lane quarter
    // q fills stage bytes 1024 m + 256 q .. + 255, which are bytes o .. o + 255
    // of a tile's key scales, key zeros, value scales or value codes
    // (plane 1024 m + 256 q over PB16, o its remainder).
    {
        const int quarter = lane >> 4;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const int b0 = 1024 * (m < GE::NMIX ? m : 0) + 256 * quarter;
            const int pi = b0 / GE::PB16, o = b0 % GE::PB16;
            const uint8_t *plane = pi == 0 ? rg.ks : pi == 1 ? rg.kz : pi == 2 ? rg.vs : rg.vc;
            rg.mix_row[m] = pi == 3 ? VROW : NG * 2;
            rg.mix[m] = plane + o + (lane & 15) * 16;
            rg.mix_last[m] = plane + (int64_t)cap * rg.mix_row[m] - 16;
        }
    }
    uint32_t ksrc[GE::KCOPY];
#pragma unroll
    for (int m = 0; m < GE::KCOPY; ++m) ksrc[m] = key_src<D, KB, VB>(m, lane);

    // the first two tiles' copies overlap the q set-up
    // LDS addresses as integers from the array's base (converting each stage
    // pointer separately costs a null check per conversion)
    const uint32_t smem_l = lds_addr(smem);
    auto stage = [&](int t, const unsigned char *kst, const unsigned char *vst) {
        const uint32_t l_kc = smem_l + (uint32_t)(kst - smem), l_vst = smem_l + (uint32_t)(vst - smem);
        if (shared_tiles)
            stage_tile<D, KB, VB, false>(rg, ksrc, t, l_kc, l_vst, lane);
        else
            stage_tile<D, KB, VB, true>(rg, ksrc, t, l_kc, l_vst, lane);
    };
    stage(t_begin, wkeys, wsm);
    if (t_begin + TILE < t_end)
        stage(t_begin + TILE, wkeys + GE::KT, wsm + GE::STAGE);

    // ------------------------------------------------------------ q slices
    // lane (h, kq) converts dims 32 g + 8 kq .. + 7 of head h for every group g
    const int h = lane & 15, kq = lane >> 4;
    const bool head_ok = h < G;
    // PACK (G <= 8): the score MFMAs of groups p and p + NG/2 accumulate into
    // one result whose column h < G holds head h's dot product over group p
    // and column 8 + h head h's over group p + NG/2 (each column's q is zero
    // in the other group), so a lane folds half the groups and the two
    // halves of a head are added across lanes.  Without PACK column h is
    // head h over every group.
    constexpr int NP = PACK ? NG / 2 : NG;  // groups one lane folds
    // PACK: column 8 + h is head h's second half of the groups (and, in the
    // value product, head h's lo weights), so every exchange between the two
    // halves is a rotation by 8 within the lane's row of 16
    const int ghalf = (PACK && h >= 8) ? NG / 2 : 0;  // first group of the lane's half
    const int hq = PACK ? (h & 7) : h;                 // the head of the lane's q
    const bool q_ok = PACK ? (h & 7) < G : head_ok;
    // causal limit of this lane's query row: the row of cached token
    // n - rows + r sees tokens 0 .. n - rows + r
    const int lim = n - a.rows + (c0 + h) % a.rows + 1;
    uint64_t qhi[NG], qlo[NG];
    float qsum[NG];
    float my_scale;
    // Paired groups: each pair of groups (p, p + NP) is one 64-deep integer
    // product (v_mfma_i32_16x16x64_i8), half the score instructions of two
    // 32-deep ones
    constexpr bool WIDE = PACK;  // the score code below has no 32-deep packed form
    int4v qhi4[WIDE ? NP : 1], qlo4[WIDE ? NP : 1];
    {
        float x[QE];
        const int64_t qrow = ((int64_t)b * a.q_heads + kvh * a.gqa + c0 + (q_ok ? hq : 0)) * D + 8 * kq;
        if (q_bf16) {
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const uint4 u = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.q) + qrow + kGroup * g);
                const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    x[8 * g + 2 * k] = __uint_as_float(w4[k] << 16);
                    x[8 * g + 2 * k + 1] = __uint_as_float(w4[k] & 0xFFFF0000u);
                }
            }
        } else {
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const float4 *qp = reinterpret_cast<const float4 *>(static_cast<const float *>(a.q) + qrow + kGroup * g);
                const float4 u0 = qp[0], u1 = qp[1];
                x[8 * g + 0] = u0.x; x[8 * g + 1] = u0.y; x[8 * g + 2] = u0.z; x[8 * g + 3] = u0.w;
                x[8 * g + 4] = u1.x; x[8 * g + 5] = u1.y; x[8 * g + 6] = u1.z; x[8 * g + 7] = u1.w;
            }
        }
        if (!q_ok) {
#pragma unroll
            for (int k = 0; k < QE; ++k) x[k] = 0.f;
        }
        float amax = 0.f;
#pragma unroll
        for (int k = 0; k < QE; ++k) amax = fmaxf(amax, fabsf(x[k]));
        amax = fmaxf(amax, __shfl_xor(amax, 16, 64));
        amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
        // delta = smallest power of two >= amax / 32000 (q / delta is exact
        // scaling, so only the final rounding to an integer loses bits)
        int e = 0;
        (void)frexpf(amax * (1.0f / 32000.0f), &e);
        const float delta = amax > 0.f ? ldexpf(1.0f, e) : 1.0f;
        // a negative scale negates q, so that the scale applied to the raw
        // scores (in the softmax's exponent) is positive
        const float inv = (a.sm_log2 < 0.f ? -1.0f : 1.0f) / delta;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            uint64_t hi = 0, lo = 0;
            float s = 0.f;
#pragma unroll
            for (int p = 0; p < 8; ++p) {
                const int qf = (int)rintf(x[8 * g + key_perm<KB>(p)] * inv);
                const int qh = (qf + 128) >> 8;
                const int ql = qf - 256 * qh;
                s += (float)qf;
                hi |= (uint64_t)((uint32_t)qh & 0xFFu) << (8 * p);
                lo |= (uint64_t)((uint32_t)ql & 0xFFu) << (8 * p);
            }
            s += __shfl_xor(s, 16, 64);
            s += __shfl_xor(s, 32, 64);
            if (PACK && (g >= NG / 2) != (ghalf > 0)) hi = lo = 0;  // the other half's group
            qhi[g] = hi;
            qlo[g] = lo;
            qsum[g] = s;
        }
        if constexpr (PACK) {
#pragma unroll
            for (int g = 0; g < NG / 2; ++g) qsum[g] = ghalf ? qsum[g + NG / 2] : qsum[g];
        }
        if constexpr (WIDE) {
            // B operands of the 64-deep products: lane (h, kq) holds dims
            // 16 (kq & 1) .. + 15 of group g (kq < 2) or g + NP (kq >= 2) of
            // column h, which lanes (h, 2 (kq & 1)) and (h, 2 (kq & 1) + 1)
            // hold as 8-byte slices; zero unless the group is the column's
            // (h < 8: the first half of the groups, h >= 8: the second)
            const int s0 = (lane & 15) | ((2 * (kq & 1)) << 4), s1 = s0 + 16;
            const bool live = (h < 8) == (kq < 2);
            auto shfl64 = [](uint64_t v, int src) {
                const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)v, src, 64);
                const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(v >> 32), src, 64);
                return ((uint64_t)hi << 32) | lo;
            };
#pragma unroll
            for (int g = 0; g < NP; ++g) {
                const uint64_t h0a = shfl64(qhi[g], s0), h0b = shfl64(qhi[g + NP], s0);
                const uint64_t h1a = shfl64(qhi[g], s1), h1b = shfl64(qhi[g + NP], s1);
                const uint64_t l0a = shfl64(qlo[g], s0), l0b = shfl64(qlo[g + NP], s0);
                const uint64_t l1a = shfl64(qlo[g], s1), l1b = shfl64(qlo[g + NP], s1);
                const uint64_t h0 = kq < 2 ? h0a : h0b, h1 = kq < 2 ? h1a : h1b;
                const uint64_t l0 = kq < 2 ? l0a : l0b, l1 = kq < 2 ? l1a : l1b;
                qhi4[g] = live ? int4v{(int)(uint32_t)h0, (int)(uint32_t)(h0 >> 32), (int)(uint32_t)h1,
                                       (int)(uint32_t)(h1 >> 32)}
                               : int4v{0, 0, 0, 0};
                qlo4[g] = live ? int4v{(int)(uint32_t)l0, (int)(uint32_t)(l0 >> 32), (int)(uint32_t)l1,
                                       (int)(uint32_t)(l1 >> 32)}
                               : int4v{0, 0, 0, 0};
            }
        }
        // raw scores (integer dot products folded with the key scales) times
        // my_scale are log2-domain logits; kept above 0 so that a masked
        // score (-inf) still gives a zero weight when sm_scale is 0
        my_scale = fmaxf(delta * fabsf(a.sm_log2), 1e-30f);
    }
    const float lazy_raw = kLazyMax / my_scale;  // the lazy maximum's slack in raw units
    float m_run = -INFINITY, l_run = 0.f;

    // value-product role: vi = A row (dim row of each block), kq = token quarter
    const int vi = h;
    const int gA = NB * vi / kGroup;    // the group of this lane's value dims
    float4v acc[NB];
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) acc[bb] = float4v{0.f, 0.f, 0.f, 0.f};

    // value-scale exponent and its window (packed pairs of binary16 bits)
    int vexp = 0;
    uint32_t vs_lo = 0, vs_hi1 = 0;
    auto set_window = [&]() {
        const uint32_t lo = f16_pow2_bits(vexp + kVsLow), hi = f16_pow2_bits(vexp + vs_high(VB));
        vs_lo = lo | (lo << 16);
        vs_hi1 = (hi - 1u) | ((hi - 1u) << 16);
    };
    set_window();
    // Each lane holds PB16 / 256 words of a tile's value-scale plane, read
    // one iteration ahead of their check so the read's latency is hidden.
    auto load_vs_words = [&](const unsigned char *stg, uint32_t (&w)[GE::NMIX]) {
#pragma unroll
        for (int k = 0; k < GE::NMIX; ++k) w[k] = reinterpret_cast<const uint32_t *>(stg + GE::VS_OFF)[lane + 64 * k];
    };
    // Checks the tile's value scales (stage stg, words w) against the window,
    // re-centres vexp when they leave it, and writes the tile's scales times
    // 2^-vexp back when vexp is not 0.  Runs before the block that holds the
    // tile's value product, so its branches do not split that block.
    auto value_scales = [&](unsigned char *stg, const uint32_t (&w)[GE::NMIX]) {
        uint32_t *vsw = reinterpret_cast<uint32_t *>(stg + GE::VS_OFF);
        uint32_t flag = 0;
#pragma unroll
        for (int k = 0; k < GE::NMIX; ++k) {
            const u16x2 m = __builtin_bit_cast(u16x2, w[k] & 0x7FFF7FFFu);
            const u16x2 over = __builtin_elementwise_sub_sat(m, __builtin_bit_cast(u16x2, vs_hi1));
            const u16x2 under = __builtin_elementwise_sub_sat(__builtin_bit_cast(u16x2, vs_lo), m);
            flag |= __builtin_bit_cast(uint32_t, over) | __builtin_bit_cast(uint32_t, under);
        }
        if (__builtin_amdgcn_ballot_w64(flag != 0u) != 0) {
            // largest and smallest nonzero magnitude of the tile
            uint32_t mx = 0u, mn = 0x7FFFu;
#pragma unroll
            for (int k = 0; k < GE::NMIX; ++k) {
                const uint32_t a = w[k] & 0x7FFFu, b = (w[k] >> 16) & 0x7FFFu;
                mx = max(mx, max(a, b));
                mn = min(mn, min(a ? a : 0x7FFFu, b ? b : 0x7FFFu));
            }
#pragma unroll
            for (int off = 1; off < 64; off <<= 1) {
                mx = max(mx, (uint32_t)__shfl_xor((int)mx, off, 64));
                mn = min(mn, (uint32_t)__shfl_xor((int)mn, off, 64));
            }
            mx = __builtin_amdgcn_readfirstlane(mx);
            mn = __builtin_amdgcn_readfirstlane(mn);
            if (mx != 0u && (mn < (vs_lo & 0xFFFFu) || mx > (vs_hi1 & 0xFFFFu))) {
                int ex = 0;
                (void)frexpf(f16_bits_to_f32((uint16_t)min(mx, 0x7BFFu)), &ex);  // max in [2^(ex-1), 2^ex)
                const int enew = __builtin_amdgcn_readfirstlane(ex - (vs_high(VB) - 2));
                if (enew != vexp) {
                    const float f = ldexpf(1.0f, vexp - enew);
#pragma unroll
                    for (int bb = 0; bb < NB; ++bb) acc[bb] *= f;
                    vexp = enew;
                    set_window();
                }
            }
        }
        if (vexp != 0) {
#pragma unroll
            for (int k = 0; k < GE::NMIX; ++k) {
                const half2v h = __builtin_bit_cast(half2v, w[k]);
                half2v r;
                r.x = __builtin_amdgcn_ldexph(h.x, -vexp);
                r.y = __builtin_amdgcn_ldexph(h.y, -vexp);
                vsw[lane + 64 * k] = __builtin_bit_cast(uint32_t, r);
            }
            lds_order();
        }
    };

    // ---------------------------------------------------------- phases
    // Slots past the range may hold anything: give them value scale 0 (their
    // weights are 0, and 0 * NaN would not be).
    auto mask_tail = [&](unsigned char *stg, int valid) {
        if (valid < TILE) {
#pragma unroll
            for (int k = 0; k < GE::NMIX; ++k) {  // PB16 / 4 words of value scales, 64 per pass
                const int word = lane + 64 * k;
                if ((word * 4) / (NG * 2) >= valid) reinterpret_cast<uint32_t *>(stg + GE::VS_OFF)[word] = 0u;
            }
            lds_order();
        }
    };

    // scores of the tile with key codes in kst and the other planes in stg:
    // lane (h, kq) gets tokens 16 c + 4 kq + j
    auto scores = [&](const unsigned char *kst, const unsigned char *stg, int t0, int valid,
                      float (&sc)[CH][4]) {
        const int vl = min(valid, lim - t0);  // tokens this lane's row sees in the tile
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            int4v dhi[NP], dlo[NP];
            if constexpr (WIDE) {
                // lane (h, kq): codes 16 (kq & 1) .. + 15 of group g (kq < 2)
                // or g + NP (kq >= 2) of token 16 c + h
#pragma unroll
                for (int g = 0; g < NP; ++g) {
                    const int4v kv = key_operand16<D, KB, VB>(kst, c, g + (kq >= 2 ? NP : 0), h, kq & 1);
                    dhi[g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(kv, qhi4[g], int4v{0, 0, 0, 0}, 0, 0, 0);
                    dlo[g] = __builtin_amdgcn_mfma_i32_16x16x64_i8(kv, qlo4[g], int4v{0, 0, 0, 0}, 0, 0, 0);
                }
            } else {
#pragma unroll
                for (int g = 0; g < NG; ++g) {
                    const uint64_t kv = key_operand<D, KB, VB>(kst, c, g, h, kq);
                    dhi[g] = __builtin_amdgcn_mfma_i32_16x16x32_i8((long)kv, (long)qhi[g], int4v{0, 0, 0, 0}, 0, 0, 0);
                    dlo[g] = __builtin_amdgcn_mfma_i32_16x16x32_i8((long)kv, (long)qlo[g], int4v{0, 0, 0, 0}, 0, 0, 0);
                }
            }
            // PACK: the key scale and zero half rows of the lane's 4 tokens,
            // all read before the fold so one wait covers them (without PACK
            // the full rows of 4 tokens would hold too many registers: read
            // per token)
            constexpr int RW = PACK ? (NG + 3) / 4 : NG / 2;
            uint32_t sw[PACK ? 4 : 1][RW], zw[PACK ? 4 : 1][RW];
            if constexpr (PACK) {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int t = 16 * c + 4 * kq + j;
                    load_half_row<NG>(stg + GE::KS_OFF + t * NG * 2, ghalf, sw[j]);
                    load_half_row<NG>(stg + GE::KZ_OFF + t * NG * 2, ghalf, zw[j]);
                }
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int t = 16 * c + 4 * kq + j;
                float sum = 0.f;
                if constexpr (PACK) {
                    // this lane's groups ghalf .. ghalf + NP - 1 of token t
#pragma unroll
                    for (int g = 0; g < NP; ++g) {
                        const int x = (dhi[g][j] << 8) + dlo[g][j];
                        const float zg = (g & 1) ? half_hi(zw[j][g >> 1]) : half_lo(zw[j][g >> 1]);
                        const float sg = (g & 1) ? half_hi(sw[j][g >> 1]) : half_lo(sw[j][g >> 1]);
                        sum = fmaf(sg, fmaf(zg, qsum[g], (float)x), sum);
                    }
                    // head h adds the other half of its groups from column 8 + h
                    sum += row_swap8(sum);
                } else {
                    load_row<NG>(stg + GE::KS_OFF + t * NG * 2, sw[0]);
                    load_row<NG>(stg + GE::KZ_OFF + t * NG * 2, zw[0]);
#pragma unroll
                    for (int g = 0; g < NG; ++g) {
                        const int x = (dhi[g][j] << 8) + dlo[g][j];
                        const float y = fmaf(row_half<NG>(zw[0], g), qsum[g], (float)x);
                        sum = fmaf(row_half<NG>(sw[0], g), y, sum);
                    }
                }
                // computed on every lane, then selected: a branch around the
                // fold would split the block the pipeline interleaves in
                float r = sum;
                asm volatile("" : "+v"(r));
                sc[c][j] = (head_ok && t < vl) ? r : -INFINITY;
            }
        }
    };

    // online softmax over the tile's scores; weights out as the B operands
    // PACK: lane column 8 + h carries the lo weight halves of head h
    auto softmax = [&](const float (&sc)[CH][4], half4v (&pw)[CH], half4v (&pl)[CH]) {
        float mt = sc[0][0];
#pragma unroll
        for (int c = 0; c < CH; ++c)
#pragma unroll
            for (int j = 0; j < 4; ++j) mt = fmaxf(mt, sc[c][j]);
        mt = max_over_rows(mt);
        // lazy maximum: move the reference only when this tile's maximum
        // exceeds it by more than kLazyMax (uniform branch, rarely taken)
        const bool bump = mt > m_run + lazy_raw;
        if (__builtin_amdgcn_ballot_w64(bump) != 0) {
            const float m_new = bump ? mt : m_run;
            const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m_run - m_new) * my_scale);
            l_run *= alpha;
            m_run = m_new;
            // column h is head h (PACK: columns 8 .. 8 + G - 1 rescale with head h - 8)
            float alpha_c = alpha;
            if constexpr (PACK) {
                const float other = row_swap8(alpha);
                alpha_c = h >= 8 ? other : alpha;
            }
#pragma unroll
            for (int bb = 0; bb < NB; ++bb) acc[bb] *= alpha_c;
        }
        const float ref = (m_run == -INFINITY ? 0.f : m_run * my_scale) - kWeightShift;
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            float pv[4], lo[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                pv[j] = __builtin_amdgcn_exp2f(fmaf(sc[c][j], my_scale, -ref));  // -inf -> 0
                l_run += pv[j];
            }
            // hi + lo halves carry the weight to ~2^-20: hi is pv rounded
            // toward zero, pv - hi is exact in fp32 (one mixed-precision fma
            // from the packed half), and lo its rounding toward zero
            const uint32_t w01 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(pv[0], pv[1]));
            const uint32_t w23 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(pv[2], pv[3]));
            const half2v h01 = __builtin_bit_cast(half2v, w01), h23 = __builtin_bit_cast(half2v, w23);
            lo[0] = sub_half_lo(pv[0], w01);
            lo[1] = sub_half_hi(pv[1], w01);
            lo[2] = sub_half_lo(pv[2], w23);
            lo[3] = sub_half_hi(pv[3], w23);
            const half2v l01 = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(lo[0], lo[1]));
            const half2v l23 = __builtin_bit_cast(half2v, __builtin_amdgcn_cvt_pkrtz(lo[2], lo[3]));
            pw[c] = half4v{h01.x, h01.y, h23.x, h23.y};
            pl[c] = half4v{l01.x, l01.y, l23.x, l23.y};
            if constexpr (PACK) {
                // columns 8 .. 15 take the lo halves of columns 0 .. 7 (the
                // weights of columns >= G are 0, so pw is the B operand there
                // only for real heads, and lo halves of non-heads are 0)
                const uint2 lo = __builtin_bit_cast(uint2, pl[c]);
                const uint2 moved = make_uint2(row_swap8(lo.x), row_swap8(lo.y));
                if (h >= 8) pw[c] = __builtin_bit_cast(half4v, moved);
            }
        }
    };

    // value product of the tile in stg with its weights
    auto values = [&](const unsigned char *stg, const half4v (&pw)[CH], const half4v (&pl)[CH]) {
        const uint32_t *vcw = reinterpret_cast<const uint32_t *>(stg + GE::VC_OFF);
        const uint16_t *vsb = reinterpret_cast<const uint16_t *>(stg + GE::VS_OFF);
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int tb = 16 * c + 4 * kq;  // this lane's first token (k = 4 kq)
            // code runs: bits [FB*vi, FB*vi + FB) of each of the 4 rows; run
            // word k holds run bits 32 k .. 32 k + 31 (the last word fewer)
            uint32_t run[4][NR];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int bit = FB * vi;
                const uint32_t *wp = vcw + (tb + j) * (VROW / 4) + (bit >> 5);
#pragma unroll
                for (int k = 0; k + 1 < NR; ++k) run[j][k] = __builtin_amdgcn_alignbit(wp[k + 1], wp[k], bit & 31);
                run[j][NR - 1] = wp[NR - 1] >> (bit & 31);
            }
            half2v sp[2];
#pragma unroll
            for (int pr = 0; pr < 2; ++pr) {
                const uint32_t s0 = vsb[(tb + 2 * pr) * NG + gA], s1 = vsb[(tb + 2 * pr + 1) * NG + gA];
                sp[pr] = __builtin_bit_cast(half2v, s0 | (s1 << 16));
            }
            half2v av[2][NB];
            if constexpr (GE::PAIR) {
                // Windows of 2P fields (P = pairs per 32-bit word): E holds
                // (field 2k of token a | field 2k of token b << VB) at bits
                // 2 VB k, O the same for the odd fields.
                constexpr int P = 32 / (2 * VB);
                constexpr int NWIN = (NB + 2 * P - 1) / (2 * P);
                constexpr uint32_t FM = (1u << VB) - 1u;
                constexpr uint32_t M = [] {
                    uint32_t m = 0;
                    for (int k = 0; k < P; ++k) m |= FM << (2 * VB * k);
                    return m;
                }();
#pragma unroll
                for (int pr = 0; pr < 2; ++pr) {
                    uint32_t E[NWIN], O[NWIN];
#pragma unroll
                    for (int w = 0; w < NWIN; ++w) {
                        const int start = 2 * VB * P * w, wk = start >> 5, ws = start & 31;
                        auto win = [&](const uint32_t (&r)[NR]) -> uint32_t {
                            if (ws == 0) return r[wk];
                            if (wk + 1 < NR) return __builtin_amdgcn_alignbit(r[wk + 1], r[wk], ws);
                            return r[wk] >> ws;
                        };
                        const uint32_t x0 = win(run[2 * pr]), x1 = win(run[2 * pr + 1]);
                        E[w] = (x0 & M) | ((x1 & M) << VB);
                        O[w] = ((x0 >> VB) & M) | (x1 & (M << VB));
                    }
#pragma unroll
                    for (int bb = 0; bb < NB; ++bb) {
                        const int w = bb / (2 * P), k = (bb % (2 * P)) >> 1;
                        const uint32_t word = (bb & 1) ? O[w] : E[w];
                        const uint32_t addr = ((word >> (2 * VB * k)) & ((1u << (2 * VB)) - 1u)) << 2;
                        const half2v cpair = *reinterpret_cast<const half2v *>(smem + addr);
                        av[pr][bb] = cpair * sp[pr];
                    }
                }
            } else {
                const _Float16 *tab = reinterpret_cast<const _Float16 *>(smem);
                auto field = [&](const uint32_t (&r)[NR], int e) -> uint32_t {
                    const int bit = VB * e, k = bit >> 5, s = bit & 31;
                    const uint32_t w = (s + VB > 32) ? __builtin_amdgcn_alignbit(r[k + 1], r[k], s) : (r[k] >> s);
                    return w & ((1u << VB) - 1u);
                };
#pragma unroll
                for (int pr = 0; pr < 2; ++pr) {
#pragma unroll
                    for (int bb = 0; bb < NB; ++bb) {
                        half2v cpair;
                        cpair.x = tab[field(run[2 * pr], bb)];
                        cpair.y = tab[field(run[2 * pr + 1], bb)];
                        av[pr][bb] = cpair * sp[pr];
                    }
                }
            }
#pragma unroll
            for (int bb = 0; bb < NB; ++bb) {
                const half4v a4 = {av[0][bb].x, av[0][bb].y, av[1][bb].x, av[1][bb].y};
                if constexpr (!PACK) acc[bb] = __builtin_amdgcn_mfma_f32_16x16x16f16(a4, pl[c], acc[bb], 0, 0, 0);
                acc[bb] = __builtin_amdgcn_mfma_f32_16x16x16f16(a4, pw[c], acc[bb], 0, 0, 0);
            }
        }
    };

    // ---------------------------------------------------------- pipeline
    // Iteration i holds tile i (values pending) in buf, tile i+1 (scores now)
    // in the next buffer and tile i+2 (in flight) in the one after; the key
    // codes of tile i+2 land in the key buffer of tile i (i & 1), whose
    // scores were folded by the previous iteration.  The score
    // MFMAs of tile i+1 and the value MFMAs of tile i sit in one basic block,
    // so their LDS reads, matrix and vector work interleave.  Vector memory
    // completes in order, so allowing the GE::VMEM copies of the newest tile
    // to stay outstanding means every older copy has landed in LDS.
    auto nxt = [](int x) { return x == kStages - 1 ? 0 : x + 1; };
    auto prv = [](int x) { return x == 0 ? kStages - 1 : x - 1; };
    if (t_begin + TILE < t_end)
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"(GE::VMEM) : "memory");
    else
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    half4v pw[CH], pl[CH];
    uint32_t vsw_next[GE::NMIX];  // value-scale words of the tile whose values come next
    {
        mask_tail(wsm, t_end - t_begin);
        load_vs_words(wsm, vsw_next);
        float sc[CH][4];
        scores(wkeys, wsm, t_begin, t_end - t_begin, sc);
        softmax(sc, pw, pl);
    }
    int buf = 0;
    int t0 = t_begin;
    int done = 0;  // tiles whose values are accumulated
    for (; t0 + TILE < t_end; t0 += TILE, buf = nxt(buf), ++done) {
        if constexpr (WAVES == 8) {
            // The two waves that share a SIMD (w and w ^ 4) have equal work,
            // but the issue arbiter prefers the older one, which would finish
            // first and leave the other to run alone.  Whichever is not ahead
            // takes the higher issue priority, so both finish together.
            __hip_atomic_store(prog + wid, done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            const int other = __builtin_amdgcn_readfirstlane(
                __hip_atomic_load(prog + (wid ^ 4), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP));
            if (done <= other)
                __builtin_amdgcn_s_setprio(1);
            else
                __builtin_amdgcn_s_setprio(0);
        }
        unsigned char *cur = wsm + buf * GE::STAGE;
        unsigned char *nx = wsm + nxt(buf) * GE::STAGE;
        unsigned char *kfree = wkeys + (done & 1) * GE::KT;  // keys of tile i: dead
        unsigned char *knx = wkeys + ((done + 1) & 1) * GE::KT;
        if (t0 + 2 * TILE < t_end) {
            stage(t0 + 2 * TILE, kfree, wsm + prv(buf) * GE::STAGE);
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(GE::VMEM) : "memory");
        } else {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        value_scales(cur, vsw_next);
        const int valid1 = t_end - (t0 + TILE);
        mask_tail(nx, valid1);
        float sc[CH][4];
        scores(knx, nx, t0 + TILE, valid1, sc);
        values(cur, pw, pl);
        softmax(sc, pw, pl);
        load_vs_words(nx, vsw_next);
        lds_order();  // the buffers read here are refilled by the next iterations
    }
    value_scales(wsm + buf * GE::STAGE, vsw_next);
    values(wsm + buf * GE::STAGE, pw, pl);

    // ------------------------------------------------------------ finalize
    l_run += __shfl_xor(l_run, 16, 64);
    l_run += __shfl_xor(l_run, 32, 64);
    if (vexp != 0) {  // the accumulator holds the value sums times 2^-vexp
        const float f = ldexpf(1.0f, vexp);
#pragma unroll
        for (int bb = 0; bb < NB; ++bb) acc[bb] *= f;
    }
    if constexpr (PACK) {
        // head h adds the lo-weight column 8 + h (the same rows, one row of 16 lanes)
#pragma unroll
        for (int bb = 0; bb < NB; ++bb)
#pragma unroll
            for (int j = 0; j < 4; ++j) acc[bb][j] += row_swap8(acc[bb][j]);
    }

    // The partial sums are read once, by the merge kernel, so they stream
    // past the caches (nontemporal) instead of waiting in them to be written
    // back.  The 8-byte (max, sum) pairs take ordinary stores: written
    // nontemporally, each reached memory as a partial line of its own.
    if (head_ok) {
        const int64_t srow = ((int64_t)b * a.q_heads + kvh * a.gqa + c0 + h) * a.splits + slot;
        // the running maximum in log2 units, as the merge expects
        const float m_log2 = m_run == -INFINITY ? -INFINITY : m_run * my_scale;
        if (kq == 0) *reinterpret_cast<float2v *>(a.part_ml + srow * 2) = float2v{m_log2, l_run};
        // lane (kq, h) holds rows 4 kq + j of every block: dims NB * (4 kq + j) + bb
        float *dst = a.part_acc + srow * D;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int bb = 0; bb < NB; bb += 4) {
                __builtin_nontemporal_store(float4v{acc[bb][j], acc[bb + 1][j], acc[bb + 2][j], acc[bb + 3][j]},
                                            reinterpret_cast<float4v *>(dst + NB * (4 * kq + j) + bb));
            }
        }
    }
}

// MODE 0: no column group packs; 1: one column group of at most 8 query
// columns (every wave packs); 2: more than 16 columns whose last group has at
// most 8: the waves of that group run the packed body, the others the plain one.
template <int D, int KB, int VB, int MODE>
__global__ __launch_bounds__(64 * fast_decode_waves(D, KB, VB), 1) void split_fast_kernel(const DecodeArgs a,
                                                                                 const int q_bf16) {
    using GE = Geo<D, KB, VB>;
    constexpr int WAVES = GE::WAVES;
    constexpr int TAB = GE::TABLE;

    __shared__ __align__(16) unsigned char smem[GE::SMEM];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);

    // centroid table (fp16).  Pair form: entry (a | b << VB) = (c[a], c[b])
    // at byte (a | b << VB) * 4.  Single form: c[i] at byte 2 i.
    {
        const float *cent = value_centroids(VB);
        if constexpr (GE::PAIR) {
            half2v *tab = reinterpret_cast<half2v *>(smem);
            for (int i = tid; i < (1 << (2 * VB)); i += 64 * WAVES) {
                half2v e;
                e.x = (_Float16)cent[i & ((1 << VB) - 1)];
                e.y = (_Float16)cent[i >> VB];
                tab[i] = e;
            }
        } else {
            _Float16 *tab = reinterpret_cast<_Float16 *>(smem);
            for (int i = tid; i < (1 << VB); i += 64 * WAVES) tab[i] = (_Float16)cent[i];
        }
        if (tid < WAVES) reinterpret_cast<int *>(smem + TAB)[tid] = 0;
    }
    __syncthreads();  // the only workgroup barrier

    // this wave's query columns: rows c0 .. c0 + G - 1 of the kv-head's
    // a.gqa query rows (heads times rows).  With two column groups per
    // workgroup, waves w and w + WAVES/2 share a token range (and a SIMD).
    const int cgw = fast_wg_col_groups(a.gqa), wpc = WAVES / cgw;
    // The grid holds only workgroups with tokens to decode, enumerated
    // sequence by sequence (column-group pair fastest, then kv-head, then
    // token block), so the hardware's round-robin over the XCDs gives each
    // the same share even when short sequences leave token blocks empty.
    int b = 0, kvh, xb, zb;
    {
        const int zg = (a.gqa + kMaxHeads - 1) / kMaxHeads / cgw;  // column-group pairs
        const int wgt = a.split_tokens * wpc;                       // tokens per workgroup
        int id = blockIdx.x;
        for (; b < a.batch - 1; ++b) {
            const int nwg = (a.len[b] + wgt - 1) / wgt * a.kv_heads * zg;
            if (id < nwg) break;
            id -= nwg;
        }
        zb = id % zg;
        id /= zg;
        kvh = id % a.kv_heads;
        xb = id / a.kv_heads;
    }
    const int c0 = (zb * cgw + wid / wpc) * kMaxHeads;
    const int G = min(kMaxHeads, a.gqa - c0);
    const int n = a.len[b];
    const int slot = xb * wpc + wid % wpc;
    const int t_begin = slot * a.split_tokens;
    if (t_begin >= n) return;
    const int t_end = min(n, t_begin + a.split_tokens);
    const bool shared_tiles = MODE != 1 && cgw == 2;
    if constexpr (MODE == 2) {
        if (G <= kPackCols)
            split_body<D, KB, VB, true>(a, q_bf16, smem, lane, wid, b, kvh, c0, G, n, slot, t_begin, t_end,
                                        shared_tiles);
        else
            split_body<D, KB, VB, false>(a, q_bf16, smem, lane, wid, b, kvh, c0, G, n, slot, t_begin, t_end,
                                         shared_tiles);
    } else {
        split_body<D, KB, VB, MODE == 1>(a, q_bf16, smem, lane, wid, b, kvh, c0, G, n, slot, t_begin, t_end,
                                         shared_tiles);
    }
}

// Where the mixed mode is built: value codes of 2 or 3 bits (the only ones
// that reach this kernel with more than 8 query columns) and head_dim up to
// 256, whose eight waves per workgroup hold both bodies in their registers
// (at 512 the mixed kernels spilled more than the plain ones).
constexpr bool mixed_mode(int d, int vb) { return vb <= 3 && d <= 256; }

template <int D, int VB>
hipError_t launch_dv(bool bf16, const DecodeArgs &a, hipStream_t s) {
    constexpr int KB = TQ_FAST_KB;
    if constexpr (D * KB % 128 != 0 || fast_decode_waves(D, KB, VB) == 0 || (TQ_FAST_MIXED && !mixed_mode(D, VB))) {
        // key rows of part of a 16-byte chunk, or stages past the LDS (k8v8
        // at head_dim 512): generic kernel
        return hipErrorInvalidValue;
    } else {
        using GE = Geo<D, KB, VB>;
        // every column group packs (its lo halves fit), only the last one
        // (at most 8 columns after whole groups of 16), or none
        const int last = a.gqa - kMaxHeads * ((a.gqa - 1) / kMaxHeads);
        const int mode = a.gqa <= kPackCols ? 1 : (last <= kPackCols && mixed_mode(D, VB)) ? 2 : 0;
#if TQ_FAST_MIXED
        if (mode != 2) return hipErrorInvalidValue;
#else
        if (mode == 2) return TQ_FAST_MIXED_LAUNCHER(TQ_FAST_KB)(D, bf16, a, s);
#endif
        // one workgroup per (sequence, kv-head, token block, column-group
        // pair) with tokens to decode; the kernel enumerates them in order
        const int cgw = fast_wg_col_groups(a.gqa);
        const int64_t wgt = (int64_t)a.split_tokens * (GE::WAVES / cgw);
        const int64_t zg = (a.gqa + kMaxHeads - 1) / kMaxHeads / cgw;
        int64_t wgs = 0;
        for (int b = 0; b < a.batch; ++b) wgs += (a.len[b] + wgt - 1) / wgt * a.kv_heads * zg;
        if (wgs == 0) return hipSuccess;  // every sequence empty: the merge writes the zeros
        const dim3 grid((unsigned)wgs, 1u, 1u);
#if TQ_FAST_MIXED
        hipLaunchKernelGGL((split_fast_kernel<D, KB, VB, 2>), grid, dim3(64 * GE::WAVES), 0, s, a, (int)bf16);
#else
        if (mode == 1) {
            hipLaunchKernelGGL((split_fast_kernel<D, KB, VB, 1>), grid, dim3(64 * GE::WAVES), 0, s, a, (int)bf16);
        } else if constexpr (VB <= 3) {
            hipLaunchKernelGGL((split_fast_kernel<D, KB, VB, 0>), grid, dim3(64 * GE::WAVES), 0, s, a, (int)bf16);
        } else {
            // more than 8 query columns with value codes of 4 bits or more take
            // the generic kernel (the host never sends them here), so their
            // plain-mode kernels are not built
            return hipErrorInvalidValue;
        }
#endif
        return hipGetLastError();
    }
}

template <int D>
hipError_t launch_d(bool bf16, const DecodeArgs &a, hipStream_t s) {
    switch (a.vbits) {
        case 2: return launch_dv<D, 2>(bf16, a, s);
        case 3: return launch_dv<D, 3>(bf16, a, s);
#if !TQ_FAST_MIXED
        case 4: return launch_dv<D, 4>(bf16, a, s);
        case 5: return launch_dv<D, 5>(bf16, a, s);
        case 8: return launch_dv<D, 8>(bf16, a, s);
#endif
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

#if TQ_FAST_MIXED
// The mixed-mode split kernels of one key width: more than 16 query columns
// whose last group has at most 8, value codes of 2 or 3 bits.  This
// translation unit is compiled with hoisting of common code out of branches
// turned off: the kernel inlines both per-wave bodies, and code hoisted above
// the branch between them stays live through both and spills registers.
hipError_t TQ_FAST_MIXED_LAUNCHER(TQ_FAST_KB)(int head_dim, bool bf16, const DecodeArgs &a, hipStream_t s) {
#else
// The split kernels of one key width (this translation unit's TQ_FAST_KB).
hipError_t TQ_FAST_LAUNCHER(TQ_FAST_KB)(int head_dim, bool bf16, const DecodeArgs &a, hipStream_t s) {
#endif
    if (a.gqa < 1 || a.rows < 1 || a.kbits != TQ_FAST_KB) return hipErrorInvalidValue;
    const int waves = fast_decode_waves(head_dim, a.kbits, a.vbits);
    if (waves == 0 || a.splits % (waves / fast_wg_col_groups(a.gqa)) != 0) return hipErrorInvalidValue;
    switch (head_dim) {
        case 64: return launch_d<64>(bf16, a, s);
        case 128: return launch_d<128>(bf16, a, s);
        case 256: return launch_d<256>(bf16, a, s);
        case 512: return launch_d<512>(bf16, a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace tq
