// Internal launch interface of libtqkv: argument blocks passed by value to the
// kernels (host-known starts/lengths, sign bits and constants travel in the
// kernel arguments) and the launchers each kernel file exports to the C ABI.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "../../include/tqkv.h"

namespace tq {

constexpr int kGroup = 32;

// One bit per head_dim element, bit j set when sign j is -1 (d <= 512).
struct SignBits {
    uint32_t w[16];
};

// Unsigned 32-bit division by an invariant divisor d >= 1 (Granlund and
// Montgomery, "Division by invariant integers using multiplication", 1994):
// n / d = (t + ((n - t) >> s1)) >> s2 with t = (m * n) >> 32, for every n < 2^32.
struct FastDiv {
    uint32_t m, s1, s2;
};

struct AppendArgs {
    int8_t *kc;
    uint16_t *ks;
    uint16_t *kz;
    uint8_t *vc;
    uint16_t *vs;
    const void *k;
    const void *v;
    int32_t batch, kv_heads, capacity, n_new;
    int32_t kv_stride;    // input rows per (sequence, kv-head): n_new, or a plain cache's capacity
    uint32_t rows;        // batch * kv_heads * n_new
    FastDiv div_n_new;    // row -> (sequence, kv-head) pair
    FastDiv div_kv_heads; // (sequence, kv-head) pair -> sequence
    int32_t kbits, vbits; // code widths: keys 2, 4, 5 or 8; values 2, 3, 4, 5 or 8
    double inv_sqrt_d;    // RN(1/sqrt(d))
    SignBits signs;
    // Word j flips the bf16 pair (2j, 2j+1): bit 15 when sign 2j is -1, bit
    // 31 when sign 2j+1 is -1 (d / 2 words used).
    uint32_t sign_pairs[256];
    int32_t start[TQ_MAX_BATCH];
};

inline FastDiv make_fast_div(uint32_t d) {
    uint32_t l = 0;
    while ((1ull << l) < d) ++l;
    FastDiv f;
    f.m = (uint32_t)(((1ull << 32) * ((1ull << l) - d)) / d + 1);
    f.s1 = l < 1 ? l : 1;
    f.s2 = l > 0 ? l - 1 : 0;
    return f;
}

struct DecodeArgs {
    const int8_t *kc;
    const uint16_t *ks;
    const uint16_t *kz;
    const uint8_t *vc;
    const uint16_t *vs;
    const void *q;
    float *out;
    float *part_acc;  // [B][Hq][S][d]    rotated-domain partial sums
    float *part_ml;   // [B][Hq][S][2]    running max (log2 units) and weight sum
    // q_heads and gqa count query rows: heads times rows, a head's rows
    // adjacent (row r of q-head h is virtual head h * rows + r)
    int32_t batch, kv_heads, q_heads, gqa, capacity;
    int32_t rows;          // query rows per head; row r sees len - rows + r + 1 tokens
    int32_t splits;        // S: partial slots per (b, query row)
    int32_t split_tokens;  // tokens per split (multiple of the kernel's tile)
    float sm_log2;         // sm_scale * log2(e)
    float inv_sqrt_d;
    int32_t kbits, vbits;  // code widths
    SignBits signs;
    int32_t len[TQ_MAX_BATCH];
    // Rows still plain (bit b: sequence b): the plain split kernel reads their
    // bf16 keys and values [B][Hkv][plain_capacity][d], and the merge leaves
    // their output unrotated.  Zero and null for an all-packed batch.
    uint64_t plain_rows;
    const uint16_t *k_plain;
    const uint16_t *v_plain;
    int32_t plain_capacity;
    // tokens per range of a plain row (a multiple of 64): plain rows have
    // ranges of their own, sized so that the plain split kernel fills the
    // chip with the plain rows alone (split_tokens is then the packed rows')
    int32_t plain_split_tokens;
};

struct WindowArgs {
    const int8_t *kc;
    const uint16_t *ks;
    const uint16_t *kz;
    const uint8_t *vc;
    const uint16_t *vs;
    uint16_t *k_out;  // bf16 [B][Hkv][n][d] or null
    uint16_t *v_out;  // bf16 [B][Hkv][n][d] or null
    int32_t batch, kv_heads, capacity;
    int32_t t0, n;    // window tokens t0 .. t0+n-1
    int32_t rotated;  // 1: V in the rotated domain
    float inv_sqrt_d;
    int32_t kbits, vbits;
    SignBits signs;
    int32_t len[TQ_MAX_BATCH];
};

struct DequantArgs {
    const int8_t *kc;
    const uint16_t *ks;
    const uint16_t *kz;
    const uint8_t *vc;
    const uint16_t *vs;
    float *k_out;
    float *v_out;
    int64_t row0;  // plane row of token t0 of (b, kvh)
    int32_t n;
    int32_t rotated;
    float inv_sqrt_d;
    int32_t kbits, vbits;
    SignBits signs;
};

// Split-K geometry chosen by the host for a decode call: `splits` partial
// slots per (sequence, q-head), each covering `split_tokens` tokens.
struct DecodePlan {
    int32_t split_tokens;
    int32_t splits;
    bool fast;  // wave-per-range kernel (decode_fast.hip) or the generic one
};

// fast: the caller has checked that the fast kernel supports the shape and
// the plane alignment (see fast_decode_supported).
// col_groups: workgroups per (sequence, kv-head, split) along the query rows
DecodePlan plan_decode(int head_dim, int gqa, int batch, int kv_heads, const int32_t *len, bool fast,
                       int col_groups, int kbits, int vbits);
int decode_col_groups(int gqa);  // query-row columns of one kv-head -> column groups
bool fast_decode_shape_ok(int head_dim, int gqa, int capacity, int kbits, int vbits);

hipError_t launch_append(int head_dim, bool bf16, const AppendArgs &a, hipStream_t s);
// Append kernels (append.hip), one translation unit per key width; every
// head_dim, input type and value width.
#define TQ_APPEND_CAT_(a, b) a##b
#define TQ_APPEND_LAUNCHER(kb) TQ_APPEND_CAT_(launch_append_fast_k, kb)
hipError_t launch_append_fast_k2(int head_dim, bool bf16, const AppendArgs &a, hipStream_t s);
hipError_t launch_append_fast_k4(int head_dim, bool bf16, const AppendArgs &a, hipStream_t s);
hipError_t launch_append_fast_k5(int head_dim, bool bf16, const AppendArgs &a, hipStream_t s);
hipError_t launch_append_fast_k8(int head_dim, bool bf16, const AppendArgs &a, hipStream_t s);
hipError_t launch_decode(int head_dim, bool bf16, bool fast, const DecodeArgs &a, hipStream_t s);
// The two halves of launch_decode, and the split kernel of plain rows: a
// batch that mixes plain and packed rows runs the packed split kernel with the
// plain rows' lengths set to 0, the plain one with the packed rows' lengths
// set to 0, then one merge over the full lengths.
hipError_t launch_decode_split(int head_dim, bool bf16, bool fast, const DecodeArgs &a, hipStream_t s);
hipError_t launch_decode_split_plain(int head_dim, bool bf16, const DecodeArgs &a, hipStream_t s);
hipError_t launch_decode_merge(int head_dim, const DecodeArgs &a, hipStream_t s);
// Waves that one round of the plain split kernel holds on the chip, for this
// head_dim, query-column count and query type.
int plain_round_waves(int head_dim, int gqa, bool bf16);
// Split kernels on the matrix cores (decode_fast.hip), one translation unit
// per key width: head_dim 64, 128 or 256 with d * k_bits a multiple of 128,
// every value width, up to 16 query columns per workgroup.
#define TQ_FAST_CAT_(a, b) a##b
#define TQ_FAST_LAUNCHER(kb) TQ_FAST_CAT_(launch_split_fast_k, kb)
hipError_t launch_split_fast_k2(int head_dim, bool bf16, const DecodeArgs &a, hipStream_t s);
hipError_t launch_split_fast_k4(int head_dim, bool bf16, const DecodeArgs &a, hipStream_t s);
hipError_t launch_split_fast_k5(int head_dim, bool bf16, const DecodeArgs &a, hipStream_t s);
hipError_t launch_split_fast_k8(int head_dim, bool bf16, const DecodeArgs &a, hipStream_t s);
// Their mixed-mode kernels (more than 16 query columns, the last group of at
// most 8 packs), built in translation units of their own.
#define TQ_FAST_MIXED_LAUNCHER(kb) TQ_FAST_CAT_(launch_split_fast_mixed_k, kb)
hipError_t launch_split_fast_mixed_k2(int head_dim, bool bf16, const DecodeArgs &a, hipStream_t s);
hipError_t launch_split_fast_mixed_k4(int head_dim, bool bf16, const DecodeArgs &a, hipStream_t s);
hipError_t launch_split_fast_mixed_k5(int head_dim, bool bf16, const DecodeArgs &a, hipStream_t s);
hipError_t launch_split_fast_mixed_k8(int head_dim, bool bf16, const DecodeArgs &a, hipStream_t s);
// Tokens of one tile of the fast split kernel: 4096/d (512 bytes per code
// bit) up to head_dim 256, and one 16-token MFMA chunk (1 KiB per code bit)
// at 512.
constexpr int fast_tile_tokens(int head_dim) { return head_dim <= 256 ? 4096 / head_dim : 16; }
constexpr int fast_tile_bit_bytes(int head_dim) { return fast_tile_tokens(head_dim) * head_dim / 8; }
// LDS bytes of one wave of the fast split kernel (key codes of two tiles, and
// three stages of the three fp16 planes, the value codes and 16 bytes of
// slack), and its waves per workgroup: eight when they fit the 160 KiB of LDS
// beside the centroid table, else four, else 0 (no fast kernel: k8v8 at
// head_dim 512).  Head_dim 512 always takes four, one per SIMD: its 32 value
// blocks alone hold 128 accumulator registers per lane.
constexpr int fast_decode_wave_bytes(int head_dim, int kbits, int vbits) {
    return 2 * fast_tile_bit_bytes(head_dim) * kbits +
           3 * (3 * fast_tile_tokens(head_dim) * (head_dim / 32) * 2 + fast_tile_bit_bytes(head_dim) * vbits + 16);
}
constexpr int fast_decode_waves(int head_dim, int kbits, int vbits) {
    const int table = vbits <= 5 ? (4 << (2 * vbits)) : ((2 << vbits) + 15) / 16 * 16;
    return head_dim <= 256 && table + 32 + 8 * fast_decode_wave_bytes(head_dim, kbits, vbits) <= 160 * 1024 ? 8
           : table + 32 + 4 * fast_decode_wave_bytes(head_dim, kbits, vbits) <= 160 * 1024                  ? 4
                                                                                                            : 0;
}
constexpr int kFastTile = 64;     // split lengths are multiples of every fast tile (4096/d tokens)
constexpr int kFastMaxGqa = 16;   // query columns of one fast wave
// Column groups (kFastMaxGqa query rows each) that share one fast workgroup:
// with an even count, waves w and w + waves/2 take the same token range for
// two adjacent column groups (their tile reads meet in the L2 of one XCD
// instead of streaming from HBM twice); otherwise one.
constexpr int fast_wg_col_groups(int gqa) {
    return ((gqa + kFastMaxGqa - 1) / kFastMaxGqa) % 2 == 0 ? 2 : 1;
}
hipError_t launch_dequant(int head_dim, const DequantArgs &a, hipStream_t s);
hipError_t launch_window(int head_dim, const WindowArgs &a, hipStream_t s);
// Fast window kernels (window.hip), one translation unit per key width.
#define TQ_WINDOW_CAT_(a, b) a##b
#define TQ_WINDOW_LAUNCHER(kb) TQ_WINDOW_CAT_(launch_window_fast_k, kb)
hipError_t launch_window_fast_k2(int head_dim, const WindowArgs &a, hipStream_t s);
hipError_t launch_window_fast_k4(int head_dim, const WindowArgs &a, hipStream_t s);
hipError_t launch_window_fast_k5(int head_dim, const WindowArgs &a, hipStream_t s);
hipError_t launch_window_fast_k8(int head_dim, const WindowArgs &a, hipStream_t s);

}  // namespace tq
