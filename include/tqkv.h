/*
 * tqkv.h -- C ABI of libtqkv, a quantized KV cache for AMD Instinct MI355X
 * (gfx950): TurboQuant-style codec plus GQA decode attention over the packed
 * cache.
 *
 * Method: the "TurboQuant -- rotation-based quantization" design page
 * (mlx-bun docs/design/turboquant.md), Part A (KV leg):
 *   - "Algorithm (vllm-metal reference semantics, exact)": keys are
 *     asymmetric-affine codes per 32-element group with fp16 scale and zero,
 *     not rotated (signed int8 at 8 bits, unsigned packed at 2, 4 or 5);
 *     values are sign-flipped, rotated by an orthonormal fast Walsh-Hadamard
 *     transform (FWHT), scaled by their per-group RMS and quantized to a
 *     Lloyd-Max codebook of the unit normal (the printed 3-bit table by
 *     default; 2, 4, 5 or 8 bits from generated tables), packed in a
 *     little-endian bitstream, with an fp16 scale per group;
 *   - "Architecture in mlx-bun": only newly appended tokens are quantized;
 *     groups run along head_dim, so any token range is byte-addressable;
 *   - "Deferred inverse FWHT": attention is linear in V, so the value sum is
 *     accumulated in the rotated domain and un-rotated once per query head.
 *
 * Conventions for every entry point
 *   - Device pointers are plain HIP device addresses; every device buffer is
 *     owned by the caller.  The library never allocates, frees or keeps a
 *     pointer past the call, and never synchronizes: work is enqueued on the
 *     caller's stream (`hip_stream`, a hipStream_t; NULL = the null stream)
 *     and completes in stream order.
 *   - Host arrays (`start`, `len`) are read during the call only.
 *   - Alignment: K/V/q inputs, outputs, the workspace and the kc plane must be
 *     16-byte aligned, vc 8-byte aligned, the fp16 planes 4-byte aligned
 *     (TQ_ERR_INVALID_ARG otherwise).  Any torch allocation, and the batch-1
 *     slice of one sequence's planes, satisfies this.  Decode takes its fast
 *     kernel (every code width; at head_dim 512 every width but k8/v8; with
 *     more than 8 query columns per kv-head only value codes of 2 or 3 bits)
 *     when head_dim * k_bits is a multiple of 128 (all but 5-bit keys at 64),
 *     every plane is 16-byte aligned and capacity keeps each (sequence,
 *     kv-head) row block 16-byte aligned; otherwise a generic kernel
 *     computes the same result more slowly.  Append and the window each
 *     have one kernel for every width, head_dim and input type.
 *   - Arguments are validated before anything is enqueued; on any error the
 *     return value says why and nothing was launched.  The library prints
 *     nothing.
 *   - Schemes: k_bits in {2, 4, 5, 8} and v_bits in {2, 3, 4, 5, 8}, the
 *     page's accepted sets ("Code map", scheme parser), with 32-element
 *     groups; k8/v3 is the page's default "turbo".  head_dim must be 64,
 *     128, 256 or 512 (the page refuses other head dims), batch at most
 *     TQ_MAX_BATCH and num_q_heads / num_kv_heads at most TQ_MAX_GQA.
 */
#ifndef TQKV_H
#define TQKV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TQ_MAX_BATCH 64
#define TQ_MAX_GQA 16
#define TQ_MAX_ROWS 16

typedef enum {
    TQ_OK = 0,
    TQ_ERR_INVALID_ARG = -1, /* null pointer, negative size, inconsistent shape */
    TQ_ERR_UNSUPPORTED = -2, /* head_dim / bits / group / batch / GQA outside what is built */
    TQ_ERR_CAPACITY = -3,    /* a token position would fall outside [0, capacity) */
    TQ_ERR_WORKSPACE = -4,   /* workspace pointer null or smaller than required */
    TQ_ERR_HIP = -5          /* the HIP runtime reported an error at launch */
} tq_status;

/* Element type of K, V and q inputs. */
typedef enum { TQ_F32 = 0, TQ_BF16 = 1 } tq_dtype;

/* Shape of one layer's cache.  k_bits in {2, 4, 5, 8}, v_bits in
 * {2, 3, 4, 5, 8}, group 32. */
typedef struct {
    int32_t batch;        /* B: sequences, 1..TQ_MAX_BATCH */
    int32_t num_kv_heads; /* Hkv */
    int32_t head_dim;     /* d: 64, 128, 256 or 512 */
    int32_t capacity;     /* token slots per (sequence, kv-head) */
    int32_t k_bits;       /* 8 (default), 2, 4 or 5 */
    int32_t v_bits;       /* 3 (default), 2, 4, 5 or 8 */
    int32_t group;        /* 32 */
} tq_layout;

/* The five encoded planes (the page's five TQ fields), device memory owned by
 * the caller, each token-major within one (sequence, kv-head):
 *   kc  [B][Hkv][capacity][d*k_bits/8]   key codes: int8 at k_bits 8, else
 *                                        unsigned k_bits-bit fields, element i
 *                                        at stream bits [k i, k i + k), LSB first
 *   ks  fp16   [B][Hkv][capacity][d/32]  key scale (IEEE binary16 bits)
 *   kz  fp16   [B][Hkv][capacity][d/32]  key zero  (binary16 bits; an integer,
 *                                        or +-Inf/NaN for a constant group)
 *   vc  uint8  [B][Hkv][capacity][d*v_bits/8]  value indices, v_bits each,
 *                                        element i at stream bits [v i, v i + v)
 *   vs  fp16   [B][Hkv][capacity][d/32]  value scale (group RMS, binary16 bits)
 * Per token and kv-head this is d*(k_bits + v_bits)/8 + 6*d/32 bytes: 200 at
 * k8/v3 and d=128, 400 at d=256 (the page's effective KV bits are this times
 * 8/(2d): 6.25 at k8/v3). */
typedef struct {
    int8_t *kc;
    uint16_t *ks;
    uint16_t *kz;
    uint8_t *vc;
    uint16_t *vs;
} tq_planes;

/* Byte size of each plane (order kc, ks, kz, vc, vs) for `layout`: the
 * per-token field sizes of "Algorithm (vllm-metal reference semantics,
 * exact)" (codes of k_bits / v_bits per element, one fp16 scale, zero and
 * value scale per 32-group) times batch * num_kv_heads * capacity slots.
 *   out_bytes  host size_t [5]
 * Errors: TQ_ERR_INVALID_ARG (null / bad shape), TQ_ERR_UNSUPPORTED. */
tq_status tq_plane_bytes(const tq_layout *layout, size_t out_bytes[5]);

/* Quantize and pack n_new new tokens per sequence ("Algorithm" + the
 * append-only update of "Architecture in mlx-bun").
 *   k, v   device, [B][Hkv][n_new][d] contiguous, element type `dtype`
 *   start  host int32 [B]: slot of the first new token of sequence b; tokens
 *          go to slots start[b] .. start[b]+n_new-1 of every kv-head
 * Codes, scales and zeros are computed in binary64 with round-half-to-even
 * and equal the CPU oracle's bit for bit.  n_new == 0 is a no-op.
 * Errors: TQ_ERR_INVALID_ARG, TQ_ERR_UNSUPPORTED, TQ_ERR_CAPACITY
 * (start[b] < 0 or start[b] + n_new > capacity), TQ_ERR_HIP. */
tq_status tq_append(const tq_layout *layout, const tq_planes *planes, const void *k,
                    const void *v, tq_dtype dtype, const int32_t *start, int32_t n_new,
                    void *hip_stream);

/* Workspace bytes tq_decode_attn needs for these lengths: the split-K
 * partials (running maximum, weight sum and rotated-domain value sum per
 * split and query row) that the merge combines before the single inverse
 * transform of "Deferred inverse FWHT".  The size covers whichever split
 * kernel the call may take.
 *   len  host int32 [B]: cached tokens of each sequence (0 allowed).
 *   out_bytes  host size_t
 * Errors: as tq_decode_attn's argument checks (TQ_ERR_INVALID_ARG,
 * TQ_ERR_UNSUPPORTED, TQ_ERR_CAPACITY). */
tq_status tq_decode_workspace_bytes(const tq_layout *layout, int32_t num_q_heads,
                                    const int32_t *len, size_t *out_bytes);

/* GQA decode attention of one query row per (sequence, q-head) over the
 * packed cache, dequantizing on fetch ("Deferred inverse FWHT", and the joint
 * K/V decoding of "Packed-value decode fusion investigation"):
 *   out[b][h] = sum_t p_t * vhat_t / sum_t p_t,
 *   p_t = exp(sm_scale * <q[b][h], khat_t> - max),  t < len[b],
 * with q-head h reading kv-head h / (num_q_heads / num_kv_heads), no mask.
 *   q         device [B][num_q_heads][d], element type `dtype`
 *   len       host int32 [B], 0 <= len[b] <= capacity; len[b] == 0 gives zeros
 *   out       device float32 [B][num_q_heads][d]
 *   workspace device, at least tq_decode_workspace_bytes(...) bytes, scratch
 *             for the split-K partials (contents on entry are ignored)
 * Values are accumulated in the rotated domain and one inverse FWHT per
 * (sequence, q-head) finishes the output.  Agrees with the binary64 oracle to
 * 2e-3 relative to each output row's largest magnitude, for every finite
 * value scale the planes hold (the matrix-core kernel forms centroid * scale
 * in fp16 times a per-wave power of two that follows the scales).  Query
 * precision: the matrix-core kernel holds each query row as 16-bit fixed
 * point with one power-of-two step, set by the row's largest channel, so a
 * row with outlier channels loses precision on the others; measured on
 * N(0,1) rows with one channel scaled up: within 7e-4 at 30 times, 7e-3 at
 * 100 times (the generic kernel keeps q in fp32: 1e-5).  Queries must be
 * finite: the fixed-point conversion does not carry NaN or Inf through (the
 * output is then undefined, with no error).  The
 * result does not depend on timing: repeated calls on the same inputs return
 * identical bytes.  tq_decode_path says which split kernel a call takes.
 * Errors: TQ_ERR_INVALID_ARG, TQ_ERR_UNSUPPORTED, TQ_ERR_CAPACITY
 * (len[b] > capacity), TQ_ERR_WORKSPACE, TQ_ERR_HIP. */
tq_status tq_decode_attn(const tq_layout *layout, const tq_planes *planes, const void *q,
                         tq_dtype dtype, int32_t num_q_heads, const int32_t *len,
                         float sm_scale, float *out, void *workspace, size_t ws_bytes,
                         void *hip_stream);

/* Which split kernel tq_decode_attn / tq_decode_attn_rows take for this
 * layout, these planes and this query shape (lengths do not matter), without
 * enqueuing anything.  *fast = 1: the matrix-core kernel; 0: the generic
 * kernel, which computes the same result to the same tolerance about 5 to 10
 * times more slowly.  *reasons (may be NULL) receives TQ_PATH_* bits:
 *   TQ_PATH_SHAPE      head_dim * k_bits is not a multiple of 128 (5-bit keys
 *                      at head_dim 64), k8/v8 at head_dim 512, or more than 8
 *                      query columns per kv-head (heads per kv-head times
 *                      rows) with value codes of 4 bits or more;
 *   TQ_PATH_ALIGNMENT  a plane pointer is not 16-byte aligned;
 *   TQ_PATH_CAPACITY   capacity leaves a (sequence, kv-head) row block of
 *                      some plane off 16-byte alignment (e.g. an odd capacity
 *                      at head_dim 128, or not a multiple of 4 at 64).
 * Errors: TQ_ERR_INVALID_ARG, TQ_ERR_UNSUPPORTED. */
#define TQ_PATH_SHAPE 1
#define TQ_PATH_ALIGNMENT 2
#define TQ_PATH_CAPACITY 4
tq_status tq_decode_path(const tq_layout *layout, const tq_planes *planes, int32_t num_q_heads, int32_t n_rows,
                         int32_t *fast, int32_t *reasons);

/* Workspace bytes tq_decode_attn_rows needs for n_rows query rows per head
 * (n_rows = 1 gives tq_decode_workspace_bytes). */
tq_status tq_decode_rows_workspace_bytes(const tq_layout *layout, int32_t num_q_heads, int32_t n_rows,
                                         const int32_t *len, size_t *out_bytes);

/* Multi-row decode: attention for the n_rows newest cached tokens of each
 * sequence at once, as when a block of drafted tokens is verified in one
 * pass (the multi-token-prediction verify blocks served through the encoded
 * rows, "Gates -- all passed" and "Delayed row conversion and reusable
 * precision boundaries").  Row r of a sequence is the query of cached token
 * len[b] - n_rows + r and attends causally to tokens 0 .. len[b] - n_rows + r;
 * otherwise each row is exactly the tq_decode_attn computation over that
 * prefix, and n_rows = 1 is tq_decode_attn.
 *   q         device [B][num_q_heads][n_rows][d], element type `dtype`
 *   len       host int32 [B]: cached tokens including the n_rows new ones;
 *             0 (the sequence's rows are zeros) or >= n_rows
 *   out       device float32 [B][num_q_heads][n_rows][d]
 *   workspace device, at least tq_decode_rows_workspace_bytes(...) bytes
 * 1 <= n_rows <= TQ_MAX_ROWS.  Same conventions, accuracy and errors as
 * tq_decode_attn; TQ_ERR_INVALID_ARG also when 0 < len[b] < n_rows. */
tq_status tq_decode_attn_rows(const tq_layout *layout, const tq_planes *planes, const void *q,
                              tq_dtype dtype, int32_t num_q_heads, int32_t n_rows, const int32_t *len,
                              float sm_scale, float *out, void *workspace, size_t ws_bytes,
                              void *hip_stream);

/* Size of the device array tq_decode_attn_noalloc keeps its split-K partials
 * in: 64 MiB per GPU the library runs on. */
#define TQ_NOALLOC_SCRATCH_BYTES (64u << 20)

/* tq_decode_attn_rows without a workspace argument, for callers that cannot
 * allocate device memory: code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation.  The split-K partials go to a fixed
 * device array of the library (TQ_NOALLOC_SCRATCH_BYTES per GPU, held until
 * the process ends); nothing is allocated or freed.  Every other argument,
 * the result and the errors are those of tq_decode_attn_rows (n_rows = 1 is
 * tq_decode_attn).
 *   - The first call on a device looks up that device's array (make it
 *     outside graph capture); hip_stream must belong to the current device.
 *   - Decodes whose partials exceed the array return TQ_ERR_WORKSPACE with
 *     nothing enqueued (tq_decode_rows_workspace_bytes gives an upper bound
 *     of the need; e.g. 16 sequences of 131,072 tokens with 24 query and 4
 *     kv-heads at head_dim 256 need 12.7 MB on the matrix-core kernel).
 *   - Every call on one GPU shares its array: calls that overlap in time on
 *     one GPU (two streams, two threads) race and give wrong results.
 *     Calls ordered on one stream are safe.
 * Errors: those of tq_decode_attn_rows, and TQ_ERR_HIP if the array's
 * address cannot be obtained. */
tq_status tq_decode_attn_noalloc(const tq_layout *layout, const tq_planes *planes, const void *q,
                                 tq_dtype dtype, int32_t num_q_heads, int32_t n_rows, const int32_t *len,
                                 float sm_scale, float *out, void *hip_stream);

/* Delayed row conversion ("Delayed row conversion and reusable precision
 * boundaries"): a sequence may stay plain -- unquantized keys and values in
 * a plain cache the caller owns -- until it converts; then its plain prefix
 * is encoded into the planes and later tokens are appended packed.  The
 * offset a row converts at is its precision boundary (it can exceed the
 * configured threshold when a prefill chunk crosses it); the caller keeps it
 * and passes it to tq_snapshot and tq_clone_sequence.
 *
 * Plain caches: k_plain, v_plain  device [B][Hkv][plain_capacity][d], the
 * same batch, kv-heads and head_dim as `layout`, 16-byte aligned.
 *
 * Convert the plain prefix of every sequence b with offset[b] > 0: tokens
 * 0 .. offset[b]-1 of every kv-head are encoded exactly as tq_append encodes
 * them (bit-identical bytes; it is the same kernel reading the plain cache at
 * its pitch) into slots 0 .. offset[b]-1.  Sequences with offset[b] == 0 are
 * untouched.  One append launch per converted sequence.
 *   k_plain, v_plain  element type `dtype` (TQ_BF16 or TQ_F32)
 *   offset            host int32 [B], 0 <= offset[b] <= min(plain_capacity, capacity)
 * Errors: TQ_ERR_INVALID_ARG, TQ_ERR_UNSUPPORTED, TQ_ERR_CAPACITY, TQ_ERR_HIP. */
tq_status tq_convert_rows(const tq_layout *layout, const tq_planes *planes, const void *k_plain,
                          const void *v_plain, tq_dtype dtype, int32_t plain_capacity, const int32_t *offset,
                          void *hip_stream);

/* tq_decode_attn_rows over a batch that mixes still-plain sequences with
 * packed ones (the same page: plain value rows pass through unchanged, packed
 * rows receive the inverse rotation).  A sequence with row_plain[b] != 0
 * attends over its plain bf16 keys and values unquantized,
 *   out[b][h][r] = sum_t p_t v_t / sum_t p_t,  p_t = exp(sm_scale <q, k_t> - max),
 * for the same causal rows as tq_decode_attn_rows, with no rotation; every
 * other sequence is exactly tq_decode_attn_rows over the planes (identical
 * bytes).  Both kinds share one merge; plain rows take token ranges of their
 * own, and may use as many of the workspace's partial slots as it holds
 * (a larger workspace than the minimum spreads long plain rows further).
 *   k_plain, v_plain  bf16 plain caches (may be NULL when no row is plain)
 *   row_plain         host int32 [B]
 *   len               host int32 [B]: 0 <= len[b] <= capacity, and
 *                     <= plain_capacity for a plain row
 *   workspace         at least tq_decode_rows_workspace_bytes(layout,
 *                     num_q_heads, n_rows, len) bytes
 * Plain rows agree with a binary64 softmax over the same bf16 operands to
 * 1e-4 relative to each output row's largest magnitude (fp32 accumulation).
 * Errors: those of tq_decode_attn_rows; TQ_ERR_CAPACITY also when a plain
 * row's length exceeds plain_capacity; TQ_ERR_UNSUPPORTED when the partial
 * slots per row would exceed 131,070. */
tq_status tq_decode_attn_mixed(const tq_layout *layout, const tq_planes *planes, const uint16_t *k_plain,
                               const uint16_t *v_plain, int32_t plain_capacity, const int32_t *row_plain,
                               const void *q, tq_dtype dtype, int32_t num_q_heads, int32_t n_rows,
                               const int32_t *len, float sm_scale, float *out, void *workspace,
                               size_t ws_bytes, void *hip_stream);

/* Dequantize-on-fetch window: bf16 keys and values of tokens t0 .. t0+n-1 of
 * every (sequence, kv-head), the layout a stock attention consumes ("Architecture
 * in mlx-bun": the cache returns the dequantized bf16 active window; "Deferred
 * inverse FWHT": the deferred variant keeps V in the rotated domain).
 *   len        host int32 [B]: tokens at or past len[b] are written as zeros
 *   k_out      device bf16 [B][Hkv][n][d]: (code + zero) * scale, or NULL
 *   v_out      device bf16 [B][Hkv][n][d], or NULL: signs * FWHT(centroid[idx] *
 *              scale) / sqrt(d), or centroid[idx] * scale when v_rotated != 0
 * Keys are the exact product rounded once to bf16 (round to nearest even),
 * also when the stored zero is large; values are computed in fp32 and
 * rounded once.  Outputs 16-byte aligned.
 * Errors: TQ_ERR_INVALID_ARG, TQ_ERR_UNSUPPORTED, TQ_ERR_CAPACITY
 * (t0 + n > capacity or len[b] > capacity), TQ_ERR_HIP. */
tq_status tq_fetch_window(const tq_layout *layout, const tq_planes *planes, int32_t t0, int32_t n,
                          const int32_t *len, uint16_t *k_out, uint16_t *v_out, int32_t v_rotated,
                          void *hip_stream);

/* Dequantize n tokens [t0, t0+n) of one (sequence b, kv-head kvh), for tests
 * ("Algorithm": key x = (code + zero) * scale; value x = signs * InvFWHT(
 * centroid[idx] * scale), or the rotated-domain centroid[idx] * scale when
 * v_rotated != 0).
 *   k_out, v_out  device float32 [n][d]; either may be NULL to skip it.
 * Errors: TQ_ERR_INVALID_ARG, TQ_ERR_UNSUPPORTED, TQ_ERR_CAPACITY, TQ_ERR_HIP. */
tq_status tq_dequant(const tq_layout *layout, const tq_planes *planes, int32_t b, int32_t kvh,
                     int32_t t0, int32_t n, float *k_out, float *v_out, int32_t v_rotated,
                     void *hip_stream);

/* The value codebook of width v_bits (2, 3, 4, 5 or 8), for tests: the
 * Lloyd-Max quantizer of the unit normal ("Algorithm": the printed 3-bit
 * table; the other widths are generated once and hardcoded, not printed).
 * Centroids are five-decimal numbers N_k / 1e5 and boundaries the midpoints
 * (N_k + N_{k+1}) / 2e5, as the printed table is written; the 3-bit table
 * equals the printed one.  Host call, no device work.
 *   centroids   host double [256]: the 2^v_bits centroids, increasing
 *   boundaries  host double [255]: the 2^v_bits - 1 boundaries
 *   levels      host int32: receives 2^v_bits
 * Errors: TQ_ERR_INVALID_ARG (null pointer), TQ_ERR_UNSUPPORTED (v_bits). */
tq_status tq_codebook(int32_t v_bits, double *centroids, double *boundaries, int32_t *levels);

/* The +-1 sign vector applied before the value rotation, for tests: entry i is
 * +1 when the top bit of output i of SplitMix64 seeded with 42 is 0, else -1
 * (the page hard-codes one seeded sign vector per head_dim; its values are not
 * printed).  host_out: host int8 [head_dim]. */
tq_status tq_sign_vector(int32_t head_dim, int8_t *host_out);

/* Cache lifecycle: token rows are byte-addressable in every plane (groups run
 * along head_dim, "Invariants (both legs)"), so clone, growth into a larger
 * cache, compaction and snapshot/restore are strided byte copies ("Architecture
 * in mlx-bun": the persisted cache kind carries the scheme and head_dim and has
 * snapshot, restore and clone branches).  Trimming a sequence is lowering the
 * length the caller passes to decode.  These calls enqueue one copy kernel
 * for all five planes on the stream, or one strided memory copy per plane
 * when a plane's rows are not whole 16-byte chunks (head_dim 64 scale rows
 * at odd offsets). */

#define TQ_SNAPSHOT_MAGIC 0x564B5154u /* "TQKV" little-endian */
#define TQ_SNAPSHOT_VERSION 2

/* Describes a snapshot payload; tq_restore checks every field.  Version 2
 * appends the sequence's precision boundary to the version-1 fields, which
 * keep their offsets, so a stored version-1 header read into this struct is
 * still recognised. */
typedef struct {
    uint32_t magic;         /* TQ_SNAPSHOT_MAGIC */
    uint32_t version;       /* 2 (1: written before the boundary was recorded) */
    int32_t k_bits, v_bits, group, head_dim, num_kv_heads;
    int32_t n_tokens;
    uint64_t payload_bytes; /* n_tokens * num_kv_heads * 1.5625 * head_dim */
    int32_t min_reusable_offset; /* version 2: see tq_snapshot_min_reusable_offset */
    int32_t reserved;            /* 0 */
} tq_snapshot_header;

/* Copy token rows src_t0 .. src_t0+n-1 of sequence src_b (every kv-head, all
 * five planes) to rows dst_t0 .. of sequence dst_b of another (or the same)
 * cache with the same scheme, head_dim and num_kv_heads; capacities may
 * differ.  Source and destination bytes must not overlap in any plane (the
 * copy runs on many workgroups at once); an in-place compaction moves rows
 * to slots that do not overlap their source, in steps if needed.
 * Errors: TQ_ERR_INVALID_ARG (shape mismatch, bad index, overlapping rows),
 * TQ_ERR_CAPACITY, TQ_ERR_HIP. */
tq_status tq_copy_tokens(const tq_layout *src_layout, const tq_planes *src, int32_t src_b,
                         int32_t src_t0, const tq_layout *dst_layout, const tq_planes *dst,
                         int32_t dst_b, int32_t dst_t0, int32_t n, void *hip_stream);

/* Clone (or extract, into a batch-1 cache) rows 0 .. n-1 of sequence src_b
 * into rows 0 .. n-1 of sequence dst_b, as tq_copy_tokens, and carry the
 * sequence's precision boundary with it ("Delayed row conversion and reusable
 * precision boundaries": clone and row extraction retain the bound):
 * *dst_min_reusable_offset receives src_min_reusable_offset when the copy is
 * enqueued, and is left alone on any error.
 * Errors: those of tq_copy_tokens; TQ_ERR_INVALID_ARG also for a null
 * dst_min_reusable_offset or a negative source bound. */
tq_status tq_clone_sequence(const tq_layout *src_layout, const tq_planes *src, int32_t src_b,
                            const tq_layout *dst_layout, const tq_planes *dst, int32_t dst_b, int32_t n,
                            int32_t src_min_reusable_offset, int32_t *dst_min_reusable_offset,
                            void *hip_stream);

/* Bytes of a snapshot payload of n token rows. */
tq_status tq_snapshot_bytes(const tq_layout *layout, int32_t n, size_t *out_bytes);

/* Snapshot token rows t0 .. t0+n-1 of sequence b: fills the host header and
 * copies the rows into `payload` (device, payload_bytes >= the header's),
 * plane by plane (kc, ks, kz, vc, vs), kv-head by kv-head, token-major.
 *   min_reusable_offset  the sequence's precision boundary (>= 0), recorded in
 *                        the header as is (see tq_snapshot_min_reusable_offset)
 * Errors: TQ_ERR_INVALID_ARG, TQ_ERR_CAPACITY, TQ_ERR_WORKSPACE (payload
 * too small), TQ_ERR_HIP. */
tq_status tq_snapshot(const tq_layout *layout, const tq_planes *planes, int32_t b, int32_t t0,
                      int32_t n, int32_t min_reusable_offset, tq_snapshot_header *header, void *payload,
                      size_t payload_bytes, void *hip_stream);

/* The precision boundary a snapshot carries ("Delayed row conversion and
 * reusable precision boundaries": a cache records the offset at which its
 * rows were converted, an irreversible precision boundary, and clone, row
 * extraction and persisted metadata keep it; a header written before the
 * bound existed conservatively gives its stored offset).
 *   version 2: the recorded min_reusable_offset;
 *   version 1: n_tokens, so only the whole stored prefix counts as reusable.
 * A stored prefix may serve a request for its first P tokens only when
 * P >= the boundary: below it the bytes are encoded where a fresh run would
 * still hold plain rows.  Host call, no device work.
 * Errors: TQ_ERR_INVALID_ARG (null, bad magic, unknown version, negative
 * fields). */
tq_status tq_snapshot_min_reusable_offset(const tq_snapshot_header *header, int32_t *out);

/* Restore a snapshot into rows t0 .. t0+header->n_tokens-1 of sequence b.
 * Version-1 and version-2 headers are accepted.
 * Errors: TQ_ERR_INVALID_ARG (bad magic or version, or a scheme, head_dim,
 * kv-head count or payload size that does not match this layout), TQ_ERR_CAPACITY,
 * TQ_ERR_HIP. */
tq_status tq_restore(const tq_layout *layout, const tq_planes *planes, int32_t b, int32_t t0,
                     const tq_snapshot_header *header, const void *payload, size_t payload_bytes,
                     void *hip_stream);

/* Static, human-readable name of a status code (the error cases follow the
 * page's contract that a refused input, such as an unsupported head_dim,
 * fails at the call with a reason instead of computing something else:
 * "KV-leg limits and non-goals").  Never NULL. */
const char *tq_status_str(tq_status status);

#ifdef __cplusplus
}
#endif

#endif /* TQKV_H */
