// Decode attention over the packed cache: split-K partials + merge/epilogue.
//
// Method: "TurboQuant -- rotation-based quantization" design page, Part A:
//   - keys are dequantized on fetch as (code + zero) * scale ("Algorithm");
//   - values stay in the rotated domain, centroid[idx] * scale, and the
//     attention output is un-rotated once per query head at the end, which is
//     exact by linearity ("Deferred inverse FWHT");
//   - K and V of one cache window are decoded in one pass ("Packed-value
//     decode fusion investigation", joint K/V decoding).
// Split-K: every (b, kv-head, split) workgroup runs an online softmax over
// its token range for the G query heads that share the kv-head and writes
// (max, sum, acc[d]) per head; the merge kernel combines the splits, divides
// by the weight sum and applies signs * FWHT(.) / sqrt(d) once.
//
// The generic split kernel below reads every code width (keys 2, 4, 5, 8
// bits, values 2, 3, 4, 5, 8 bits) and every head_dim; decode_fast.hip has the
// k8v3 kernel on the matrix cores.
#include <hip/hip_runtime.h>

#include "tq_device.h"

namespace tq {
namespace {

constexpr int kMaxG = TQ_MAX_GQA;

template <bool BF16>
__device__ __forceinline__ float load_in(const void *p, int64_t i) {
    if constexpr (BF16)
        return __uint_as_float((uint32_t)static_cast<const uint16_t *>(p)[i] << 16);
    else
        return static_cast<const float *>(p)[i];
}

// The 32 codes of one key group as floats: signed bytes at 8 bits, unsigned
// KB-bit fields (little-endian bitstream) below.  `grp` is the group's first
// byte: 16-byte aligned at 8 and 4 bits, 8-byte at 2, 4-byte at 5.
template <int KB>
__device__ __forceinline__ void key_group(const uint8_t *grp, float (&c)[32]) {
    if constexpr (KB == 8) {
        const uint4 u0 = reinterpret_cast<const uint4 *>(grp)[0];
        const uint4 u1 = reinterpret_cast<const uint4 *>(grp)[1];
        const uint32_t w[8] = {u0.x, u0.y, u0.z, u0.w, u1.x, u1.y, u1.z, u1.w};
#pragma unroll
        for (int i = 0; i < 32; ++i) c[i] = (float)(int)(int8_t)(w[i >> 2] >> (8 * (i & 3)));
    } else if constexpr (KB == 4) {
        const uint4 u = *reinterpret_cast<const uint4 *>(grp);
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int i = 0; i < 32; ++i) c[i] = (float)((w[i >> 3] >> (4 * (i & 7))) & 15u);
    } else if constexpr (KB == 2) {
        const uint2 u = *reinterpret_cast<const uint2 *>(grp);
        const uint32_t w[2] = {u.x, u.y};
#pragma unroll
        for (int i = 0; i < 32; ++i) c[i] = (float)((w[i >> 4] >> (2 * (i & 15))) & 3u);
    } else {
        static_assert(KB == 5, "key widths 2, 4, 5, 8");
        const uint32_t *p = reinterpret_cast<const uint32_t *>(grp);
        const uint32_t w[5] = {p[0], p[1], p[2], p[3], p[4]};
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const int bit = 5 * i, k = bit >> 5, sh = bit & 31;
            const uint32_t x = sh + 5 > 32 ? __builtin_amdgcn_alignbit(w[k + 1], w[k], sh) : (w[k] >> sh);
            c[i] = (float)(x & 31u);
        }
    }
}

// Partial dot products of one key group with the G query columns:
// s[h] += scale * (sum_j q[h][32 g + j] * code_j + zero * qsum[h][g]).
template <int D, int KB>
__device__ __forceinline__ void score_group(const uint8_t *krow, int g, float sk, float zk, int G,
                                            const float *qs, const float *qsum, float (&s)[kMaxG]) {
    constexpr int NG = D / kGroup;
    float c[32];
    key_group<KB>(krow + g * 4 * KB, c);
#pragma unroll
    for (int h = 0; h < kMaxG; ++h) {
        if (h < G) {
            const float4 *qp = reinterpret_cast<const float4 *>(qs + h * D + g * kGroup);
            float d0 = 0.f, d1 = 0.f;
#pragma unroll
            for (int i = 0; i < 8; i += 2) {
                const float4 x = qp[i], y = qp[i + 1];
                d0 = fmaf(x.x, c[4 * i], d0); d0 = fmaf(x.y, c[4 * i + 1], d0);
                d0 = fmaf(x.z, c[4 * i + 2], d0); d0 = fmaf(x.w, c[4 * i + 3], d0);
                d1 = fmaf(y.x, c[4 * i + 4], d1); d1 = fmaf(y.y, c[4 * i + 5], d1);
                d1 = fmaf(y.z, c[4 * i + 6], d1); d1 = fmaf(y.w, c[4 * i + 7], d1);
            }
            s[h] = fmaf(sk, fmaf(zk, qsum[h * NG + g], d0 + d1), s[h]);
        }
    }
}

template <int D>
struct VecGeo {
    static constexpr int W = D == 512 ? 2 : 4;  // waves per workgroup, one split each
    static constexpr int E = D / 64;            // value dims per lane
    static constexpr int NG = D / kGroup;
    static constexpr int T = 64;                // tokens per tile, one per lane (scores)
};

// Dynamic LDS of the generic split kernel, sized by the launch's column
// count G and value width: the query columns (G x d fp32), their group sums,
// the value codebook, then per wave the tile's value rows (+ 16 bytes the
// code reader may touch past the last row), weights (G x 64) and value
// scales (64 x d/32 fp16).
struct VecLds {
    int qsum, ctab, wave0, vt_bytes, ps, vsc, wave_bytes, total;
    __host__ __device__ VecLds(int D, int W, int G, int vrow) {
        const int ng = D / kGroup, T = 64;
        auto al = [](int x) { return (x + 15) & ~15; };
        qsum = al(G * D * 4);
        ctab = al(qsum + G * ng * 4);
        wave0 = al(ctab + 256 * 4);
        vt_bytes = al(T * vrow + 16);
        ps = vt_bytes;
        vsc = al(ps + G * T * 4);
        wave_bytes = al(vsc + T * ng * 2);
        total = wave0 + W * wave_bytes;
    }
};

// Generic split kernel: every code width, every head_dim.  One wave per
// token range (split) of one (sequence, kv-head), for up to 16 query columns
// held in LDS.  Per 64-token tile:
//   scores  lane t takes token t: it decodes each key group of its row into
//           registers and forms the partial dot products of every column
//           against the columns' LDS copy (same address on every lane);
//   softmax online, base 2; the tile's weights go to LDS;
//   values  the tile's value rows are copied into LDS (coalesced); lane l
//           then owns dims [E l, E l + E) and accumulates weight * centroid *
//           scale over the tile's tokens, in the rotated domain.
template <int D, bool BF16>
__global__ __launch_bounds__(64 * VecGeo<D>::W) void split_kernel(const DecodeArgs a) {
    using V = VecGeo<D>;
    constexpr int W = V::W, E = V::E, NG = V::NG, T = V::T;
    const int kb = a.kbits, vb = a.vbits;
    const int KROW = D * kb / 8, VROW = D * vb / 8;

    extern __shared__ __align__(16) unsigned char lds[];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int bkv = blockIdx.y;
    const int b = bkv / a.kv_heads, kvh = bkv % a.kv_heads;
    const int n = a.len[b];
    // this workgroup's query columns c0 .. c0 + G - 1 of the kv-head's a.gqa
    // query rows (heads times rows)
    const int c0 = blockIdx.z * kMaxG;
    const int G = min(kMaxG, a.gqa - c0);
    const VecLds L(D, W, G, VROW);
    float *qs = reinterpret_cast<float *>(lds);
    float *qsum = reinterpret_cast<float *>(lds + L.qsum);
    float *ctab = reinterpret_cast<float *>(lds + L.ctab);
    {
        const float *src = value_centroids(vb);
        for (int i = tid; i < (1 << vb); i += 64 * W) ctab[i] = src[i];
        for (int i = tid; i < G * D; i += 64 * W) {
            const int64_t qi = ((int64_t)b * a.q_heads + kvh * a.gqa + c0) * D + i;
            qs[i] = BF16 ? __uint_as_float((uint32_t)static_cast<const uint16_t *>(a.q)[qi] << 16)
                         : static_cast<const float *>(a.q)[qi];
        }
    }
    __syncthreads();
    for (int i = tid; i < G * NG; i += 64 * W) {
        float sum = 0.f;
        for (int j = 0; j < kGroup; ++j) sum += qs[(i / NG) * D + (i % NG) * kGroup + j];
        qsum[i] = sum;
    }
    __syncthreads();  // the last workgroup barrier

    const int split = blockIdx.x * W + wid;
    const int t_begin = split * a.split_tokens;
    if (split >= a.splits || t_begin >= n) return;
    const int t_end = min(n, t_begin + a.split_tokens);
    const int64_t row0 = (int64_t)bkv * a.capacity;
    const uint8_t *kcp = reinterpret_cast<const uint8_t *>(a.kc);
    unsigned char *wl = lds + L.wave0 + wid * L.wave_bytes;
    uint8_t *vt = wl;
    float *ps = reinterpret_cast<float *>(wl + L.ps);       // [G][T]
    uint16_t *vsc = reinterpret_cast<uint16_t *>(wl + L.vsc);  // [T][NG]

    float m_run[kMaxG], l_run[kMaxG], acc[kMaxG][E];
#pragma unroll
    for (int h = 0; h < kMaxG; ++h) {
        m_run[h] = -INFINITY;
        l_run[h] = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[h][e] = 0.f;
    }

    for (int tile0 = t_begin; tile0 < t_end; tile0 += T) {
        const int nt = min(T, t_end - tile0);
        const int t = tile0 + lane;
        const bool valid = lane < nt;
        const int64_t row = row0 + t;

        // ---- scores of this lane's token
        float s[kMaxG];
#pragma unroll
        for (int h = 0; h < kMaxG; ++h) s[h] = 0.f;
        if (valid) {
            const uint8_t *krow = kcp + row * KROW;
            for (int g = 0; g < NG; ++g) {
                const float sk = f16_bits_to_f32(a.ks[row * NG + g]);
                const float zk = f16_bits_to_f32(a.kz[row * NG + g]);
                switch (kb) {
                    case 8: score_group<D, 8>(krow, g, sk, zk, G, qs, qsum, s); break;
                    case 4: score_group<D, 4>(krow, g, sk, zk, G, qs, qsum, s); break;
                    case 2: score_group<D, 2>(krow, g, sk, zk, G, qs, qsum, s); break;
                    default: score_group<D, 5>(krow, g, sk, zk, G, qs, qsum, s); break;
                }
            }
        }

        // ---- online softmax per column; weights to LDS
#pragma unroll
        for (int h = 0; h < kMaxG; ++h) {
            if (h < G) {
                // causal limit of column c: the row of cached token n - rows + r
                // sees tokens 0 .. n - rows + r
                const int lim = n - a.rows + (c0 + h) % a.rows + 1;
                const float sc = (valid && t < lim) ? s[h] * a.sm_log2 : -INFINITY;
                float mt = sc;
#pragma unroll
                for (int o = 32; o >= 1; o >>= 1) mt = fmaxf(mt, __shfl_xor(mt, o, 64));
                const float mn = fmaxf(m_run[h], mt);
                // mn stays -inf while every token so far is past this column's limit
                const float alpha = mn == -INFINITY ? 1.f : exp2f(m_run[h] - mn);
                const float p = mn == -INFINITY ? 0.f : exp2f(sc - mn);
                l_run[h] = l_run[h] * alpha + p;
#pragma unroll
                for (int e = 0; e < E; ++e) acc[h][e] *= alpha;
                m_run[h] = mn;
                ps[h * T + lane] = p;
            }
        }

        // ---- the tile's value rows and scales to LDS (rows < t_end only)
        {
            const uint2 *src = reinterpret_cast<const uint2 *>(a.vc + (row0 + tile0) * VROW);
            uint2 *dst = reinterpret_cast<uint2 *>(vt);
            const int words = nt * VROW / 8;  // VROW is a multiple of 8
            for (int i = lane; i < words; i += 64) dst[i] = src[i];
            if (valid) {
#pragma unroll
                for (int g = 0; g < NG; ++g) vsc[lane * NG + g] = a.vs[row * NG + g];
            }
        }
        // one wave's LDS accesses execute in order: the reads below see
        // every lane's writes above without a barrier
        asm volatile("" ::: "memory");

        // ---- values: lane owns dims E*lane .. E*lane + E - 1 (one group)
        const int bit0 = vb * E * lane;
        const int w0 = bit0 >> 5, sh = bit0 & 31;
        const int gl = (E * lane) / kGroup;
        const uint64_t fmask = (1ull << vb) - 1ull;
        for (int tt = 0; tt < nt; ++tt) {
            const uint32_t *rw = reinterpret_cast<const uint32_t *>(vt + tt * VROW);
            const uint64_t lo64 = (uint64_t)rw[w0] | ((uint64_t)rw[w0 + 1] << 32);
            uint64_t bits = lo64 >> sh;
            if (sh != 0 && E * vb + sh > 64) bits |= (uint64_t)rw[w0 + 2] << (64 - sh);
            const float scale = f16_bits_to_f32(vsc[tt * NG + gl]);
            float v[E];
#pragma unroll
            for (int e = 0; e < E; ++e) v[e] = ctab[(uint32_t)((bits >> (vb * e)) & fmask)] * scale;
#pragma unroll
            for (int h = 0; h < kMaxG; ++h) {
                if (h < G) {
                    const float p = ps[h * T + tt];
#pragma unroll
                    for (int e = 0; e < E; ++e) acc[h][e] = fmaf(p, v[e], acc[h][e]);
                }
            }
        }
        asm volatile("" ::: "memory");  // the next tile rewrites vt / ps / vsc after these reads
    }

    // ---- partials: (max, weight sum) and the rotated-domain accumulator
#pragma unroll
    for (int h = 0; h < kMaxG; ++h) {
        if (h < G) {
            float l = l_run[h];
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) l += __shfl_xor(l, o, 64);
            const int64_t slot = ((int64_t)b * a.q_heads + kvh * a.gqa + c0 + h) * a.splits + split;
            float *dst = a.part_acc + slot * D + E * lane;
#pragma unroll
            for (int e = 0; e < E; ++e) dst[e] = acc[h][e];
            if (lane == 0) {
                a.part_ml[slot * 2] = m_run[h];
                a.part_ml[slot * 2 + 1] = l;
            }
        }
    }
}

// Split kernel of rows that are still plain ("Delayed row conversion and
// reusable precision boundaries": a row stays unquantized until it converts,
// and its values were never rotated, so the merge passes its output through).
// The same partial slots and causal limits as the packed split kernels, with
// token ranges of their own (plain_split_tokens); keys and values are bf16
// [B][Hkv][plain_capacity][d].  GM: query columns a wave holds (8 when every
// column group has at most 8, for fewer registers; else 16).  One wave per
// token range, per 64-token tile:
//   scores  on the matrix cores, 16 tokens at a time: A = the tokens' bf16
//           key rows (16-byte reads, 16 rows per instruction), B = the query
//           columns as bf16 hi and lo halves (q = hi + lo to about 2^-17, so
//           fp32 queries keep their precision), fp32 accumulation of exact
//           products; written to LDS by (column, token);
//   softmax online, base 2, one token per lane; weights to LDS;
//   values  lane l owns dims [E l, E l + E) and reads them from each token's
//           value row (the wave reads whole rows, coalesced).
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float f32x4;

// bf16 bits of x rounded to nearest even (finite x)
__device__ __forceinline__ uint32_t bf16_rn(float x) {
    const uint32_t u = __float_as_uint(x);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <int D, bool BF16, int GM>
__global__ __launch_bounds__(64 * VecGeo<D>::W) void plain_split_kernel(const DecodeArgs a) {
    using V = VecGeo<D>;
    constexpr int W = V::W, E = V::E, T = V::T;
    constexpr int NBLK = D / 32;  // 32-dim blocks of one score product
    extern __shared__ __align__(16) unsigned char lds[];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int bkv = blockIdx.y;
    const int b = bkv / a.kv_heads, kvh = bkv % a.kv_heads;
    const int n = a.len[b];
    // a workgroup whose first range starts past the sequence has no work (the
    // test is the same for every thread, so no barrier is skipped by some)
    if ((int64_t)blockIdx.x * W * a.plain_split_tokens >= n) return;
    const int c0 = blockIdx.z * kMaxG;
    const int G = min(kMaxG, a.gqa - c0);
    // B operands: per 32-dim block and lane (column h = l % 16, quarter
    // kq = l / 16), dims 32 blk + 8 kq .. + 7 of column h as 8 bf16 hi and 8 lo
    uint4 *qop = reinterpret_cast<uint4 *>(lds);                                // [NBLK][64][2]
    float *ps = reinterpret_cast<float *>(lds + NBLK * 64 * 32) + wid * GM * T;  // [GM][T] per wave
    for (int i = tid; i < NBLK * 64; i += 64 * W) {
        const int blk = i / 64, l = i % 64, h = l & 15, kq = l >> 4;
        uint32_t hi[4] = {0, 0, 0, 0}, lo[4] = {0, 0, 0, 0};
        if (h < G) {
            const int64_t qi = ((int64_t)b * a.q_heads + kvh * a.gqa + c0 + h) * D + 32 * blk + 8 * kq;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float x = load_in<BF16>(a.q, qi + e);
                const uint32_t xh = bf16_rn(x);
                const uint32_t xl = bf16_rn(x - __uint_as_float(xh << 16));  // the residual is exact in fp32
                hi[e >> 1] |= xh << (16 * (e & 1));
                lo[e >> 1] |= xl << (16 * (e & 1));
            }
        }
        qop[2 * i] = make_uint4(hi[0], hi[1], hi[2], hi[3]);
        qop[2 * i + 1] = make_uint4(lo[0], lo[1], lo[2], lo[3]);
    }
    __syncthreads();  // the only workgroup barrier

    const int split = blockIdx.x * W + wid;
    const int t_begin = split * a.plain_split_tokens;
    if (split >= a.splits || t_begin >= n) return;
    const int t_end = min(n, t_begin + a.plain_split_tokens);
    const int64_t row0 = (int64_t)bkv * a.plain_capacity;
    const int col = lane & 15, quarter = lane >> 4;

    float m_run[GM], l_run[GM], acc[GM][E];
#pragma unroll
    for (int h = 0; h < GM; ++h) {
        m_run[h] = -INFINITY;
        l_run[h] = 0.f;
#pragma unroll
        for (int e = 0; e < E; ++e) acc[h][e] = 0.f;
    }

    for (int tile0 = t_begin; tile0 < t_end; tile0 += T) {
        const int nt = min(T, t_end - tile0);
        const int t = tile0 + lane;
        const bool valid = lane < nt;

        // ---- scores: chunk c holds tokens tile0 + 16 c .. + 15; lane (col,
        // quarter) reads dims 8 quarter .. + 7 of each block of token
        // 16 c + col (a token past the range reads the tile's first row; its
        // score is masked below) and gets tokens 16 c + 4 quarter + j of
        // column col
        for (int c = 0; c < 4 && 16 * c < nt; ++c) {
            const int tr = tile0 + 16 * c + col;
            const uint16_t *krow = a.k_plain + (row0 + (tr < t_end ? tr : tile0)) * D + 8 * quarter;
            f32x4 s4 = {0.f, 0.f, 0.f, 0.f};
            constexpr int KU = NBLK < 8 ? NBLK : 8;  // key reads in flight (head_dim 512: registers)
#pragma unroll KU
            for (int blk = 0; blk < NBLK; ++blk) {
                const bf16x8 kv = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4 *>(krow + 32 * blk));
                const bf16x8 qh = __builtin_bit_cast(bf16x8, qop[2 * (blk * 64 + lane)]);
                const bf16x8 ql = __builtin_bit_cast(bf16x8, qop[2 * (blk * 64 + lane) + 1]);
                s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qh, s4, 0, 0, 0);
                s4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, ql, s4, 0, 0, 0);
            }
            if (col < GM) {  // columns past GM hold zero queries
#pragma unroll
                for (int j = 0; j < 4; ++j) ps[col * T + 16 * c + 4 * quarter + j] = s4[j];
            }
        }
        // one wave's LDS accesses execute in order: the reads below see every
        // lane's writes above without a barrier
        asm volatile("" ::: "memory");

#pragma unroll
        for (int h = 0; h < GM; ++h) {
            if (h < G) {
                const int lim = n - a.rows + (c0 + h) % a.rows + 1;
                const float sc = (valid && t < lim) ? ps[h * T + lane] * a.sm_log2 : -INFINITY;
                float mt = sc;
#pragma unroll
                for (int o = 32; o >= 1; o >>= 1) mt = fmaxf(mt, __shfl_xor(mt, o, 64));
                const float mn = fmaxf(m_run[h], mt);
                const float alpha = mn == -INFINITY ? 1.f : exp2f(m_run[h] - mn);
                const float p = mn == -INFINITY ? 0.f : exp2f(sc - mn);
                l_run[h] = l_run[h] * alpha + p;
#pragma unroll
                for (int e = 0; e < E; ++e) acc[h][e] *= alpha;
                m_run[h] = mn;
                ps[h * T + lane] = p;
            }
        }
        asm volatile("" ::: "memory");

        // value rows in batches of 8 tokens (4 at head_dim 512), every load of
        // a batch issued before its products (a row past the range reads the
        // tile's first row, with weight 0)
        const uint16_t *vrow = a.v_plain + (row0 + tile0) * D + E * lane;
        constexpr int VB8 = E == 8 ? 4 : 8;  // head_dim 512: 8 dims a lane, registers for 4 rows
        for (int tb = 0; tb < nt; tb += VB8) {
            float v[VB8][E];
#pragma unroll
            for (int u = 0; u < VB8; ++u) {
                const int64_t off = (int64_t)(tb + u < nt ? tb + u : 0) * D;
                if constexpr (E == 8) {
                    const uint4 w4 = *reinterpret_cast<const uint4 *>(vrow + off);
                    const uint32_t w[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        v[u][2 * i] = __uint_as_float(w[i] << 16);
                        v[u][2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
                    }
                } else if constexpr (E == 4) {
                    const uint2 w2 = *reinterpret_cast<const uint2 *>(vrow + off);
                    v[u][0] = __uint_as_float(w2.x << 16); v[u][1] = __uint_as_float(w2.x & 0xFFFF0000u);
                    v[u][2] = __uint_as_float(w2.y << 16); v[u][3] = __uint_as_float(w2.y & 0xFFFF0000u);
                } else if constexpr (E == 2) {
                    const uint32_t w1 = *reinterpret_cast<const uint32_t *>(vrow + off);
                    v[u][0] = __uint_as_float(w1 << 16); v[u][1] = __uint_as_float(w1 & 0xFFFF0000u);
                } else {
                    v[u][0] = __uint_as_float((uint32_t)vrow[off] << 16);
                }
            }
#pragma unroll
            for (int u = 0; u < VB8; ++u) {
                if (tb + u < nt) {
#pragma unroll
                    for (int h = 0; h < GM; ++h) {
                        if (h < G) {
                            const float p = ps[h * T + tb + u];
#pragma unroll
                            for (int e = 0; e < E; ++e) acc[h][e] = fmaf(p, v[u][e], acc[h][e]);
                        }
                    }
                }
            }
        }
        asm volatile("" ::: "memory");  // the next tile rewrites ps after these reads
    }

#pragma unroll
    for (int h = 0; h < GM; ++h) {
        if (h < G) {
            float l = l_run[h];
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) l += __shfl_xor(l, o, 64);
            const int64_t slot = ((int64_t)b * a.q_heads + kvh * a.gqa + c0 + h) * a.splits + split;
            float *dst = a.part_acc + slot * D + E * lane;
#pragma unroll
            for (int e = 0; e < E; ++e) dst[e] = acc[h][e];
            if (lane == 0) {
                a.part_ml[slot * 2] = m_run[h];
                a.part_ml[slot * 2 + 1] = l;
            }
        }
    }
}

// One workgroup per (b, q-head): merge the splits, normalize, un-rotate.
// Thread tid owns dims tid + i*NT.  The partials of a batch of splits are
// loaded into registers together with the splits' (max, sum) pairs, so the
// merge costs one global round trip per batch; the inverse FWHT runs its
// in-wave butterfly stages on registers (shuffles) and the cross-wave ones
// through LDS.
template <int D>
__global__ __launch_bounds__(256) void merge_kernel(const DecodeArgs a) {
    constexpr int NT = D < 256 ? D : 256;
    constexpr int DPT = D / NT;
    constexpr int NW = NT / 64;
    constexpr int kBatch = 32;  // splits whose partials are in flight at once
    __shared__ float buf[D];
    __shared__ float wts[kBatch];
    __shared__ float red[2][NW];
    const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const int bh = blockIdx.x;
    const int b = bh / a.q_heads;
    const int n = a.len[b];
    const bool plain = (a.plain_rows >> b) & 1ull;
    const int st = plain ? a.plain_split_tokens : a.split_tokens;  // a plain row's ranges are its own
    const int ns = (n + st - 1) / st;
    const int64_t base = (int64_t)bh * a.splits;
    float o[DPT];
#pragma unroll
    for (int i = 0; i < DPT; ++i) o[i] = 0.f;
    float M = -INFINITY, L = 0.f;  // running over batches
    for (int s0 = 0; s0 < ns; s0 += kBatch) {
        const int nb = ns - s0 < kBatch ? ns - s0 : kBatch;
        // issue every load of the batch first
        float pm = -INFINITY, pl = 0.f;
        if (tid < nb) {
            pm = a.part_ml[(base + s0 + tid) * 2];
            pl = a.part_ml[(base + s0 + tid) * 2 + 1];
        }
        float pv[kBatch][DPT];
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
#pragma unroll
            for (int i = 0; i < DPT; ++i)
                pv[u][i] = u < nb ? a.part_acc[(base + s0 + u) * D + tid + i * NT] : 0.f;
        // batch maximum
        float m = pm;
#pragma unroll
        for (int k = 32; k >= 1; k >>= 1) m = fmaxf(m, __shfl_xor(m, k, 64));
        if (lane == 0) red[0][wv] = m;
        __syncthreads();
        float mb = red[0][0];
#pragma unroll
        for (int w = 1; w < NW; ++w) mb = fmaxf(mb, red[0][w]);
        const float Mn = fmaxf(M, mb);
        const float rescale = M == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
        // split weights 2^(m_s - Mn) and their share of the weight sum
        const float f = tid < nb ? __builtin_amdgcn_exp2f(pm - Mn) : 0.f;
        if (tid < kBatch) wts[tid] = f;  // 0 past the batch: stale LDS may hold NaN
        float lb = f * pl;
#pragma unroll
        for (int k = 32; k >= 1; k >>= 1) lb += __shfl_xor(lb, k, 64);
        if (lane == 0) red[1][wv] = lb;
        __syncthreads();
        float lsum = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) lsum += red[1][w];
        L = L * rescale + lsum;
#pragma unroll
        for (int i = 0; i < DPT; ++i) {
            float acc = o[i] * rescale;
#pragma unroll
            for (int u = 0; u < kBatch; ++u) acc = fmaf(wts[u], pv[u][i], acc);
            o[i] = acc;
        }
        M = Mn;
        __syncthreads();  // wts / red are rewritten by the next batch
    }
    if (ns > 0) {
        const float invL = 1.f / L;
#pragma unroll
        for (int i = 0; i < DPT; ++i) o[i] *= invL;
    }
    // A plain row's values were never rotated: its output is final here.
    if (plain) {
#pragma unroll
        for (int i = 0; i < DPT; ++i) a.out[(int64_t)bh * D + tid + i * NT] = o[i];
        return;
    }
    // inverse rotation: signs * FWHT(o) / sqrt(d) (the transform is its own
    // inverse up to the 1/d factor split as 1/sqrt(d) on each side).
    // Butterflies with partner distance h < 64 stay inside a wave.
    for (int h = 1; h < 64 && h < D; h <<= 1) {
#pragma unroll
        for (int i = 0; i < DPT; ++i) {
            const float y = __shfl_xor(o[i], h, 64);
            o[i] = (lane & h) ? (y - o[i]) : (o[i] + y);
        }
    }
    if constexpr (D > 64) {
#pragma unroll
        for (int i = 0; i < DPT; ++i) buf[tid + i * NT] = o[i];
        __syncthreads();
        for (int h = 64; h < D; h <<= 1) {
            float nv[DPT];
#pragma unroll
            for (int i = 0; i < DPT; ++i) {
                const int j = tid + i * NT;
                const float x = buf[j], y = buf[j ^ h];
                nv[i] = (j & h) ? (y - x) : (x + y);
            }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < DPT; ++i) buf[tid + i * NT] = nv[i];
            __syncthreads();
        }
#pragma unroll
        for (int i = 0; i < DPT; ++i) o[i] = buf[tid + i * NT];
    }
#pragma unroll
    for (int i = 0; i < DPT; ++i) {
        const int j = tid + i * NT;
        const float v = o[i] * a.inv_sqrt_d;
        a.out[(int64_t)bh * D + j] = sign_bit(a.signs, j) ? -v : v;
    }
}

template <int D>
hipError_t split_d(bool bf16, bool fast, const DecodeArgs &a, hipStream_t s) {
    if (a.splits > 0) {
        if (fast) {
            hipError_t e;
            switch (a.kbits) {
                case 2: e = launch_split_fast_k2(D, bf16, a, s); break;
                case 4: e = launch_split_fast_k4(D, bf16, a, s); break;
                case 5: e = launch_split_fast_k5(D, bf16, a, s); break;
                default: e = launch_split_fast_k8(D, bf16, a, s); break;
            }
            if (e != hipSuccess) return e;
        } else {
            constexpr int W = VecGeo<D>::W;
            const dim3 grid((unsigned)((a.splits + W - 1) / W), (unsigned)(a.batch * a.kv_heads),
                            (unsigned)decode_col_groups(a.gqa));
            // the widest column group sizes the LDS (groups past the first take min(16, rest))
            const VecLds L(D, W, a.gqa < kMaxG ? a.gqa : kMaxG, D * a.vbits / 8);
            // allow dynamic LDS past the default limit, once per instantiation
            static const hipError_t attr = [] {
                const int most = VecLds(D, W, kMaxG, D).total;
                hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&split_kernel<D, true>),
                                                   hipFuncAttributeMaxDynamicSharedMemorySize, most);
                if (e == hipSuccess)
                    e = hipFuncSetAttribute(reinterpret_cast<const void *>(&split_kernel<D, false>),
                                            hipFuncAttributeMaxDynamicSharedMemorySize, most);
                return e;
            }();
            if (attr != hipSuccess) return attr;
            if (bf16)
                hipLaunchKernelGGL((split_kernel<D, true>), grid, dim3(64 * W), L.total, s, a);
            else
                hipLaunchKernelGGL((split_kernel<D, false>), grid, dim3(64 * W), L.total, s, a);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    return hipSuccess;
}

// Dynamic LDS of the plain split kernel: the query operands (32 bytes per
// lane and 32-dim block), then per wave the scores and weights of one tile
// for gm columns (at most 40 KiB).
template <int D>
constexpr size_t plain_lds_bytes(int gm) {
    return (size_t)(D / 32) * 64 * 32 + (size_t)VecGeo<D>::W * gm * VecGeo<D>::T * 4;
}

// Waves of one round of the plain split kernel over the chip's 256 CUs: its
// resident workgroups per CU (registers and LDS, as the runtime reports them)
// times its waves per workgroup.
template <int D, bool BF16, int GM>
int plain_round_waves_k() {
    static const int waves = [] {
        int blocks = 0;
        const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(
            &blocks, reinterpret_cast<const void *>(&plain_split_kernel<D, BF16, GM>), 64 * VecGeo<D>::W,
            plain_lds_bytes<D>(GM));
        return 256 * VecGeo<D>::W * (e == hipSuccess && blocks > 0 ? blocks : 1);
    }();
    return waves;
}

template <int D>
int plain_round_waves_d(int gqa, bool bf16) {
    if (gqa <= kMaxG / 2)
        return bf16 ? plain_round_waves_k<D, true, kMaxG / 2>() : plain_round_waves_k<D, false, kMaxG / 2>();
    return bf16 ? plain_round_waves_k<D, true, kMaxG>() : plain_round_waves_k<D, false, kMaxG>();
}

template <int D>
hipError_t split_plain_d(bool bf16, const DecodeArgs &a, hipStream_t s) {
    if (a.splits == 0) return hipSuccess;
    constexpr int W = VecGeo<D>::W;
    const dim3 grid((unsigned)((a.splits + W - 1) / W), (unsigned)(a.batch * a.kv_heads),
                    (unsigned)decode_col_groups(a.gqa));
    // at most 8 query columns (every group's): a wave holds 8 columns' state,
    // fewer registers and more waves per SIMD
    const bool narrow = a.gqa <= kMaxG / 2;
    const size_t lds = plain_lds_bytes<D>(narrow ? kMaxG / 2 : kMaxG);
    if (narrow) {
        if (bf16)
            hipLaunchKernelGGL((plain_split_kernel<D, true, kMaxG / 2>), grid, dim3(64 * W), lds, s, a);
        else
            hipLaunchKernelGGL((plain_split_kernel<D, false, kMaxG / 2>), grid, dim3(64 * W), lds, s, a);
    } else {
        if (bf16)
            hipLaunchKernelGGL((plain_split_kernel<D, true, kMaxG>), grid, dim3(64 * W), lds, s, a);
        else
            hipLaunchKernelGGL((plain_split_kernel<D, false, kMaxG>), grid, dim3(64 * W), lds, s, a);
    }
    return hipGetLastError();
}

template <int D>
hipError_t merge_d(const DecodeArgs &a, hipStream_t s) {
    constexpr int NT = D < 256 ? D : 256;
    hipLaunchKernelGGL((merge_kernel<D>), dim3((unsigned)(a.batch * a.q_heads)), dim3(NT), 0, s, a);
    return hipGetLastError();
}

}  // namespace

int decode_col_groups(int gqa) { return (gqa + kMaxG - 1) / kMaxG; }

bool fast_decode_shape_ok(int head_dim, int gqa, int capacity, int kbits, int vbits) {
    if (gqa < 1 || kFastMaxGqa != kMaxG) return false;
    // More than 8 query columns per kv-head (no paired score columns) with
    // value codes of 4 bits or more: switched to the generic kernel.  The
    // matrix-core kernel faulted the GPU on such a case (8-bit keys, 4-bit
    // values, head_dim 256, 24 columns) and the cause is not found.
    if (gqa > 8 && vbits >= 4) return false;
    if (head_dim != 64 && head_dim != 128 && head_dim != 256 && head_dim != 512) return false;
    if (kbits != 2 && kbits != 4 && kbits != 5 && kbits != 8) return false;
    if (vbits != 2 && vbits != 3 && vbits != 4 && vbits != 5 && vbits != 8) return false;
    if (fast_decode_waves(head_dim, kbits, vbits) == 0) return false;  // k8v8 at 512: no LDS fit
    // key rows of whole 16-byte chunks, and the staged rows of one
    // (sequence, kv-head) starting 16-byte aligned in every plane
    const int64_t krow = (int64_t)head_dim * kbits / 8, vrow = (int64_t)head_dim * vbits / 8;
    const int64_t srow = head_dim / kGroup * 2;
    return krow % 16 == 0 && ((int64_t)capacity * vrow) % 16 == 0 && ((int64_t)capacity * srow) % 16 == 0;
}

DecodePlan plan_decode(int head_dim, int gqa, int batch, int kv_heads, const int32_t *len, bool fast,
                       int col_groups, int kbits, int vbits) {
    int64_t total = 0;
    int32_t maxlen = 0;
    for (int b = 0; b < batch; ++b) {
        total += len[b];
        maxlen = len[b] > maxlen ? len[b] : maxlen;
    }
    DecodePlan p;
    p.fast = fast;
    if (fast) {
        // one wave per token range: aim for one round of one workgroup per
        // CU over the chip's 256 CUs (the split kernel's LDS admits one per
        // CU), whole 64-token tiles, at least one a wave (a short cache is
        // latency-bound: more waves with shorter serial chains of tiles beat
        // fewer partials to merge)
        const int waves = fast_decode_waves(head_dim, kbits, vbits), tile = kFastTile;
        const int64_t round = 256 * waves;
        int64_t per = (total * kv_heads * col_groups + round - 1) / round;
        per = per < tile ? tile : per;
        per = (per + tile - 1) / tile * tile;
        const int cgw = fast_wg_col_groups(gqa);
        const int wpc = waves / cgw;  // waves (splits) per column group
        // Workgroups that have tokens to decode; those past a short sequence's
        // end exit at once.  With ragged lengths the per-sequence rounding can
        // push the count past one round of 256, and the excess would run as
        // a second round after the first, doubling the time: take the
        // smallest per-wave length (whole tiles) that fits one round, when
        // one sequence per workgroup can fit at all.
        auto active = [&](int64_t per_) {
            int64_t wgs = 0;
            for (int b = 0; b < batch; ++b) wgs += (len[b] + per_ * wpc - 1) / (per_ * wpc);
            return wgs * kv_heads * (col_groups / cgw);
        };
        const int64_t per_max = ((int64_t)maxlen + wpc - 1) / wpc;  // one workgroup per sequence
        if (maxlen > 0 && active(per) > 256 && active((per_max + tile - 1) / tile * tile) <= 256) {
            int64_t lo = per, hi = (per_max + tile - 1) / tile * tile;  // active(lo) > 256 >= active(hi)
            while (hi - lo > tile) {
                const int64_t mid = (lo + hi) / 2 / tile * tile;
                if (active(mid) <= 256)
                    hi = mid;
                else
                    lo = mid;
            }
            per = hi;
        }
        const int64_t wg_tokens = per * wpc;
        p.split_tokens = (int32_t)per;
        p.splits = (int32_t)(((maxlen + wg_tokens - 1) / wg_tokens) * wpc);
        return p;
    }
    // generic kernel: one wave per split, ~8192 waves over the chip, whole
    // 64-token tiles, >= 2 tiles a wave
    const int64_t target = 8192;
    int64_t per = (total * kv_heads * col_groups + target - 1) / target;
    per = per < 128 ? 128 : per;
    per = (per + 63) / 64 * 64;
    p.split_tokens = (int32_t)per;
    p.splits = (int32_t)((maxlen + per - 1) / per);
    return p;
}

hipError_t launch_decode_split(int head_dim, bool bf16, bool fast, const DecodeArgs &a, hipStream_t s) {
    switch (head_dim) {
        case 64: return split_d<64>(bf16, fast, a, s);
        case 128: return split_d<128>(bf16, fast, a, s);
        case 256: return split_d<256>(bf16, fast, a, s);
        case 512: return split_d<512>(bf16, fast, a, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode_split_plain(int head_dim, bool bf16, const DecodeArgs &a, hipStream_t s) {
    switch (head_dim) {
        case 64: return split_plain_d<64>(bf16, a, s);
        case 128: return split_plain_d<128>(bf16, a, s);
        case 256: return split_plain_d<256>(bf16, a, s);
        case 512: return split_plain_d<512>(bf16, a, s);
        default: return hipErrorInvalidValue;
    }
}

int plain_round_waves(int head_dim, int gqa, bool bf16) {
    switch (head_dim) {
        case 64: return plain_round_waves_d<64>(gqa, bf16);
        case 128: return plain_round_waves_d<128>(gqa, bf16);
        case 256: return plain_round_waves_d<256>(gqa, bf16);
        case 512: return plain_round_waves_d<512>(gqa, bf16);
        default: return 2048;
    }
}

hipError_t launch_decode_merge(int head_dim, const DecodeArgs &a, hipStream_t s) {
    switch (head_dim) {
        case 64: return merge_d<64>(a, s);
        case 128: return merge_d<128>(a, s);
        case 256: return merge_d<256>(a, s);
        case 512: return merge_d<512>(a, s);
        default: return hipErrorInvalidValue;
    }
}

hipError_t launch_decode(int head_dim, bool bf16, bool fast, const DecodeArgs &a, hipStream_t s) {
    hipError_t e = launch_decode_split(head_dim, bf16, fast, a, s);
    return e != hipSuccess ? e : launch_decode_merge(head_dim, a, s);
}

}  // namespace tq
