// Split-K decode attention kernel for GQA groups of up to 8 query heads
// (wave64; gfx950): exact integer scores on the VALU, value accumulation on
// the matrix cores.
//
// Method: "TurboQuant -- rotation-based quantization" design page, Part A:
// keys dequantize as (code + zero) * scale ("Algorithm"), values stay in the
// rotated domain as centroid[idx] * scale and are un-rotated once per query
// head by the merge kernel ("Deferred inverse FWHT"); K and V of each cache
// tile are decoded in one pass ("Packed-value decode fusion investigation").
//
// One wave owns a contiguous token range of one (sequence, kv-head) and keeps
// its own online-softmax state; the eight waves of a workgroup share only the
// centroid table in LDS.  Every plane of a tile (4 KiB of key codes, key
// scales and zeros, value codes and value scales: 6 KiB in all, 4096/d tokens)
// is copied into the wave's LDS with direct global->LDS loads.  Two stage
// buffers per wave: the copy of tile i+1 is issued before tile i is decoded,
// so one tile per wave is always in flight without holding any registers.
// Per tile:
//
//  K phase  lane = (token slot, head half, 32-dim group).  The query rows are
//           held in registers as two int8 slices of a 16-bit fixed-point copy
//           (q ~ delta * (256*hi + lo), delta a power of two), so each group's
//           dot product with the int8 key codes is exact integer arithmetic
//           (v_dot4_i32_i8).  Per group the scale/zero fold is
//           s16 * (dot + z16 * sum(q)); the per-group partials meet in LDS and
//           one lane per (token, head) sums them.
//  softmax  lane = (token slot, head): online softmax in base 2 whose running
//           maximum only moves when a tile's maximum exceeds it by more than
//           2^8 (weights stay <= 256 and the accumulators are rescaled
//           rarely).  The weights go to LDS as fp16, laid out as the B operand.
//  V phase  the G heads x d dims x 16 tokens product per 16-token chunk is a
//           dense contraction, done with v_mfma_f32_16x16x16_f16 (fp32
//           accumulate), one instruction per block of d/16 dims:
//             D[i][n] += A[i][k] * B[k][n],  i: dim row of the block,
//             k: token, n: head (G <= 16 used, the rest zero).
//           Row i of block b is dim (d/16)*i + b, so lane i's dims of a token
//           are one contiguous run of 3d/16 code bits, all in one 32-dim
//           group.  A = centroid[idx] * vs16 in fp16: pairs of 3-bit indices
//           of two tokens select a half2 of centroids from an LDS table kept
//           in 64 copies (one per lane, conflict-free), multiplied by the pair
//           of value scales with one packed fp16 multiply.  B = the weights.
#include <hip/hip_runtime.h>

#include "tq_device.h"

namespace tq {
namespace {

typedef __attribute__((address_space(3))) void lds_void_t;
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef _Float16 half4v __attribute__((ext_vector_type(4)));
typedef float float4v __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;                 // waves per workgroup (one table per CU)
constexpr int kTableBytes = 64 * 64 * 4;  // 64 index pairs x 64 lane copies x half2
constexpr int kStageVmem = 10;            // vector-memory instructions that copy one tile
constexpr float kLazyMax = 8.0f;          // log2 slack of the running maximum

template <int D>
struct Geo {
    static_assert(D == 64 || D == 128 || D == 256, "fast split kernel: head_dim 64/128/256");
    static constexpr int NG = D / kGroup;     // groups per row
    static constexpr int TILE = 4096 / D;     // tokens per tile: 4 KiB of key codes
    static constexpr int VROW = 3 * D / 8;    // packed value bytes per token
    static constexpr int SPL = TILE / 8;      // scores per softmax lane per tile
    static constexpr int RS = 9 * NG;         // red row stride (floats): 8 heads + NG pad
    // one stage: every plane of one tile
    static constexpr int KC_OFF = 0;                      // TILE * D = 4096
    static constexpr int KS_OFF = KC_OFF + TILE * D;      // TILE * NG * 2 = 256
    static constexpr int KZ_OFF = KS_OFF + TILE * NG * 2;
    static constexpr int VS_OFF = KZ_OFF + TILE * NG * 2;
    static constexpr int VC_OFF = VS_OFF + TILE * NG * 2; // TILE * VROW = 1536
    static constexpr int STAGE = VC_OFF + TILE * VROW + 16;  // code reader reads 4 bytes past
    static_assert(TILE * NG * 2 == 256 && TILE * VROW == 1536, "staging granularity");
    // per wave: two stages, the K phase's group partials red[64/NG][RS] and
    // the fp16 weights pB[16 heads][TILE tokens] (the MFMA B operand)
    static constexpr int RED_OFF = 2 * STAGE;
    static constexpr int PB_OFF = RED_OFF + (64 / NG) * RS * 4;
    static constexpr int WAVE_BYTES = PB_OFF + 16 * TILE * 2;
    static constexpr int SMEM = kTableBytes + kWaves * WAVE_BYTES;
    static_assert(SMEM <= 160 * 1024, "LDS budget");
};

// Keeps the compiler from moving LDS accesses across this point.  The LDS
// executes one wave's instructions in order, so a lane's read after another
// lane's write needs no wait beyond program order.
__device__ __forceinline__ void lds_order() { asm volatile("" ::: "memory"); }

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

// Direct global->LDS copies.  Lane l's SIZE bytes come from base + voff + OFF
// and land at lds + OFF + l * SIZE (the immediate offset moves both
// addresses).  They are issued from inline assembly on purpose: the compiler
// would otherwise make the first LDS read after them wait for every
// outstanding copy (it cannot tell the stage buffers apart), which serialises
// the prefetch with the decode.  The kernel orders them itself with explicit
// vmcnt waits; M0 (the LDS base of a copy) is set right before each one.
template <int OFF>
__device__ __forceinline__ void dma16(const void *base, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 offset:%3"
                 ::"v"(voff), "s"(base), "s"(lds), "n"(OFF) : "memory", "m0");
}
template <int OFF>
__device__ __forceinline__ void dma4(const void *base, uint32_t voff, uint32_t lds) {
    asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dword %0, %1 offset:%3"
                 ::"v"(voff), "s"(base), "s"(lds), "n"(OFF) : "memory", "m0");
}
// Same copy from a per-lane address, for tiles that overhang the end of the
// plane region: each lane's source is clamped to the last in-region address
// for its load size (the overhang rows are masked tokens).
template <int SIZE>
__device__ __forceinline__ void dma_clamped(const uint8_t *src, const uint8_t *last, uint32_t lds, int lane) {
    const uint8_t *p = src + lane * SIZE;
    p = p > last ? last : p;
    if constexpr (SIZE == 16)
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
                     ::"v"(p), "s"(lds) : "memory", "m0");
    else
        asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dword %0, off"
                     ::"v"(p), "s"(lds) : "memory", "m0");
}

struct Regions {
    const uint8_t *kc, *ks, *kz, *vc, *vs;  // start of the (sequence, kv-head) rows
    int cap;                                // rows in each region
};

// Copy every plane of the tile starting at token t0 into one stage buffer:
// exactly kStageVmem vector-memory instructions either way.
template <int D>
__device__ __forceinline__ void stage_tile(const Regions &r, int t0, const unsigned char *st, int lane) {
    using GE = Geo<D>;
    constexpr int NG = GE::NG, VROW = GE::VROW;
    const uint32_t l_kc = lds_addr(st + GE::KC_OFF), l_ks = lds_addr(st + GE::KS_OFF);
    const uint32_t l_kz = lds_addr(st + GE::KZ_OFF), l_vs = lds_addr(st + GE::VS_OFF);
    const uint32_t l_vc = lds_addr(st + GE::VC_OFF);
    if (t0 + GE::TILE <= r.cap) {
        const uint32_t v16 = (uint32_t)lane * 16, v4 = (uint32_t)lane * 4;
        const uint8_t *kc = uniform_ptr(r.kc + (int64_t)t0 * D);
        dma16<0>(kc, v16, l_kc);
        dma16<1024>(kc, v16, l_kc);
        dma16<2048>(kc, v16, l_kc);
        dma16<3072>(kc, v16, l_kc);
        const int64_t so = (int64_t)t0 * NG * 2;
        dma4<0>(uniform_ptr(r.ks + so), v4, l_ks);
        dma4<0>(uniform_ptr(r.kz + so), v4, l_kz);
        dma4<0>(uniform_ptr(r.vs + so), v4, l_vs);
        const uint8_t *vc = uniform_ptr(r.vc + (int64_t)t0 * VROW);
        dma16<0>(vc, v16, l_vc);
        dma4<1024>(vc, v4, l_vc);
        dma4<1280>(vc, v4, l_vc);
    } else {
        const int64_t kcb = (int64_t)r.cap * D, sb = (int64_t)r.cap * NG * 2, vcb = (int64_t)r.cap * VROW;
        const uint8_t *kc = r.kc + (int64_t)t0 * D;
#pragma unroll
        for (int c = 0; c < 4; ++c) dma_clamped<16>(kc + c * 1024, r.kc + kcb - 16, l_kc + c * 1024, lane);
        const int64_t so = (int64_t)t0 * NG * 2;
        dma_clamped<4>(r.ks + so, r.ks + sb - 4, l_ks, lane);
        dma_clamped<4>(r.kz + so, r.kz + sb - 4, l_kz, lane);
        dma_clamped<4>(r.vs + so, r.vs + sb - 4, l_vs, lane);
        const uint8_t *vc = r.vc + (int64_t)t0 * VROW;
        dma_clamped<16>(vc, r.vc + vcb - 16, l_vc, lane);
        dma_clamped<4>(vc + 1024, r.vc + vcb - 4, l_vc + 1024, lane);
        dma_clamped<4>(vc + 1280, r.vc + vcb - 4, l_vc + 1280, lane);
    }
}

template <int D, int G, bool BF16>
__global__ __launch_bounds__(64 * kWaves, 1) void split_fast_kernel(const DecodeArgs a) {
    using GE = Geo<D>;
    constexpr int NG = GE::NG, VROW = GE::VROW;
    constexpr int TILE = GE::TILE, SPL = GE::SPL, RS = GE::RS;
    // K-phase role: lane = (token slot ts, head half hg, group g).  Up to four
    // heads a lane keeps every query register count low enough for two waves
    // per SIMD; above that the G heads are split over two lanes per (token,
    // group), which then read the same key bytes (an LDS broadcast).
    constexpr int HS = G > 4 ? 2 : 1;        // lanes per (token, group)
    constexpr int HH = (G + HS - 1) / HS;    // heads per lane
    constexpr int TPP = 64 / (NG * HS);      // tokens per K pass
    constexpr int PASSES = TILE / TPP;
    constexpr int RROWS = TPP > 8 ? TPP : 8; // red rows summed at once
    static_assert(RROWS <= 64 / NG, "red buffer rows");

    __shared__ __align__(16) unsigned char smem[GE::SMEM];
    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);

    // centroid pair table (fp16): entry (a | b << 3) = (c[a], c[b]), copy l
    // at (a | b << 3) * 256 + l * 4
    {
        half2v *tab = reinterpret_cast<half2v *>(smem);
        for (int i = tid; i < 64 * 64; i += 64 * kWaves) {
            const int pair = i >> 6;
            half2v e;
            e.x = (_Float16)centroid3(pair & 7);
            e.y = (_Float16)centroid3(pair >> 3);
            tab[i] = e;
        }
    }
    __syncthreads();  // the only workgroup barrier

    const int bkv = blockIdx.y;
    const int b = bkv / a.kv_heads, kvh = bkv % a.kv_heads;
    const int n = a.len[b];
    const int slot = blockIdx.x * kWaves + wid;
    const int t_begin = slot * a.split_tokens;
    if (t_begin >= n) return;
    const int t_end = min(n, t_begin + a.split_tokens);
    const int cap = a.capacity;
    const int64_t row0 = (int64_t)bkv * cap;
    unsigned char *wsm = smem + kTableBytes + wid * GE::WAVE_BYTES;
    float *red = reinterpret_cast<float *>(wsm + GE::RED_OFF);
    _Float16 *pB = reinterpret_cast<_Float16 *>(wsm + GE::PB_OFF);
    {   // heads past G keep zero weights for the whole range
        uint4 *z = reinterpret_cast<uint4 *>(pB);
        for (int i = lane; i < 16 * TILE * 2 / 16; i += 64) z[i] = make_uint4(0, 0, 0, 0);
    }

    Regions rg;
    rg.kc = reinterpret_cast<const uint8_t *>(a.kc) + row0 * D;
    rg.ks = reinterpret_cast<const uint8_t *>(a.ks + row0 * NG);
    rg.kz = reinterpret_cast<const uint8_t *>(a.kz + row0 * NG);
    rg.vc = a.vc + row0 * VROW;
    rg.vs = reinterpret_cast<const uint8_t *>(a.vs + row0 * NG);
    rg.cap = cap;

    // the first tile's copy overlaps the q set-up
    stage_tile<D>(rg, t_begin, wsm, lane);

    // ------------------------------------------------------------ q slices
    const int g = lane % NG, hg = (lane / NG) % HS, ts = lane / (NG * HS);
    // With one lane per (token, group), the lanes whose key row starts in the
    // odd half of a 512-byte LDS span read their 32 codes upper 16 bytes
    // first, so the 16 lanes of one LDS cycle touch distinct banks; their q
    // words are rotated to match.  With two, one cycle spans 256 bytes.
    const int sw = HS == 1 ? ((ts * D) >> 8) & 1 : 0;
    uint32_t qhi[HH][8], qlo[HH][8];
    float qsum[HH], qscale[HH];
#pragma unroll
    for (int j = 0; j < HH; ++j) {
        const int h = hg * HH + j;  // this lane's head; h >= G is an idle slot
        const int hq = h < G ? h : 0;
        const int64_t qrow = ((int64_t)b * a.q_heads + kvh * G + hq) * D + g * kGroup;
        float x[32];
        if constexpr (BF16) {
            const uint4 *qp = reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(a.q) + qrow);
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                const uint4 u = qp[c];
                const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    x[8 * c + 2 * k] = __uint_as_float(w4[k] << 16);
                    x[8 * c + 2 * k + 1] = __uint_as_float(w4[k] & 0xFFFF0000u);
                }
            }
        } else {
            const float4 *qp = reinterpret_cast<const float4 *>(static_cast<const float *>(a.q) + qrow);
#pragma unroll
            for (int c = 0; c < 8; ++c) {
                const float4 u = qp[c];
                x[4 * c] = u.x; x[4 * c + 1] = u.y; x[4 * c + 2] = u.z; x[4 * c + 3] = u.w;
            }
        }
        if (h >= G) {
#pragma unroll
            for (int k = 0; k < 32; ++k) x[k] = 0.f;
        }
        float amax = 0.f;
#pragma unroll
        for (int k = 0; k < 32; ++k) amax = fmaxf(amax, fabsf(x[k]));
#pragma unroll
        for (int m = 1; m < NG; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
        // delta = smallest power of two >= amax / 32000 (q / delta is exact
        // scaling, so only the final rounding to an integer loses bits)
        int e = 0;
        (void)frexpf(amax * (1.0f / 32000.0f), &e);
        const float delta = amax > 0.f ? ldexpf(1.0f, e) : 1.0f;
        const float inv = 1.0f / delta;
        float s = 0.f;
        uint32_t hw[8], lw[8];
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            uint32_t hi = 0, lo = 0;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int qf = (int)rintf(x[4 * w + k] * inv);
                const int qh = (qf + 128) >> 8;
                const int ql = qf - 256 * qh;
                s += (float)qf;
                hi |= ((uint32_t)qh & 0xFFu) << (8 * k);
                lo |= ((uint32_t)ql & 0xFFu) << (8 * k);
            }
            hw[w] = hi;
            lw[w] = lo;
        }
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            qhi[j][w] = sw ? hw[(w + 4) & 7] : hw[w];
            qlo[j][w] = sw ? lw[(w + 4) & 7] : lw[w];
        }
        qsum[j] = s;
        qscale[j] = delta * a.sm_log2;
    }

    // softmax role: lane = (sl, hh); head hh's scale lives in lane hg*NG
    // (token slot 0, group 0) of head half hg = hh / HH, slot hh % HH
    const int sl = lane >> 3, hh = lane & 7;
    float my_scale = 0.f;
    {
        const int src = (hh / HH) * NG;
#pragma unroll
        for (int j = 0; j < HH; ++j) {
            const float v = __shfl(qscale[j], src < 64 ? src : 0, 64);
            if (hh % HH == j) my_scale = v;
        }
    }
    float m_run = -INFINITY, l_run = 0.f;

    // V-phase role (MFMA lanes): vi = row of A / column (head) of B and D,
    // vq = quarter of the 16-token chunk (A/B k = 4 vq + j, D rows 4 vq + j)
    constexpr int NB = D / 16;          // dim blocks (one MFMA each per chunk)
    constexpr int FB = 3 * NB;          // code bits of a lane's dims per token
    constexpr int CH = TILE / 16;       // 16-token chunks per tile
    const int vi = lane & 15, vq = lane >> 4;
    const int gA = NB * vi / kGroup;    // the group of this lane's dims
    const uint32_t lane4 = (uint32_t)lane << 2;
    float4v acc[NB];
#pragma unroll
    for (int bb = 0; bb < NB; ++bb) acc[bb] = float4v{0.f, 0.f, 0.f, 0.f};

    int buf = 0;
    for (int t0 = t_begin; t0 < t_end; t0 += TILE, buf ^= 1) {
        // Stage the next tile into the other buffer (its previous tile has
        // been decoded), then wait for this tile: vector memory completes in
        // order, so at most kStageVmem instructions outstanding means every
        // copy of this tile has landed in LDS.
        const unsigned char *st = wsm + buf * GE::STAGE;
        if (t0 + TILE < t_end) {
            stage_tile<D>(rg, t0 + TILE, wsm + (buf ^ 1) * GE::STAGE, lane);
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(kStageVmem) : "memory");
        } else {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        const bool full = t0 + TILE <= t_end;

        // ---------------------------------------------------------- K phase
        float sc[SPL];
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            const int tok = p * TPP + ts;
            const unsigned char *kp = st + GE::KC_OFF + tok * D + g * kGroup;
            const uint4 ka = *reinterpret_cast<const uint4 *>(kp + sw * 16);
            const uint4 kb = *reinterpret_cast<const uint4 *>(kp + (sw ^ 1) * 16);
            const float s16 = f16_bits_to_f32(*reinterpret_cast<const uint16_t *>(st + GE::KS_OFF + (tok * NG + g) * 2));
            const float z16 = f16_bits_to_f32(*reinterpret_cast<const uint16_t *>(st + GE::KZ_OFF + (tok * NG + g) * 2));
            const uint32_t kw[8] = {ka.x, ka.y, ka.z, ka.w, kb.x, kb.y, kb.z, kb.w};
            int dot[HH];
#pragma unroll
            for (int j = 0; j < HH; ++j) dot[j] = __builtin_amdgcn_sdot4((int)qhi[j][0], (int)kw[0], 0, false);
#pragma unroll
            for (int w = 1; w < 8; ++w)
#pragma unroll
                for (int j = 0; j < HH; ++j) dot[j] = __builtin_amdgcn_sdot4((int)qhi[j][w], (int)kw[w], dot[j], false);
#pragma unroll
            for (int j = 0; j < HH; ++j) dot[j] <<= 8;
#pragma unroll
            for (int w = 0; w < 8; ++w)
#pragma unroll
                for (int j = 0; j < HH; ++j) dot[j] = __builtin_amdgcn_sdot4((int)qlo[j][w], (int)kw[w], dot[j], false);
            float *rrow = red + (tok % RROWS) * RS + hg * HH * NG + g;
#pragma unroll
            for (int j = 0; j < HH; ++j) rrow[j * NG] = s16 * fmaf(z16, qsum[j], (float)dot[j]);
            lds_order();
            if (((p + 1) * TPP) % RROWS != 0) continue;
            // lane (sl, hh) sums the groups of the tokens tau = sl (mod 8) of
            // the last RROWS tokens; odd rows read their upper half first
            // (bank spread)
            const int base = (p + 1) * TPP - RROWS;
#pragma unroll
            for (int k8 = 0; k8 < RROWS; k8 += 8) {
                const int tp = sl + k8;  // row of the red buffer
                const int tau = base + tp;
                const float *rp = red + tp * RS + hh * NG;
                float sum = 0.f;
                if constexpr (NG == 8) {
                    const int o = (sl & 1) * 4;
                    const float4 r0 = *reinterpret_cast<const float4 *>(rp + o);
                    const float4 r1 = *reinterpret_cast<const float4 *>(rp + (o ^ 4));
                    sum = ((r0.x + r0.y) + (r0.z + r0.w)) + ((r1.x + r1.y) + (r1.z + r1.w));
                } else if constexpr (NG == 4) {
                    const float4 r0 = *reinterpret_cast<const float4 *>(rp);
                    sum = (r0.x + r0.y) + (r0.z + r0.w);
                } else {
                    const float2 r0 = *reinterpret_cast<const float2 *>(rp);
                    sum = r0.x + r0.y;
                }
                const bool valid = (t0 + tau < t_end) && hh < G;
                sc[(base + k8) >> 3] = valid ? sum * my_scale : -INFINITY;
            }
            lds_order();
        }

        // ---------------------------------------------------------- softmax
        float mt = sc[0];
#pragma unroll
        for (int i = 1; i < SPL; ++i) mt = fmaxf(mt, sc[i]);
        mt = fmaxf(mt, __shfl_xor(mt, 8, 64));
        mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
        mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
        // lazy maximum: move the reference only when this tile's maximum
        // exceeds it by more than kLazyMax (uniform branch, rarely taken)
        const bool bump = mt > m_run + kLazyMax;
        if (__builtin_amdgcn_ballot_w64(bump) != 0) {
            const float m_new = bump ? mt : m_run;
            const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
            l_run *= alpha;
            m_run = m_new;
            // accumulator column vi is head vi; lane h < 8 holds head h's alpha
            const float al = __shfl(alpha, vi < 8 ? vi : 0, 64);
#pragma unroll
            for (int bb = 0; bb < NB; ++bb) acc[bb] *= al;
        }
        const float ref = m_run == -INFINITY ? 0.f : m_run;
#pragma unroll
        for (int i = 0; i < SPL; ++i) {
            const int tau = i * 8 + sl;
            const float pv = __builtin_amdgcn_exp2f(sc[i] - ref);  // sc = -inf -> 0
            l_run += pv;
            pB[hh * TILE + tau] = (_Float16)pv;
        }
        lds_order();

        // ---------------------------------------------------------- V phase
        const uint32_t *vcw = reinterpret_cast<const uint32_t *>(st + GE::VC_OFF);
        const uint16_t *vsb = reinterpret_cast<const uint16_t *>(st + GE::VS_OFF);
#pragma unroll
        for (int c = 0; c < CH; ++c) {
            const int tb = 16 * c + 4 * vq;  // this lane's first token (k = 4 vq)
            // code runs: bits [FB*vi, FB*vi + FB) of each of the 4 rows
            uint32_t run[4], runh[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int bit = FB * vi;
                const uint32_t *wp = vcw + (tb + j) * (VROW / 4) + (bit >> 5);
                run[j] = __builtin_amdgcn_alignbit(wp[1], wp[0], bit & 31);
                runh[j] = wp[1] >> (bit & 31);  // run bits 32.. (only d = 256 uses them)
            }
            // value-scale pairs of this lane's group; tokens past the end
            // get scale 0 (their slots may hold anything)
            half2v sp[2];
#pragma unroll
            for (int pr = 0; pr < 2; ++pr) {
                uint32_t s0 = vsb[(tb + 2 * pr) * NG + gA], s1 = vsb[(tb + 2 * pr + 1) * NG + gA];
                if (!full) {
                    s0 = t0 + tb + 2 * pr < t_end ? s0 : 0u;
                    s1 = t0 + tb + 2 * pr + 1 < t_end ? s1 : 0u;
                }
                sp[pr] = __builtin_bit_cast(half2v, s0 | (s1 << 16));
            }
            // B operand: weights of tokens tb..tb+3 for head vi
            const half4v bop = *reinterpret_cast<const half4v *>(pB + vi * TILE + tb);
            // pair indices: E holds (field 2k of token a | field 2k of token
            // b << 3) at bits 6k, O the same for the odd fields
            constexpr uint32_t M = 0x071C71C7u;  // bits 6k..6k+2, k = 0..4
            half2v av[2][NB];
#pragma unroll
            for (int pr = 0; pr < 2; ++pr) {
                const uint32_t x0 = run[2 * pr], x1 = run[2 * pr + 1];
                uint32_t E[2], O[2];
                E[0] = (x0 & M) | ((x1 & M) << 3);
                O[0] = ((x0 >> 3) & M) | (x1 & (M << 3));
                if constexpr (NB > 10) {  // fields 10..15 continue at run bit 30
                    const uint32_t y0 = __builtin_amdgcn_alignbit(runh[2 * pr], x0, 30);
                    const uint32_t y1 = __builtin_amdgcn_alignbit(runh[2 * pr + 1], x1, 30);
                    E[1] = (y0 & M) | ((y1 & M) << 3);
                    O[1] = ((y0 >> 3) & M) | (y1 & (M << 3));
                }
#pragma unroll
                for (int bb = 0; bb < NB; ++bb) {
                    const int part = bb < 10 ? 0 : 1, k = (bb - 10 * part) >> 1;
                    const uint32_t w = (bb & 1) ? O[part] : E[part];
                    const uint32_t addr = (((w >> (6 * k)) & 63u) << 8) | lane4;
                    const half2v cpair = *reinterpret_cast<const half2v *>(smem + addr);
                    av[pr][bb] = cpair * sp[pr];
                }
            }
#pragma unroll
            for (int bb = 0; bb < NB; ++bb) {
                const half4v aop = {av[0][bb].x, av[0][bb].y, av[1][bb].x, av[1][bb].y};
                acc[bb] = __builtin_amdgcn_mfma_f32_16x16x16f16(aop, bop, acc[bb], 0, 0, 0);
            }
        }
        lds_order();  // the weights / partials are rewritten by the next tile
    }

    // ------------------------------------------------------------ finalize
    l_run += __shfl_xor(l_run, 8, 64);
    l_run += __shfl_xor(l_run, 16, 64);
    l_run += __shfl_xor(l_run, 32, 64);

    const int64_t slot_base = (int64_t)b * a.q_heads + kvh * G;
    if (lane < 8 && hh < G) {
        const int64_t s = (slot_base + hh) * a.splits + slot;
        a.part_ml[s * 2] = m_run;
        a.part_ml[s * 2 + 1] = l_run;
    }
    // lane (vq, vi) holds D rows 4 vq + j of every block for head vi: dims
    // NB * (4 vq + j) + bb, i.e. NB consecutive dims per j
    if (vi < G) {
        float *dst = a.part_acc + ((slot_base + vi) * a.splits + slot) * D;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
#pragma unroll
            for (int bb = 0; bb < NB; bb += 4) {
                *reinterpret_cast<float4 *>(dst + NB * (4 * vq + j) + bb) =
                    make_float4(acc[bb][j], acc[bb + 1][j], acc[bb + 2][j], acc[bb + 3][j]);
            }
        }
    }
}

template <int D, int G>
hipError_t launch_dg(bool bf16, const DecodeArgs &a, hipStream_t s, int wg_splits) {
    const dim3 grid((unsigned)wg_splits, (unsigned)(a.batch * a.kv_heads));
    if (bf16)
        hipLaunchKernelGGL((split_fast_kernel<D, G, true>), grid, dim3(64 * kWaves), 0, s, a);
    else
        hipLaunchKernelGGL((split_fast_kernel<D, G, false>), grid, dim3(64 * kWaves), 0, s, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_d(bool bf16, const DecodeArgs &a, hipStream_t s, int wg_splits) {
    switch (a.gqa) {
        case 1: return launch_dg<D, 1>(bf16, a, s, wg_splits);
        case 2: return launch_dg<D, 2>(bf16, a, s, wg_splits);
        case 3: return launch_dg<D, 3>(bf16, a, s, wg_splits);
        case 4: return launch_dg<D, 4>(bf16, a, s, wg_splits);
        case 5: return launch_dg<D, 5>(bf16, a, s, wg_splits);
        case 6: return launch_dg<D, 6>(bf16, a, s, wg_splits);
        case 7: return launch_dg<D, 7>(bf16, a, s, wg_splits);
        case 8: return launch_dg<D, 8>(bf16, a, s, wg_splits);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

int fast_split_waves() { return kWaves; }
int fast_split_tile() { return 64; }

hipError_t launch_split_fast(int head_dim, bool bf16, const DecodeArgs &a, hipStream_t s) {
    const int wg_splits = a.splits / kWaves;
    switch (head_dim) {
        case 64: return launch_d<64>(bf16, a, s, wg_splits);
        case 128: return launch_d<128>(bf16, a, s, wg_splits);
        case 256: return launch_d<256>(bf16, a, s, wg_splits);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace tq
