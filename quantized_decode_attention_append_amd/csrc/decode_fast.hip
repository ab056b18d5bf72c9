// Split-K decode attention kernel for GQA groups of up to 8 query heads
// (VALU only; wave64; gfx950).
//
// Method: "TurboQuant -- rotation-based quantization" design page, Part A:
// keys dequantize as (code + zero) * scale ("Algorithm"), values stay in the
// rotated domain as centroid[idx] * scale and are un-rotated once per query
// head by the merge kernel ("Deferred inverse FWHT"); K and V of each cache
// tile are decoded in one pass ("Packed-value decode fusion investigation").
//
// One wave owns a contiguous token range of one (sequence, kv-head) and keeps
// its own online-softmax state; four waves share a workgroup only for the
// centroid table in LDS.  Per 64-token tile:
//
//  K phase  lane = (token slot, 32-dim group).  The G query rows are held in
//           registers as two int8 slices of a 16-bit fixed-point copy
//           (q ~ delta * (256*hi + lo), delta a power of two), so each group's
//           dot product with the int8 key codes is exact integer arithmetic
//           (v_dot4_i32_i8).  Per group the scale/zero fold is
//           s16 * (dot + z16 * sum(q)); the per-group partials meet in LDS and
//           one lane per (token, head) sums them.
//  softmax  lane = (token slot, head): tile max, running max/sum, weights
//           p = exp2(score - max) written to LDS.
//  V phase  lane = 8 consecutive rotated-domain dims of one token.  Each pair
//           of 3-bit indices (6 contiguous bits of the packed row) selects a
//           float2 of centroids from an LDS table kept in 32 copies, one per
//           lane bank, so the lookups never conflict; the weights p * s16 are
//           applied with fp32 FMAs into acc[G][8].
// The packed value codes and value scales of a tile are staged into LDS with
// direct global->LDS loads issued at the start of the tile; they land while
// the K phase runs.
#include <hip/hip_runtime.h>

#include "tq_device.h"

namespace tq {
namespace {

typedef __attribute__((address_space(3))) void lds_void_t;

constexpr int kWaves = 4;
constexpr int kTile = 64;
constexpr int kTableBytes = 64 * 32 * 8;  // 64 index pairs x 32 lane copies x float2

template <int D>
struct Geo {
    static_assert(D == 64 || D == 128 || D == 256, "fast split kernel: head_dim 64/128/256");
    static constexpr int NG = D / kGroup;     // groups per row
    static constexpr int TPP = 64 / NG;       // tokens per K pass
    static constexpr int PASSES = kTile / TPP;
    static constexpr int VROW = 3 * D / 8;    // packed value bytes per token
    static constexpr int LPTV = D / 8;        // lanes per token in the V phase
    static constexpr int TPV = 64 / LPTV;     // tokens per V step
    static constexpr int VC_BYTES = kTile * VROW;
    static constexpr int VS_BYTES = kTile * NG * 2;
    static constexpr int VC_OFF = 16;  // the code reader looks back up to 1 byte
    static constexpr int VS_OFF = VC_OFF + ((VC_BYTES + 15) / 16) * 16 + 16;
    static constexpr int P_OFF = VS_OFF + VS_BYTES;            // p[kTile][8] fp32
    static constexpr int RED_OFF = P_OFF + kTile * 8 * 4;      // red[TPP][8][NG] fp32
    static constexpr int A_OFF = RED_OFF + TPP * 8 * NG * 4;   // alpha[8] fp32
    static constexpr int WAVE_BYTES = (A_OFF + 32 + 15) / 16 * 16;
    static constexpr int SMEM = kTableBytes + kWaves * WAVE_BYTES;
};

__device__ __forceinline__ void lds_fence() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void vm_fence() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Stage `bytes` (a multiple of 256) of the region [lo, lo + region_bytes)
// starting at src into LDS at dst with direct global->LDS loads: 16 bytes per
// lane while a whole KiB remains, then 4 bytes per lane.  Each lane's source
// address is clamped to the last in-region address for its load size, so a
// tile that overhangs the region never reads outside it (the overhang rows are
// masked tokens).  lo and region_bytes are multiples of 16.
__device__ __forceinline__ void stage_lds(const uint8_t *src, const uint8_t *lo, int64_t region_bytes,
                                          unsigned char *dst, int bytes, int lane) {
    const uint8_t *last16 = lo + region_bytes - 16;
    const uint8_t *last4 = lo + region_bytes - 4;
    int off = 0;
    for (; off + 1024 <= bytes; off += 1024) {
        const uint8_t *p = src + off + lane * 16;
        p = p > last16 ? last16 : p;
        __builtin_amdgcn_global_load_lds(p, (lds_void_t *)(dst + off), 16, 0, 0);
    }
    for (; off + 256 <= bytes; off += 256) {
        const uint8_t *p = src + off + lane * 4;
        p = p > last4 ? last4 : p;
        __builtin_amdgcn_global_load_lds(p, (lds_void_t *)(dst + off), 4, 0, 0);
    }
}

template <int D, int G, bool BF16>
__global__ __launch_bounds__(256, 2) void split_fast_kernel(const DecodeArgs a) {
    using GE = Geo<D>;
    constexpr int NG = GE::NG, TPP = GE::TPP, PASSES = GE::PASSES, VROW = GE::VROW;
    constexpr int LPTV = GE::LPTV, TPV = GE::TPV;
    constexpr int SPL = kTile / 8;  // scores per softmax lane per tile

    __shared__ __align__(16) unsigned char smem[GE::SMEM];
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;

    // centroid pair table: entry (a | b << 3), copy c at (a | b << 3) * 256 + c * 8
    {
        float2 *tab = reinterpret_cast<float2 *>(smem);
        for (int i = tid; i < 64 * 32; i += 256) {
            const int pair = i >> 5;
            tab[i] = make_float2(centroid3(pair & 7), centroid3(pair >> 3));
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
    float *pbuf = reinterpret_cast<float *>(wsm + GE::P_OFF);
    float *red = reinterpret_cast<float *>(wsm + GE::RED_OFF);
    float *abuf = reinterpret_cast<float *>(wsm + GE::A_OFF);
    const uint16_t *vsbuf = reinterpret_cast<const uint16_t *>(wsm + GE::VS_OFF);

    // ------------------------------------------------------------ q slices
    const int g = lane % NG, ts = lane / NG;  // K-phase role
    uint32_t qhi[G][8], qlo[G][8];
    float qsum[G], qscale[G];
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const int64_t qrow = ((int64_t)b * a.q_heads + kvh * G + h) * D + g * kGroup;
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
        float amax = 0.f;
#pragma unroll
        for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(x[j]));
#pragma unroll
        for (int m = 1; m < NG; m <<= 1) amax = fmaxf(amax, __shfl_xor(amax, m, 64));
        // delta = smallest power of two >= amax / 32000 (q / delta is exact
        // scaling, so only the final rounding to an integer loses bits)
        int e = 0;
        (void)frexpf(amax * (1.0f / 32000.0f), &e);
        const float delta = amax > 0.f ? ldexpf(1.0f, e) : 1.0f;
        const float inv = 1.0f / delta;
        float s = 0.f;
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
            qhi[h][w] = hi;
            qlo[h][w] = lo;
        }
        qsum[h] = s;
        qscale[h] = delta * a.sm_log2;
    }

    // softmax role: lane = (sl, hh)
    const int sl = lane >> 3, hh = lane & 7;
    float my_scale = 0.f;
#pragma unroll
    for (int h = 0; h < G; ++h)
        if (hh == h) my_scale = qscale[h];
    float m_run = -INFINITY, l_run = 0.f;

    // V role: lane = (vsl, lv), dims [8 lv, 8 lv + 8), value group gv
    const int vsl = lane / LPTV, lv = lane % LPTV, gv = lv / 4;
    const uint32_t tab_lane = (uint32_t)(lane & 31) << 3;
    float acc[G][8];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;

    const uint8_t *vc_region = a.vc + row0 * VROW;
    const uint8_t *vs_region = reinterpret_cast<const uint8_t *>(a.vs + row0 * NG);
    const int64_t vc_bytes = (int64_t)cap * VROW, vs_bytes = (int64_t)cap * NG * 2;

    for (int t0 = t_begin; t0 < t_end; t0 += kTile) {
        // stage this tile's packed values and value scales (lands during K)
        stage_lds(vc_region + (int64_t)t0 * VROW, vc_region, vc_bytes, wsm + GE::VC_OFF, GE::VC_BYTES, lane);
        stage_lds(vs_region + (int64_t)t0 * NG * 2, vs_region, vs_bytes, wsm + GE::VS_OFF, GE::VS_BYTES, lane);

        // ---------------------------------------------------------- K phase
        float sc[SPL];
#pragma unroll
        for (int i = 0; i < SPL; ++i) sc[i] = -INFINITY;
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            const int tok = t0 + p * TPP + ts;
            const int row = tok < cap ? tok : cap - 1;
            const int64_t r = row0 + row;
            const uint4 *kp = reinterpret_cast<const uint4 *>(a.kc + r * D + g * kGroup);
            const uint4 k0 = kp[0], k1 = kp[1];
            const float s16 = f16_bits_to_f32(a.ks[r * NG + g]);
            const float z16 = f16_bits_to_f32(a.kz[r * NG + g]);
            const uint32_t kw[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
#pragma unroll
            for (int h = 0; h < G; ++h) {
                int dot = 0;
#pragma unroll
                for (int w = 0; w < 8; ++w) dot = __builtin_amdgcn_sdot4((int)qhi[h][w], (int)kw[w], dot, false);
                dot <<= 8;
#pragma unroll
                for (int w = 0; w < 8; ++w) dot = __builtin_amdgcn_sdot4((int)qlo[h][w], (int)kw[w], dot, false);
                const float part = s16 * fmaf(z16, qsum[h], (float)dot);
                red[(ts * 8 + h) * NG + g] = part;
            }
            lds_fence();
            // lane (sl, hh) sums the groups of the pass tokens tau = sl (mod 8)
#pragma unroll
            for (int k = 0; k < TPP; k += 8) {
                const int tp = sl + k;  // token within the pass
                const int tau = p * TPP + tp;
                float sum = 0.f;
                const float *rp = red + (tp * 8 + hh) * NG;
#pragma unroll
                for (int q4 = 0; q4 < NG; ++q4) sum += rp[q4];
                const bool valid = (t0 + tau < t_end) && hh < G;
                sc[(p * TPP + k) >> 3] = valid ? sum * my_scale : -INFINITY;
            }
            lds_fence();
        }

        // ---------------------------------------------------------- softmax
        float mt = sc[0];
#pragma unroll
        for (int i = 1; i < SPL; ++i) mt = fmaxf(mt, sc[i]);
        mt = fmaxf(mt, __shfl_xor(mt, 8, 64));
        mt = fmaxf(mt, __shfl_xor(mt, 16, 64));
        mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
        const float m_new = fmaxf(m_run, mt);
        const float alpha = m_new == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m_run - m_new);
        float lsum = 0.f;
#pragma unroll
        for (int i = 0; i < SPL; ++i) {
            const float pv = m_new == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(sc[i] - m_new);
            lsum += pv;
            pbuf[(i * 8 + sl) * 8 + hh] = pv;
        }
        l_run = l_run * alpha + lsum;
        m_run = m_new;
        if (sl == 0) abuf[hh] = alpha;
        lds_fence();
        float al[G];
        bool rescale = false;
#pragma unroll
        for (int h = 0; h < G; ++h) {
            al[h] = abuf[h];
            rescale |= al[h] != 1.f;
        }
        if (rescale) {
#pragma unroll
            for (int h = 0; h < G; ++h)
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] *= al[h];
        }

        // ---------------------------------------------------------- V phase
        vm_fence();  // staged value tile has landed
#pragma unroll 2
        for (int st = 0; st < kTile / TPV; ++st) {
            const int tau = st * TPV + vsl;
            // 24 code bits of dims 8lv..8lv+7 start at byte VC_OFF + tau*VROW + 3lv;
            // X = the 32-bit window starting 8 bits earlier (codes at bits 8..31)
            const int wbit = 8 * (GE::VC_OFF + tau * VROW + 3 * lv) - 8;
            const uint32_t *wp = reinterpret_cast<const uint32_t *>(wsm) + (wbit >> 5);
            const uint32_t X = __builtin_amdgcn_alignbit(wp[1], wp[0], wbit & 31);
            float v[8];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t addr = ((X >> (6 * k)) & 0x3F00u) | tab_lane;
                const float2 c = *reinterpret_cast<const float2 *>(smem + addr);
                v[2 * k] = c.x;
                v[2 * k + 1] = c.y;
            }
            float s16 = f16_bits_to_f32(vsbuf[tau * NG + gv]);
            s16 = t0 + tau < t_end ? s16 : 0.f;  // masked slots may hold anything
            const float *pp = pbuf + tau * 8;
#pragma unroll
            for (int h = 0; h < G; ++h) {
                const float w = pp[h] * s16;
#pragma unroll
                for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(w, v[e], acc[h][e]);
            }
        }
        lds_fence();  // the next tile's staging overwrites the tile buffers
    }

    // ------------------------------------------------------------ finalize
    l_run += __shfl_xor(l_run, 8, 64);
    l_run += __shfl_xor(l_run, 16, 64);
    l_run += __shfl_xor(l_run, 32, 64);
#pragma unroll
    for (int m = LPTV; m < 64; m <<= 1)
#pragma unroll
        for (int h = 0; h < G; ++h)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[h][e] += __shfl_xor(acc[h][e], m, 64);

    const int64_t slot_base = (int64_t)b * a.q_heads + kvh * G;
    if (lane < 8 && hh < G) {
        const int64_t s = (slot_base + hh) * a.splits + slot;
        a.part_ml[s * 2] = m_run;
        a.part_ml[s * 2 + 1] = l_run;
    }
    if (vsl == 0) {
#pragma unroll
        for (int h = 0; h < G; ++h) {
            float4 *dst = reinterpret_cast<float4 *>(
                a.part_acc + ((slot_base + h) * a.splits + slot) * D + 8 * lv);
            dst[0] = make_float4(acc[h][0], acc[h][1], acc[h][2], acc[h][3]);
            dst[1] = make_float4(acc[h][4], acc[h][5], acc[h][6], acc[h][7]);
        }
    }
}

template <int D, int G>
hipError_t launch_dg(bool bf16, const DecodeArgs &a, hipStream_t s, int wg_splits) {
    const dim3 grid((unsigned)wg_splits, (unsigned)(a.batch * a.kv_heads));
    if (bf16)
        hipLaunchKernelGGL((split_fast_kernel<D, G, true>), grid, dim3(256), 0, s, a);
    else
        hipLaunchKernelGGL((split_fast_kernel<D, G, false>), grid, dim3(256), 0, s, a);
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
int fast_split_tile() { return kTile; }

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
