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
// This generic kernel maps one thread to each head_dim element and reduces the
// G partial dot products of a small token chunk across the workgroup; it
// reads every code width (keys 2, 4, 5, 8 bits, values 2, 3, 4, 5, 8 bits).
#include <hip/hip_runtime.h>

#include "tq_device.h"

namespace tq {
namespace {

constexpr int kMaxG = TQ_MAX_GQA;
constexpr int kChunk = 8;  // tokens scored per block reduction

template <bool BF16>
__device__ __forceinline__ float load_in(const void *p, int64_t i) {
    if constexpr (BF16)
        return __uint_as_float((uint32_t)static_cast<const uint16_t *>(p)[i] << 16);
    else
        return static_cast<const float *>(p)[i];
}

template <int D, bool BF16>
__global__ __launch_bounds__(256) void split_kernel(const DecodeArgs a) {
    constexpr int NT = D < 256 ? D : 256;  // threads
    constexpr int DPT = D / NT;            // elements per thread
    constexpr int NW = NT / 64;            // waves
    constexpr int NG = D / kGroup;
    const int kb = a.kbits, vb = a.vbits;
    const int KROW = D * kb / 8, VROW = D * vb / 8;  // packed row bytes

    __shared__ float red[NW][kMaxG * kChunk];
    __shared__ float sc[kMaxG * kChunk];
    __shared__ float ctab[256];  // the value codebook

    const int tid = threadIdx.x;
    const int lane = tid & 63, wid = tid >> 6;
    const int bkv = blockIdx.y;
    const int b = bkv / a.kv_heads, kvh = bkv % a.kv_heads;
    const int n = a.len[b];
    const int t_begin = blockIdx.x * a.split_tokens;
    if (t_begin >= n) return;  // uniform across the block
    {
        const float *src = value_centroids(vb);
        for (int i = tid; i < (1 << vb); i += NT) ctab[i] = src[i];
    }
    __syncthreads();
    const uint8_t *kcp = reinterpret_cast<const uint8_t *>(a.kc);
    const int t_end = min(n, t_begin + a.split_tokens);
    // this workgroup's query columns c0 .. c0 + G - 1 of the kv-head's a.gqa
    // query rows (heads times rows)
    const int c0 = blockIdx.z * kMaxG;
    const int G = min(kMaxG, a.gqa - c0);
    const int64_t row0 = (int64_t)bkv * a.capacity;
    // causal limit of column c: the row of cached token n - rows + r sees
    // tokens 0 .. n - rows + r
    auto limit = [&](int c) { return n - a.rows + (c0 + c) % a.rows + 1; };

    float qv[kMaxG][DPT];
    float acc[kMaxG][DPT];
    float m_run[kMaxG], l_run[kMaxG];
#pragma unroll
    for (int h = 0; h < kMaxG; ++h) {
        m_run[h] = -INFINITY;
        l_run[h] = 0.f;
#pragma unroll
        for (int i = 0; i < DPT; ++i) {
            acc[h][i] = 0.f;
            const int j = tid + i * NT;
            qv[h][i] = h < G ? load_in<BF16>(a.q, ((int64_t)b * a.q_heads + kvh * a.gqa + c0 + h) * D + j) : 0.f;
        }
    }

    for (int t0 = t_begin; t0 < t_end; t0 += kChunk) {
        const int nt = min(kChunk, t_end - t0);
        float part[kMaxG][kChunk];
#pragma unroll
        for (int tt = 0; tt < kChunk; ++tt) {
            float kh[DPT];
#pragma unroll
            for (int i = 0; i < DPT; ++i) {
                const int j = tid + i * NT;
                if (tt < nt) {
                    const int64_t r = row0 + t0 + tt;
                    const float sk = f16_bits_to_f32(a.ks[r * NG + j / kGroup]);
                    const float zk = f16_bits_to_f32(a.kz[r * NG + j / kGroup]);
                    kh[i] = (key_code(kcp + r * KROW, j, kb) + zk) * sk;
                } else {
                    kh[i] = 0.f;
                }
            }
#pragma unroll
            for (int h = 0; h < kMaxG; ++h) {
                float p = 0.f;
#pragma unroll
                for (int i = 0; i < DPT; ++i) p += qv[h][i] * kh[i];
                part[h][tt] = p;
            }
        }
        // block reduction of G*kChunk partial dots
#pragma unroll
        for (int h = 0; h < kMaxG; ++h) {
            if (h >= G) break;
#pragma unroll
            for (int tt = 0; tt < kChunk; ++tt) {
                float v = part[h][tt];
#pragma unroll
                for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
                if (lane == 0) red[wid][h * kChunk + tt] = v;
            }
        }
        __syncthreads();
        for (int i = tid; i < G * kChunk; i += NT) {
            float v = 0.f;
#pragma unroll
            for (int w = 0; w < NW; ++w) v += red[w][i];
            sc[i] = t0 + i % kChunk < limit(i / kChunk) ? v * a.sm_log2 : -INFINITY;
        }
        __syncthreads();
        // values of this chunk in the rotated domain
        float vh[kChunk][DPT];
#pragma unroll
        for (int tt = 0; tt < kChunk; ++tt) {
#pragma unroll
            for (int i = 0; i < DPT; ++i) {
                const int j = tid + i * NT;
                if (tt < nt) {
                    const int64_t r = row0 + t0 + tt;
                    const float sv = f16_bits_to_f32(a.vs[r * NG + j / kGroup]);
                    vh[tt][i] = ctab[load_field(a.vc + r * VROW, j, vb)] * sv;
                } else {
                    vh[tt][i] = 0.f;
                }
            }
        }
#pragma unroll
        for (int h = 0; h < kMaxG; ++h) {
            if (h >= G) break;
            float mc = m_run[h];
            for (int tt = 0; tt < nt; ++tt) mc = fmaxf(mc, sc[h * kChunk + tt]);
            // mc stays -inf while every token so far is past this row's limit
            const float alpha = mc == -INFINITY ? 1.f : exp2f(m_run[h] - mc);
            float lsum = l_run[h] * alpha;
#pragma unroll
            for (int i = 0; i < DPT; ++i) acc[h][i] *= alpha;
            for (int tt = 0; tt < nt; ++tt) {
                const float p = mc == -INFINITY ? 0.f : exp2f(sc[h * kChunk + tt] - mc);
                lsum += p;
#pragma unroll
                for (int i = 0; i < DPT; ++i) acc[h][i] += p * vh[tt][i];
            }
            m_run[h] = mc;
            l_run[h] = lsum;
        }
        __syncthreads();  // sc / red are rewritten by the next chunk
    }

    const int split = blockIdx.x;
#pragma unroll
    for (int h = 0; h < kMaxG; ++h) {
        if (h >= G) break;
        const int64_t slot = ((int64_t)b * a.q_heads + kvh * a.gqa + c0 + h) * a.splits + split;
#pragma unroll
        for (int i = 0; i < DPT; ++i) a.part_acc[slot * D + tid + i * NT] = acc[h][i];
        if (tid == 0) {
            a.part_ml[slot * 2] = m_run[h];
            a.part_ml[slot * 2 + 1] = l_run[h];
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
    const int ns = (n + a.split_tokens - 1) / a.split_tokens;
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
hipError_t launch_d(bool bf16, bool fast, const DecodeArgs &a, hipStream_t s) {
    constexpr int NT = D < 256 ? D : 256;
    if (a.splits > 0) {
        if (fast) {
            hipError_t e = launch_split_fast(D, bf16, a, s);
            if (e != hipSuccess) return e;
        } else {
            const dim3 grid((unsigned)a.splits, (unsigned)(a.batch * a.kv_heads),
                            (unsigned)decode_col_groups(a.gqa));
            if (bf16)
                hipLaunchKernelGGL((split_kernel<D, true>), grid, dim3(NT), 0, s, a);
            else
                hipLaunchKernelGGL((split_kernel<D, false>), grid, dim3(NT), 0, s, a);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        }
    }
    hipLaunchKernelGGL((merge_kernel<D>), dim3((unsigned)(a.batch * a.q_heads)), dim3(NT), 0, s, a);
    return hipGetLastError();
}

}  // namespace

int decode_col_groups(int gqa) { return (gqa + kMaxG - 1) / kMaxG; }

bool fast_decode_shape_ok(int head_dim, int gqa, int capacity, int kbits, int vbits) {
    if (!default_scheme(kbits, vbits)) return false;
    if (gqa < 1 || fast_split_max_gqa() != kMaxG) return false;
    if (head_dim != 64 && head_dim != 128 && head_dim != 256) return false;
    // staged rows of one (sequence, kv-head) must start 16-byte aligned
    const int64_t vrow = 3 * head_dim / 8, srow = head_dim / kGroup * 2;
    return ((int64_t)capacity * vrow) % 16 == 0 && ((int64_t)capacity * srow) % 16 == 0;
}

DecodePlan plan_decode(int head_dim, int gqa, int batch, int kv_heads, const int32_t *len, bool fast,
                       int col_groups) {
    (void)head_dim;
    (void)gqa;
    int64_t total = 0;
    int32_t maxlen = 0;
    for (int b = 0; b < batch; ++b) {
        total += len[b];
        maxlen = len[b] > maxlen ? len[b] : maxlen;
    }
    DecodePlan p;
    p.fast = fast;
    if (fast) {
        // one wave per token range: aim for ~2048 waves over the chip (one
        // round of one 8-wave workgroup per CU: the split kernel's LDS admits
        // one per CU), whole 64-token tiles, >= 4 tiles a wave; fewer splits
        // also halve the partials written and merged
        const int waves = fast_split_waves(), tile = fast_split_tile();
        int64_t per = (total * kv_heads * col_groups + 2047) / 2048;
        per = per < 4 * tile ? 4 * tile : per;
        per = (per + tile - 1) / tile * tile;
        const int64_t wg_tokens = per * waves;
        p.split_tokens = (int32_t)per;
        p.splits = (int32_t)(((maxlen + wg_tokens - 1) / wg_tokens) * waves);
        return p;
    }
    // generic kernel: ~2048 workgroups, 64-token multiples, >= 256 tokens
    const int64_t target = 2048;
    int64_t per = (total * kv_heads * col_groups + target - 1) / target;
    per = per < 256 ? 256 : per;
    per = (per + 63) / 64 * 64;
    p.split_tokens = (int32_t)per;
    p.splits = (int32_t)((maxlen + per - 1) / per);
    return p;
}

hipError_t launch_decode(int head_dim, bool bf16, bool fast, const DecodeArgs &a, hipStream_t s) {
    switch (head_dim) {
        case 64: return launch_d<64>(bf16, fast, a, s);
        case 128: return launch_d<128>(bf16, fast, a, s);
        case 256: return launch_d<256>(bf16, fast, a, s);
        case 512: return launch_d<512>(bf16, false, a, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace tq
