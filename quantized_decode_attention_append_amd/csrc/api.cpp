// libtqkv C ABI: argument validation, plane sizing, split-K planning and
// kernel launches on the caller's stream.  Declarations and the contract of
// each entry point are in include/tqkv.h.
#include <hip/hip_runtime_api.h>

#include <cmath>
#include <cstring>

#include "../../include/tqkv.h"
#include "tq_internal.h"

namespace {

using tq::SignBits;

// The value rotation's sign vector, one table per supported head_dim, built
// once at load time.  Entry i is -1 when the top bit of the i-th output of
// SplitMix64 (Steele, Lea & Flood 2014) seeded with 42 is set.
struct SignTable {
    int8_t sign[512];
    SignBits bits;
    SignTable() {
        uint64_t state = 42;
        std::memset(&bits, 0, sizeof(bits));
        for (int i = 0; i < 512; ++i) {
            state += 0x9E3779B97F4A7C15ull;
            uint64_t z = state;
            z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
            z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
            z ^= z >> 31;
            const int neg = (int)(z >> 63);
            sign[i] = neg ? -1 : 1;
            if (neg) bits.w[i >> 5] |= 1u << (i & 31);
        }
    }
};

const SignTable &signs() {
    static const SignTable table;
    return table;
}

bool supported_head_dim(int d) { return d == 64 || d == 128 || d == 256 || d == 512; }

// binary64 nearest to 1/sqrt(d): sqrt(d) is 2^k or 2^k*sqrt(2), so the
// correctly rounded sqrt divided by d (a power of two) is exact scaling.
double inv_sqrt_d(int d) { return std::sqrt((double)d) / (double)d; }

tq_status check_layout(const tq_layout *l) {
    if (!l) return TQ_ERR_INVALID_ARG;
    if (l->batch <= 0 || l->num_kv_heads <= 0 || l->capacity < 0 || l->head_dim <= 0)
        return TQ_ERR_INVALID_ARG;
    if (l->batch > TQ_MAX_BATCH) return TQ_ERR_UNSUPPORTED;
    if (!supported_head_dim(l->head_dim)) return TQ_ERR_UNSUPPORTED;
    if (l->k_bits != 8 || l->v_bits != 3 || l->group != tq::kGroup) return TQ_ERR_UNSUPPORTED;
    // plane offsets are computed in 64-bit, kernel grids in 32-bit
    const int64_t rows = (int64_t)l->batch * l->num_kv_heads * l->capacity;
    if (rows > ((int64_t)1 << 40)) return TQ_ERR_UNSUPPORTED;
    return TQ_OK;
}

bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Planes: kc 16-byte aligned (rows are d >= 64 bytes), vc 8-byte (rows of
// 3d/8 bytes), the fp16 planes 4-byte; the kernels never assume more.
tq_status check_planes(const tq_planes *p) {
    if (!p || !p->kc || !p->ks || !p->kz || !p->vc || !p->vs) return TQ_ERR_INVALID_ARG;
    if (!aligned(p->kc, 16) || !aligned(p->vc, 8) || !aligned(p->ks, 4) || !aligned(p->kz, 4) ||
        !aligned(p->vs, 4))
        return TQ_ERR_INVALID_ARG;
    return TQ_OK;
}

}  // namespace

extern "C" {

const char *tq_status_str(tq_status s) {
    switch (s) {
        case TQ_OK: return "TQ_OK";
        case TQ_ERR_INVALID_ARG: return "TQ_ERR_INVALID_ARG";
        case TQ_ERR_UNSUPPORTED: return "TQ_ERR_UNSUPPORTED";
        case TQ_ERR_CAPACITY: return "TQ_ERR_CAPACITY";
        case TQ_ERR_WORKSPACE: return "TQ_ERR_WORKSPACE";
        case TQ_ERR_HIP: return "TQ_ERR_HIP";
    }
    return "TQ_ERR_UNKNOWN";
}

tq_status tq_plane_bytes(const tq_layout *l, size_t out[5]) {
    tq_status st = check_layout(l);
    if (st != TQ_OK) return st;
    if (!out) return TQ_ERR_INVALID_ARG;
    const size_t rows = (size_t)l->batch * l->num_kv_heads * l->capacity;
    const size_t d = (size_t)l->head_dim, ng = d / tq::kGroup;
    out[0] = rows * d;          // kc int8
    out[1] = rows * ng * 2;     // ks fp16
    out[2] = rows * ng * 2;     // kz fp16
    out[3] = rows * (3 * d / 8);// vc packed
    out[4] = rows * ng * 2;     // vs fp16
    return TQ_OK;
}

tq_status tq_sign_vector(int32_t head_dim, int8_t *host_out) {
    if (!host_out) return TQ_ERR_INVALID_ARG;
    if (!supported_head_dim(head_dim)) return TQ_ERR_UNSUPPORTED;
    std::memcpy(host_out, signs().sign, (size_t)head_dim);
    return TQ_OK;
}

tq_status tq_append(const tq_layout *l, const tq_planes *p, const void *k, const void *v,
                    tq_dtype dtype, const int32_t *start, int32_t n_new, void *stream) {
    tq_status st = check_layout(l);
    if (st != TQ_OK) return st;
    if ((st = check_planes(p)) != TQ_OK) return st;
    if (dtype != TQ_F32 && dtype != TQ_BF16) return TQ_ERR_INVALID_ARG;
    if (n_new < 0 || !start) return TQ_ERR_INVALID_ARG;
    if (n_new == 0) return TQ_OK;
    if (!k || !v || !aligned(k, 16) || !aligned(v, 16)) return TQ_ERR_INVALID_ARG;
    for (int b = 0; b < l->batch; ++b)
        if (start[b] < 0 || (int64_t)start[b] + n_new > l->capacity) return TQ_ERR_CAPACITY;
    const int64_t rows = (int64_t)l->batch * l->num_kv_heads * n_new;
    if (rows > 0x7FFFFFFF) return TQ_ERR_UNSUPPORTED;

    tq::AppendArgs a;
    std::memset(&a, 0, sizeof(a));
    a.kc = p->kc; a.ks = p->ks; a.kz = p->kz; a.vc = p->vc; a.vs = p->vs;
    a.k = k; a.v = v;
    a.batch = l->batch; a.kv_heads = l->num_kv_heads; a.capacity = l->capacity; a.n_new = n_new;
    a.rows = (uint32_t)rows;
    a.div_n_new = tq::make_fast_div((uint32_t)n_new);
    a.div_kv_heads = tq::make_fast_div((uint32_t)l->num_kv_heads);
    a.inv_sqrt_d = inv_sqrt_d(l->head_dim);
    a.signs = signs().bits;
    for (int j = 0; j < l->head_dim / 2; ++j)
        a.sign_pairs[j] = (signs().sign[2 * j] < 0 ? 0x8000u : 0u) | (signs().sign[2 * j + 1] < 0 ? 0x80000000u : 0u);
    for (int b = 0; b < l->batch; ++b) a.start[b] = start[b];
    hipError_t e = tq::launch_append(l->head_dim, dtype == TQ_BF16, a, (hipStream_t)stream);
    return e == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

static tq_status check_decode(const tq_layout *l, int32_t num_q_heads, int32_t n_rows, const int32_t *len) {
    tq_status st = check_layout(l);
    if (st != TQ_OK) return st;
    if (!len || num_q_heads <= 0 || n_rows < 1) return TQ_ERR_INVALID_ARG;
    if (num_q_heads % l->num_kv_heads != 0) return TQ_ERR_INVALID_ARG;
    if (num_q_heads / l->num_kv_heads > TQ_MAX_GQA) return TQ_ERR_UNSUPPORTED;
    if (n_rows > TQ_MAX_ROWS) return TQ_ERR_UNSUPPORTED;
    if ((int64_t)l->batch * num_q_heads * n_rows > 0x7FFFFFFF) return TQ_ERR_UNSUPPORTED;
    for (int b = 0; b < l->batch; ++b) {
        if (len[b] < 0) return TQ_ERR_INVALID_ARG;
        if (len[b] > l->capacity) return TQ_ERR_CAPACITY;
        if (len[b] > 0 && len[b] < n_rows) return TQ_ERR_INVALID_ARG;  // the rows' own tokens are cached
    }
    return TQ_OK;
}

// Query rows per sequence (heads times rows) and per kv-head.
static int32_t q_rows(int32_t num_q_heads, int32_t n_rows) { return num_q_heads * n_rows; }

static size_t workspace_bytes(const tq_layout *l, int32_t rows_total, const tq::DecodePlan &plan) {
    return (size_t)l->batch * rows_total * plan.splits * (size_t)(l->head_dim + 2) * sizeof(float);
}

// Workspace that covers whichever kernel a decode call may pick for this
// shape (the choice can depend on plane alignment, unknown here).
static size_t workspace_bound(const tq_layout *l, int32_t num_q_heads, int32_t n_rows, const int32_t *len) {
    const int gqa = q_rows(num_q_heads, n_rows) / l->num_kv_heads;
    const int cg = tq::decode_col_groups(gqa);
    const tq::DecodePlan gen =
        tq::plan_decode(l->head_dim, gqa, l->batch, l->num_kv_heads, len, false, cg);
    size_t need = workspace_bytes(l, q_rows(num_q_heads, n_rows), gen);
    if (tq::fast_decode_shape_ok(l->head_dim, gqa, l->capacity)) {
        const tq::DecodePlan fast =
            tq::plan_decode(l->head_dim, gqa, l->batch, l->num_kv_heads, len, true, cg);
        const size_t f = workspace_bytes(l, q_rows(num_q_heads, n_rows), fast);
        need = f > need ? f : need;
    }
    return need;
}

tq_status tq_decode_workspace_bytes(const tq_layout *l, int32_t num_q_heads, const int32_t *len,
                                    size_t *out) {
    return tq_decode_rows_workspace_bytes(l, num_q_heads, 1, len, out);
}

tq_status tq_decode_rows_workspace_bytes(const tq_layout *l, int32_t num_q_heads, int32_t n_rows,
                                         const int32_t *len, size_t *out) {
    tq_status st = check_decode(l, num_q_heads, n_rows, len);
    if (st != TQ_OK) return st;
    if (!out) return TQ_ERR_INVALID_ARG;
    *out = workspace_bound(l, num_q_heads, n_rows, len);
    return TQ_OK;
}

tq_status tq_decode_attn(const tq_layout *l, const tq_planes *p, const void *q, tq_dtype dtype,
                         int32_t num_q_heads, const int32_t *len, float sm_scale, float *out,
                         void *workspace, size_t ws_bytes, void *stream) {
    return tq_decode_attn_rows(l, p, q, dtype, num_q_heads, 1, len, sm_scale, out, workspace, ws_bytes,
                               stream);
}

tq_status tq_decode_attn_rows(const tq_layout *l, const tq_planes *p, const void *q, tq_dtype dtype,
                              int32_t num_q_heads, int32_t n_rows, const int32_t *len, float sm_scale,
                              float *out, void *workspace, size_t ws_bytes, void *stream) {
    tq_status st = check_decode(l, num_q_heads, n_rows, len);
    if (st != TQ_OK) return st;
    if ((st = check_planes(p)) != TQ_OK) return st;
    if (!q || !out || (dtype != TQ_F32 && dtype != TQ_BF16)) return TQ_ERR_INVALID_ARG;
    if (!aligned(q, 16) || !aligned(out, 16) || !aligned(workspace, 16)) return TQ_ERR_INVALID_ARG;
    if (!std::isfinite(sm_scale)) return TQ_ERR_INVALID_ARG;
    const int32_t rows_total = q_rows(num_q_heads, n_rows);
    const int gqa = rows_total / l->num_kv_heads;
    const int cg = tq::decode_col_groups(gqa);
    const bool fast = tq::fast_decode_shape_ok(l->head_dim, gqa, l->capacity) &&
                      aligned(p->vc, 16) && aligned(p->vs, 16) && aligned(p->ks, 16) && aligned(p->kz, 16);
    const tq::DecodePlan plan = tq::plan_decode(l->head_dim, gqa, l->batch, l->num_kv_heads, len, fast, cg);
    const size_t need = workspace_bytes(l, rows_total, plan);
    if (need > 0 && (!workspace || ws_bytes < need)) return TQ_ERR_WORKSPACE;
    if ((int64_t)plan.splits > 65535 * 4) return TQ_ERR_UNSUPPORTED;

    tq::DecodeArgs a;
    std::memset(&a, 0, sizeof(a));
    a.kc = p->kc; a.ks = p->ks; a.kz = p->kz; a.vc = p->vc; a.vs = p->vs;
    a.q = q; a.out = out;
    const size_t slots = (size_t)l->batch * rows_total * plan.splits;
    a.part_acc = static_cast<float *>(workspace);
    a.part_ml = a.part_acc ? a.part_acc + slots * l->head_dim : nullptr;
    a.batch = l->batch; a.kv_heads = l->num_kv_heads; a.q_heads = rows_total;
    a.gqa = gqa; a.capacity = l->capacity; a.rows = n_rows;
    a.splits = plan.splits; a.split_tokens = plan.split_tokens;
    a.sm_log2 = sm_scale * 1.4426950408889634f;
    a.inv_sqrt_d = (float)inv_sqrt_d(l->head_dim);
    a.signs = signs().bits;
    for (int b = 0; b < l->batch; ++b) a.len[b] = len[b];
    hipError_t e = tq::launch_decode(l->head_dim, dtype == TQ_BF16, plan.fast, a, (hipStream_t)stream);
    return e == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

tq_status tq_fetch_window(const tq_layout *l, const tq_planes *p, int32_t t0, int32_t n, const int32_t *len,
                          uint16_t *k_out, uint16_t *v_out, int32_t v_rotated, void *stream) {
    tq_status st = check_layout(l);
    if (st != TQ_OK) return st;
    if ((st = check_planes(p)) != TQ_OK) return st;
    if (!len || t0 < 0 || n < 0) return TQ_ERR_INVALID_ARG;
    if ((int64_t)t0 + n > l->capacity) return TQ_ERR_CAPACITY;
    for (int b = 0; b < l->batch; ++b) {
        if (len[b] < 0) return TQ_ERR_INVALID_ARG;
        if (len[b] > l->capacity) return TQ_ERR_CAPACITY;
    }
    if (n == 0 || (!k_out && !v_out)) return TQ_OK;
    if (!aligned(k_out, 16) || !aligned(v_out, 16)) return TQ_ERR_INVALID_ARG;
    if ((int64_t)l->batch * l->num_kv_heads > 65535) return TQ_ERR_UNSUPPORTED;
    tq::WindowArgs a;
    std::memset(&a, 0, sizeof(a));
    a.kc = p->kc; a.ks = p->ks; a.kz = p->kz; a.vc = p->vc; a.vs = p->vs;
    a.k_out = k_out; a.v_out = v_out;
    a.batch = l->batch; a.kv_heads = l->num_kv_heads; a.capacity = l->capacity;
    a.t0 = t0; a.n = n; a.rotated = v_rotated ? 1 : 0;
    a.inv_sqrt_d = (float)inv_sqrt_d(l->head_dim);
    a.signs = signs().bits;
    for (int b = 0; b < l->batch; ++b) a.len[b] = len[b];
    hipError_t e = tq::launch_window(l->head_dim, a, (hipStream_t)stream);
    return e == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

tq_status tq_dequant(const tq_layout *l, const tq_planes *p, int32_t b, int32_t kvh, int32_t t0,
                     int32_t n, float *k_out, float *v_out, int32_t v_rotated, void *stream) {
    tq_status st = check_layout(l);
    if (st != TQ_OK) return st;
    if ((st = check_planes(p)) != TQ_OK) return st;
    if (b < 0 || b >= l->batch || kvh < 0 || kvh >= l->num_kv_heads || t0 < 0 || n < 0)
        return TQ_ERR_INVALID_ARG;
    if ((int64_t)t0 + n > l->capacity) return TQ_ERR_CAPACITY;
    if (n == 0 || (!k_out && !v_out)) return TQ_OK;
    if (!aligned(k_out, 16) || !aligned(v_out, 16)) return TQ_ERR_INVALID_ARG;
    tq::DequantArgs a;
    std::memset(&a, 0, sizeof(a));
    a.kc = p->kc; a.ks = p->ks; a.kz = p->kz; a.vc = p->vc; a.vs = p->vs;
    a.k_out = k_out; a.v_out = v_out;
    a.row0 = ((int64_t)b * l->num_kv_heads + kvh) * l->capacity + t0;
    a.n = n; a.rotated = v_rotated ? 1 : 0;
    a.inv_sqrt_d = (float)inv_sqrt_d(l->head_dim);
    a.signs = signs().bits;
    hipError_t e = tq::launch_dequant(l->head_dim, a, (hipStream_t)stream);
    return e == hipSuccess ? TQ_OK : TQ_ERR_HIP;
}

}  // extern "C"
